"""Oracle of the int8 cache ("10.3 - KV cache implementation details", section 4.4) against hand-worked
rows, invariants, a closed form and planted mistakes.

The hand rows are chosen so every binary32 step is exact, so the expected codes follow from the
definition on paper: amax / 127 is the scale, x * (127 / amax) rounded half to even is the code.
"""

import numpy as np
import pytest

from oracle import attention as att
from oracle import cache_bytes as cb
from oracle import quant


def bf16_bits(values):
    """float values exactly representable in bf16 -> their bf16 bit patterns."""
    f = np.asarray(values, dtype=np.float32)
    bits = f.view(np.uint32)
    assert not np.any(bits & np.uint32(0xFFFF)), "value not exact in bf16"
    return (bits >> np.uint32(16)).astype(np.uint16)


# (row, expected codes, expected scale), worked by hand:
HAND = [
    # amax 127: 127/amax = 1, codes = x rounded half to even (-63.5 -> -64, 2.5 -> 2, -0.5 -> 0, 3.5 -> 4)
    ([127, -63.5, 2.5, -0.5, 3.5, 0, 1, -127], [127, -64, 2, 0, 4, 0, 1, -127], 1.0),
    # amax 254: 127/amax = 0.5; 1 -> 0.5 -> 0, 3 -> 1.5 -> 2, -5 -> -2.5 -> -2
    ([254, 1, 3, -5, 0, 0, 0, 0], [127, 0, 2, -2, 0, 0, 0, 0], 2.0),
    # amax 8: 127/8 = 15.875; 4 -> 63.5 -> 64, 2 -> 31.75 -> 32, 0.125 -> 1.984375 -> 2
    ([-8, 4, 2, 1, 0.5, 0.25, 0.125, 0], [-127, 64, 32, 16, 8, 4, 2, 0], np.float32(8) / np.float32(127)),
    # zeros: scale 0, codes 0
    ([0, 0, 0, 0, 0, 0, 0, 0], [0] * 8, 0.0),
]


@pytest.mark.parametrize("as_bits", [False, True])
def test_hand_rows(as_bits):
    rows = np.array([r for r, _, _ in HAND], dtype=np.float32)
    x = bf16_bits(rows) if as_bits else rows
    codes, scale = quant.quantize_rows(x)
    assert codes.dtype == np.int8 and scale.dtype == np.float32
    assert codes.tolist() == [c for _, c, _ in HAND]
    assert scale.tolist() == [float(np.float32(s)) for _, _, s in HAND]
    # dequantised values of the first two rows, by hand
    deq = quant.dequantize(codes, scale)
    assert deq[0].tolist() == [127, -64, 2, 0, 4, 0, 1, -127]
    assert deq[1].tolist() == [254, 0, 4, -4, 0, 0, 0, 0]


def test_row_wise_not_column_wise():
    """Each row has its own scale: a large row does not coarsen a small one."""
    x = np.array([[1000, 1, 2, 3], [0.5, 0.25, -0.5, 0.125]], dtype=np.float32)
    codes, scale = quant.quantize_rows(x)
    assert codes[1].tolist() == [127, 64, -127, 32]  # 0.25 * 254 = 63.5 -> 64; 0.125 * 254 = 31.75 -> 32
    assert scale[1] == np.float32(0.5) / np.float32(127)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_invariants_random(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((64, 128)) * rng.uniform(1e-3, 1e3, size=(64, 1))).astype(np.float32)
    x[5] = 0.0
    codes, scale = quant.quantize_rows(x)
    c = codes.astype(np.int64)
    assert np.all(np.abs(c) <= 127)
    amax = np.abs(x).max(axis=1)
    assert np.array_equal(scale, (amax / np.float32(127)).astype(np.float32))
    # the largest element of every non-zero row is +-127 with its sign
    i = np.abs(x).argmax(axis=1)
    nz = amax > 0
    assert np.all(c[np.arange(64), i][nz] == 127 * np.sign(x[np.arange(64), i][nz]))
    # signs agree, and the error is at most half a step (plus binary32 rounding of the scale)
    assert np.all(c * np.sign(x) >= 0)
    err = np.abs(x.astype(np.float64) - quant.dequantize(codes, scale))
    assert np.all(err <= scale[:, None].astype(np.float64) * (0.5 + 1e-5))
    assert not codes[5].any() and scale[5] == 0


def test_cache_fill_append_semantics():
    L, B, Hkv, S, D = 2, 3, 2, 6, 8
    cache = quant.RefQuantCache(L, B, Hkv, S, D)
    assert not cache.codes.any() and not cache.scales.any()
    hand = np.array([r for r, _, _ in HAND], dtype=np.float32)          # [4, 8]
    k = bf16_bits(np.broadcast_to(hand[None, None, :3], (B, Hkv, 3, D)))  # rows A, B, C of HAND
    v = bf16_bits(np.broadcast_to(-hand[None, None, :3], (B, Hkv, 3, D)))
    cache.fill(1, k, v, 2)
    assert cache.codes[1, 0, 2, 1, 3].tolist() == HAND[1][1]
    assert cache.codes[1, 1, 0, 0, 4].tolist() == [-c for c in HAND[2][1]]
    assert cache.scales[1, 0, 1, 1, 2] == np.float32(1.0) and cache.scales[1, 1, 0, 0, 3] == np.float32(2.0)
    assert not cache.codes[0].any() and not cache.codes[1, :, :, :, :2].any() and not cache.codes[1, :, :, :, 5:].any()
    # append one row per sequence; b = 1 is out of range and left untouched
    before = cache.codes.copy(), cache.scales.copy()
    kn = bf16_bits(np.broadcast_to(hand[None, None, 0:1], (B, Hkv, 1, D)))
    vn = bf16_bits(np.broadcast_to(hand[None, None, 1:2], (B, Hkv, 1, D)))
    skipped = cache.append(1, kn, vn, np.array([0, 6, 5]))
    assert skipped == [1]
    assert cache.codes[1, 0, 0, :, 0].tolist() == [HAND[0][1]] * Hkv
    assert cache.codes[1, 1, 2, :, 5].tolist() == [HAND[1][1]] * Hkv
    assert np.array_equal(cache.codes[:, :, 1], before[0][:, :, 1]) and np.array_equal(cache.scales[:, :, 1], before[1][:, :, 1])
    changed = np.argwhere(np.any(cache.codes != before[0], axis=-1) | (cache.scales != before[1]))
    assert {tuple(x) for x in changed.tolist()} <= {(1, kv, b, g, r) for kv in (0, 1) for b, r in ((0, 0), (2, 5)) for g in range(Hkv)}
    # keys() are the dequantised codes
    assert cache.keys(1)[0, 0, 0].tolist() == [127, -64, 2, 0, 4, 0, 1, -127]
    assert cache.values(1)[2, 1, 5].tolist() == [254, 0, 4, -4, 0, 0, 0, 0]


def test_decode_closed_form():
    """Equal keys give equal weights: the output is the plain mean of the dequantised values."""
    B, Hkv, S, D, H = 1, 1, 4, 8, 2
    cache = quant.RefQuantCache(1, B, Hkv, S, D)
    hand = np.array([r for r, _, _ in HAND], dtype=np.float32)
    k = bf16_bits(np.broadcast_to(hand[None, None, 0:1], (B, Hkv, 2, D)))
    v = bf16_bits(hand[None, None, 0:2])
    cache.fill(0, k, v, 0)
    q = bf16_bits(np.array([[[1, 0, 0, 0, 0, 0, 0, 0], [0, 0.5, 0, 0, 0, 0, 0, 0]]], dtype=np.float32))
    out = att.decode_attention(q, cache.keys(0), cache.values(0), [2], 0.125)
    want = [(a + b) / 2 for a, b in zip([127, -64, 2, 0, 4, 0, 1, -127], [254, 0, 4, -4, 0, 0, 0, 0])]
    assert np.allclose(out[0, 0], want, rtol=0, atol=1e-12) and np.allclose(out[0, 1], want, rtol=0, atol=1e-12)


def test_int8_cache_bytes():
    """Codes at p_cache = 1 (section 4.4) plus a 4-byte scale per cached row of K and of V."""
    codes = cb.kv_cache_bytes(32, 8, 128, 4096, 16, 1)
    assert codes * 2 == cb.kv_cache_bytes(32, 8, 128, 4096, 16, 2)
    assert quant.int8_cache_bytes(32, 8, 128, 4096, 16) == codes + 2 * 32 * 8 * 4096 * 16 * 4
    assert quant.int8_cache_bytes(1, 1, 8, 6, 3) == 2 * 6 * 3 * (8 + 4)


# ---- planted mistakes: each must be caught by the hand rows ----------------

def _mutant(flaw):
    def q(x):
        x = quant._to_f32(x)
        amax = np.max(np.abs(x), axis=-1)
        zero = amax == 0
        safe = np.where(zero, np.float32(1), amax)
        levels = np.float32(255 if flaw == "levels_255" else 127)
        axis_max = np.max(np.abs(x), axis=0, keepdims=True) if flaw == "column_scale" else None
        inv = (levels / safe).astype(np.float32)
        s = x * (inv[..., None] if axis_max is None else (levels / np.where(axis_max == 0, 1, axis_max)))
        if flaw == "half_away":
            c = np.sign(s) * np.floor(np.abs(s) + 0.5)
        elif flaw == "truncate":
            c = np.trunc(s)
        else:
            c = np.rint(s)
        c = np.clip(c, -127, 127)
        c = np.where(zero[..., None], 0, c).astype(np.int8)
        return c, np.where(zero, 0, amax / levels).astype(np.float32)
    return q


@pytest.mark.parametrize("flaw", ["levels_255", "column_scale", "half_away", "truncate"])
def test_pins_catch_planted_mistakes(flaw, monkeypatch):
    monkeypatch.setattr(quant, "quantize_rows", _mutant(flaw))
    with pytest.raises(AssertionError):
        test_hand_rows(False)
