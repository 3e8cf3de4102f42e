"""Oracle buffer model against a brute-force element-by-element model."""

import numpy as np
import pytest

from oracle import cache_bytes as cb
from oracle.buffer import RefCache, RefLatentCache
from static_kv_cache_amd import synthetic


def _brute(shape, ops):
    """Dict of element writes keyed by (l, kv, b, g, s, d); unspecified = 0."""
    mem = {}
    L, _, B, Hkv, S, D = shape
    for op in ops:
        if op[0] == "fill":
            _, l, k, v, start = op
            for b in range(B):
                for g in range(Hkv):
                    for i in range(k.shape[2]):
                        for d in range(D):
                            mem[(l, 0, b, g, start + i, d)] = int(k[b, g, i, d])
                            mem[(l, 1, b, g, start + i, d)] = int(v[b, g, i, d])
        else:
            _, l, k, v, ci = op
            for b in range(B):
                c = int(ci[b])
                if c < 0 or c + k.shape[2] > S:
                    continue
                for g in range(Hkv):
                    for i in range(k.shape[2]):
                        for d in range(D):
                            mem[(l, 0, b, g, c + i, d)] = int(k[b, g, i, d])
                            mem[(l, 1, b, g, c + i, d)] = int(v[b, g, i, d])
    out = np.zeros(shape, dtype=np.int64)
    for key, val in mem.items():
        out[key] = val
    return out


@pytest.mark.parametrize("storage", ["bf16", "f32"])
def test_fill_append_matches_brute_force(storage):
    rng = np.random.default_rng(21)
    L, B, Hkv, S, D = 2, 3, 2, 6, 4
    cache = RefCache(L, B, Hkv, S, D, storage)
    assert cache.buf.nbytes == cb.kv_cache_bytes(L, Hkv, D, S, B, 2 if storage == "bf16" else 4)

    def bits(shape):
        x = synthetic.draw(rng, shape, storage)
        return x.view(np.uint32) if storage == "f32" else x

    ops = [("fill", 1, bits((B, Hkv, 3, D)), bits((B, Hkv, 3, D)), 0),
           ("append", 1, bits((B, Hkv, 1, D)), bits((B, Hkv, 1, D)), np.array([3, 5, 6])),  # b=2 out of range
           ("append", 0, bits((B, Hkv, 2, D)), bits((B, Hkv, 2, D)), np.array([0, 4, -1])),  # b=2 negative
           ("fill", 0, bits((B, Hkv, 1, D)), bits((B, Hkv, 1, D)), 5)]
    for op in ops:
        if op[0] == "fill":
            cache.fill(op[1], op[2], op[3], op[4])
        else:
            skipped = cache.append(op[1], op[2], op[3], op[4])
            assert skipped == [2]
    assert np.array_equal(cache.buf.astype(np.int64), _brute(cache.shape, ops))


def test_fill_rejects_capacity_overflow():
    cache = RefCache(1, 1, 1, 4, 2, "bf16")
    with pytest.raises(ValueError):
        cache.fill(0, np.zeros((1, 1, 3, 2), np.uint16), np.zeros((1, 1, 3, 2), np.uint16), 2)
    assert not cache.buf.any()


def test_latent_cache_rows():
    rng = np.random.default_rng(22)
    L, B, S, W = 1, 2, 5, 6
    c = RefLatentCache(L, B, S, W, "bf16")
    assert c.buf.nbytes == cb.mla_cache_bytes(L, W, S, B, 2)
    rows = synthetic.draw(rng, (B, 4, W), "bf16")
    c.fill(0, rows, 0)
    new = synthetic.draw(rng, (B, 1, W), "bf16")
    assert c.append(0, new, np.array([4, 5])) == [1]
    assert np.array_equal(c.buf[0, 0, :4], rows[0]) and np.array_equal(c.buf[0, 0, 4], new[0, 0])
    assert np.array_equal(c.buf[0, 1, :4], rows[1]) and not c.buf[0, 1, 4].any()
