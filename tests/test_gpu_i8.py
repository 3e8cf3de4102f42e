"""int8 cache (dtype "i8", "10.3 - KV cache implementation details" section 4.4) on the GPU.

* Quantisation at fill and append gives the oracle's codes and scales bit for bit: both sides decide
  a code in binary32 (amax / 127, x * (127 / amax) rounded half to even).
* Decode attention matches the oracle's attention over the dequantised rows (code * scale, float64)
  within the bf16 bound of the parity tests (q, out and the P operand are bf16).
* Rows past the valid length never matter; out-of-range appends are skipped and flagged.
* The fused append-decode call quantises the new rows in the kernel: its output bits, codes and
  scales equal those of kvc_append followed by kvc_decode_attn.
"""

import numpy as np
import pytest
import torch

from gpu_util import bits_of, device, say, to_f64, tol_check
from oracle import attention as oatt
from oracle.quant import RefQuantCache
from static_kv_cache_amd import kvc, synthetic

pytestmark = pytest.mark.gpu


def varied_rows(rng, shape):
    """bf16 bits of N(0,1) rows with per-row magnitudes from 1e-3 to 1e3, a few zero rows,
    and a few rows built from exact ties (x * 127 / amax lands on .5)."""
    x = rng.standard_normal(shape, dtype=np.float32)
    mag = (10.0 ** rng.uniform(-3, 3, size=shape[:-1] + (1,))).astype(np.float32)
    x = (x * mag).astype(np.float32)
    flat = x.reshape(-1, shape[-1])
    n = flat.shape[0]
    for r in range(0, n, 7):
        flat[r] = 0.0
    for r in range(3, n, 11):  # amax 254: every odd integer element is a tie at x * 0.5
        flat[r] = rng.integers(-254, 255, size=shape[-1]).astype(np.float32)
        flat[r, 0] = 254.0
    return synthetic.f32_to_bf16_bits(x)


def codes_scales(cache, layer):
    k, v = cache.layer_tensors(layer)
    ks, vs = cache.layer_scales(layer)
    return (k.cpu().numpy(), v.cpu().numpy(), ks.cpu().numpy(), vs.cpu().numpy())


def assert_same_as_ref(cache, layer, ref, rl=0):
    k, v, ks, vs = codes_scales(cache, layer)
    assert np.array_equal(k, ref.codes[rl, 0]), "K codes differ from the oracle"
    assert np.array_equal(v, ref.codes[rl, 1]), "V codes differ from the oracle"
    assert np.array_equal(ks.view(np.uint32), ref.scales[rl, 0].view(np.uint32)), "K scales differ"
    assert np.array_equal(vs.view(np.uint32), ref.scales[rl, 1].view(np.uint32)), "V scales differ"


@pytest.mark.parametrize("D", [64, 128, 256])
def test_fill_and_append_bit_exact(D):
    dev = device()
    rng = np.random.default_rng(100 + D)
    L, B, Hkv, S, T = 2, 5, 3, 40, 17
    say(f"i8 fill/append: D={D}")
    cache = kvc.Cache(kvc.gqa_desc(L, B, 2 * Hkv, Hkv, D, S, "i8"))
    ref = RefQuantCache(1, B, Hkv, S, D)
    k, v = varied_rows(rng, (B, Hkv, T, D)), varied_rows(rng, (B, Hkv, T, D))
    cache.prefill_fill(1, kvc.to_device(k, dev), kvc.to_device(v, dev), 4)
    ref.fill(0, k, v, 4)
    assert_same_as_ref(cache, 1, ref)
    # append two rows per sequence at per-sequence positions; b = 3 is out of range
    ci = np.array([0, 21, S - 2, S - 1, 30], dtype=np.int32)
    kn, vn = varied_rows(rng, (B, Hkv, 2, D)), varied_rows(rng, (B, Hkv, 2, D))
    cache.append(1, kvc.to_device(kn, dev), kvc.to_device(vn, dev), kvc.to_device(ci, dev))
    skipped = ref.append(0, kn, vn, ci)
    assert skipped == [3]
    assert cache.check_status() == kvc.KVC_ERR_DEVICE_RANGE
    assert_same_as_ref(cache, 1, ref)
    # layer 0 untouched
    k0, v0, ks0, vs0 = codes_scales(cache, 0)
    assert not k0.any() and not v0.any() and not ks0.any() and not vs0.any()
    cache.free()


SHAPES = [  # (B, H, Hkv, D, S)
    (3, 32, 8, 128, 600),
    (2, 64, 2, 128, 300),    # 32 heads per kv head: two head chunks
    (4, 8, 8, 64, 130),      # MHA
    (2, 16, 1, 256, 90),     # MQA, widest rows
    (5, 4, 4, 64, 70),
]


def run_decode(dev, case, B, H, Hkv, D, S, workgroups=None):
    cache = kvc.Cache(kvc.gqa_desc(1, B, H, Hkv, D, S, "i8"))
    if workgroups is not None:
        cache.set_workgroups(workgroups)
    cache.prefill_fill(0, kvc.to_device(case["k_fill"], dev), kvc.to_device(case["v_fill"], dev), 0)
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    cache.decode_attn(0, kvc.to_device(case["q"], dev), out, valid_lens=kvc.to_device(case["valid_lens"], dev),
                      sm_scale=case["sm_scale"])
    status = cache.check_status()
    cache.free()
    return out, status


def oracle_for(case, B, Hkv, D, S):
    ref = RefQuantCache(1, B, Hkv, S, D)
    ref.fill(0, case["k_fill"], case["v_fill"], 0)
    return oatt.decode_attention(case["q"], ref.keys(0), ref.values(0), case["valid_lens"], case["sm_scale"])


@pytest.mark.parametrize("B,H,Hkv,D,S", SHAPES)
def test_decode_matches_oracle_ragged(B, H, Hkv, D, S):
    dev = device()
    lens = [S, 1, 0, S // 2 + 3, 17][:B]
    say(f"i8 decode: B={B} H={H} Hkv={Hkv} D={D} S={S} lens={lens}")
    case = synthetic.random_gqa_case(S + D + H, B, H, Hkv, D, S, "i8", valid_lens=lens)
    out, status = run_decode(dev, case, B, H, Hkv, D, S)
    assert status == kvc.KVC_OK
    want = oracle_for(case, B, Hkv, D, S)
    err = tol_check(to_f64(out), want, "bf16", "i8 decode")
    say(f"  max abs err {err:.3e}")
    for b, n in enumerate(lens):
        if n == 0:
            assert not to_f64(out)[b].any(), "an empty sequence must give zeros"


@pytest.mark.parametrize("workgroups", [1, 7, 333, 2048])
def test_decode_grid_invariance_within_bound(workgroups):
    dev = device()
    B, H, Hkv, D, S = 3, 16, 4, 128, 1000
    case = synthetic.random_gqa_case(77, B, H, Hkv, D, S, "i8", valid_lens=[1000, 333, 65])
    say(f"i8 workgroups={workgroups}")
    out, status = run_decode(dev, case, B, H, Hkv, D, S, workgroups)
    assert status == kvc.KVC_OK
    tol_check(to_f64(out), oracle_for(case, B, Hkv, D, S), "bf16", f"workgroups {workgroups}")


def test_rows_past_valid_length_do_not_matter():
    dev = device()
    B, H, Hkv, D, S = 2, 8, 2, 128, 256
    case = synthetic.random_gqa_case(5, B, H, Hkv, D, S, "i8", valid_lens=[100, 37])
    big = dict(case)
    for key in ("k_fill", "v_fill"):
        x = synthetic.f32_to_bf16_bits(np.full(case[key].shape, 3.0e4, dtype=np.float32))
        x[:, :, :100] = case[key][:, :, :100]
        big[key] = x
    a, _ = run_decode(dev, case, B, H, Hkv, D, S)
    b, _ = run_decode(dev, big, B, H, Hkv, D, S)
    # sequence 1 attends 37 rows: rows 37..99 differ between the two caches only past its length
    big2 = dict(big)
    for key in ("k_fill", "v_fill"):
        x = big[key].copy()
        x[1, :, :37] = case[key][1, :, :37]
        big2[key] = x
    c, _ = run_decode(dev, big2, B, H, Hkv, D, S)
    assert np.array_equal(bits_of(a, "bf16"), bits_of(b, "bf16"))
    assert np.array_equal(bits_of(a, "bf16")[1], bits_of(c, "bf16")[1])


def test_single_row_is_the_dequantised_row():
    """n = 1: the output is the single row's dequantised values, rounded to bf16."""
    dev = device()
    B, H, Hkv, D, S = 2, 4, 2, 64, 8
    case = synthetic.random_gqa_case(9, B, H, Hkv, D, S, "i8", valid_lens=[1, 1])
    out, _ = run_decode(dev, case, B, H, Hkv, D, S)
    want = oracle_for(case, B, Hkv, D, S)
    # the oracle's value is code * scale exactly; the device result is that value through a bf16 P
    # operand of 1 * scale_v, so it equals bf16(code * bf16(scale_v)) up to one bf16 rounding
    tol_check(to_f64(out), want, "bf16", "n = 1")


def test_append_then_decode_step_on_device():
    dev = device()
    B, H, Hkv, D, S = 3, 8, 2, 128, 64
    case = synthetic.random_gqa_case(21, B, H, Hkv, D, S, "i8", valid_lens=[10, 30, 64])
    cache = kvc.Cache(kvc.gqa_desc(1, B, H, Hkv, D, S, "i8"))
    ref = RefQuantCache(1, B, Hkv, S, D)
    cache.prefill_fill(0, kvc.to_device(case["k_fill"], dev), kvc.to_device(case["v_fill"], dev), 0)
    ref.fill(0, case["k_fill"], case["v_fill"], 0)
    ci = np.array([9, 29, 63], dtype=np.int32)
    cache.append(0, kvc.to_device(case["k_new"], dev), kvc.to_device(case["v_new"], dev), kvc.to_device(ci, dev))
    ref.append(0, case["k_new"], case["v_new"], ci)
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    cache.decode_attn(0, kvc.to_device(case["q"], dev), out, cache_index=kvc.to_device(ci, dev),
                      sm_scale=case["sm_scale"])
    assert cache.check_status() == kvc.KVC_OK
    assert_same_as_ref(cache, 0, ref)
    want = oatt.decode_attention(case["q"], ref.keys(0), ref.values(0), ci + 1, case["sm_scale"])
    tol_check(to_f64(out), want, "bf16", "append then decode")
    cache.free()


def garbage_case(seed, B, H, Hkv, D, S, ci):
    """Rows from each sequence's new row on hold large finite garbage (3e4): the new row must come
    from k_new / v_new, and nothing past it may be attended."""
    case = synthetic.random_gqa_case(seed, B, H, Hkv, D, S, "i8", valid_lens=np.maximum(np.asarray(ci) + 1, 1))
    case["cache_index"] = np.asarray(ci, dtype=np.int32)
    junk = synthetic.f32_to_bf16_bits(np.float32(3.0e4))
    for b, c in enumerate(ci):
        if 0 <= c < S:
            case["k_fill"][b, :, c:] = junk
            case["v_fill"][b, :, c:] = junk
    return case


def two_ways(dev, case, B, H, Hkv, D, S, workgroups=None):
    """(fused out bits, its codes/scales, separate out bits, its codes/scales, statuses, fused out f64)."""
    res = []
    for fused in (True, False):
        cache = kvc.Cache(kvc.gqa_desc(1, B, H, Hkv, D, S, "i8"))
        if workgroups is not None:
            cache.set_workgroups(workgroups)
        cache.prefill_fill(0, kvc.to_device(case["k_fill"], dev), kvc.to_device(case["v_fill"], dev), 0)
        kn, vn = kvc.to_device(case["k_new"], dev), kvc.to_device(case["v_new"], dev)
        q, ci = kvc.to_device(case["q"], dev), kvc.to_device(case["cache_index"], dev)
        out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
        if fused:
            cache.append_decode_attn(0, kn, vn, q, out, ci, case["sm_scale"])
        else:
            cache.append(0, kn, vn, ci)
            cache.decode_attn(0, q, out, cache_index=ci, sm_scale=case["sm_scale"])
        status = cache.check_status()
        res.append((bits_of(out, "bf16"), codes_scales(cache, 0), status, to_f64(out)))
        cache.free()
    return res


def same_codes(a, b):
    return all(np.array_equal(x.view(np.uint8) if x.dtype == np.int8 else x.view(np.uint32),
                              y.view(np.uint8) if y.dtype == np.int8 else y.view(np.uint32)) for x, y in zip(a, b))


FUSED_SHAPES = [(3, 32, 8, 128, 600), (2, 64, 2, 128, 300), (4, 8, 8, 64, 130), (2, 16, 1, 256, 90)]


@pytest.mark.parametrize("B,H,Hkv,D,S", FUSED_SHAPES)
def test_fused_equals_append_then_decode(B, H, Hkv, D, S):
    dev = device()
    ci = [0, S - 1, S // 2, 16][:B]
    say(f"i8 fused: B={B} H={H} Hkv={Hkv} D={D} S={S} ci={ci}")
    case = garbage_case(S + D + H, B, H, Hkv, D, S, ci)
    (fo, fc, fs, fout), (so, sc, ss, _) = two_ways(dev, case, B, H, Hkv, D, S)
    assert fs == ss == kvc.KVC_OK
    assert same_codes(fc, sc), "codes or scales differ from append + decode"
    assert np.array_equal(fo, so), "output bits differ from append + decode"
    ref = RefQuantCache(1, B, Hkv, S, D)
    ref.fill(0, case["k_fill"], case["v_fill"], 0)
    ref.append(0, case["k_new"], case["v_new"], case["cache_index"])
    want = oatt.decode_attention(case["q"], ref.keys(0), ref.values(0), np.asarray(ci) + 1, case["sm_scale"])
    tol_check(fout, want, "bf16", "i8 fused")


@pytest.mark.parametrize("workgroups", [1, 7, 333])
def test_fused_grid_invariance(workgroups):
    dev = device()
    B, H, Hkv, D, S = 3, 16, 4, 128, 1000
    case = garbage_case(91, B, H, Hkv, D, S, [999, 332, 16])
    say(f"i8 fused workgroups={workgroups}")
    (fo, fc, _, _), (so, sc, _, _) = two_ways(dev, case, B, H, Hkv, D, S, workgroups)
    assert np.array_equal(fo, so) and same_codes(fc, sc)


def test_fused_out_of_range_is_skipped_and_flagged():
    dev = device()
    B, H, Hkv, D, S = 3, 8, 2, 64, 50
    case = synthetic.random_gqa_case(92, B, H, Hkv, D, S, "i8", valid_lens=[10, 1, 1])
    case["cache_index"] = np.array([9, -1, S], dtype=np.int32)
    (fo, fc, fs, fout), (so, sc, ss, _) = two_ways(dev, case, B, H, Hkv, D, S)
    assert fs == kvc.KVC_ERR_DEVICE_RANGE
    assert same_codes(fc, sc), "skipped sequences must be left untouched"
    assert not fout[1:].any(), "skipped sequences give zeros"
    assert np.array_equal(fo[0], so[0])


def test_llama3_8b_shape_full_size():
    """Llama-3-8B-shaped int8 cache at full size (B=16, H=32, H_kv=8, d_h=128, S=4096,
    valid_len ~ U[1024, 4096]): codes and scales bit-exact, every (b, h) output within the bound."""
    dev = device()
    cfg = synthetic.WORKLOADS["llama3_8b_gqa_i8"]
    B, H, Hkv, D, S = cfg["batch"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["max_context"]
    say(f"llama3_8b_gqa_i8: {cfg}")
    cache = kvc.Cache(kvc.gqa_desc(2, B, H, Hkv, D, S, "i8"))
    c = synthetic.gqa_layer(cfg, seed_offset=1)
    ref = RefQuantCache(1, B, Hkv, S, D)
    cache.prefill_fill(1, kvc.to_device(c["k_fill"], dev), kvc.to_device(c["v_fill"], dev), 0)
    ref.fill(0, c["k_fill"], c["v_fill"], 0)
    ci = kvc.to_device(c["cache_index"], dev)
    cache.append(1, kvc.to_device(c["k_new"], dev), kvc.to_device(c["v_new"], dev), ci)
    ref.append(0, c["k_new"], c["v_new"], c["cache_index"])
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    cache.decode_attn(1, kvc.to_device(c["q"], dev), out, valid_lens=kvc.to_device(c["valid_lens"], dev),
                      sm_scale=c["sm_scale"])
    cache.check()
    assert_same_as_ref(cache, 1, ref)
    want = oatt.decode_attention(c["q"], ref.keys(0), ref.values(0), c["valid_lens"], c["sm_scale"])
    err = tol_check(to_f64(out), want, "bf16", "llama3 i8")
    say(f"  max abs err {err:.3e}")
    cache.free()
