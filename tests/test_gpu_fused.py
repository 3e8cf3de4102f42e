"""kvc_append_decode_attn (append and decode in one launch) on the GPU.

The fused call must give exactly what kvc_append followed by kvc_decode_attn
gives: the same output bits and the same cache bytes, whatever the cache held
at the appended row before (NaN garbage there and past it included), and the
oracle's result within the usual bound. Out-of-range positions are skipped
and flagged as by kvc_append.
"""

import numpy as np
import pytest
import torch

from gpu_util import bits_of, device, oracle_decode, say, to_f64, tol_check
from oracle.buffer import RefCache
from static_kv_cache_amd import kvc, synthetic

pytestmark = pytest.mark.gpu

NAN = {"bf16": np.uint16(0x7FC0), "f32": np.float32(np.nan)}


def garbage_case(seed, B, H, Hkv, D, S, dtype, ci):
    case = synthetic.random_gqa_case(seed, B, H, Hkv, D, S, dtype, valid_lens=np.maximum(np.asarray(ci) + 1, 1))
    case["cache_index"] = np.asarray(ci, dtype=np.int32)
    for b, c in enumerate(ci):
        if 0 <= c < S:
            case["k_fill"][b, :, c:] = NAN[dtype]   # the appended row and everything past it
            case["v_fill"][b, :, c:] = NAN[dtype]
    return case


def two_ways(dev, case, dtype, workgroups=None):
    """(fused out, fused cache layer, separate out, separate cache layer)."""
    B, Hkv, S, D = case["k_fill"].shape
    H = case["q"].shape[1]
    res = []
    for fused in (True, False):
        cache = kvc.Cache(kvc.gqa_desc(1, B, H, Hkv, D, S, dtype))
        if workgroups is not None:
            cache.set_workgroups(workgroups)
        cache.prefill_fill(0, kvc.to_device(case["k_fill"], dev), kvc.to_device(case["v_fill"], dev), 0)
        kn, vn = kvc.to_device(case["k_new"], dev), kvc.to_device(case["v_new"], dev)
        q, ci = kvc.to_device(case["q"], dev), kvc.to_device(case["cache_index"], dev)
        out = torch.empty((B, H, D), dtype=kvc.torch_dtype(dtype), device=dev)
        if fused:
            cache.append_decode_attn(0, kn, vn, q, out, ci, case["sm_scale"])
        else:
            cache.append(0, kn, vn, ci)
            cache.decode_attn(0, q, out, cache_index=ci, sm_scale=case["sm_scale"])
        status = cache.check_status()
        k, v = cache.layer_tensors(0)
        res.append((bits_of(out, dtype), bits_of(k, dtype), bits_of(v, dtype), status, to_f64(out)))
        cache.free()
    return res


SHAPES = [
    ("bf16", 3, 32, 8, 128, 600),
    ("bf16", 2, 64, 2, 128, 300),   # 32 heads per kv head: two head chunks
    ("bf16", 4, 8, 8, 64, 130),
    ("bf16", 2, 16, 1, 256, 90),
    ("f32", 3, 8, 2, 128, 200),
    ("f32", 2, 4, 4, 32, 70),
]


@pytest.mark.parametrize("dtype,B,H,Hkv,D,S", SHAPES)
def test_fused_equals_append_then_decode(dtype, B, H, Hkv, D, S):
    dev = device()
    ci = [0, S - 1, S // 2, 16, 15, 63][:B]
    say(f"fused: {dtype} B={B} H={H} Hkv={Hkv} D={D} S={S} ci={ci}")
    case = garbage_case(S + D + H, B, H, Hkv, D, S, dtype, ci)
    (fo, fk, fv, fs, fout), (so, sk, sv, ss, sout) = two_ways(dev, case, dtype)
    assert fs == ss == kvc.KVC_OK
    assert np.array_equal(fk, sk) and np.array_equal(fv, sv), "cache bytes differ"
    assert np.array_equal(fo, so), "output bits differ from append + decode"
    ref = RefCache(1, B, Hkv, S, D, dtype)
    ref.fill(0, case["k_fill"], case["v_fill"], 0)
    ref.append(0, case["k_new"], case["v_new"], case["cache_index"])
    want = oracle_decode(ref, 0, case["q"], np.asarray(ci) + 1, case["sm_scale"])
    tol_check(fout, want, dtype, "fused")


@pytest.mark.parametrize("workgroups", [1, 7, 333])
def test_fused_grid_invariance(workgroups):
    dev = device()
    B, H, Hkv, D, S = 3, 16, 4, 128, 1000
    case = garbage_case(91, B, H, Hkv, D, S, "bf16", [999, 332, 16])
    say(f"fused workgroups={workgroups}")
    (fo, fk, fv, fs, fout), (so, sk, sv, ss, sout) = two_ways(dev, case, "bf16", workgroups)
    assert np.array_equal(fo, so) and np.array_equal(fk, sk) and np.array_equal(fv, sv)


def test_fused_out_of_range_is_skipped_and_flagged():
    dev = device()
    B, H, Hkv, D, S = 3, 8, 2, 64, 50
    case = synthetic.random_gqa_case(92, B, H, Hkv, D, S, "bf16", valid_lens=[10, 1, 1])
    case["cache_index"] = np.array([9, -1, S], dtype=np.int32)
    (fo, fk, fv, fs, fout), (so, sk, sv, ss, sout) = two_ways(dev, case, "bf16")
    assert fs == kvc.KVC_ERR_DEVICE_RANGE
    assert np.array_equal(fk, sk) and np.array_equal(fv, sv), "skipped sequences must be left untouched"
    assert not fout[1:].any(), "skipped sequences give zeros"
    assert np.array_equal(fo[0], so[0])
