"""kvc_decode_attn_noalloc (decode attention with the library's static
workspace, for callers that cannot allocate) against kvc_decode_attn on the
same layer: the same kernels on the same grid, so the outputs must be equal
bit for bit, and within the bound of the oracle. Calls in a row with
different shapes (the second smaller) share the static workspace: each must
still be right, and repeating the first shape gives its bits again."""

import numpy as np
import pytest
import torch

from gpu_util import bits_of, device, oracle_decode, say, to_f64, tol_check
from oracle.buffer import RefCache
from static_kv_cache_amd import kvc, synthetic

pytestmark = pytest.mark.gpu


def layer(dev, seed, B, H, Hkv, D, S, dtype, lens):
    """A one-layer cache filled and appended as a decode step; returns the
    cache, its layer copies, the inputs, kvc_decode_attn's output and the
    oracle's."""
    case = synthetic.random_gqa_case(seed, B, H, Hkv, D, S, dtype, valid_lens=np.maximum(lens, 1))
    case["valid_lens"] = np.asarray(lens, dtype=np.int32)
    case["cache_index"] = np.maximum(case["valid_lens"] - 1, 0).astype(np.int32)
    desc = kvc.gqa_desc(1, B, H, Hkv, D, S, dtype)
    cache = kvc.Cache(desc)
    ref = RefCache(1, B, Hkv, S, D, dtype)
    cache.prefill_fill(0, kvc.to_device(case["k_fill"], dev), kvc.to_device(case["v_fill"], dev), 0)
    ref.fill(0, case["k_fill"], case["v_fill"], 0)
    ci = kvc.to_device(case["cache_index"], dev)
    cache.append(0, kvc.to_device(case["k_new"], dev), kvc.to_device(case["v_new"], dev), ci)
    ref.append(0, case["k_new"], case["v_new"], case["cache_index"])
    q = kvc.to_device(case["q"], dev)
    vl = kvc.to_device(case["valid_lens"], dev)
    out = torch.empty((B, H, D), dtype=kvc.torch_dtype(dtype), device=dev)
    cache.decode_attn(0, q, out, valid_lens=vl, sm_scale=case["sm_scale"])
    cache.check()
    k_dev, v_dev = cache.layer_tensors(0)
    want = oracle_decode(ref, 0, case["q"], case["valid_lens"], case["sm_scale"])
    return desc, cache, k_dev, v_dev, q, vl, case, out, want


def noalloc(dev, desc, k_dev, v_dev, q, vl, case):
    out = torch.full(tuple(q.shape), 7.0, dtype=q.dtype, device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    kvc.decode_attn_noalloc(desc, k_dev, v_dev, q, out, valid_lens=vl, sm_scale=case["sm_scale"], err_flag=flag)
    torch.cuda.synchronize()
    return out, int(flag.item())


SHAPES = [
    # seed, B, H, Hkv, D, S, dtype, lengths
    (301, 16, 32, 8, 128, 4096, "bf16", None),           # the Llama-3-8B-shaped layer
    (302, 3, 8, 2, 64, 300, "bf16", [300, 0, 1]),        # smaller: empty and one-row sequences
    (303, 2, 4, 4, 32, 97, "f32", [97, 40]),             # smaller still, fp32
]


def test_noalloc_matches_decode_attn_calls_in_a_row():
    dev = device()
    rng = np.random.default_rng(300)
    first = None
    for i, (seed, B, H, Hkv, D, S, dtype, lens) in enumerate(SHAPES + SHAPES[:1]):
        if lens is None:
            lens = np.random.default_rng(seed).integers(1024, S + 1, size=B)
        say(f"no-alloc call {i}: {dtype} B={B} H={H} H_kv={Hkv} D={D} S={S} lengths {list(lens)[:8]}")
        desc, cache, k_dev, v_dev, q, vl, case, want_bits, want = layer(dev, seed, B, H, Hkv, D, S, dtype, lens)
        got, flag = noalloc(dev, desc, k_dev, v_dev, q, vl, case)
        assert flag == 0
        assert np.array_equal(bits_of(got, dtype), bits_of(want_bits, dtype)), f"call {i}: bits differ"
        tol_check(to_f64(got), want, dtype, f"call {i}")
        if i == 0:
            first = bits_of(got, dtype).copy()
        if i == len(SHAPES):
            assert np.array_equal(bits_of(got, dtype), first), "the repeated first shape changed"
        del k_dev, v_dev
        cache.free()


def test_noalloc_out_of_range_length_flags_and_zeros():
    dev = device()
    desc, cache, k_dev, v_dev, q, vl, case, _, want = layer(dev, 304, 3, 8, 2, 128, 200, "bf16", [200, 50, 7])
    bad = kvc.to_device(np.array([200, 201, 7], dtype=np.int32), dev)
    got, flag = noalloc(dev, desc, k_dev, v_dev, q, bad, case)
    assert flag == 1
    g = to_f64(got)
    assert not g[1].any(), "the out-of-range sequence gives zeros"
    tol_check(g[[0, 2]], want[[0, 2]], "bf16", "in-range sequences")
    del k_dev, v_dev
    cache.free()
