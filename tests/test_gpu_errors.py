"""Error behaviour of the C ABI: host-checkable misuse returns a status and
enqueues nothing; device-side out-of-range indices skip the sequence and
raise the sticky flag reported by kvc_check."""

import ctypes

import numpy as np
import pytest
import torch

from gpu_util import bits_of, device, say, to_f64
from static_kv_cache_amd import kvc, synthetic

pytestmark = pytest.mark.gpu


def _cache(dev, dtype="bf16", B=2, H=4, Hkv=2, D=32, S=16, L=2):
    desc = kvc.gqa_desc(L, B, H, Hkv, D, S, dtype)
    region = torch.zeros(kvc.cache_bytes(desc), dtype=torch.uint8, device=dev)
    return kvc.Cache(desc, external=region), region


def test_host_checked_errors_enqueue_nothing():
    dev = device()
    say("host-checked errors")
    cache, region = _cache(dev)
    lib = kvc.load()
    h = cache.handle
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    k = torch.ones((2, 2, 4, 32), dtype=torch.bfloat16, device=dev)
    kp = ctypes.c_void_p(k.data_ptr())
    ci = torch.zeros(2, dtype=torch.int32, device=dev)
    cip = ctypes.c_void_p(ci.data_ptr())
    q = torch.ones((2, 4, 32), dtype=torch.bfloat16, device=dev)
    out = torch.full((2, 4, 32), 7.0, dtype=torch.bfloat16, device=dev)
    qp, op = ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(out.data_ptr())
    E = kvc
    assert lib.kvc_prefill_fill(h, 0, kp, kp, 13, 4, st) == E.KVC_ERR_CAPACITY      # 13 + 4 > 16
    assert lib.kvc_prefill_fill(h, 0, kp, kp, -1, 4, st) == E.KVC_ERR_CAPACITY
    assert lib.kvc_prefill_fill(h, 0, kp, kp, 0, 0, st) == E.KVC_ERR_INVALID_ARG
    assert lib.kvc_prefill_fill(h, 2, kp, kp, 0, 4, st) == E.KVC_ERR_INVALID_ARG    # bad layer
    assert lib.kvc_prefill_fill(h, -1, kp, kp, 0, 4, st) == E.KVC_ERR_INVALID_ARG
    assert lib.kvc_prefill_fill(h, 0, kp, None, 0, 4, st) == E.KVC_ERR_INVALID_ARG  # GQA needs v
    assert lib.kvc_append(h, 0, kp, kp, None, 1, st) == E.KVC_ERR_INVALID_ARG
    assert lib.kvc_append(h, 0, kp, kp, cip, 0, st) == E.KVC_ERR_INVALID_ARG
    assert lib.kvc_append(h, 0, kp, kp, cip, 17, st) == E.KVC_ERR_CAPACITY
    assert lib.kvc_decode_attn(h, 0, qp, op, None, None, ctypes.c_float(1.0), st) == E.KVC_ERR_INVALID_ARG
    assert lib.kvc_decode_attn(h, 0, None, op, cip, cip, ctypes.c_float(1.0), st) == E.KVC_ERR_INVALID_ARG
    assert lib.kvc_decode_attn(h, 0, qp, op, cip, cip, ctypes.c_float(0.0), st) == E.KVC_ERR_INVALID_ARG
    assert lib.kvc_decode_attn(h, 0, qp, op, cip, cip, ctypes.c_float(float("nan")), st) == E.KVC_ERR_INVALID_ARG
    assert lib.kvc_decode_attn(h, 5, qp, op, cip, cip, ctypes.c_float(1.0), st) == E.KVC_ERR_INVALID_ARG
    assert lib.kvc_mla_decode(h, 0, qp, qp, qp, qp, op, cip, cip, ctypes.c_float(1.0), st) == E.KVC_ERR_INVALID_ARG
    assert lib.kvc_set_workgroups(h, -1) == E.KVC_ERR_INVALID_ARG
    assert lib.kvc_set_workgroups(h, cache.workgroups()[1] + 1) == E.KVC_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert not region.any().item(), "a rejected call wrote to the cache"
    assert (out.float() == 7.0).all().item(), "a rejected call wrote the output"
    assert cache.check_status() == E.KVC_OK
    cache.free()


def test_decode_out_of_range_length_gives_zeros_and_flag():
    dev = device()
    say("decode out-of-range length")
    B, H, Hkv, D, S = 3, 4, 2, 32, 16
    cache, region = _cache(dev, B=B, S=S)
    rng = np.random.default_rng(2)
    k = synthetic.draw(rng, (B, Hkv, S, D), "bf16")
    cache.prefill_fill(0, kvc.to_device(k, dev), kvc.to_device(k, dev), 0)
    q = kvc.to_device(synthetic.draw(rng, (B, H, D), "bf16"), dev)
    out = torch.full((B, H, D), 3.0, dtype=torch.bfloat16, device=dev)
    valid = kvc.to_device(np.array([S + 1, 4, -2], dtype=np.int32), dev)
    cache.decode_attn(0, q, out, valid_lens=valid, sm_scale=0.2)
    assert cache.check_status() == kvc.KVC_ERR_DEVICE_RANGE
    o = to_f64(out)
    assert not o[0].any() and not o[2].any() and o[1].any()
    assert cache.check_status() == kvc.KVC_OK
    cache.free()


def test_absurd_allocation_reports_oom():
    device()
    say("absurd allocation")
    desc = kvc.gqa_desc(1 << 12, 64, 64, 64, 128, 1 << 16, "bf16")     # 2^49 bytes
    with pytest.raises(kvc.KvcError) as e:
        kvc.Cache(desc)
    assert e.value.status == kvc.KVC_ERR_OOM


def test_external_buffer_must_be_aligned():
    dev = device()
    desc = kvc.gqa_desc(1, 1, 4, 4, 32, 16, "bf16")
    raw = torch.zeros(kvc.cache_bytes(desc) + 512, dtype=torch.uint8, device=dev)
    lib = kvc.load()
    h = ctypes.c_void_p()
    st = lib.kvc_alloc(ctypes.byref(desc), ctypes.c_void_p(raw.data_ptr() + 16), ctypes.byref(h))
    assert st == kvc.KVC_ERR_INVALID_ARG and not h.value
