"""Append and prefill fill are bit copies: the whole device buffer must equal
the oracle's buffer model byte for byte after every call."""

import numpy as np
import pytest
import torch

from gpu_util import bits_of, device, ref_cache_like, say
from static_kv_cache_amd import kvc, synthetic

pytestmark = pytest.mark.gpu


def whole_buffer_bits(ext, dtype):
    return bits_of(ext, dtype)


@pytest.mark.parametrize("dtype,L,B,H,Hkv,D,S", [
    ("f32", 1, 1, 4, 4, 32, 128),
    ("bf16", 3, 4, 8, 2, 32, 40),
    ("bf16", 2, 3, 16, 4, 128, 67),
    ("f32", 2, 2, 4, 1, 256, 33),
    ("bf16", 1, 2, 4, 4, 64, 16),
])
def test_fill_and_append_bit_exact(dtype, L, B, H, Hkv, D, S):
    dev = device()
    say(f"append bit-exact: {dtype} L={L} B={B} H={H} Hkv={Hkv} D={D} S={S}")
    rng = np.random.default_rng(100 + D + S)
    desc = kvc.gqa_desc(L, B, H, Hkv, D, S, dtype)
    nbytes = kvc.cache_bytes(desc)
    # external buffer with guard canaries on both sides of the cache region
    guard = 4096
    raw = torch.full((nbytes + 2 * guard,), 0x5A, dtype=torch.uint8, device=dev)
    region = raw[guard:guard + nbytes]
    region.zero_()
    cache = kvc.Cache(desc, external=region)
    ref = ref_cache_like(desc, dtype)
    el = torch.float32 if dtype == "f32" else torch.bfloat16
    view = region.view(el)

    def cmp(what):
        torch.cuda.synchronize()
        got = bits_of(view, dtype)
        want = ref.buf.reshape(-1)
        assert np.array_equal(got, want if dtype == "bf16" else want.view(np.uint32)), what
        g = raw.cpu().numpy()
        assert (g[:guard] == 0x5A).all() and (g[guard + nbytes:] == 0x5A).all(), "canary overwritten"

    for layer in range(L):
        t = int(rng.integers(1, S + 1))
        start = int(rng.integers(0, S - t + 1))
        k = synthetic.draw(rng, (B, Hkv, t, D), dtype)
        v = synthetic.draw(rng, (B, Hkv, t, D), dtype)
        cache.prefill_fill(layer, kvc.to_device(k, dev), kvc.to_device(v, dev), start)
        ref.fill(layer, k, v, start)
        cmp(f"fill layer {layer} start {start} t {t}")
    for step in range(4):
        layer = step % L
        t_new = 1 if step < 3 else min(3, S)
        ci = rng.integers(0, S - t_new + 1, size=B).astype(np.int32)
        k = synthetic.draw(rng, (B, Hkv, t_new, D), dtype)
        v = synthetic.draw(rng, (B, Hkv, t_new, D), dtype)
        cache.append(layer, kvc.to_device(k, dev), kvc.to_device(v, dev), kvc.to_device(ci, dev))
        assert ref.append(layer, k, v, ci) == []
        cmp(f"append step {step} layer {layer} ci {ci.tolist()}")
    cache.check()
    cache.free()


def test_append_out_of_range_is_skipped_and_flagged():
    dev = device()
    say("append out of range: skipped + flagged")
    B, H, Hkv, D, S = 4, 4, 2, 32, 24
    desc = kvc.gqa_desc(1, B, H, Hkv, D, S, "bf16")
    region = torch.zeros(kvc.cache_bytes(desc), dtype=torch.uint8, device=dev)
    cache = kvc.Cache(desc, external=region)
    ref = ref_cache_like(desc, "bf16")
    rng = np.random.default_rng(5)
    k = synthetic.draw(rng, (B, Hkv, 2, D), "bf16")
    v = synthetic.draw(rng, (B, Hkv, 2, D), "bf16")
    ci = np.array([0, S - 1, -3, S - 2], dtype=np.int32)   # b=1 overflows by one, b=2 negative
    cache.append(0, kvc.to_device(k, dev), kvc.to_device(v, dev), kvc.to_device(ci, dev))
    assert ref.append(0, k, v, ci) == [1, 2]
    assert cache.check_status() == kvc.KVC_ERR_DEVICE_RANGE
    assert cache.check_status() == kvc.KVC_OK  # the flag clears once reported
    assert np.array_equal(bits_of(region.view(torch.bfloat16), "bf16"), ref.buf.reshape(-1))
    cache.free()


def test_owned_allocation_layer_pointers_and_zero_fill():
    dev = device()
    say("owned allocation: zero-filled, per-layer regions")
    B, H, Hkv, D, S, L = 2, 8, 4, 64, 48, 3
    cache = kvc.Cache(kvc.gqa_desc(L, B, H, Hkv, D, S, "bf16"))
    ptrs = [cache.layer_ptrs(l) for l in range(L)]
    layer_bytes = 2 * B * Hkv * S * D * 2
    for l in range(L):
        assert ptrs[l][1] - ptrs[l][0] == layer_bytes // 2
        if l:
            assert ptrs[l][0] - ptrs[l - 1][0] == layer_bytes
    k, v = cache.layer_tensors(1)
    assert not k.float().abs().sum().item() and not v.float().abs().sum().item()
    rng = np.random.default_rng(9)
    kk = synthetic.draw(rng, (B, Hkv, S, D), "bf16")
    vv = synthetic.draw(rng, (B, Hkv, S, D), "bf16")
    cache.prefill_fill(1, kvc.to_device(kk, dev), kvc.to_device(vv, dev), 0)
    k, v = cache.layer_tensors(1)
    assert np.array_equal(bits_of(k, "bf16"), kk) and np.array_equal(bits_of(v, "bf16"), vv)
    k0, _ = cache.layer_tensors(0)
    assert not k0.float().abs().sum().item()
    assert cache.logical_bytes([5, 48]) == 3 * 2 * Hkv * D * 2 * 53
    cache.free()
