"""kvc_prefill_attn on the GPU: the chunk's rows land in the cache bit for bit, and its causal
attention matches the oracle (each query is the decode of its own position over the cache)."""

import numpy as np
import pytest
import torch

from gpu_util import bits_of, device, say, to_f64, tol_check
from oracle import attention as oatt
from oracle.buffer import RefCache
from static_kv_cache_amd import kvc, synthetic

pytestmark = pytest.mark.gpu


def run_prefill(dev, B, H, Hkv, D, S, start, t, seed):
    rng = np.random.default_rng(seed)
    pre_k = synthetic.draw(rng, (B, Hkv, max(start, 1), D), "bf16")
    pre_v = synthetic.draw(rng, (B, Hkv, max(start, 1), D), "bf16")
    k = synthetic.draw(rng, (B, Hkv, t, D), "bf16")
    v = synthetic.draw(rng, (B, Hkv, t, D), "bf16")
    q = synthetic.draw(rng, (B, H, t, D), "bf16")
    scale = 1.0 / np.sqrt(D)
    cache = kvc.Cache(kvc.gqa_desc(1, B, H, Hkv, D, S, "bf16"))
    ref = RefCache(1, B, Hkv, S, D, "bf16")
    if start > 0:
        cache.prefill_fill(0, kvc.to_device(pre_k[:, :, :start], dev), kvc.to_device(pre_v[:, :, :start], dev), 0)
        ref.fill(0, pre_k[:, :, :start], pre_v[:, :, :start], 0)
    out = torch.empty((B, H, t, D), dtype=torch.bfloat16, device=dev)
    cache.prefill_attn(0, kvc.to_device(q, dev), kvc.to_device(k, dev), kvc.to_device(v, dev), out, start, scale)
    assert cache.check_status() == kvc.KVC_OK
    ref.fill(0, k, v, start)
    kd, vd = cache.layer_tensors(0)
    assert np.array_equal(bits_of(kd, "bf16"), ref.keys(0)) and np.array_equal(bits_of(vd, "bf16"), ref.values(0))
    cache.free()
    return out, q, ref, scale


SHAPES = [  # B, H, Hkv, D, S, start, t
    (2, 8, 2, 128, 256, 0, 100),    # GQA (G = 4: four heads per workgroup, 16 positions each)
    (1, 4, 4, 64, 128, 0, 70),      # MHA (one head per workgroup, 64 positions)
    (2, 16, 1, 128, 64, 0, 33),     # MQA (G = 16)
    (1, 12, 4, 128, 96, 0, 50),     # G = 3: one head per workgroup
    (1, 4, 2, 128, 96, 0, 61),      # G = 2
    (2, 8, 2, 256, 80, 0, 40),      # widest rows
    (2, 8, 2, 128, 200, 37, 60),    # a chunk after 37 cached rows
    (1, 8, 8, 64, 300, 200, 1),     # a one-token chunk (a decode step written as prefill)
]


@pytest.mark.parametrize("B,H,Hkv,D,S,start,t", SHAPES)
def test_prefill_matches_oracle(B, H, Hkv, D, S, start, t):
    dev = device()
    say(f"prefill: B={B} H={H} Hkv={Hkv} D={D} S={S} start={start} t={t}")
    out, q, ref, scale = run_prefill(dev, B, H, Hkv, D, S, start, t, 1000 + t + D)
    want = oatt.prefill_attention(q, ref.keys(0), ref.values(0), start, scale)
    err = tol_check(to_f64(out), want, "bf16", "prefill")
    say(f"  max abs err {err:.3e}")


def test_prefill_position_zero_is_its_own_value_row():
    """The first position attends only itself: its output is its V row (one bf16 rounding)."""
    dev = device()
    out, q, ref, scale = run_prefill(dev, 1, 8, 2, 128, 64, 0, 20, 7)
    want = np.repeat(ref.values(0)[0, :, 0], 4, axis=0)
    assert np.array_equal(bits_of(out, "bf16")[0, :, 0], want)


def test_prefill_llama3_prompt_full_size():
    """Llama-3-8B-shaped prompt of 4096 tokens (B=1, H=32, H_kv=8, d_h=128): every head at every
    position against the oracle, and the cache rows bit for bit."""
    dev = device()
    B, H, Hkv, D, S, t = 1, 32, 8, 128, 4096, 4096
    rng = np.random.default_rng(4096)
    k = synthetic.draw(rng, (B, Hkv, t, D), "bf16")
    v = synthetic.draw(rng, (B, Hkv, t, D), "bf16")
    q = synthetic.draw(rng, (B, H, t, D), "bf16")
    scale = 1.0 / np.sqrt(D)
    cache = kvc.Cache(kvc.gqa_desc(1, B, H, Hkv, D, S, "bf16"))
    out = torch.empty((B, H, t, D), dtype=torch.bfloat16, device=dev)
    cache.prefill_attn(0, kvc.to_device(q, dev), kvc.to_device(k, dev), kvc.to_device(v, dev), out, 0, scale)
    cache.check()
    k_dev, v_dev = cache.layer_tensors(0)
    assert np.array_equal(bits_of(k_dev, "bf16"), k) and np.array_equal(bits_of(v_dev, "bf16"), v)
    del k_dev, v_dev
    cache.free()
    got = to_f64(out)
    ref = RefCache(1, B, Hkv, S, D, "bf16")
    ref.fill(0, k, v, 0)
    want = oatt.prefill_attention(q, ref.keys(0), ref.values(0), 0, scale)
    err = tol_check(got, want, "bf16", "4096-token prompt, every position")
    say(f"  max abs err {err:.3e}")


def test_prefill_errors():
    dev = device()
    c = kvc.Cache(kvc.gqa_desc(1, 1, 4, 2, 64, 32, "bf16"))
    q = torch.zeros((1, 4, 8, 64), dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(q)
    with pytest.raises(kvc.KvcError) as e:
        c.prefill_attn(0, q, kv, kv, out, 25, 0.125)
    assert e.value.status == kvc.KVC_ERR_CAPACITY
    c.free()
    f = kvc.Cache(kvc.gqa_desc(1, 1, 4, 2, 64, 32, "f32"))
    qf = torch.zeros((1, 4, 8, 64), dtype=torch.float32, device=dev)
    kvf = torch.zeros((1, 2, 8, 64), dtype=torch.float32, device=dev)
    with pytest.raises(kvc.KvcError) as e:
        f.prefill_attn(0, qf, kvf, kvf, torch.empty_like(qf), 0, 0.125)
    assert e.value.status == kvc.KVC_ERR_UNSUPPORTED
    f.free()
