"""Oracle decode attention against its pins (library routine, closed forms,
invariants) and the no-cache recomputation."""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle_pins as pins
from oracle import attention as att
from oracle.buffer import RefCache
from static_kv_cache_amd import synthetic


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_decode_attention_pins(check):
    check(att.decode_attention)


def test_gqa_equals_repeated_mha():
    """GQA is MHA with each key/value head repeated over its contiguous group."""
    rng = np.random.default_rng(11)
    B, H, H_kv, D, S = 2, 12, 3, 8, 7
    q = rng.standard_normal((B, H, D))
    k = rng.standard_normal((B, H_kv, S, D))
    v = rng.standard_normal((B, H_kv, S, D))
    n = np.array([3, 7])
    a = att.decode_attention(q, k, v, n, 0.3)
    b = att.decode_attention(q, att.repeat_kv_heads(k, H // H_kv), att.repeat_kv_heads(v, H // H_kv), n, 0.3)
    assert np.allclose(a, b, rtol=0, atol=1e-13)


def test_stored_dtypes_are_widened_exactly():
    """bf16 bits and fp32 values reach the math as the exact stored values."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((1, 2, 5, 4)).astype(np.float32)
    bits = synthetic.f32_to_bf16_bits(x)
    wide = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q = synthetic.f32_to_bf16_bits(rng.standard_normal((1, 2, 4)).astype(np.float32))
    qw = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    a = att.decode_attention(q, bits, bits, [5], 0.5)
    b = att.decode_attention(qw, wide, wide, [5], 0.5)
    assert np.array_equal(a, b)


def test_cached_decode_equals_nocache_and_library_causal():
    """The tiny fp32 workload: prefill 64 tokens into the static buffer, then 16
    decode steps that append at cache_index = 64 + i and attend 65 + i rows.
    Each step must equal (a) the no-cache recomputation and (b) torch's causal
    SDPA over the whole sequence (KV-Cache Mechanics, 'Disabling the Cache')."""
    cfg = synthetic.WORKLOADS["tiny_mha_f32"]
    d = synthetic.tiny_sequence(cfg)
    P, steps, S = cfg["prefill"], cfg["steps"], cfg["max_context"]
    k, v, q = d["k"], d["v"], d["q"]          # k,v [1,H_kv,T,D]; q [steps,1,H,D]
    cache = RefCache(1, 1, cfg["n_kv_heads"], S, cfg["head_dim"], "f32")
    cache.fill(0, k[:, :, :P], v[:, :, :P], 0)
    # full-sequence queries for the no-cache path: only decode positions are compared
    T = P + steps
    q_full = np.zeros((T, cfg["n_heads"], cfg["head_dim"]), dtype=np.float32)
    q_full[P:] = q[:, 0]
    nocache = att.causal_attention_nocache(q_full, k[0].transpose(1, 0, 2), v[0].transpose(1, 0, 2), 1.0)
    lib = F.scaled_dot_product_attention(
        torch.from_numpy(q_full.astype(np.float64)).permute(1, 0, 2)[None],
        torch.from_numpy(k.astype(np.float64)), torch.from_numpy(v.astype(np.float64)),
        is_causal=True, scale=1.0)[0].permute(1, 0, 2).numpy()
    for i in range(steps):
        ci = P + i
        assert cache.append(0, k[:, :, ci:ci + 1], v[:, :, ci:ci + 1], [ci]) == []
        o = att.decode_attention(q[i], cache.keys(0).view(np.float32), cache.values(0).view(np.float32),
                                 [ci + 1], 1.0)
        assert np.allclose(o[0], nocache[ci], rtol=0, atol=1e-12)
        assert np.allclose(o[0], lib[ci], rtol=0, atol=1e-12)


def test_permutation_and_linearity():
    """Attention is invariant to the order of the valid rows and linear in V."""
    rng = np.random.default_rng(13)
    B, H, H_kv, D, S = 1, 4, 2, 8, 9
    q = rng.standard_normal((B, H, D))
    k = rng.standard_normal((B, H_kv, S, D))
    v = rng.standard_normal((B, H_kv, S, D))
    o = att.decode_attention(q, k, v, [S], 0.5)
    perm = rng.permutation(S)
    assert np.allclose(att.decode_attention(q, k[:, :, perm], v[:, :, perm], [S], 0.5), o, atol=1e-13)
    assert np.allclose(att.decode_attention(q, k, 3.0 * v + 1.0, [S], 0.5), 3.0 * o + 1.0, atol=1e-12)


def test_brute_force_tiny():
    """Pure-Python loops (math.exp, running sums) on a tiny case."""
    rng = np.random.default_rng(14)
    B, H, H_kv, D, S = 1, 2, 1, 3, 4
    q = rng.standard_normal((B, H, D))
    k = rng.standard_normal((B, H_kv, S, D))
    v = rng.standard_normal((B, H_kv, S, D))
    o = att.decode_attention(q, k, v, [3], 0.9)
    for h in range(H):
        w = [math.exp(0.9 * sum(q[0, h, d] * k[0, 0, j, d] for d in range(D))) for j in range(3)]
        z = sum(w)
        for d in range(D):
            assert abs(o[0, h, d] - sum(w[j] * v[0, 0, j, d] for j in range(3)) / z) < 1e-12


def test_prefill_attention_equals_nocache_causal():
    """Prefill of a chunk [start, start + t) equals the last t rows of the no-cache causal attention
    over the whole sequence (growing lists, no buffer); start = 0 is the plain prompt. Also against
    torch's causal SDPA in float64 for start = 0."""
    rng = np.random.default_rng(31)
    B, H, Hkv, D, S = 2, 4, 2, 8, 12
    k = rng.standard_normal((B, Hkv, S, D))
    v = rng.standard_normal((B, Hkv, S, D))
    q = rng.standard_normal((B, H, S, D))
    for start, t in ((0, 7), (5, 7), (11, 1)):
        got = att.prefill_attention(q[:, :, start:start + t], k, v, start, 0.3)
        for b in range(B):
            full = att.causal_attention_nocache(q[b].transpose(1, 0, 2), k[b].transpose(1, 0, 2),
                                                v[b].transpose(1, 0, 2), 0.3)   # [S, H, D]
            want = full[start:start + t].transpose(1, 0, 2)
            assert np.allclose(got[b], want, rtol=0, atol=1e-12)
    sd = F.scaled_dot_product_attention(torch.from_numpy(q[:, :, :7]), torch.from_numpy(att.repeat_kv_heads(k[:, :, :7], 2)),
                                        torch.from_numpy(att.repeat_kv_heads(v[:, :, :7], 2)), is_causal=True,
                                        scale=0.3).numpy()
    assert np.allclose(att.prefill_attention(q[:, :, :7], k, v, 0, 0.3), sd, rtol=0, atol=1e-12)


def test_prefill_attention_rows_are_decodes():
    """Every row of the prefill equals the decode of its position (valid length start + i + 1),
    GQA with groups of 3, chunks after cached rows and a one-token chunk."""
    rng = np.random.default_rng(32)
    B, H, Hkv, D, S = 2, 6, 2, 16, 40
    k = rng.standard_normal((B, Hkv, S, D))
    v = rng.standard_normal((B, Hkv, S, D))
    for start, t in ((0, 40), (13, 9), (39, 1)):
        q = rng.standard_normal((B, H, t, D))
        got = att.prefill_attention(q, k, v, start, 0.25)
        for i in range(t):
            want = att.decode_attention(q[:, :, i], k, v, np.full(B, start + i + 1), 0.25)
            assert np.allclose(got[:, :, i], want, rtol=0, atol=1e-12), (start, t, i)
