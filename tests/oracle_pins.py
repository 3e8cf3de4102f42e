"""Pins for the oracle's decode attention, written as reusable checks.

Each check takes a decode-attention implementation with the oracle's
signature ``fn(q, k_cache, v_cache, valid_lens, sm_scale) -> [B, H, D]``
and raises AssertionError if it disagrees with something the pages or the
mathematics fix independently of that implementation:

* library routine: torch's CPU float64 scaled_dot_product_attention
  (explicit scale, enable_gqa for grouped heads) on the valid prefix;
* closed forms: n = 1 gives value row 0; q = 0 gives the mean of the value
  rows; two rows give a logistic blend; a dominant logit picks its row;
* invariants: garbage past valid_len changes nothing; the no-cache
  recomputation ("KV-Cache Mechanics", "Disabling the Cache") matches the
  cached decode step by step (checked in the test modules).

``tests/test_oracle_mutations.py`` feeds deliberately broken copies of the
oracle through the same checks to show each plausible mistake is caught.
"""

import math

import numpy as np
import torch
import torch.nn.functional as F

RTOL = 1e-12


def _close(a, b, tol=RTOL):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * scale, f"max abs err {err:.3e} > {tol:.1e} * {scale:.3g}"


def _rand(rng, shape):
    return rng.standard_normal(shape)


def sdpa_reference(q, k, v, valid_lens, sm_scale):
    """torch CPU float64 SDPA on each sequence's valid prefix."""
    B, H, D = q.shape
    H_kv = k.shape[1]
    out = np.zeros((B, H, D))
    for b in range(B):
        n = int(valid_lens[b])
        if n == 0:
            continue
        qt = torch.from_numpy(np.ascontiguousarray(q[b][:, None, :]))          # [H,1,D]
        kt = torch.from_numpy(np.ascontiguousarray(k[b, :, :n, :]))             # [H_kv,n,D]
        vt = torch.from_numpy(np.ascontiguousarray(v[b, :, :n, :]))
        o = F.scaled_dot_product_attention(qt[None], kt[None], vt[None], scale=sm_scale,
                                           enable_gqa=(H != H_kv))
        out[b] = o[0, :, 0, :].numpy()
    return out


def check_library(fn, seed=0):
    rng = np.random.default_rng(seed)
    for (B, H, H_kv, D, S) in [(2, 4, 4, 8, 9), (3, 8, 2, 16, 17), (2, 6, 1, 4, 5), (1, 8, 4, 32, 33)]:
        q = _rand(rng, (B, H, D))
        k = _rand(rng, (B, H_kv, S, D))
        v = _rand(rng, (B, H_kv, S, D))
        n = rng.integers(1, S + 1, size=B)
        scale = 1.0 / math.sqrt(D) * (1.0 + 0.5 * rng.random())
        _close(fn(q, k, v, n, scale), sdpa_reference(q, k, v, n, scale))


def check_single_row(fn, seed=1):
    """n = 1: softmax of one logit is 1, so every head returns value row 0 of its group."""
    rng = np.random.default_rng(seed)
    B, H, H_kv, D, S = 2, 8, 2, 8, 6
    q = _rand(rng, (B, H, D))
    k = _rand(rng, (B, H_kv, S, D))
    v = _rand(rng, (B, H_kv, S, D))
    o = fn(q, k, v, np.array([1, 1]), 0.7)
    G = H // H_kv
    for b in range(B):
        for h in range(H):
            assert np.array_equal(o[b, h], v[b, h // G, 0]), "n=1 must return value row 0 exactly"


def check_zero_query(fn, seed=2):
    """q = 0: all logits equal, output is the mean of the n value rows."""
    rng = np.random.default_rng(seed)
    B, H, H_kv, D, S = 2, 4, 2, 8, 10
    q = np.zeros((B, H, D))
    k = _rand(rng, (B, H_kv, S, D))
    v = _rand(rng, (B, H_kv, S, D))
    n = np.array([7, 10])
    o = fn(q, k, v, n, 0.5)
    G = H // H_kv
    for b in range(B):
        for h in range(H):
            _close(o[b, h], v[b, h // G, :n[b]].mean(axis=0))


def check_two_rows(fn, seed=3):
    """n = 2: o = v0 + (v1 - v0) * sigmoid(scale * q.(k1 - k0))."""
    rng = np.random.default_rng(seed)
    B, H, H_kv, D, S = 1, 4, 4, 8, 4
    q = _rand(rng, (B, H, D))
    k = _rand(rng, (B, H_kv, S, D))
    v = _rand(rng, (B, H_kv, S, D))
    scale = 0.37
    o = fn(q, k, v, np.array([2]), scale)
    for h in range(H):
        z = scale * float(q[0, h] @ (k[0, h, 1] - k[0, h, 0]))
        w = 1.0 / (1.0 + math.exp(-z))
        _close(o[0, h], v[0, h, 0] + (v[0, h, 1] - v[0, h, 0]) * w)


def check_dominant(fn, seed=4):
    """One key aligned with q at huge scale: the output is that key's value row."""
    rng = np.random.default_rng(seed)
    B, H, H_kv, D, S = 1, 2, 1, 8, 12
    q = _rand(rng, (B, H, D))
    k = 0.01 * _rand(rng, (B, H_kv, S, D))
    v = _rand(rng, (B, H_kv, S, D))
    j = 5
    k[0, 0, j] = 100.0 * q[0, 0] / np.linalg.norm(q[0, 0])
    o = fn(q, k, v, np.array([S]), 1.0)
    _close(o[0, 0], v[0, 0, j], tol=1e-9)


def check_garbage_beyond_valid(fn, seed=5):
    """Rows >= n_b never influence the output (reads stop at the valid length)."""
    rng = np.random.default_rng(seed)
    B, H, H_kv, D, S = 3, 4, 2, 8, 16
    q = _rand(rng, (B, H, D))
    k = _rand(rng, (B, H_kv, S, D))
    v = _rand(rng, (B, H_kv, S, D))
    n = np.array([5, 16, 1])
    ref = fn(q, k, v, n, 0.4)
    for junk in (np.nan, np.inf, -np.inf, 1e30, 0.0):
        k2, v2 = k.copy(), v.copy()
        for b in range(B):
            k2[b, :, n[b]:] = junk
            v2[b, :, n[b]:] = junk
        assert np.array_equal(fn(q, k2, v2, n, 0.4), ref), f"garbage {junk} changed the output"


def check_empty(fn):
    """n_b = 0 gives an all-zero row (reading taken: empty softmax -> 0)."""
    q = np.ones((2, 2, 4))
    k = np.ones((2, 1, 3, 4))
    v = np.ones((2, 1, 3, 4))
    o = fn(q, k, v, np.array([0, 3]), 1.0)
    assert np.array_equal(o[0], np.zeros((2, 4)))
    _close(o[1], np.ones((2, 4)))


ALL_CHECKS = [check_library, check_single_row, check_zero_query, check_two_rows,
              check_dominant, check_garbage_beyond_valid, check_empty]
