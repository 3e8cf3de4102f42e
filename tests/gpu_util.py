"""Helpers for the GPU tests: device fixture, tolerances, oracle runs."""

import sys

import numpy as np
import pytest

from oracle import attention as oatt
from oracle.buffer import RefCache

# Tolerances (written here, used by every parity test):
#  fp32 cache: |o - r| <= 1e-5 * (|r| + max_d |r[b,h,:]|)  (1e-5 relative to the
#              output row's scale, so entries near zero from cancellation pass)
#  bf16 cache: |o - r| <= 1e-2 + 1e-2 * |r|
#  and, for every bf16 path, each output row (b, h) within a relative L2
#  norm of the oracle's row: BF16_ROW_RTOL for the GQA paths (bf16, int8,
#  block-table), whose result is rounded to bf16 twice (the softmax weights
#  P entering the p.v product, and the output), each a relative step of at
#  most 2^-9, so a row is off by about 2e-3 at worst; the latent path sets
#  its own bound (it rounds five times). The element-wise bound alone is
#  looser than the output itself at long context (output RMS ~0.009 at
#  32,768 rows), where a dropped row or tile would pass it.
F32_RTOL = 1e-5
BF16_ATOL = 1e-2
BF16_RTOL = 1e-2
BF16_ROW_RTOL = 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from static_kv_cache_amd import kvc
    kvc.load()  # fails loudly if the library is not built
    return torch.device("cuda:0")


def to_f64(t):
    """Device tensor (bf16 / fp32) -> float64 numpy."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def tol_check(got, want, dtype, what="", row_rtol=None):
    """The element-wise bound of `dtype`; for bf16 also the per-row L2 bound
    (BF16_ROW_RTOL unless `row_rtol` is given). Returns the max abs error."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    err = np.abs(got - want)
    if dtype == "f32":
        row = np.max(np.abs(want), axis=-1, keepdims=True)
        bound = F32_RTOL * (np.abs(want) + row)
    else:
        bound = BF16_ATOL + BF16_RTOL * np.abs(want)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} out of tolerance; first at "
                             f"{tuple(idx)}: got {got[tuple(idx)]!r} want {want[tuple(idx)]!r}; "
                             f"max err {err.max():.3e}")
    if dtype != "f32":
        row_l2_check(got, want, BF16_ROW_RTOL if row_rtol is None else row_rtol, what)
    return float(err.max())


def row_l2_check(got, want, rtol, what=""):
    """Every output row (last axis) within `rtol` of the oracle's in relative
    L2 norm; rows the oracle gives as exactly zero must be exactly zero.
    Returns the worst relative error."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    num = np.linalg.norm(got - want, axis=-1)
    den = np.linalg.norm(want, axis=-1)
    live = den > 0
    rel = num[live] / den[live]
    worst = float(rel.max()) if rel.size else 0.0
    if not worst <= rtol:
        idx = np.argwhere(live)[int(np.argmax(rel))]
        raise AssertionError(f"{what}: worst row relative L2 error {worst:.3e} > {rtol:.1e} at row {tuple(idx)}")
    assert np.all(num[~live] == 0), f"{what}: rows that must be zero are not"
    return worst


def oracle_decode(ref, layer, q, valid_lens, sm_scale):
    return oatt.decode_attention(q, ref.keys(layer), ref.values(layer), valid_lens, sm_scale)


def bits_of(t, dtype):
    """Raw element bits of a device tensor as numpy (uint16 bf16 / uint32 fp32)."""
    a = t.detach().cpu()
    import torch
    if dtype == "bf16":
        return a.view(torch.int16).numpy().view(np.uint16)
    return a.view(torch.int32).numpy().view(np.uint32)


def ref_cache_like(desc, dtype):
    return RefCache(desc.n_layers, desc.batch, desc.n_kv_heads, desc.max_context, desc.head_dim, dtype)
