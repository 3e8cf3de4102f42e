"""Latent (MLA) decode on the GPU against the CPU float64 oracle.

Two entry points are covered: kvc_decode_attn on a latent cache (absorbed
queries in, latent output out) against oracle.mla.latent_attention, and the
whole step kvc_mla_decode (absorb, latent attention, up-projection) against
oracle.mla.mla_decode_absorbed, which the CPU tests pin to the materialised
form. Besides the element-wise bf16 bound, every (b, h) output row must be
within 2e-2 of the oracle in relative L2 norm: the GPU path rounds to bf16
five times (q~, p, the piece partials, o~, out), each a relative 2^-9 step,
and the element-wise bound alone is loose against outputs of size ~0.02.
"""

import math

import numpy as np
import pytest
import torch

from gpu_util import bits_of, device, row_l2_check, say, to_f64, tol_check
from oracle import mla as omla
from static_kv_cache_amd import kvc, synthetic

pytestmark = pytest.mark.gpu

ROW_RTOL = 2e-2


def row_norm_check(got, want, what):
    return row_l2_check(got, want, ROW_RTOL, what)


def mla_cfg(B, H, S, seed=0, valid=None):
    cfg = dict(synthetic.WORKLOADS["mla_latent_bf16"])
    cfg.update(batch=B, n_heads=H, max_context=S, seed=seed)
    rng = np.random.default_rng(seed)
    d = synthetic.mla_layer(cfg, rng=rng)
    if valid is not None:
        d["valid_lens"] = np.asarray(valid, dtype=np.int32)
        d["cache_index"] = np.maximum(d["valid_lens"] - 1, 0).astype(np.int32)
    return cfg, d


def make_cache(dev, cfg, d, workgroups=None, layers=1, layer=0):
    B, H, S = cfg["batch"], cfg["n_heads"], cfg["max_context"]
    desc = kvc.mla_desc(layers, B, H, S)
    cache = kvc.Cache(desc)
    if workgroups is not None:
        cache.set_workgroups(workgroups)
    cache.prefill_fill(layer, kvc.to_device(d["rows_fill"], dev), None, 0)
    return cache


def run_latent(dev, cfg, d, q_abs_bits, workgroups=None):
    """kvc_decode_attn on a latent cache; returns (gpu o~, oracle o~)."""
    B, H = cfg["batch"], cfg["n_heads"]
    cache = make_cache(dev, cfg, d, workgroups)
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    cache.decode_attn(0, kvc.to_device(q_abs_bits, dev), out,
                      valid_lens=kvc.to_device(d["valid_lens"], dev), sm_scale=d["sm_scale"])
    cache.check()
    got = to_f64(out)
    cache.free()
    want = omla.latent_attention(q_abs_bits, d["rows_fill"], d["valid_lens"], d["sm_scale"], 512)
    return got, want


def random_q_abs(seed, B, H):
    """Absorbed queries drawn at the scale the absorb step gives them."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, 576)).astype(np.float32)
    q[..., :512] *= np.float32(math.sqrt(128) * 0.02)
    return synthetic.f32_to_bf16_bits(q)


@pytest.mark.parametrize("B,H,S", [(5, 16, 300), (3, 8, 97), (2, 32, 200), (4, 1, 64)])
def test_latent_attention_ragged(B, H, S):
    """Latent attention over ragged lengths including 0, 1 and tile edges."""
    dev = device()
    special = [0, 1, 31, 32, 33, S]
    valid = [special[i % len(special)] for i in range(B)]
    valid[-1] = S
    cfg, d = mla_cfg(B, H, S, seed=B * 100 + H, valid=valid)
    say(f"latent attention: B={B} H={H} S={S} valid={valid}")
    q_abs = random_q_abs(B + H + S, B, H)
    got, want = run_latent(dev, cfg, d, q_abs)
    tol_check(got, want, "bf16", "latent", row_rtol=ROW_RTOL)
    worst = row_norm_check(got, want, "latent")
    assert not got[np.asarray(valid) == 0].any(), "empty sequence must give zeros"
    say(f"  worst row rel err {worst:.3e}")


@pytest.mark.parametrize("workgroups", [1, 3, 64, 333, 2048])
def test_latent_workgroup_invariance(workgroups):
    """Any persistent grid size: one workgroup streams everything, large
    counts cut each sequence into many pieces merged by the second kernel."""
    dev = device()
    B, H, S = 3, 16, 1000
    cfg, d = mla_cfg(B, H, S, seed=7, valid=[1000, 333, 17])
    c = kvc.Cache(kvc.mla_desc(1, B, H, S))
    wg = min(workgroups, c.workgroups()[1])
    c.free()
    say(f"latent workgroups={wg}")
    got, want = run_latent(dev, cfg, d, random_q_abs(8, B, H), workgroups=wg)
    tol_check(got, want, "bf16", f"workgroups {wg}", row_rtol=ROW_RTOL)
    row_norm_check(got, want, f"workgroups {wg}")


def test_latent_single_row_is_exact():
    """n = 1: the only weight is exactly 1, so o~ is the latent of row 0 bit
    for bit (the partial o~ / l and the merge weight are exact too)."""
    dev = device()
    B, H, S = 4, 16, 64
    cfg, d = mla_cfg(B, H, S, seed=9, valid=[1] * B)
    cache = make_cache(dev, cfg, d)
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    cache.decode_attn(0, kvc.to_device(random_q_abs(10, B, H), dev), out,
                      valid_lens=kvc.to_device(d["valid_lens"], dev), sm_scale=d["sm_scale"])
    cache.check()
    got = bits_of(out, "bf16")
    want = np.broadcast_to(d["rows_fill"][:, 0:1, :512], (B, H, 512))
    assert np.array_equal(got, want)
    cache.free()


def test_latent_garbage_beyond_valid_is_bit_identical():
    """NaN, inf and huge values in rows at or past n_b change nothing."""
    dev = device()
    B, H, S = 3, 16, 160
    valid = [100, 31, 1]
    cfg, d = mla_cfg(B, H, S, seed=11, valid=valid)
    q = kvc.to_device(random_q_abs(12, B, H), dev)
    outs = []
    for garbage in (False, True):
        rows = d["rows_fill"].copy()
        for b, n in enumerate(valid):
            if garbage:
                rows[b, n:] = np.uint16(0x7FC0)        # NaN
                rows[b, n::3] = np.uint16(0x7F80)      # +inf
                rows[b, n + 1::5] = np.uint16(0x7E80)  # ~1.7e38
            else:
                rows[b, n:] = 0
        cache = kvc.Cache(kvc.mla_desc(1, B, H, S))
        cache.prefill_fill(0, kvc.to_device(rows, dev), None, 0)
        out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
        cache.decode_attn(0, q, out, valid_lens=kvc.to_device(d["valid_lens"], dev), sm_scale=d["sm_scale"])
        cache.check()
        outs.append(bits_of(out, "bf16"))
        cache.free()
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("B,H,S", [(3, 16, 130), (2, 32, 64)])
def test_mla_decode_step_small(B, H, S):
    """Append of the new latent row, then the whole absorbed decode step
    (kvc_mla_decode) against the float64 absorbed oracle; the append is
    bit-exact against the buffer model."""
    dev = device()
    cfg, d = mla_cfg(B, H, S, seed=B * 10 + H)
    say(f"mla decode step: B={B} H={H} S={S} valid={d['valid_lens'].tolist()}")
    cache = make_cache(dev, cfg, d, layers=2, layer=1)
    ci = d["cache_index"]
    cache.append(1, kvc.to_device(d["rows_new"], dev), None, kvc.to_device(ci, dev))
    rows = d["rows_fill"].copy()
    for b in range(B):
        rows[b, ci[b]] = d["rows_new"][b, 0]
    out = torch.empty((B, H, 128), dtype=torch.bfloat16, device=dev)
    cache.mla_decode(1, kvc.to_device(d["q_nope"], dev), kvc.to_device(d["q_rope"], dev),
                     kvc.to_device(d["w_uk"], dev), kvc.to_device(d["w_uv"], dev), out,
                     cache_index=kvc.to_device(ci, dev), sm_scale=d["sm_scale"])
    cache.check()
    got_rows = bits_of(cache.layer_tensors(1)[0], "bf16")
    assert np.array_equal(got_rows, rows), "append must be bit-exact"
    want = omla.mla_decode_absorbed(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], rows,
                                    ci + 1, d["sm_scale"])
    got = to_f64(out)
    tol_check(got, want, "bf16", "mla step", row_rtol=ROW_RTOL)
    worst = row_norm_check(got, want, "mla step")
    say(f"  worst row rel err {worst:.3e}")
    cache.free()


def test_mla_latent_workload_full_size():
    """The 32-sequence, 16-head, 4096-row latent workload at full size in the
    benchmark's launch configuration, every output compared."""
    dev = device()
    cfg = synthetic.WORKLOADS["mla_latent_bf16"]
    d = synthetic.mla_layer(cfg)
    B, H, S = cfg["batch"], cfg["n_heads"], cfg["max_context"]
    say(f"mla full size: B={B} H={H} S={S}")
    cache = kvc.Cache(kvc.mla_desc(1, B, H, S))
    cache.prefill_fill(0, kvc.to_device(d["rows_fill"], dev), None, 0)
    ci = d["cache_index"]
    cache.append(0, kvc.to_device(d["rows_new"], dev), None, kvc.to_device(ci, dev))
    rows = d["rows_fill"].copy()
    rows[np.arange(B), ci] = d["rows_new"][:, 0]
    out = torch.empty((B, H, 128), dtype=torch.bfloat16, device=dev)
    cache.mla_decode(0, kvc.to_device(d["q_nope"], dev), kvc.to_device(d["q_rope"], dev),
                     kvc.to_device(d["w_uk"], dev), kvc.to_device(d["w_uv"], dev), out,
                     valid_lens=kvc.to_device(d["valid_lens"], dev), sm_scale=d["sm_scale"])
    cache.check()
    want = omla.mla_decode_absorbed(d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"], rows,
                                    d["valid_lens"], d["sm_scale"])
    got = to_f64(out)
    tol_check(got, want, "bf16", "mla full size", row_rtol=ROW_RTOL)
    worst = row_norm_check(got, want, "mla full size")
    say(f"  worst row rel err {worst:.3e}")
    cache.free()
