"""Seeded synthetic inputs for the static KV-cache decode path.

This module only draws numbers and rounds them to the storage type; it holds
none of the method's arithmetic (no attention, no cache bookkeeping) and
imports neither the oracle nor the HIP binding. Both sides receive the same
stored bits from here.

Recipe (every workload): ``numpy.random.default_rng(seed)``;
``standard_normal(..., dtype=float32)`` draws; bf16 values are the float32
draws rounded to nearest-even on their bit patterns. Draw order per layer
is fixed: K fill rows, V fill rows, K new row, V new row, q (and, for the
latent cache, latent rows, new latent row, q_nope, q_rope, W_UK, W_UV).

Workloads (one dict each in ``WORKLOADS``) follow the shapes of the pages'
examples: the DantinoX model (12 layers, 8 heads of width 32, context 512),
a Llama-3-8B-shaped GQA layer stack, a long-context GQA layer sized like
the Llama-2-70B byte example, and a DeepSeek-V2-shaped latent cache
(d_c = 512, 16 heads of width 128). No public dataset is involved.
"""

import math

import numpy as np

WORKLOADS = {
    # tiny MHA in fp32: prefill 64 tokens then 16 decode steps; q pre-scaled
    # by 1/sqrt(d_h) and sm_scale = 1
    "tiny_mha_f32": dict(attn="gqa", dtype="f32", n_layers=1, batch=1, n_heads=4,
                         n_kv_heads=4, head_dim=32, max_context=128, prefill=64,
                         steps=16, seed=0),
    # DantinoX-shaped, all sequences valid to 512 (fill 511, append at 511)
    "dantinox_mha_bf16": dict(attn="gqa", dtype="bf16", n_layers=12, batch=8, n_heads=8,
                              n_kv_heads=8, head_dim=32, max_context=512, seed=1),
    "dantinox_gqa_bf16": dict(attn="gqa", dtype="bf16", n_layers=12, batch=8, n_heads=8,
                              n_kv_heads=2, head_dim=32, max_context=512, seed=1),
    # Llama-3-8B-shaped GQA, valid_len ~ U[1024, 4096] per sequence
    "llama3_8b_gqa_bf16": dict(attn="gqa", dtype="bf16", n_layers=32, batch=16, n_heads=32,
                               n_kv_heads=8, head_dim=128, max_context=4096,
                               valid_lo=1024, valid_hi=4096, seed=2),
    # the same shape on an int8 cache (rows, queries and new rows drawn as bf16)
    "llama3_8b_gqa_i8": dict(attn="gqa", dtype="i8", n_layers=32, batch=16, n_heads=32,
                             n_kv_heads=8, head_dim=128, max_context=4096,
                             valid_lo=1024, valid_hi=4096, seed=2),
    # long context: cache sized for 80 layers, one layer-step at a time
    "longctx_gqa_bf16": dict(attn="gqa", dtype="bf16", n_layers=80, batch=1, n_heads=64,
                             n_kv_heads=8, head_dim=128, max_context=32768, seed=3),
    # latent cache: d_c = 512 latent + 64 rotary key per row, 16 heads
    "mla_latent_bf16": dict(attn="mla", dtype="bf16", n_layers=1, batch=32, n_heads=16,
                            latent_dim=512, rope_dim=64, nope_dim=128, v_dim=128,
                            max_context=4096, w_std=0.02, seed=4),
}


def f32_to_bf16_bits(x):
    """float32 array -> bf16 bit patterns (uint16), round to nearest, ties to even.

    NaN becomes the quiet NaN 0x7FC0 (sign kept); overflow rounds to +-inf.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) & np.uint32(0x8000)).astype(np.uint16) | np.uint16(0x7FC0)
    return r


def draw(rng, shape, dtype, std=1.0):
    """N(0, std^2) draws stored as fp32 (float32 array) or bf16 (uint16 bits)."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x = (x * np.float32(std)).astype(np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def gqa_valid_lens(cfg, rng):
    """Per-sequence valid lengths of a decode step (the appended row included)."""
    B, S = cfg["batch"], cfg["max_context"]
    if "valid_lo" in cfg:
        return rng.integers(cfg["valid_lo"], cfg["valid_hi"] + 1, size=B).astype(np.int32)
    return np.full(B, S, dtype=np.int32)


def gqa_layer(cfg, seed_offset=0, fill_rows=None, rng=None):
    """One layer's worth of inputs for a decode step on a GQA/MHA/MQA cache.

    Returns a dict:
      k_fill, v_fill  [B, H_kv, fill_rows, D]  rows written by the prefill fill
      k_new, v_new    [B, H_kv, 1, D]           the appended token
      q               [B, H, D]
      valid_lens      [B] int32  (n_b, appended row included)
      cache_index     [B] int32  (= n_b - 1: append, then attend [0, n_b))
      sm_scale        float
    """
    if rng is None:
        rng = np.random.default_rng(cfg["seed"] + 1000 * seed_offset)
    B, H, Hkv, D, S = (cfg["batch"], cfg["n_heads"], cfg["n_kv_heads"],
                       cfg["head_dim"], cfg["max_context"])
    dt = "bf16" if cfg["dtype"] == "i8" else cfg["dtype"]  # an int8 cache takes bf16 rows
    T = S if fill_rows is None else fill_rows
    valid = gqa_valid_lens(cfg, rng)
    out = dict(
        k_fill=draw(rng, (B, Hkv, T, D), dt),
        v_fill=draw(rng, (B, Hkv, T, D), dt),
        k_new=draw(rng, (B, Hkv, 1, D), dt),
        v_new=draw(rng, (B, Hkv, 1, D), dt),
        q=draw(rng, (B, H, D), dt),
        valid_lens=valid,
        cache_index=(valid - 1).astype(np.int32),
        sm_scale=1.0 / math.sqrt(D),
    )
    return out


def tiny_sequence(cfg):
    """The tiny fp32 MHA case: one sequence of prefill + steps tokens.

    Returns k, v [B, H_kv, T, D] for all T = prefill + steps tokens and
    q [steps, B, H, D] already multiplied by 1/sqrt(D) (fp32), sm_scale = 1.
    """
    rng = np.random.default_rng(cfg["seed"])
    B, H, Hkv, D = cfg["batch"], cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    T = cfg["prefill"] + cfg["steps"]
    k = draw(rng, (B, Hkv, T, D), "f32")
    v = draw(rng, (B, Hkv, T, D), "f32")
    q = draw(rng, (cfg["steps"], B, H, D), "f32")
    q = (q * np.float32(1.0 / math.sqrt(D))).astype(np.float32)
    return dict(k=k, v=v, q=q, sm_scale=1.0)


def mla_layer(cfg, seed_offset=0, fill_rows=None, rng=None):
    """One layer's worth of inputs for a decode step on a latent (MLA) cache.

    Returns a dict:
      rows_fill  [B, fill_rows, d_c + d_R]   latent + rotary key rows
      rows_new   [B, 1, d_c + d_R]
      q_nope     [B, H, nope_dim];  q_rope [B, H, d_R]
      w_uk       [H, nope_dim, d_c]; w_uv [H, d_c, v_dim]   (std w_std)
      valid_lens, cache_index [B] int32; sm_scale = 1/sqrt(nope_dim + d_R)
    """
    if rng is None:
        rng = np.random.default_rng(cfg["seed"] + 1000 * seed_offset)
    B, H, S = cfg["batch"], cfg["n_heads"], cfg["max_context"]
    dc, dr, dn, dv = cfg["latent_dim"], cfg["rope_dim"], cfg["nope_dim"], cfg["v_dim"]
    dt = cfg["dtype"]
    T = S if fill_rows is None else fill_rows
    if "valid_lo" in cfg:
        valid = rng.integers(cfg["valid_lo"], cfg["valid_hi"] + 1, size=B).astype(np.int32)
    else:
        valid = np.full(B, S, dtype=np.int32)
    return dict(
        rows_fill=draw(rng, (B, T, dc + dr), dt),
        rows_new=draw(rng, (B, 1, dc + dr), dt),
        q_nope=draw(rng, (B, H, dn), dt),
        q_rope=draw(rng, (B, H, dr), dt),
        w_uk=draw(rng, (H, dn, dc), dt, std=cfg["w_std"]),
        w_uv=draw(rng, (H, dc, dv), dt, std=cfg["w_std"]),
        valid_lens=valid,
        cache_index=(valid - 1).astype(np.int32),
        sm_scale=1.0 / math.sqrt(dn + dr),
    )


def random_gqa_case(seed, batch, n_heads, n_kv_heads, head_dim, max_context, dtype,
                    valid_lens=None, fill_rows=None):
    """Small random case for parity tests; valid_lens default U[1, S]."""
    rng = np.random.default_rng(seed)
    cfg = dict(batch=batch, n_heads=n_heads, n_kv_heads=n_kv_heads, head_dim=head_dim,
               max_context=max_context, dtype=dtype, seed=seed)
    if valid_lens is None:
        valid_lens = rng.integers(1, max_context + 1, size=batch)
    d = gqa_layer(cfg, fill_rows=fill_rows, rng=rng)
    d["valid_lens"] = np.asarray(valid_lens, dtype=np.int32)
    d["cache_index"] = (d["valid_lens"] - 1).astype(np.int32)
    return d
