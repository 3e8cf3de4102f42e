"""Oracle latent (MLA) decode: absorbed vs materialised identity and a
library-routine pin."""

import numpy as np
import torch
import torch.nn.functional as F

from oracle import mla
from oracle.attention import decode_attention
from static_kv_cache_amd import synthetic


def _case(seed=31, B=2, H=4, S=9, dc=16, dr=4, dn=8, dv=8):
    rng = np.random.default_rng(seed)
    return dict(q_nope=rng.standard_normal((B, H, dn)), q_rope=rng.standard_normal((B, H, dr)),
                w_uk=0.3 * rng.standard_normal((H, dn, dc)), w_uv=0.3 * rng.standard_normal((H, dc, dv)),
                rows=rng.standard_normal((B, S, dc + dr)), valid=np.array([S, 4][:B]), scale=0.45)


def test_absorbed_equals_materialized():
    c = _case()
    a = mla.mla_decode_absorbed(c["q_nope"], c["q_rope"], c["w_uk"], c["w_uv"], c["rows"], c["valid"], c["scale"])
    m = mla.mla_decode_materialized(c["q_nope"], c["q_rope"], c["w_uk"], c["w_uv"], c["rows"], c["valid"], c["scale"])
    assert np.allclose(a, m, rtol=0, atol=1e-12)


def test_materialized_matches_library_sdpa():
    """Rebuild per-head keys [W_UK c ; kR] and values W_UV^T c explicitly with
    torch, then torch's float64 SDPA must match the oracle."""
    c = _case(seed=32)
    dc = c["w_uk"].shape[2]
    out = mla.mla_decode_absorbed(c["q_nope"], c["q_rope"], c["w_uk"], c["w_uv"], c["rows"], c["valid"], c["scale"])
    B, H, _ = c["q_nope"].shape
    for b in range(B):
        n = int(c["valid"][b])
        r = torch.from_numpy(c["rows"][b, :n])
        lat, kr = r[:, :dc], r[:, dc:]
        wuk = torch.from_numpy(c["w_uk"])
        wuv = torch.from_numpy(c["w_uv"])
        keys = torch.cat([torch.einsum("hic,jc->hji", wuk, lat), kr[None].expand(H, n, -1)], dim=2)
        vals = torch.einsum("hcv,jc->hjv", wuv, lat)
        q = torch.cat([torch.from_numpy(c["q_nope"][b]), torch.from_numpy(c["q_rope"][b])], dim=1)[:, None]
        o = F.scaled_dot_product_attention(q[None], keys[None], vals[None], scale=c["scale"])[0, :, 0]
        assert np.allclose(out[b], o.numpy(), rtol=0, atol=1e-12)


def test_latent_attention_reduces_to_mqa():
    """The latent part of the cache acts as one shared key AND value head: with
    d_R = 0, latent attention equals decode attention with H_kv = 1 and K = V."""
    rng = np.random.default_rng(33)
    B, H, S, dc = 2, 4, 6, 8
    rows = rng.standard_normal((B, S, dc))
    q = rng.standard_normal((B, H, dc))
    n = np.array([6, 2])
    a = mla.latent_attention(q, rows, n, 0.6, dc)
    kv = rows[:, None]                       # [B, 1, S, dc]
    assert np.allclose(a, decode_attention(q, kv, kv, n, 0.6), rtol=0, atol=1e-13)


def test_rope_part_scores_but_is_not_a_value():
    """The rotary key columns move the scores but never appear in the output."""
    rng = np.random.default_rng(34)
    B, H, S, dc, dr = 1, 2, 5, 6, 3
    rows = rng.standard_normal((B, S, dc + dr))
    q = rng.standard_normal((B, H, dc + dr))
    a = mla.latent_attention(q, rows, [S], 0.5, dc)
    assert a.shape == (B, H, dc)
    q0 = q.copy()
    q0[..., dc:] = 0.0
    b = mla.latent_attention(q0, rows, [S], 0.5, dc)
    assert np.allclose(b, mla.latent_attention(q0[..., :dc], rows[..., :dc], [S], 0.5, dc), atol=1e-13)
    assert not np.allclose(a, b)


def test_workload_inputs_shapes():
    cfg = dict(synthetic.WORKLOADS["mla_latent_bf16"], batch=2, max_context=8)
    d = synthetic.mla_layer(cfg)
    assert d["rows_fill"].shape == (2, 8, 576) and d["w_uk"].shape == (16, 128, 512)
    assert d["w_uv"].shape == (16, 512, 128) and abs(d["sm_scale"] - 1 / np.sqrt(192)) < 1e-15
