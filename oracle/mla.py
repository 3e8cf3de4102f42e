"""Latent (MLA) decode attention (oracle; test infrastructure only).

Sources:
* "10.3 - KV cache implementation details", section 4.3: cache a latent
  c in R^{d_c} per token and rebuild keys and values from it with low-rank
  up-projections; DeepSeek-V2 uses d_c = 512 against 16 heads of width 128.
* "KV-Cache Mechanics", "AR Static KV-Cache" note and the MHA/GQA/MLA
  comparison: MLA stores a compressed latent per token and decompresses it
  during attention, paying an "absorb" overhead per decode step.

Readings taken (the pages do not spell them out):
* per-head up-projections W_UK[h] of shape [d_nope, d_c] (key) and
  W_UV[h] of shape [d_c, d_v] (value), d_nope = d_v = 128;
* each cache row holds the latent c_j (d_c entries) followed by a decoupled
  rotary key kR_j (d_R entries) shared by all heads, stored already rotated;
* head h's key for token j is [W_UK[h] c_j ; kR_j] and its value is
  W_UV[h]^T c_j; the query is [q_nope ; q_rope];
* "absorbing" W_UK into the query (q~ = W_UK[h]^T q_nope) and W_UV into the
  output (o = W_UV[h]^T o~) gives the same result by associativity.

Functions
---------
mla_decode_materialized  rebuild k, v per head, then plain attention
mla_decode_absorbed      absorbed form: attention over the latent rows
latent_attention         attention of absorbed queries over latent rows
                         (the part that reads the cache)
absorb_query             q~ = [W_UK[h]^T q_nope ; q_rope]
"""

import numpy as np

from .codec import widen
from .attention import softmax_weighted_sum


def absorb_query(q_nope, q_rope, w_uk):
    """q_nope [B,H,dn], q_rope [B,H,dR], w_uk [H,dn,dc] -> q~ [B,H,dc+dR] float64."""
    q_nope = widen(q_nope)
    q_rope = widen(q_rope)
    w_uk = widen(w_uk)
    B, H, _ = q_nope.shape
    d_c = w_uk.shape[2]
    q_lat = np.zeros((B, H, d_c), dtype=np.float64)
    for h in range(H):
        q_lat[:, h, :] = q_nope[:, h, :] @ w_uk[h]          # sum_i q_i W_UK[h, i, c]
    return np.concatenate([q_lat, q_rope], axis=2)


def latent_attention(q_abs, rows, valid_lens, sm_scale, latent_dim):
    """Attention of absorbed queries over the latent rows.

    q_abs: [B, H, d_c + d_R]; rows: [B, S, d_c + d_R] (one layer of the latent
    cache). The score of token j is sm_scale * q_abs . row_j (latent and rope
    parts together); the value of token j is the latent part row_j[:d_c].
    Returns the latent output o~ [B, H, d_c] float64; n_b = 0 gives zeros.
    """
    q_abs = widen(q_abs)
    B, H, W = q_abs.shape
    out = np.zeros((B, H, latent_dim), dtype=np.float64)
    for b in range(B):
        n = int(valid_lens[b])
        if n == 0:
            continue
        r = widen(rows[b, :n])                 # [n, W]
        for h in range(H):
            scores = sm_scale * (r @ q_abs[b, h])
            out[b, h] = softmax_weighted_sum(scores, r[:, :latent_dim])
    return out


def mla_decode_absorbed(q_nope, q_rope, w_uk, w_uv, rows, valid_lens, sm_scale):
    """Absorbed MLA decode: q~ = W_UK^T q_nope, attend over latents, o = W_UV^T o~."""
    w_uv = widen(w_uv)
    d_c = w_uv.shape[1]
    q_abs = absorb_query(q_nope, q_rope, w_uk)
    o_lat = latent_attention(q_abs, rows, valid_lens, sm_scale, d_c)
    B, H, _ = o_lat.shape
    out = np.zeros((B, H, w_uv.shape[2]), dtype=np.float64)
    for h in range(H):
        out[:, h, :] = o_lat[:, h, :] @ w_uv[h]             # sum_c o~_c W_UV[h, c, i]
    return out


def mla_decode_materialized(q_nope, q_rope, w_uk, w_uv, rows, valid_lens, sm_scale):
    """MLA decode with keys and values rebuilt per head from the latent."""
    q_nope = widen(q_nope)
    q_rope = widen(q_rope)
    w_uk = widen(w_uk)
    w_uv = widen(w_uv)
    B, H, _ = q_nope.shape
    d_c = w_uk.shape[2]
    d_v = w_uv.shape[2]
    out = np.zeros((B, H, d_v), dtype=np.float64)
    for b in range(B):
        n = int(valid_lens[b])
        if n == 0:
            continue
        r = widen(rows[b, :n])
        c = r[:, :d_c]                         # latents  [n, d_c]
        k_rope = r[:, d_c:]                    # rotary keys [n, d_R]
        for h in range(H):
            k_nope = c @ w_uk[h].T             # [n, d_nope]: W_UK[h] c_j
            keys = np.concatenate([k_nope, k_rope], axis=1)
            vals = c @ w_uv[h]                 # [n, d_v]: W_UV[h]^T c_j
            q = np.concatenate([q_nope[b, h], q_rope[b, h]])
            scores = sm_scale * (keys @ q)
            out[b, h] = softmax_weighted_sum(scores, vals)
    return out
