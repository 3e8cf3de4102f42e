"""Decode attention over the static cache, and the no-cache reference
(oracle; test infrastructure only).

Sources:
* "10.3 - KV cache implementation details", section 5 step 2: the query of a
  decode step is one row; keys and values are the whole cache;
  attn = softmax(q K^T / sqrt(d_head)) V; this is the only place the cache is
  read. Section 4.2: g key/value groups, each shared by n_heads / g query
  heads; section 4.1: MQA is the case of a single key/value head.
* "KV Cache Optimization: GQA Audit, In-Place Buffers, Persistent Prompts",
  "#2 ... After": reads slice the buffer to the valid length, so rows past it
  are never attended.
* "KV-Cache Mechanics", "Disabling the Cache": generation without the cache
  recomputes everything and must give the same result.

Readings taken where the pages are silent (each listed in the design notes):
* head h uses key/value head g = h // (H / H_kv) (contiguous groups);
* n_b = 0 gives an all-zero output row;
* the softmax scale is an explicit argument (1/sqrt(d_head) on the page).

The decode function computes the plain definition (the GPU path reaches the
same real-number result by re-association: split context, online softmax,
merge). Subtracting the maximum logit before exponentiating is the usual
exact rewriting of softmax and does not change the value.
"""

import numpy as np

from .codec import widen


def softmax_weighted_sum(scores, values):
    """softmax(scores) @ values for one query; scores [n], values [n, D]; n >= 1."""
    m = np.max(scores)
    p = np.exp(scores - m)
    return (p @ values) / np.sum(p)


def decode_attention(q, k_cache, v_cache, valid_lens, sm_scale):
    """Single-query attention of every query head against cache rows [0, n_b).

    q:        [B, H, D]        stored values (fp32 / bf16 bits / float64)
    k_cache:  [B, H_kv, S, D]  one layer of the cache
    v_cache:  [B, H_kv, S, D]
    valid_lens: [B] integers, 0 <= n_b <= S
    Returns float64 [B, H, D].
    """
    q = widen(q)
    B, H, D = q.shape
    H_kv = k_cache.shape[1]
    if H % H_kv != 0:
        raise ValueError("n_heads must be a multiple of n_kv_heads")
    group = H // H_kv
    out = np.zeros((B, H, D), dtype=np.float64)
    for b in range(B):
        n = int(valid_lens[b])
        if n == 0:
            continue
        for h in range(H):
            g = h // group
            keys = widen(k_cache[b, g, :n])      # [n, D]; rows >= n never touched
            vals = widen(v_cache[b, g, :n])
            scores = sm_scale * (keys @ q[b, h])
            out[b, h] = softmax_weighted_sum(scores, vals)
    return out


def causal_attention_nocache(q_seq, k_seq, v_seq, sm_scale):
    """Generation without a cache: recompute attention for every position.

    q_seq: [T, H, D]; k_seq, v_seq: [T, H_kv, D] (one sequence). Position i
    attends positions 0..i. Keys and values are gathered by growing a Python
    list token by token (concatenation semantics, no pre-allocated buffer),
    which shares nothing with the buffer model.
    Returns float64 [T, H, D].
    """
    q_seq = widen(q_seq)
    k_seq = widen(k_seq)
    v_seq = widen(v_seq)
    T, H, D = q_seq.shape
    H_kv = k_seq.shape[1]
    group = H // H_kv
    out = np.zeros((T, H, D), dtype=np.float64)
    past_k, past_v = [], []
    for i in range(T):
        past_k.append(k_seq[i])
        past_v.append(v_seq[i])
        keys = np.stack(past_k)   # [i+1, H_kv, D]
        vals = np.stack(past_v)
        for h in range(H):
            g = h // group
            scores = sm_scale * (keys[:, g, :] @ q_seq[i, h])
            out[i, h] = softmax_weighted_sum(scores, vals[:, g, :])
    return out


def prefill_attention(q, k_cache, v_cache, start, sm_scale):
    """Causal attention of t new queries over a cache that already holds their rows.

    "KV-Cache Mechanics", "AR Static KV-Cache": the prompt's forward pass fills
    the cache from cache_index 0 (a later chunk continues at cache_index =
    start); "10.3 - KV cache implementation details", section 3: query i of
    the chunk (position start + i) attends positions 0 .. start + i.
    q: [B, H, t, D]; k_cache, v_cache: [B, H_kv, S, D] holding rows
    [0, start + t). Written as the masked matrix form of that definition:
    for each (b, h), scores = sm_scale * Q K^T over the n = start + t rows,
    entries with key position > query position removed (weight 0), a
    row-wise softmax and the product with V; each row is then the decode of
    its position with valid length start + i + 1. Returns float64 [B, H, t, D].
    """
    q = widen(q)
    B, H, t, D = q.shape
    H_kv = k_cache.shape[1]
    group = H // H_kv
    n = start + t
    allowed = np.arange(n)[None, :] <= (start + np.arange(t))[:, None]   # [t, n]
    out = np.zeros((B, H, t, D), dtype=np.float64)
    for b in range(B):
        for g in range(H_kv):
            keys = widen(k_cache[b, g, :n])      # [n, D]; rows >= n never touched
            vals = widen(v_cache[b, g, :n])
            for h in range(g * group, (g + 1) * group):
                scores = np.where(allowed, sm_scale * (q[b, h] @ keys.T), -np.inf)
                m = np.max(scores, axis=1, keepdims=True)
                p = np.exp(scores - m)              # exp(-inf) = 0 for the removed entries
                out[b, h] = (p @ vals) / np.sum(p, axis=1, keepdims=True)
    return out


def repeat_kv_heads(x, group):
    """[B, H_kv, S, D] -> [B, H_kv * group, S, D], each key/value head repeated
    ``group`` times contiguously (GQA written as MHA)."""
    return np.repeat(np.asarray(x), group, axis=1)
