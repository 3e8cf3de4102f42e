"""Byte accounting of a static KV cache (oracle; test infrastructure only).

Sources:
* "10.3 - KV cache implementation details", section 2 (boxed formula
  2 * n_layers * n_heads * d_head * n_ctx * B * p), section 2.2 (bytes per
  token), section 4.1-4.4 (MQA / GQA / MLA / quantised variants) and
  section 9 item 1 (the formula written with n_kv_heads).
* "KV-Cache Mechanics", "Memory Formula" (L * 2 * S * H_kv * d_h * bytes).
* "Key-value cache" lesson record, "Payload estimate" and the science
  equation (M_KV = 2 B L T Hkv Dh s; per-token growth 2 L Hkv Dh s).

All results are exact Python integers (p may be 0.5 for int4, in which case
the product is still an integer for any even element count; a non-integer
result raises).
"""

from fractions import Fraction


def _exact(x):
    x = Fraction(x)
    if x.denominator != 1:
        raise ValueError(f"byte count {x} is not an integer")
    return int(x)


def kv_cache_bytes(n_layers, n_kv_heads, head_dim, n_ctx, batch, bytes_per_elem):
    """Physical bytes of K and V for every layer: 2 * L * H_kv * d_h * S * B * p.

    The leading 2 counts the two tensors (keys and values). For MHA pass
    n_kv_heads = n_heads; for MQA pass 1; for GQA pass the group count g.
    """
    return _exact(2 * n_layers * n_kv_heads * head_dim * n_ctx * batch * Fraction(bytes_per_elem))


def kv_bytes_per_token(n_layers, n_kv_heads, head_dim, bytes_per_elem):
    """Growth per retained position of one sequence: 2 * L * H_kv * d_h * p."""
    return _exact(2 * n_layers * n_kv_heads * head_dim * Fraction(bytes_per_elem))


def mla_cache_bytes(n_layers, latent_dim, n_ctx, batch, bytes_per_elem, rope_dim=0):
    """Latent (MLA) cache: n_layers * (d_c + d_R) * n_ctx * B * p.

    One tensor only (no factor 2): the latent is stored once per token and
    keys/values are reconstructed from it. ``rope_dim`` is the width of a
    decoupled rotary key stored beside the latent in the same row; with
    rope_dim = 0 this is exactly the page's formula.
    """
    return _exact(n_layers * (latent_dim + rope_dim) * n_ctx * batch * Fraction(bytes_per_elem))


def logical_kv_bytes(n_layers, n_kv_heads, head_dim, valid_lens, bytes_per_elem):
    """Bytes that the live prefixes occupy: 2 * L * H_kv * d_h * p * sum_b n_b.

    This is the page's formula with n_ctx * B replaced by the per-sequence
    valid lengths (the pre-allocated buffer's logical, as opposed to
    physical, size).
    """
    total = sum(int(n) for n in valid_lens)
    return _exact(2 * n_layers * n_kv_heads * head_dim * total * Fraction(bytes_per_elem))


def logical_mla_bytes(n_layers, latent_dim, valid_lens, bytes_per_elem, rope_dim=0):
    total = sum(int(n) for n in valid_lens)
    return _exact(n_layers * (latent_dim + rope_dim) * total * Fraction(bytes_per_elem))
