"""int8 storage of the static cache, one float32 scale per row (oracle; test infrastructure only).

Sources:
* "10.3 - KV cache implementation details", section 4.4: independently of
  the attention kind, the cache itself can be stored in lower precision;
  int8 instead of 16-bit halves the memory at a small quality cost, and the
  byte formula takes p_cache = 1.
* "KV Cache Optimization: GQA Audit, In-Place Buffers, Persistent Prompts",
  "#2 ... Mutual exclusion": a quantisation that needs runtime
  re-quantisation does not compose with a fixed-capacity buffer. Here every
  row is quantised exactly once, when it is written, and never again, so
  the in-place append of "#2 ... After" is unchanged: it slice-assigns the
  new rows' codes and scales and no other byte of the cache changes.

Readings taken where the pages are silent (listed in the design notes):
* granularity: one scale per cached row of one key/value head (per token,
  per head, separately for K and V); symmetric, no zero point;
* codes: with amax = max_i |x_i| over the row's head_dim elements,
      scale  = amax / 127
      code_i = round_half_even(x_i * (127 / amax)), clamped to [-127, 127]
  every operation in IEEE binary32, the precision the kernel uses, so the
  oracle and the kernel decide identical codes (a quantised code is an
  integer decided by floating point). A row of zeros gets scale 0 and codes 0.
* the value a stored element stands for is code_i * scale (exact in
  float64), and attention is the plain definition over those values;
* the interface types stay bf16: the rows handed in and the queries and
  outputs are bf16, only the cache is int8.
Inputs are finite; a row holding inf or NaN has no defined codes.
"""

import numpy as np

from .codec import widen


def _to_f32(x):
    """bf16 bit patterns (uint16) or float32 values -> float32 values (exact)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if x.dtype == np.float32:
        return x
    raise TypeError(f"expected bf16 bits or float32, got {x.dtype}")


def quantize_rows(x):
    """Per-row symmetric int8 codes of x [..., D]: returns (codes int8 [..., D], scale float32 [...])."""
    x = _to_f32(x)
    amax = np.max(np.abs(x), axis=-1)                       # float32, exact
    zero = amax == np.float32(0)
    safe = np.where(zero, np.float32(1), amax)
    with np.errstate(over="ignore"):
        inv = (np.float32(127) / safe).astype(np.float32)   # binary32 division
        scaled = (x * inv[..., None]).astype(np.float32)    # binary32 product, no fusion
    codes = np.clip(np.rint(scaled), -127, 127)             # rint: round half to even
    codes = np.where(zero[..., None], 0, codes).astype(np.int8)
    scale = np.where(zero, np.float32(0), (amax / np.float32(127)).astype(np.float32)).astype(np.float32)
    return codes, scale


def dequantize(codes, scale):
    """The values the stored rows stand for: code * scale, float64 [..., D]."""
    return np.asarray(codes).astype(np.float64) * np.asarray(scale).astype(np.float64)[..., None]


class RefQuantCache:
    """Static int8 K/V cache: codes [L][2][B][H_kv][S][D] and scales [L][2][B][H_kv][S] (float32)."""

    def __init__(self, n_layers, batch, n_kv_heads, max_context, head_dim):
        self.shape = (n_layers, 2, batch, n_kv_heads, max_context, head_dim)
        # allocated once, zero-filled (codes 0, scale 0 = value 0), never resized
        self.codes = np.zeros(self.shape, dtype=np.int8)
        self.scales = np.zeros(self.shape[:-1], dtype=np.float32)

    @property
    def max_context(self):
        return self.shape[4]

    def keys(self, layer):
        """float64 [B, H_kv, S, D] values the key rows stand for."""
        return dequantize(self.codes[layer, 0], self.scales[layer, 0])

    def values(self, layer):
        return dequantize(self.codes[layer, 1], self.scales[layer, 1])

    def _write(self, layer, kv, b_sel, rows, x):
        codes, scale = quantize_rows(x)
        self.codes[layer, kv, b_sel, :, rows, :] = codes
        self.scales[layer, kv, b_sel, :, rows] = scale

    def fill(self, layer, k, v, start):
        """Quantise and write rows [start, start + t) of every (b, g) from k, v [B, H_kv, t, D] (bf16 bits)."""
        k = _to_f32(k)
        v = _to_f32(v)
        t = k.shape[2]
        if start < 0 or t < 1 or start + t > self.max_context:
            raise ValueError("fill outside the allocated capacity")
        for kv, x in ((0, k), (1, v)):
            codes, scale = quantize_rows(x)
            self.codes[layer, kv, :, :, start:start + t, :] = codes
            self.scales[layer, kv, :, :, start:start + t] = scale

    def append(self, layer, k_new, v_new, cache_index):
        """Quantise and slice-assign rows [ci_b, ci_b + t_new) of sequence b; returns the skipped sequences."""
        k_new = _to_f32(k_new)
        v_new = _to_f32(v_new)
        t_new = k_new.shape[2]
        skipped = []
        for b, ci in enumerate(np.asarray(cache_index).tolist()):
            if ci < 0 or ci + t_new > self.max_context:
                skipped.append(b)
                continue
            for kv, x in ((0, k_new), (1, v_new)):
                codes, scale = quantize_rows(x[b])
                self.codes[layer, kv, b, :, ci:ci + t_new, :] = codes
                self.scales[layer, kv, b, :, ci:ci + t_new] = scale
        return skipped


def int8_cache_bytes(n_layers, n_kv_heads, head_dim, n_ctx, batch):
    """Physical bytes of the int8 cache: the section 4.4 formula at p_cache = 1 for the
    codes, plus one float32 scale per cached row of K and of V (4 bytes each)."""
    rows = 2 * n_layers * n_kv_heads * n_ctx * batch
    return rows * head_dim * 1 + rows * 4


def widen_query(q):
    """bf16 query bits -> float64 (the queries stay bf16 on an int8 cache)."""
    return widen(q)
