"""Bit-exact model of the static, pre-allocated KV cache (oracle; test infrastructure only).

Sources:
* "KV-Cache Mechanics", "AR Static KV-Cache": one array of shape
  [B, H_kv, max_context, head_size] per layer, allocated once; prefill writes
  from cache_index = 0, each decode step writes at cache_index = T_prompt
  (then one further per step).
* "KV Cache Optimization: GQA Audit, In-Place Buffers, Persistent Prompts",
  "#2 In-place KV cache updates", "After": the buffer has fixed capacity and
  every append slice-assigns the new rows [valid, valid + tNew) of keys and
  values; nothing else changes. "#1": the persisted layout is
  [B, nKvHeads, T, headDim] (key/value heads, not query heads).
* "10.3 - KV cache implementation details", section 5 step 2: the new token's
  k and v are appended to the layer's cache before attention reads it.
* "Key-value cache" lesson record, "mechanism": store each new token's keys
  and values for every layer; release or reuse the allocation afterwards.

The model holds raw element bits (uint32 for fp32, uint16 for bf16) in the
same layout the device buffer uses, so a device buffer can be compared with
it byte for byte:

    GQA/MHA/MQA cache: [L][2 (K, V)][B][H_kv][S][D], D fastest
    MLA latent cache:  [L][B][S][W],  W = latent_dim + rope_dim, W fastest

Out-of-range appends (a sequence whose cache_index < 0 or
cache_index + t_new > S) leave that sequence untouched and are reported in
the returned list; the buffer never grows (no regrowth, no concat).
"""

import numpy as np

_BITS = {"f32": np.uint32, "bf16": np.uint16}


def _as_bits(x, storage):
    x = np.asarray(x)
    want = _BITS[storage]
    if x.dtype == want:
        return x
    if storage == "f32" and x.dtype == np.float32:
        return x.view(np.uint32)
    raise TypeError(f"expected {storage} bits, got {x.dtype}")


class RefCache:
    """Static K/V cache for MHA / GQA / MQA: [L][2][B][H_kv][S][D] stored bits."""

    def __init__(self, n_layers, batch, n_kv_heads, max_context, head_dim, storage):
        if storage not in _BITS:
            raise ValueError(storage)
        self.storage = storage
        self.shape = (n_layers, 2, batch, n_kv_heads, max_context, head_dim)
        # allocated once, zero-filled, never resized
        self.buf = np.zeros(self.shape, dtype=_BITS[storage])

    @property
    def max_context(self):
        return self.shape[4]

    def keys(self, layer):
        return self.buf[layer, 0]

    def values(self, layer):
        return self.buf[layer, 1]

    def fill(self, layer, k, v, start):
        """Write rows [start, start + t) of every (b, g) from k, v of shape [B, H_kv, t, D]."""
        k = _as_bits(k, self.storage)
        v = _as_bits(v, self.storage)
        t = k.shape[2]
        if start < 0 or t < 1 or start + t > self.max_context:
            raise ValueError("fill outside the allocated capacity")
        self.buf[layer, 0, :, :, start:start + t, :] = k
        self.buf[layer, 1, :, :, start:start + t, :] = v

    def append(self, layer, k_new, v_new, cache_index):
        """Slice-assign rows [ci_b, ci_b + t_new) of sequence b for every b.

        k_new, v_new: [B, H_kv, t_new, D]; cache_index: [B] integers.
        Returns the list of sequences skipped because they were out of range.
        """
        k_new = _as_bits(k_new, self.storage)
        v_new = _as_bits(v_new, self.storage)
        t_new = k_new.shape[2]
        skipped = []
        for b, ci in enumerate(np.asarray(cache_index).tolist()):
            if ci < 0 or ci + t_new > self.max_context:
                skipped.append(b)
                continue
            self.buf[layer, 0, b, :, ci:ci + t_new, :] = k_new[b]
            self.buf[layer, 1, b, :, ci:ci + t_new, :] = v_new[b]
        return skipped

    def as_bytes(self):
        return self.buf.tobytes()


class RefLatentCache:
    """Static latent (MLA) cache: [L][B][S][W] stored bits, W = d_c + d_R.

    "10.3 - KV cache implementation details", section 4.3: one latent vector
    per token (a single tensor, not K and V). The decoupled rotary key of
    width d_R is stored in the same row after the d_c latent entries.
    """

    def __init__(self, n_layers, batch, max_context, row_width, storage):
        if storage not in _BITS:
            raise ValueError(storage)
        self.storage = storage
        self.shape = (n_layers, batch, max_context, row_width)
        self.buf = np.zeros(self.shape, dtype=_BITS[storage])

    @property
    def max_context(self):
        return self.shape[2]

    def rows(self, layer):
        return self.buf[layer]

    def fill(self, layer, rows, start):
        """rows: [B, t, W]."""
        rows = _as_bits(rows, self.storage)
        t = rows.shape[1]
        if start < 0 or t < 1 or start + t > self.max_context:
            raise ValueError("fill outside the allocated capacity")
        self.buf[layer, :, start:start + t, :] = rows

    def append(self, layer, rows_new, cache_index):
        """rows_new: [B, t_new, W]; cache_index: [B]. Returns skipped sequences."""
        rows_new = _as_bits(rows_new, self.storage)
        t_new = rows_new.shape[1]
        skipped = []
        for b, ci in enumerate(np.asarray(cache_index).tolist()):
            if ci < 0 or ci + t_new > self.max_context:
                skipped.append(b)
                continue
            self.buf[layer, b, ci:ci + t_new, :] = rows_new[b]
        return skipped

    def as_bytes(self):
        return self.buf.tobytes()
