"""Saving and loading the live prefix of a static cache (oracle; test infrastructure only).

Sources:
* "KV Cache Optimization: GQA Audit, In-Place Buffers, Persistent Prompts",
  "#3 Persistent KV across sessions": the cache after the prompt's prefill is
  saved once and loaded by later runs, which then skip the prefill and give
  identical output; its file map: a pre-allocated cache saves only its live
  prefix, and loading sets the valid lengths from what was saved.
* "10.3 - KV cache implementation details", section 7.3: requests that share
  a prefix can reuse its K/V.

The pages fix no byte format. Readings taken (listed in the design notes):
* the image is a header followed by the payload. Header, little-endian:
  int32 words [magic, version, the ten descriptor fields (attn, dtype,
  n_layers, batch, n_heads, n_kv_heads, head_dim, max_context, latent_dim,
  rope_dim), header bytes, 0] (56 bytes), then the payload bytes as uint64,
  then from byte 64 the batch's valid lengths as int32, zero-padded to a
  multiple of 256 bytes;
* payload: for each layer, for K then V (the latent cache has one tensor),
  for each sequence, for each kv head, its rows [0, n_b) in order: the live
  rows only, packed, as stored. For an int8 cache all codes come first, then
  the float32 row scales in the same order. Its size is the cache's logical
  bytes for those lengths;
* loading writes saved sequence src[b] into rows [0, n) of sequence b of a
  cache with the same layers, kv heads, row width and dtype (batch, query
  heads and capacity may differ); src[b] = -1 leaves b alone, and several
  sequences may name one saved sequence (a shared prefix). Rows at or past n
  are not touched.
"""

import struct

import numpy as np

MAGIC = 0x3143564B  # "KVC1" as little-endian bytes
VERSION = 1
DESC_FIELDS = ("attn", "dtype", "n_layers", "batch", "n_heads", "n_kv_heads", "head_dim", "max_context",
               "latent_dim", "rope_dim")


def header_bytes(batch):
    n = 4 * (16 + batch)
    return (n + 255) // 256 * 256


def _tensors(cache):
    """The stored tensors of a cache model, each viewed as [L][KV][B][G][S][...], in payload order."""
    if hasattr(cache, "codes"):  # int8: codes [L][2][B][G][S][D], scales [L][2][B][G][S]
        return [cache.codes, cache.scales]
    if cache.buf.ndim == 4:  # latent [L][B][S][W] -> [L][1][B][1][S][W]
        return [cache.buf[:, None, :, None]]
    return [cache.buf]


def pack(cache, desc, valid_lens):
    """Image bytes of the live prefix [0, n_b) of every layer and sequence of `cache`."""
    lens = [int(x) for x in valid_lens]
    parts = []
    for t in _tensors(cache):
        L, KV, B, G = t.shape[:4]
        assert B == len(lens)
        for layer in range(L):
            for kv in range(KV):
                for b in range(B):
                    for g in range(G):
                        parts.append(np.ascontiguousarray(t[layer, kv, b, g, :lens[b]]).tobytes())
    payload = b"".join(parts)
    hdr = struct.pack("<14i", MAGIC, VERSION, *[int(desc[f]) for f in DESC_FIELDS], header_bytes(len(lens)), 0)
    hdr += struct.pack("<Q", len(payload)) + struct.pack(f"<{len(lens)}i", *lens)
    hdr += b"\0" * (header_bytes(len(lens)) - len(hdr))
    return hdr + payload


def parse_header(image):
    """(descriptor dict, lengths, header bytes, payload bytes) of an image."""
    w = struct.unpack_from("<14i", image, 0)
    if w[0] != MAGIC or w[1] != VERSION:
        raise ValueError("not a prefix image")
    desc = dict(zip(DESC_FIELDS, w[2:12]))
    hb = w[12]
    (payload,) = struct.unpack_from("<Q", image, 56)
    lens = list(struct.unpack_from(f"<{desc['batch']}i", image, 64))
    return desc, lens, hb, payload


def unpack(image, cache, src):
    """Write saved sequence src[b] into rows [0, n) of sequence b of `cache` (src[b] = -1: untouched).
    Returns the loaded length per destination (-1 where untouched)."""
    desc, lens, hb, _ = parse_header(image)
    tensors = _tensors(cache)
    out = [-1] * len(src)
    off = hb
    for t in tensors:
        L, KV, B_dst, G = t.shape[:4]
        row = t.shape[5:]
        row_bytes = int(np.prod(row, dtype=np.int64)) * t.dtype.itemsize
        # offsets of every saved (layer, kv, sequence, head) run, in payload order
        where = {}
        for layer in range(L):
            for kv in range(KV):
                for s, n in enumerate(lens):
                    for g in range(G):
                        where[layer, kv, s, g] = off
                        off += n * row_bytes
        for b, s in enumerate(src):
            if s < 0:
                continue
            n = lens[s]
            if n > t.shape[4]:
                raise ValueError("saved prefix longer than the cache")
            out[b] = n
            for layer in range(L):
                for kv in range(KV):
                    for g in range(G):
                        o = where[layer, kv, s, g]
                        rows = np.frombuffer(image, dtype=t.dtype, count=n * int(np.prod(row, dtype=np.int64)),
                                             offset=o).reshape((n,) + row)
                        t[layer, kv, b, g, :n] = rows
    return out
