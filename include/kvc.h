/*
 * kvc.h -- C ABI of the static KV-cache decode library (libkvc.so, gfx950).
 *
 * The library implements autoregressive decode over a KV cache that is
 * allocated once, at its full capacity, per layer:
 *
 *   - "KV-Cache Mechanics" (DantinoX docs), "AR Static KV-Cache": one
 *     [B, H_kv, max_context, head_size] array per layer, allocated up front so
 *     shapes never change between decode steps; prefill writes from
 *     cache_index 0, each decode step writes at cache_index.
 *   - "KV Cache Optimization: GQA Audit, In-Place Buffers, Persistent
 *     Prompts", "#2 In-place KV cache updates": new rows are slice-assigned
 *     into the fixed buffer (no concat, no regrowth); reads stop at the valid
 *     length.
 *   - "10.3 - KV cache implementation details", section 5: per layer, append
 *     the new k and v, then single-query attention
 *     softmax(q K^T / sqrt(d_head)) V over the cached rows; section 4.1-4.3
 *     for MQA, GQA and the latent (MLA) cache.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every tensor pointer is a DEVICE pointer (hipMalloc'd or a torch
 *    tensor's data_ptr) unless a parameter says "host". All tensors are dense,
 *    row-major (last dimension fastest) and 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work
 *    is enqueued asynchronously on it; the caller keeps every argument alive
 *    until that work has run.
 *  - Element type: every tensor that holds cache-typed values (k, v, q, out,
 *    latent rows, MLA weights) has the cache's dtype, except on an int8
 *    cache (KVC_I8), whose rows are stored as int8 codes but every tensor
 *    handed in or out is bf16. Nothing else is converted; there is no
 *    per-call dtype argument.
 *  - Index arrays (`cache_index`, `valid_lens`) are int32 device arrays of
 *    length B. They stay on the device so a decode step has fixed pointers
 *    and launch shapes and can be captured in a HIP graph.
 *  - Host-checkable misuse returns a status and enqueues NOTHING (the cache
 *    is unchanged). Device-side out-of-range indices cannot be seen by the
 *    host without a sync, so the kernels skip the offending sequence (append
 *    writes nothing for it, attention writes zeros for it) and raise a sticky
 *    per-cache flag that kvc_check() reports as KVC_ERR_DEVICE_RANGE.
 *  - No call allocates or synchronises except kvc_alloc, kvc_free,
 *    kvc_alloc_paged, kvc_check and the prefix save/load calls (and every
 *    call when the environment variable KVC_SYNC_CHECK=1 is set, which makes
 *    each launch synchronous and checked).
 *  - Each cache owns a workspace that its attention calls share: split
 *    partials, self-resetting arrival counters, and the split of the work
 *    cached for the last lengths seen (reused while the lengths, grid and
 *    append mode stay the same, as across the layers of one decode step).
 *    Calls on one cache must therefore not run concurrently: enqueue them on
 *    one stream, or order the streams.
 */
#ifndef KVC_H
#define KVC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVC_OK = 0,
  KVC_ERR_INVALID_ARG = 1,   /* NULL pointer, bad layer, bad shape or field */
  KVC_ERR_CAPACITY = 2,      /* host-visible rows outside [0, max_context) */
  KVC_ERR_OOM = 3,           /* device allocation failed */
  KVC_ERR_DEVICE = 4,        /* a HIP runtime call or launch failed */
  KVC_ERR_UNSUPPORTED = 5,   /* valid request this build does not implement */
  KVC_ERR_DEVICE_RANGE = 6   /* a device-side index was out of range (kvc_check) */
} kvc_status;

/* KVC_I8: "10.3 - KV cache implementation details", section 4.4 (the cache
 * stored in lower precision, p_cache = 1). Each cached row of one kv head,
 * of K and of V separately, is stored as head_dim int8 codes plus one
 * float32 scale, quantised once when the row is written (fill or append):
 *   amax = max_i |x_i|, scale = amax / 127,
 *   code_i = round_half_even(x_i * (127 / amax)) clamped to [-127, 127],
 * all in IEEE binary32 (a row of zeros: scale 0, codes 0). The row stands
 * for code_i * scale, and attention runs on those values. Rows handed in,
 * queries and outputs are bf16. GQA only, head_dim 64, 128 or 256. */
typedef enum { KVC_F32 = 0, KVC_BF16 = 1, KVC_I8 = 2 } kvc_dtype;

/* KVC_ATTN_GQA covers MHA (n_kv_heads == n_heads), GQA and MQA
 * (n_kv_heads == 1) with one code path; KVC_ATTN_MLA is the latent cache. */
typedef enum { KVC_ATTN_GQA = 0, KVC_ATTN_MLA = 1 } kvc_attn;

/* Static shape of a cache. Fields not used by the attention kind must be 0.
 *
 *  GQA: n_heads % n_kv_heads == 0; head_dim in {32, 64, 128, 256};
 *       latent_dim = rope_dim = 0.
 *       Layout: [n_layers][2 (K, V)][batch][n_kv_heads][max_context][head_dim].
 *       KVC_I8: the codes in that layout, followed by the scales
 *       [n_layers][2 (K, V)][batch][n_kv_heads][max_context] (float32).
 *  MLA: n_kv_heads = 1; latent_dim = 512, rope_dim = 64, head_dim = 128
 *       (per-head width of q_nope and of the output), bf16 only;
 *       n_heads <= 16 or a multiple of 16.
 *       Layout: [n_layers][batch][max_context][latent_dim + rope_dim], each
 *       row = latent c (latent_dim) then the rotary key kR (rope_dim).
 *  Group of query head h: kv head h / (n_heads / n_kv_heads) (contiguous). */
typedef struct {
  int32_t attn;         /* kvc_attn */
  int32_t dtype;        /* kvc_dtype */
  int32_t n_layers;     /* >= 1 */
  int32_t batch;        /* B in [1, 2048] */
  int32_t n_heads;      /* H, query heads >= 1 */
  int32_t n_kv_heads;   /* H_kv */
  int32_t head_dim;     /* d_h */
  int32_t max_context;  /* S >= 1, rows per sequence; KVC_ERR_UNSUPPORTED when
                           batch * (S + 1024) >= 2^31 or the rows of one
                           (sequence, kv head) take >= 2^30 bytes */
  int32_t latent_dim;   /* MLA d_c */
  int32_t rope_dim;     /* MLA d_R */
} kvc_desc;

typedef struct kvc_cache kvc_cache; /* opaque */

/* Physical bytes of the cache region for `desc` (pure host, no device work).
 * "10.3 - KV cache implementation details", section 2 / 4.2:
 *   GQA: 2 * n_layers * n_kv_heads * head_dim * max_context * batch * p;
 * section 4.3 (with the rotary key stored in the same row):
 *   MLA: n_layers * (latent_dim + rope_dim) * max_context * batch * p;
 * p = 4 (fp32), 2 (bf16) or 1 (int8, section 4.4), and for int8 the
 * scales add 2 * n_layers * n_kv_heads * max_context * batch * 4.
 * Returns KVC_ERR_INVALID_ARG for a bad desc. */
kvc_status kvc_bytes(const kvc_desc* desc, uint64_t* physical);

/* Allocate a cache once, at full capacity ("AR Static KV-Cache"). If
 * `external` is NULL the library hipMallocs the region and zero-fills it;
 * otherwise `external` must point to >= kvc_bytes() device bytes, 256-byte
 * aligned, which the caller owns and keeps alive until kvc_free (the library
 * neither clears nor frees it). The library also allocates a fixed
 * workspace for split-context partials and a device error flag.
 * Runs on the current HIP device; synchronous. On failure *out is NULL. */
kvc_status kvc_alloc(const kvc_desc* desc, void* external, kvc_cache** out);

/* Release the cache (and its region unless external). NULL is a no-op.
 * Synchronises the device first. */
kvc_status kvc_free(kvc_cache* cache);

/* Device pointers of one layer: GQA *k = [B][H_kv][S][d_h] keys, *v values;
 * MLA *k = [B][S][latent_dim + rope_dim] rows and *v = NULL. Host only. */
kvc_status kvc_layer_ptrs(const kvc_cache* cache, int32_t layer, void** k, void** v);

/* Device pointers of one layer's row scales on an int8 cache:
 * *k_scales, *v_scales = float32 [B][H_kv][S]. Other caches:
 * KVC_ERR_INVALID_ARG. Host only. */
kvc_status kvc_layer_scales(const kvc_cache* cache, int32_t layer, void** k_scales, void** v_scales);

/* Logical bytes of the live prefixes given HOST valid lengths [B]:
 * the byte formula with max_context * batch replaced by sum_b n_b
 * ("KV Cache Optimization ...", "File map": totalBytes reports logical bytes,
 * physicalBytes the capacity). Host only. */
kvc_status kvc_logical_bytes(const kvc_cache* cache, const int32_t* host_valid_lens, uint64_t* out);

/* Prefill fill / migration into the static buffer: copy rows
 * [start, start + t) of every sequence and KV head of `layer`.
 *  GQA: k, v = [B][H_kv][t][d_h].   MLA: k = rows [B][t][latent_dim + rope_dim],
 *  v must be NULL.
 * ("KV-Cache Mechanics", "AR Static KV-Cache": prefill fills the cache from
 * cache_index 0; "KV Cache Optimization ...", "File map": migrateToPreAlloc.)
 * Bit copy (int8 cache: bf16 rows in, each row quantised as for KVC_I8).
 * start < 0, t < 1 or start + t > max_context -> KVC_ERR_CAPACITY. */
kvc_status kvc_prefill_fill(kvc_cache* cache, int32_t layer, const void* k, const void* v,
                            int32_t start, int32_t t, void* stream);

/* In-place append of t_new new rows per sequence at a per-sequence position:
 * rows [cache_index[b], cache_index[b] + t_new) of sequence b get
 * k_new[b], v_new[b]; no other byte of the cache changes.
 *  GQA: k_new, v_new = [B][H_kv][t_new][d_h].
 *  MLA: k_new = rows [B][t_new][latent_dim + rope_dim], v_new must be NULL.
 *  cache_index: device int32 [B].
 * ("KV Cache Optimization ...", "#2 ... After": slice-assign at the valid
 * length; "10.3 ...", section 5 step 2: append k_t, v_t before attention.)
 * On an int8 cache the bf16 rows are quantised as for KVC_I8 (codes and
 * scales of those rows are written, nothing else).
 * A sequence with cache_index[b] < 0 or cache_index[b] + t_new > max_context
 * is skipped and raises the device-range flag. t_new < 1 -> INVALID_ARG. */
kvc_status kvc_append(kvc_cache* cache, int32_t layer, const void* k_new, const void* v_new,
                      const int32_t* cache_index, int32_t t_new, void* stream);

/* Single-query decode attention of every query head over rows [0, n_b):
 *   n_b = valid_lens ? valid_lens[b] : cache_index[b] + 1
 * (append at cache_index, then attend it: the new token is included).
 *  GQA: q = [B][H][d_h], out = [B][H][d_h];
 *       out[b,h] = softmax(sm_scale * K[b,g,:n_b] q[b,h]) V[b,g,:n_b],
 *       g = h / (H / H_kv)  ("10.3 ...", section 5 step 2 and section 4.2).
 *  MLA: q = absorbed queries [B][H][latent_dim + rope_dim],
 *       out = latent output [B][H][latent_dim];
 *       out[b,h] = softmax(sm_scale * R[b,:n_b] q[b,h]) R[b,:n_b,:latent_dim],
 *       R = the cached rows (latent then rotary key).
 *  int8 cache: q and out bf16; K and V are the rows' code * scale values.
 * Accumulation is fp32; out is rounded to the cache dtype (nearest-even;
 * bf16 for an int8 cache).
 * n_b == 0 gives out[b] = 0. n_b < 0 or n_b > max_context gives out[b] = 0
 * and raises the device-range flag. At least one of valid_lens and
 * cache_index must be non-NULL. sm_scale must be finite and > 0. */
kvc_status kvc_decode_attn(kvc_cache* cache, int32_t layer, const void* q, void* out,
                           const int32_t* valid_lens, const int32_t* cache_index,
                           float sm_scale, void* stream);

/* Prefill of a prompt chunk on one GQA layer ("KV-Cache Mechanics", "AR
 * Static KV-Cache": the prompt's forward pass fills the cache from
 * cache_index 0, and a later chunk continues at cache_index = start;
 * "10.3 ...", section 3: causal attention; section 4.2: shared kv heads).
 * Writes k, v = [B][H_kv][t][d_h] into rows [start, start + t) of every
 * sequence (as kvc_prefill_fill), then computes the causal attention of the
 * chunk's t queries q = [B][H][t][d_h] over the cache:
 *   out[b,h,i] = softmax(sm_scale * K[b,g,0:start+i+1] q[b,h,i]) V[b,g,0:start+i+1],
 *   g = h / (H / H_kv), out = [B][H][t][d_h]. Rows [0, start) must already
 * hold the earlier part of the prompt. bf16 GQA caches only (others:
 * KVC_ERR_UNSUPPORTED). start < 0 or start + t > max_context ->
 * KVC_ERR_CAPACITY; t < 1 or a bad argument -> KVC_ERR_INVALID_ARG. */
kvc_status kvc_prefill_attn(kvc_cache* cache, int32_t layer, const void* q, const void* k, const void* v,
                            void* out, int32_t start, int32_t t, float sm_scale, void* stream);

/* One decode step of one GQA layer in one launch: the same result as
 *   kvc_append(cache, layer, k_new, v_new, cache_index, 1, stream);
 *   kvc_decode_attn(cache, layer, q, out, NULL, cache_index, sm_scale, stream);
 * ("10.3 ...", section 5 step 2: append k_t, v_t, then attend rows 0..t),
 * i.e. the new row is written at cache_index[b] and attended together with
 * rows [0, cache_index[b]). k_new, v_new = [B][H_kv][1][d_h]; q, out as for
 * kvc_decode_attn. The new row enters the attention straight from k_new /
 * v_new, and the kernel writes it into the cache in the same launch, so the
 * output bits equal those of the two calls. A sequence with cache_index[b]
 * outside [0, max_context) is skipped (no write, zero output) and raises the
 * device-range flag. On an int8 cache the new rows are quantised as by
 * kvc_append (the same codes and scales), attended from those codes and
 * written into the cache. Latent caches: KVC_ERR_UNSUPPORTED. */
kvc_status kvc_append_decode_attn(kvc_cache* cache, int32_t layer, const void* k_new, const void* v_new,
                                  const void* q, void* out, const int32_t* cache_index, float sm_scale,
                                  void* stream);

/* Full latent (MLA) decode step for an MLA cache ("10.3 ...", section 4.3;
 * "KV-Cache Mechanics", MHA vs GQA vs MLA comparison, "absorb" overhead):
 *   q~[b,h]  = [ W_UK[h]^T q_nope[b,h] ; q_rope[b,h] ]
 *   o~[b,h]  = kvc_decode_attn(q~) over the latent rows
 *   out[b,h] = W_UV[h]^T o~[b,h]
 * which equals attention with per-head keys [W_UK[h] c_j ; kR_j] and values
 * W_UV[h]^T c_j. Shapes (d_n = d_v = head_dim):
 *   q_nope [B][H][d_n], q_rope [B][H][rope_dim], w_uk [H][d_n][latent_dim],
 *   w_uv [H][latent_dim][d_v], out [B][H][d_v]; all bf16.
 * Valid lengths, errors and rounding as kvc_decode_attn. */
kvc_status kvc_mla_decode(kvc_cache* cache, int32_t layer, const void* q_nope, const void* q_rope,
                          const void* w_uk, const void* w_uv, void* out,
                          const int32_t* valid_lens, const int32_t* cache_index,
                          float sm_scale, void* stream);

/* ---- block-table (paged) caches -----------------------------------------
 * "10.3 - KV cache implementation details", section 7.2: the cache is
 * allocated in fixed-size blocks, like virtual-memory pages, and a block
 * table maps each sequence's logical blocks to physical ones, so
 * non-contiguous blocks are logically contiguous; section 7.3: sequences
 * that share a prefix can share its blocks.
 *
 * A paged cache is a bf16 GQA cache whose desc.max_context is the logical
 * row capacity of one sequence (a multiple of block_size, at most 4096
 * blocks). block_size is a power of two in [16, 256]; num_blocks >= 1
 * physical blocks per layer, and one layer's K pool (num_blocks * n_kv_heads
 * * block_size * head_dim * 2 bytes) must stay below 2^30 bytes
 * (KVC_ERR_UNSUPPORTED otherwise). Layout:
 *   [n_layers][2 (K, V)][num_blocks][n_kv_heads][block_size][head_dim].
 * A block table is a device int32 array [batch][max_context / block_size]:
 * row r of sequence b is row r % block_size of physical block
 * table[b][r / block_size]. Tables are passed per call, so they can change
 * between steps; entries for rows a call does not touch are never read.
 * Sharing a block between sequences shares its rows (an append into it is
 * seen by all of them; two sequences that write the same row in one call
 * race, and the row holds one of the two writes). On a paged cache only the
 * calls below, kvc_layer_ptrs (the two pools), kvc_logical_bytes,
 * kvc_set/get_workgroups, kvc_check and kvc_free apply; the others return
 * KVC_ERR_INVALID_ARG. */

/* Physical bytes of a paged cache: 2 * n_layers * num_blocks * n_kv_heads
 * * block_size * head_dim * 2. Pure host. */
kvc_status kvc_bytes_paged(const kvc_desc* desc, int32_t block_size, int32_t num_blocks, uint64_t* physical);

/* Allocate a paged cache (pools zero-filled unless external), as kvc_alloc. */
kvc_status kvc_alloc_paged(const kvc_desc* desc, int32_t block_size, int32_t num_blocks, void* external,
                           kvc_cache** out);

/* kvc_append through a block table: rows [cache_index[b], cache_index[b] +
 * t_new) of sequence b get k_new[b], v_new[b] ([B][H_kv][t_new][d_h]). A
 * sequence whose rows leave [0, max_context), or reach a table entry outside
 * [0, num_blocks), is skipped (nothing written) and raises the device-range
 * flag. With t_new > 1 this is also the prefill fill of a paged cache. */
kvc_status kvc_paged_append(kvc_cache* cache, int32_t layer, const void* k_new, const void* v_new,
                            const int32_t* block_table, const int32_t* cache_index, int32_t t_new, void* stream);

/* kvc_decode_attn through a block table: the same attention over the rows
 * [0, n_b) the table maps. A row whose entry lies outside [0, num_blocks)
 * reads as zeros and raises the device-range flag. */
kvc_status kvc_paged_decode_attn(kvc_cache* cache, int32_t layer, const void* q, void* out,
                                 const int32_t* block_table, const int32_t* valid_lens,
                                 const int32_t* cache_index, float sm_scale, void* stream);

/* One decode step of one layer of a paged cache in one launch: the same
 * result as
 *   kvc_paged_append(cache, layer, k_new, v_new, block_table, cache_index, 1, stream);
 *   kvc_paged_decode_attn(cache, layer, q, out, block_table, NULL, cache_index, sm_scale, stream);
 * ("10.3 ...", section 5 step 2, through the block table of section 7.2):
 * the new row is written at cache_index[b] through the table and attended
 * with rows [0, cache_index[b]), straight from k_new / v_new, so the output
 * bits equal those of the two calls. A sequence with cache_index[b] outside
 * [0, max_context) is skipped (no write, zero output) and raises the
 * device-range flag; if the new row's table entry lies outside
 * [0, num_blocks), nothing is written, that block's rows (the new one
 * included) read as zeros and the flag is raised, as after the two calls.
 * Unlike the two calls, a sequence that reads a block into which another
 * sequence of the same call writes its new row may see that row before or
 * after the write. Shapes as for kvc_append_decode_attn. */
kvc_status kvc_paged_append_decode_attn(kvc_cache* cache, int32_t layer, const void* k_new, const void* v_new,
                                        const void* q, void* out, const int32_t* block_table,
                                        const int32_t* cache_index, float sm_scale, void* stream);

/* ---- live-prefix save and load -------------------------------------------
 * "KV Cache Optimization: GQA Audit, In-Place Buffers, Persistent Prompts",
 * "#3 Persistent KV across sessions" and its file map: the cache after a
 * prompt's prefill is saved once and loaded by later runs, which skip the
 * prefill with identical output; a pre-allocated cache saves only its live
 * prefix, and a load sets the valid lengths from what was saved. "10.3 - KV
 * cache implementation details", section 7.3: requests sharing a prefix
 * reuse its K/V.
 *
 * Image (little-endian, version 1):
 *   header: int32 [magic 0x3143564B ("KVC1"), version 1, the ten kvc_desc
 *     fields in declaration order, header bytes, 0] (56 bytes), the payload
 *     bytes as uint64 at byte 56, the batch's valid lengths as int32 from
 *     byte 64, zero padding to a multiple of 256 bytes;
 *   payload: for each layer, K then V (the latent cache: its one tensor), for
 *     each sequence, for each kv head, rows [0, n_b) as stored; for an int8
 *     cache all codes first, then the float32 row scales in the same order.
 * The payload is kvc_logical_bytes of the lengths. File I/O, naming and
 * invalidation are the caller's. Block-table caches are not supported
 * (KVC_ERR_INVALID_ARG). Both calls are ordered on `stream` and synchronise
 * it before returning. */

/* Image bytes for host_valid_lens[B] (each in [0, max_context], else
 * KVC_ERR_CAPACITY). Pure host. */
kvc_status kvc_prefix_bytes(const kvc_cache* cache, const int32_t* host_valid_lens, uint64_t* bytes);

/* Write the image of rows [0, n_b) of every layer and sequence, n_b =
 * host_valid_lens[b], to dst: device memory or pinned host memory of
 * dst_bytes >= kvc_prefix_bytes (else KVC_ERR_INVALID_ARG). */
kvc_status kvc_save_prefix(kvc_cache* cache, const int32_t* host_valid_lens, void* dst, uint64_t dst_bytes,
                           void* stream);

/* Load an image of src_bytes (device or pinned host memory): saved sequence
 * host_src_seq[b] (in [0, saved batch), or -1 to leave b alone) is written
 * into rows [0, n) of sequence b, n being its saved length, and
 * host_valid_lens[b] is set to n (left as it is for -1). Several b may name
 * one saved sequence (a shared prefix). Rows at or past n are not touched.
 * The image must come from a cache with the same attention kind, dtype,
 * n_layers, n_kv_heads, head_dim, latent_dim and rope_dim; batch, n_heads
 * and max_context may differ. A malformed or mismatched image, or a bad
 * host_src_seq entry, gives KVC_ERR_INVALID_ARG, and a saved length above
 * this cache's max_context KVC_ERR_CAPACITY; nothing is written then. */
kvc_status kvc_load_prefix(kvc_cache* cache, const void* src, uint64_t src_bytes, const int32_t* host_src_seq,
                           int32_t* host_valid_lens, void* stream);

/* Force the number of persistent workgroups attention launches (0 restores
 * the default: one per compute unit). The rows of
 * all sequences and kv heads are divided evenly among them, so this only
 * changes how the context is partitioned and the rounding order of the
 * result. n must be in [0, *max_n of kvc_get_workgroups]. Host only. */
kvc_status kvc_set_workgroups(kvc_cache* cache, int32_t n);

/* The forced workgroup count (0 = default) and, if max_n is not NULL, the
 * largest accepted value. Host only. */
kvc_status kvc_get_workgroups(const kvc_cache* cache, int32_t* n, int32_t* max_n);

/* For callers that cannot allocate (code under HIP graph capture, serving
 * loops and harnesses that forbid hipMalloc): kvc_decode_attn on a GQA layer
 * the caller holds, without a kvc_cache. Nothing is allocated: the kernels'
 * workspace (partials, arrival counters, the cached split of the work) is a
 * 16 MiB static array on each device, held until the process ends.
 *  desc:    the cache's shape (attn GQA, dtype bf16 or fp32; n_layers is not
 *           used); validated as by kvc_alloc.
 *  k_layer, v_layer: device pointers to one layer's K and V,
 *           [B][H_kv][max_context][d_h] each, in the cache dtype.
 *  q, out, valid_lens, cache_index, sm_scale: as for kvc_decode_attn, with
 *           the same result bit for bit (same kernels, same default grid).
 *  err_flag: device int32 the kernels set to 1 when a sequence's length is
 *           out of range (that sequence's outputs are zeros); never cleared
 *           by the library; may be NULL (the flag is then not reported).
 * Host-checkable errors return a status and enqueue nothing: a bad
 * descriptor or argument (KVC_ERR_INVALID_ARG / KVC_ERR_UNSUPPORTED as for
 * kvc_alloc), an MLA or int8 shape, or a shape whose workspace exceeds the
 * array (B * H > 65536, or (compute units + B * H) * 16 * (d_h + 2) * 4 bytes
 * plus the split and counters above 16 MiB): KVC_ERR_UNSUPPORTED.
 * Calls on one device share the array: calls that overlap in time on one
 * device (concurrent streams) race and must not be issued. */
kvc_status kvc_decode_attn_noalloc(const kvc_desc* desc, const void* k_layer, const void* v_layer, const void* q,
                                   void* out, const int32_t* valid_lens, const int32_t* cache_index,
                                   float sm_scale, int32_t* err_flag, void* stream);

/* Synchronise `stream`, then report and clear the sticky device-range flag:
 * KVC_ERR_DEVICE_RANGE if any kernel since the last check skipped a
 * sequence, KVC_ERR_DEVICE if the stream reported an error, else KVC_OK. */
kvc_status kvc_check(kvc_cache* cache, void* stream);

/* Static string for a status code. */
const char* kvc_strerror(kvc_status status);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
