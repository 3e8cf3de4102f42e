// Host side of libkvc.so: descriptor validation, byte accounting, the one
// static allocation, layer pointer math, split planning and launches on the
// caller's stream. Every entry point is declared in include/kvc.h.
//
// Byte formulas: "10.3 - KV cache implementation details", section 2 (and
// 4.2 for H_kv, 4.3 for the latent cache); "KV-Cache Mechanics", "Memory
// Formula". Allocation once at full capacity: "KV-Cache Mechanics", "AR
// Static KV-Cache"; "KV Cache Optimization: GQA Audit, In-Place Buffers,
// Persistent Prompts", "#2 In-place KV cache updates".

#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>

#include "kvc_internal.h"

namespace {

bool env_sync_check() {
  const char* s = getenv("KVC_SYNC_CHECK");
  return s && s[0] == '1';
}

// Bytes per stored element: fp32 4, bf16 2, int8 codes 1 ("10.3 - KV cache
// implementation details", section 4.4: p_cache).
int elem_size(int dtype) { return dtype == KVC_F32 ? 4 : (dtype == KVC_BF16 ? 2 : (dtype == KVC_I8 ? 1 : 0)); }

bool valid_gqa_head_dim(int d) { return d == 32 || d == 64 || d == 128 || d == 256; }

kvc_status validate_desc(const kvc_desc* d) {
  if (!d) return KVC_ERR_INVALID_ARG;
  if (elem_size(d->dtype) == 0) return KVC_ERR_INVALID_ARG;
  if (d->n_layers < 1 || d->batch < 1 || d->n_heads < 1 || d->max_context < 1) return KVC_ERR_INVALID_ARG;
  if (d->batch > KVC_MAX_BATCH) return KVC_ERR_UNSUPPORTED;
  // the decode row space (rows of all sequences plus per-segment start-up
  // rows) and byte offsets within one sequence's rows are 32-bit
  if ((int64_t)d->batch * ((int64_t)d->max_context + 1024) >= (int64_t)1 << 31)
    return KVC_ERR_UNSUPPORTED;
  if (d->attn == KVC_ATTN_GQA) {
    if (d->n_kv_heads < 1 || d->n_heads % d->n_kv_heads != 0) return KVC_ERR_INVALID_ARG;
    if (d->latent_dim != 0 || d->rope_dim != 0) return KVC_ERR_INVALID_ARG;
    if (!valid_gqa_head_dim(d->head_dim)) return KVC_ERR_UNSUPPORTED;
    // int8 rows: a lane takes head_dim / 4 codes of a row in 16-byte vectors
    if (d->dtype == KVC_I8 && d->head_dim < 64) return KVC_ERR_UNSUPPORTED;
    if ((int64_t)d->max_context * d->head_dim * elem_size(d->dtype) >= (int64_t)1 << 30)
      return KVC_ERR_UNSUPPORTED;
    return KVC_OK;
  }
  if (d->attn == KVC_ATTN_MLA) {
    if (d->n_kv_heads != 1) return KVC_ERR_INVALID_ARG;
    if (d->latent_dim < 1 || d->rope_dim < 0 || d->head_dim < 1) return KVC_ERR_INVALID_ARG;
    if (d->dtype != KVC_BF16 || d->latent_dim != 512 || d->rope_dim != 64 || d->head_dim != 128)
      return KVC_ERR_UNSUPPORTED;
    if (d->n_heads > 16 && d->n_heads % 16 != 0) return KVC_ERR_UNSUPPORTED;  // chunks of 16 heads
    if ((int64_t)d->max_context * (d->latent_dim + d->rope_dim) * elem_size(d->dtype) >= (int64_t)1 << 30)
      return KVC_ERR_UNSUPPORTED;
    return KVC_OK;
  }
  return KVC_ERR_INVALID_ARG;
}

// Exact product with overflow check (all factors positive).
bool mul_u64(uint64_t a, uint64_t b, uint64_t* out) {
  if (a != 0 && b > UINT64_MAX / a) return false;
  *out = a * b;
  return true;
}

kvc_status bytes_of(const kvc_desc* d, uint64_t* out) {
  uint64_t x = 1;
  uint64_t p = (uint64_t)elem_size(d->dtype);
  uint64_t factors[6];
  int n = 0;
  if (d->attn == KVC_ATTN_GQA) {
    // 2 * L * H_kv * d_h * S * B * p
    factors[n++] = 2;
    factors[n++] = (uint64_t)d->n_layers;
    factors[n++] = (uint64_t)d->n_kv_heads * (uint64_t)d->head_dim;
    factors[n++] = (uint64_t)d->max_context;
    factors[n++] = (uint64_t)d->batch;
    factors[n++] = p;
    if (d->dtype == KVC_I8) {
      // plus one float32 scale per cached row of K and of V
      uint64_t rows = 1;
      const uint64_t rf[4] = {2, (uint64_t)d->n_layers, (uint64_t)d->n_kv_heads * (uint64_t)d->max_context,
                              (uint64_t)d->batch * 4};
      for (int i = 0; i < 4; ++i)
        if (!mul_u64(rows, rf[i], &rows)) return KVC_ERR_INVALID_ARG;
      for (int i = 0; i < n; ++i)
        if (!mul_u64(x, factors[i], &x)) return KVC_ERR_INVALID_ARG;
      if (x > UINT64_MAX - rows) return KVC_ERR_INVALID_ARG;
      *out = x + rows;
      return KVC_OK;
    }
  } else {
    // L * (d_c + d_R) * S * B * p
    factors[n++] = (uint64_t)d->n_layers;
    factors[n++] = (uint64_t)(d->latent_dim + d->rope_dim);
    factors[n++] = (uint64_t)d->max_context;
    factors[n++] = (uint64_t)d->batch;
    factors[n++] = p;
  }
  for (int i = 0; i < n; ++i)
    if (!mul_u64(x, factors[i], &x)) return KVC_ERR_INVALID_ARG;
  *out = x;
  return KVC_OK;
}

kvc_status after_launch(kvc_cache* c, hipError_t e, hipStream_t stream) {
  if (e != hipSuccess) return KVC_ERR_DEVICE;
  if (c->sync_check) {
    if (hipStreamSynchronize(stream) != hipSuccess) return KVC_ERR_DEVICE;
    int32_t flag = 0;
    if (hipMemcpy(&flag, c->err_flag, sizeof(flag), hipMemcpyDeviceToHost) != hipSuccess)
      return KVC_ERR_DEVICE;
    if (flag) return KVC_ERR_DEVICE_RANGE;  // left set for kvc_check
  }
  return KVC_OK;
}

bool layer_ok(const kvc_cache* c, int32_t layer) { return layer >= 0 && layer < c->d.n_layers; }

// Static-cache calls: a live, non-paged cache and a layer in range.
bool static_ok(const kvc_cache* c, int32_t layer) { return c && !c->paged && layer_ok(c, layer); }

int log2_exact(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return (1 << s) == x ? s : -1;
}

// Block-table caches ("10.3 - KV cache implementation details", section
// 7.2): bf16 GQA pools of num_blocks blocks of block_size rows per kv head.
kvc_status validate_paged(const kvc_desc* d, int32_t block_size, int32_t num_blocks) {
  kvc_status s = validate_desc(d);
  if (s != KVC_OK) return s;
  if (block_size < 1 || num_blocks < 1) return KVC_ERR_INVALID_ARG;
  if (d->max_context % block_size != 0) return KVC_ERR_INVALID_ARG;
  if (d->attn != KVC_ATTN_GQA || d->dtype != KVC_BF16) return KVC_ERR_UNSUPPORTED;
  // a 16-row attention tile spans at most two blocks
  if (block_size < 16 || block_size > 256 || log2_exact(block_size) < 0) return KVC_ERR_UNSUPPORTED;
  if (d->max_context / block_size > KVC_MAX_TABLE) return KVC_ERR_UNSUPPORTED;
  // byte offsets within one pool are 32-bit, with room above for "no row"
  if ((int64_t)num_blocks * d->n_kv_heads * block_size * d->head_dim * 2 >= (int64_t)1 << 30)
    return KVC_ERR_UNSUPPORTED;
  return KVC_OK;
}

uint64_t paged_bytes(const kvc_desc* d, int32_t block_size, int32_t num_blocks) {
  // 2 * L * num_blocks * H_kv * block_size * d_h * 2 (each pool < 2^30 bytes)
  return 2ull * d->n_layers * ((uint64_t)num_blocks * d->n_kv_heads * block_size * d->head_dim * 2);
}

kvc_status alloc_impl(const kvc_desc* desc, void* external, uint64_t bytes, int32_t block_size,
                      int32_t num_blocks, kvc_cache** out);

// Stored bytes of one cached row position over all of a layer's tensors
// (K and V of every kv head, plus int8 row scales; the latent row).
uint64_t bytes_per_position(const kvc_cache* c) {
  uint64_t per_row = c->d.attn == KVC_ATTN_GQA ? 2ull * c->d.n_kv_heads * c->d.head_dim * c->elem
                                               : (uint64_t)c->row_elems * c->elem;
  if (c->d.dtype == KVC_I8) per_row += 2ull * c->d.n_kv_heads * sizeof(float);
  return per_row;
}

// ---- live-prefix image ("KV Cache Optimization ...", "#3 Persistent KV
// across sessions"; layout in include/kvc.h) -----------------------------
constexpr int32_t kImageMagic = 0x3143564B;  // "KVC1"
constexpr int32_t kImageVersion = 1;

uint64_t image_header_bytes(int batch) { return ((uint64_t)4 * (16 + batch) + 255) / 256 * 256; }

// The header for `lens` (batch entries) of cache c.
void image_header(const kvc_cache* c, const int32_t* lens, uint64_t payload, unsigned char* out) {
  const uint64_t hb = image_header_bytes(c->d.batch);
  memset(out, 0, hb);
  const int32_t w[14] = {kImageMagic, kImageVersion, c->d.attn, c->d.dtype, c->d.n_layers, c->d.batch,
                         c->d.n_heads, c->d.n_kv_heads, c->d.head_dim, c->d.max_context, c->d.latent_dim,
                         c->d.rope_dim, (int32_t)hb, 0};
  memcpy(out, w, sizeof(w));
  memcpy(out + 56, &payload, 8);
  memcpy(out + 64, lens, (size_t)c->d.batch * 4);
}

// One direction of the payload copy for the sequences' runs in `map_host`
// ([B][2]: rows, first image row); total_rows = rows of all saved sequences.
hipError_t prefix_copy(kvc_cache* c, uint8_t* payload, const int32_t* map_host, bool save, int64_t total_rows,
                       hipStream_t s) {
  int max_rows = 0;
  for (int b = 0; b < c->d.batch; ++b) max_rows = map_host[2 * b] > max_rows ? map_host[2 * b] : max_rows;
  hipError_t e = hipMemcpyAsync(c->ws_map, map_host, (size_t)c->d.batch * 2 * sizeof(int32_t),
                                hipMemcpyHostToDevice, s);
  if (e != hipSuccess || max_rows == 0) return e;
  const bool gqa = c->d.attn == KVC_ATTN_GQA;
  const int kv_parts = gqa ? 2 : 1;
  const int groups = gqa ? c->d.n_kv_heads : 1;
  const int row_bytes = c->row_elems * c->elem;
  e = kvc_launch_prefix_copy(c->base, payload, c->ws_map, save, c->layer_bytes, c->kv_bytes, c->d.n_layers,
                             kv_parts, c->d.batch, max_rows, groups, c->d.max_context, row_bytes, 16, total_rows, s);
  if (e == hipSuccess && c->d.dtype == KVC_I8) {
    const uint64_t codes = (uint64_t)c->d.n_layers * kv_parts * total_rows * groups * row_bytes;
    e = kvc_launch_prefix_copy(c->scales, payload + codes, c->ws_map, save, c->scale_layer_bytes,
                               c->scale_kv_bytes, c->d.n_layers, kv_parts, c->d.batch, max_rows, groups,
                               c->d.max_context, 4, 4, total_rows, s);
  }
  return e;
}

}  // namespace

extern "C" {

kvc_status kvc_bytes(const kvc_desc* desc, uint64_t* physical) {
  if (!physical) return KVC_ERR_INVALID_ARG;
  kvc_status s = validate_desc(desc);
  if (s != KVC_OK) return s;
  return bytes_of(desc, physical);
}

kvc_status kvc_alloc(const kvc_desc* desc, void* external, kvc_cache** out) {
  if (!out) return KVC_ERR_INVALID_ARG;
  *out = nullptr;
  kvc_status s = validate_desc(desc);
  if (s != KVC_OK) return s;
  uint64_t bytes = 0;
  s = bytes_of(desc, &bytes);
  if (s != KVC_OK) return s;
  return alloc_impl(desc, external, bytes, 0, 0, out);
}

kvc_status kvc_bytes_paged(const kvc_desc* desc, int32_t block_size, int32_t num_blocks, uint64_t* physical) {
  if (!physical) return KVC_ERR_INVALID_ARG;
  kvc_status s = validate_paged(desc, block_size, num_blocks);
  if (s != KVC_OK) return s;
  *physical = paged_bytes(desc, block_size, num_blocks);
  return KVC_OK;
}

kvc_status kvc_alloc_paged(const kvc_desc* desc, int32_t block_size, int32_t num_blocks, void* external,
                           kvc_cache** out) {
  if (!out) return KVC_ERR_INVALID_ARG;
  *out = nullptr;
  kvc_status s = validate_paged(desc, block_size, num_blocks);
  if (s != KVC_OK) return s;
  return alloc_impl(desc, external, paged_bytes(desc, block_size, num_blocks), block_size, num_blocks, out);
}

}  // extern "C"

namespace {

// One allocation of `bytes` (or the caller's buffer) plus the decode
// workspace; block_size = 0 for a static cache.
kvc_status alloc_impl(const kvc_desc* desc, void* external, uint64_t bytes, int32_t block_size,
                      int32_t num_blocks, kvc_cache** out) {
  if (external && ((uintptr_t)external % 256) != 0) return KVC_ERR_INVALID_ARG;
  kvc_cache* c = new (std::nothrow) kvc_cache();
  if (!c) return KVC_ERR_OOM;
  memset(c, 0, sizeof(*c));
  c->d = *desc;
  c->elem = elem_size(desc->dtype);
  c->bytes = bytes;
  c->sync_check = env_sync_check();
  if (hipGetDevice(&c->device) != hipSuccess) { delete c; return KVC_ERR_DEVICE; }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, c->device) != hipSuccess) { delete c; return KVC_ERR_DEVICE; }
  c->num_cus = prop.multiProcessorCount;

  if (block_size > 0) {
    c->paged = true;
    c->block_size = block_size;
    c->block_shift = log2_exact(block_size);
    c->num_blocks = num_blocks;
    c->table_width = desc->max_context / block_size;
    c->row_elems = desc->head_dim;
    c->kv_bytes = (uint64_t)num_blocks * desc->n_kv_heads * block_size * desc->head_dim * c->elem;
    c->layer_bytes = 2 * c->kv_bytes;
  } else if (desc->attn == KVC_ATTN_GQA) {
    c->row_elems = desc->head_dim;
    c->kv_bytes = (uint64_t)desc->batch * desc->n_kv_heads * desc->max_context * desc->head_dim * c->elem;
    c->layer_bytes = 2 * c->kv_bytes;
    if (desc->dtype == KVC_I8) {
      c->scale_kv_bytes = (uint64_t)desc->batch * desc->n_kv_heads * desc->max_context * sizeof(float);
      c->scale_layer_bytes = 2 * c->scale_kv_bytes;
    }
  } else {
    c->row_elems = desc->latent_dim + desc->rope_dim;
    c->kv_bytes = 0;
    c->layer_bytes = (uint64_t)desc->batch * desc->max_context * c->row_elems * c->elem;
  }
  c->max_workgroups = c->num_cus * KVC_MAX_WG_PER_CU;
  const int acc_width = desc->attn == KVC_ATTN_GQA ? desc->head_dim : desc->latent_dim;
  // a slot per (workgroup, segment) intersection, at most 16 heads each
  c->ws_entries = ((uint64_t)c->max_workgroups + (uint64_t)desc->batch * desc->n_heads) * 16;

  bool ok = true;
  if (external) {
    c->base = (uint8_t*)external;
    c->owns_base = false;
  } else {
    ok = hipMalloc((void**)&c->base, bytes) == hipSuccess;
    c->owns_base = ok;
    if (ok) ok = hipMemset(c->base, 0, bytes) == hipSuccess;
  }
  if (ok && desc->dtype == KVC_I8) c->scales = c->base + (uint64_t)desc->n_layers * c->layer_bytes;
  if (ok) ok = hipMalloc((void**)&c->ws_acc, c->ws_entries * acc_width * sizeof(float)) == hipSuccess;
  if (ok) ok = hipMalloc((void**)&c->ws_ml, c->ws_entries * 2 * sizeof(float)) == hipSuccess;
  const uint64_t cnt_bytes = (uint64_t)desc->batch * desc->n_heads * sizeof(int32_t);
  if (ok) ok = hipMalloc((void**)&c->ws_cnt, cnt_bytes) == hipSuccess;
  if (ok) ok = hipMemset(c->ws_cnt, 0, cnt_bytes) == hipSuccess;
  if (ok) ok = hipMalloc((void**)&c->ws_map, (uint64_t)desc->batch * 2 * sizeof(int32_t)) == hipSuccess;
  const uint64_t plan_bytes = ((uint64_t)KVC_PLAN_HEAD + (uint64_t)c->max_workgroups * KVC_PLAN_INTS) * 4;
  if (ok) ok = hipMalloc((void**)&c->ws_plan, plan_bytes) == hipSuccess;
  if (ok) ok = hipMemset(c->ws_plan, 0, plan_bytes) == hipSuccess;  // no plan yet
  if (ok) ok = hipMalloc((void**)&c->err_flag, 256) == hipSuccess;
  if (ok) ok = hipMemset(c->err_flag, 0, 256) == hipSuccess;
  if (ok && desc->attn == KVC_ATTN_MLA) {
    const uint64_t bh = (uint64_t)desc->batch * desc->n_heads;
    ok = hipMalloc((void**)&c->ws_qabs, bh * c->row_elems * sizeof(uint16_t)) == hipSuccess;
    if (ok) ok = hipMalloc((void**)&c->ws_olat, bh * desc->latent_dim * sizeof(uint16_t)) == hipSuccess;
    const uint64_t chunks = ((uint64_t)desc->n_heads + 15) / 16;
    if (ok) ok = hipMalloc((void**)&c->ws_seg, (uint64_t)desc->batch * chunks * 2 * sizeof(int32_t)) == hipSuccess;
  }
  if (ok) ok = hipDeviceSynchronize() == hipSuccess;
  if (!ok) {
    (void)hipGetLastError();
    kvc_free(c);
    return KVC_ERR_OOM;
  }
  *out = c;
  return KVC_OK;
}

}  // namespace

extern "C" {

kvc_status kvc_free(kvc_cache* c) {
  if (!c) return KVC_OK;
  hipError_t e = hipDeviceSynchronize();
  if (c->owns_base && c->base) (void)hipFree(c->base);
  if (c->ws_acc) (void)hipFree(c->ws_acc);
  if (c->ws_ml) (void)hipFree(c->ws_ml);
  if (c->ws_cnt) (void)hipFree(c->ws_cnt);
  if (c->err_flag) (void)hipFree(c->err_flag);
  if (c->ws_map) (void)hipFree(c->ws_map);
  if (c->ws_plan) (void)hipFree(c->ws_plan);
  if (c->ws_seg) (void)hipFree(c->ws_seg);
  if (c->ws_qabs) (void)hipFree(c->ws_qabs);
  if (c->ws_olat) (void)hipFree(c->ws_olat);
  delete c;
  return e == hipSuccess ? KVC_OK : KVC_ERR_DEVICE;
}

kvc_status kvc_layer_ptrs(const kvc_cache* c, int32_t layer, void** k, void** v) {
  if (!c || !k || !v || !layer_ok(c, layer)) return KVC_ERR_INVALID_ARG;
  uint8_t* l = c->base + (uint64_t)layer * c->layer_bytes;
  *k = l;
  *v = c->d.attn == KVC_ATTN_GQA ? (void*)(l + c->kv_bytes) : nullptr;
  return KVC_OK;
}

kvc_status kvc_layer_scales(const kvc_cache* c, int32_t layer, void** k_scales, void** v_scales) {
  if (!k_scales || !v_scales || !static_ok(c, layer) || c->d.dtype != KVC_I8) return KVC_ERR_INVALID_ARG;
  uint8_t* l = c->scales + (uint64_t)layer * c->scale_layer_bytes;
  *k_scales = l;
  *v_scales = l + c->scale_kv_bytes;
  return KVC_OK;
}

kvc_status kvc_logical_bytes(const kvc_cache* c, const int32_t* host_valid_lens, uint64_t* out) {
  if (!c || !host_valid_lens || !out) return KVC_ERR_INVALID_ARG;
  uint64_t total = 0;
  for (int b = 0; b < c->d.batch; ++b) {
    if (host_valid_lens[b] < 0 || host_valid_lens[b] > c->d.max_context) return KVC_ERR_CAPACITY;
    total += (uint64_t)host_valid_lens[b];
  }
  *out = (uint64_t)c->d.n_layers * bytes_per_position(c) * total;
  return KVC_OK;
}

kvc_status kvc_prefix_bytes(const kvc_cache* c, const int32_t* host_valid_lens, uint64_t* bytes) {
  if (!c || c->paged || !bytes) return KVC_ERR_INVALID_ARG;
  uint64_t payload = 0;
  kvc_status st = kvc_logical_bytes(c, host_valid_lens, &payload);
  if (st != KVC_OK) return st;
  *bytes = image_header_bytes(c->d.batch) + payload;
  return KVC_OK;
}

kvc_status kvc_save_prefix(kvc_cache* c, const int32_t* host_valid_lens, void* dst, uint64_t dst_bytes,
                           void* stream) {
  if (!c || c->paged || !dst || ((uintptr_t)dst % 16) != 0) return KVC_ERR_INVALID_ARG;
  uint64_t need = 0;
  kvc_status st = kvc_prefix_bytes(c, host_valid_lens, &need);
  if (st != KVC_OK) return st;
  if (dst_bytes < need) return KVC_ERR_INVALID_ARG;
  const uint64_t hb = image_header_bytes(c->d.batch);
  unsigned char* hdr = (unsigned char*)malloc(hb);
  int32_t* map = (int32_t*)malloc((size_t)c->d.batch * 2 * sizeof(int32_t));
  if (!hdr || !map) { free(hdr); free(map); return KVC_ERR_OOM; }
  int64_t rows = 0;
  for (int b = 0; b < c->d.batch; ++b) {
    map[2 * b] = host_valid_lens[b];
    map[2 * b + 1] = (int32_t)rows;
    rows += host_valid_lens[b];
  }
  image_header(c, host_valid_lens, need - hb, hdr);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(dst, hdr, hb, hipMemcpyDefault, s);
  if (e == hipSuccess) e = prefix_copy(c, (uint8_t*)dst + hb, map, true, rows, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  free(hdr);
  free(map);
  return e == hipSuccess ? KVC_OK : KVC_ERR_DEVICE;
}

kvc_status kvc_load_prefix(kvc_cache* c, const void* src, uint64_t src_bytes, const int32_t* host_src_seq,
                           int32_t* host_valid_lens, void* stream) {
  if (!c || c->paged || !src || ((uintptr_t)src % 16) != 0 || !host_src_seq || !host_valid_lens)
    return KVC_ERR_INVALID_ARG;
  if (src_bytes < 64) return KVC_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  unsigned char head[64];
  if (hipMemcpyAsync(head, src, 64, hipMemcpyDefault, s) != hipSuccess || hipStreamSynchronize(s) != hipSuccess)
    return KVC_ERR_DEVICE;
  int32_t w[14];
  uint64_t payload = 0;
  memcpy(w, head, sizeof(w));
  memcpy(&payload, head + 56, 8);
  // the image's descriptor: the same cache rows, any batch / query heads / capacity
  const kvc_desc& d = c->d;
  if (w[0] != kImageMagic || w[1] != kImageVersion) return KVC_ERR_INVALID_ARG;
  if (w[2] != d.attn || w[3] != d.dtype || w[4] != d.n_layers || w[7] != d.n_kv_heads || w[8] != d.head_dim ||
      w[10] != d.latent_dim || w[11] != d.rope_dim)
    return KVC_ERR_INVALID_ARG;
  const int src_batch = w[5];
  const int src_context = w[9];
  if (src_batch < 1 || src_batch > KVC_MAX_BATCH || src_context < 1) return KVC_ERR_INVALID_ARG;
  const uint64_t hb = image_header_bytes(src_batch);
  if ((uint64_t)w[12] != hb || w[13] != 0 || src_bytes < hb) return KVC_ERR_INVALID_ARG;
  int32_t* lens = (int32_t*)malloc((size_t)src_batch * sizeof(int32_t));
  int32_t* map = (int32_t*)malloc((size_t)d.batch * 2 * sizeof(int32_t));
  int64_t* first = (int64_t*)malloc((size_t)src_batch * sizeof(int64_t));
  kvc_status st = (lens && map && first) ? KVC_OK : KVC_ERR_OOM;
  int64_t rows = 0;
  if (st == KVC_OK &&
      (hipMemcpyAsync(lens, (const unsigned char*)src + 64, (size_t)src_batch * 4, hipMemcpyDefault, s) !=
           hipSuccess ||
       hipStreamSynchronize(s) != hipSuccess))
    st = KVC_ERR_DEVICE;
  for (int i = 0; st == KVC_OK && i < src_batch; ++i) {
    if (lens[i] < 0 || lens[i] > src_context) st = KVC_ERR_INVALID_ARG;
    first[i] = rows;
    rows += lens[i];
  }
  if (st == KVC_OK) {
    // the payload must be exactly the saved rows, and present
    const uint64_t want = (uint64_t)d.n_layers * bytes_per_position(c) * (uint64_t)rows;
    if (payload != want || src_bytes - hb < payload || rows > 0x7fffffffLL) st = KVC_ERR_INVALID_ARG;
  }
  for (int b = 0; st == KVC_OK && b < d.batch; ++b) {
    const int32_t sq = host_src_seq[b];
    if (sq < -1 || sq >= src_batch) { st = KVC_ERR_INVALID_ARG; break; }
    map[2 * b] = sq < 0 ? 0 : lens[sq];
    map[2 * b + 1] = sq < 0 ? 0 : (int32_t)first[sq];
    if (map[2 * b] > d.max_context) st = KVC_ERR_CAPACITY;
  }
  if (st == KVC_OK) {
    hipError_t e = prefix_copy(c, (uint8_t*)const_cast<void*>(src) + hb, map, false, rows, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) st = KVC_ERR_DEVICE;
  }
  if (st == KVC_OK)
    for (int b = 0; b < d.batch; ++b)
      if (host_src_seq[b] >= 0) host_valid_lens[b] = lens[host_src_seq[b]];
  free(lens);
  free(map);
  free(first);
  return st;
}

kvc_status kvc_prefill_fill(kvc_cache* c, int32_t layer, const void* k, const void* v, int32_t start,
                            int32_t t, void* stream) {
  if (!k || !static_ok(c, layer)) return KVC_ERR_INVALID_ARG;
  const bool gqa = c->d.attn == KVC_ATTN_GQA;
  if (gqa ? !v : v != nullptr) return KVC_ERR_INVALID_ARG;
  if (t < 1) return KVC_ERR_INVALID_ARG;
  if (start < 0 || (int64_t)start + t > c->d.max_context) return KVC_ERR_CAPACITY;
  uint8_t* kl;
  uint8_t* vl;
  kvc_layer_ptrs(c, layer, (void**)&kl, (void**)&vl);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (c->d.dtype == KVC_I8) {
    float* ks;
    float* vs;
    kvc_layer_scales(c, layer, (void**)&ks, (void**)&vs);
    e = kvc_launch_quant_rows(k, v, kl, vl, ks, vs, c->d.batch, c->d.n_kv_heads, t, c->d.head_dim,
                              c->d.max_context, nullptr, start, c->err_flag, s);
  } else {
    e = kvc_launch_copy_rows(k, v, kl, vl, c->d.batch, gqa ? c->d.n_kv_heads : 1, t, c->row_elems * c->elem,
                             c->d.max_context, nullptr, start, c->err_flag, s);
  }
  return after_launch(c, e, s);
}

kvc_status kvc_append(kvc_cache* c, int32_t layer, const void* k_new, const void* v_new,
                      const int32_t* cache_index, int32_t t_new, void* stream) {
  if (!k_new || !cache_index || !static_ok(c, layer)) return KVC_ERR_INVALID_ARG;
  const bool gqa = c->d.attn == KVC_ATTN_GQA;
  if (gqa ? !v_new : v_new != nullptr) return KVC_ERR_INVALID_ARG;
  if (t_new < 1) return KVC_ERR_INVALID_ARG;
  if (t_new > c->d.max_context) return KVC_ERR_CAPACITY;
  uint8_t* kl;
  uint8_t* vl;
  kvc_layer_ptrs(c, layer, (void**)&kl, (void**)&vl);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (c->d.dtype == KVC_I8) {
    float* ks;
    float* vs;
    kvc_layer_scales(c, layer, (void**)&ks, (void**)&vs);
    e = kvc_launch_quant_rows(k_new, v_new, kl, vl, ks, vs, c->d.batch, c->d.n_kv_heads, t_new, c->d.head_dim,
                              c->d.max_context, cache_index, 0, c->err_flag, s);
  } else {
    e = kvc_launch_copy_rows(k_new, v_new, kl, vl, c->d.batch, gqa ? c->d.n_kv_heads : 1, t_new,
                             c->row_elems * c->elem, c->d.max_context, cache_index, 0, c->err_flag, s);
  }
  return after_launch(c, e, s);
}

kvc_status kvc_decode_attn(kvc_cache* c, int32_t layer, const void* q, void* out,
                           const int32_t* valid_lens, const int32_t* cache_index, float sm_scale,
                           void* stream) {
  if (!q || !out || !static_ok(c, layer)) return KVC_ERR_INVALID_ARG;
  if (!valid_lens && !cache_index) return KVC_ERR_INVALID_ARG;
  if (!(sm_scale > 0.0f) || sm_scale > 3.0e38f) return KVC_ERR_INVALID_ARG;
  void* kl;
  void* vl;
  kvc_layer_ptrs(c, layer, &kl, &vl);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (c->d.attn == KVC_ATTN_GQA && c->d.dtype == KVC_I8) {
    float* ks;
    float* vs;
    kvc_layer_scales(c, layer, (void**)&ks, (void**)&vs);
    e = kvc_launch_gqa_decode(c, kl, vl, q, out, valid_lens, cache_index, sm_scale, s, nullptr, nullptr, ks, vs);
  } else if (c->d.attn == KVC_ATTN_GQA)
    e = kvc_launch_gqa_decode(c, kl, vl, q, out, valid_lens, cache_index, sm_scale, s);
  else
    e = kvc_launch_mla_attn(c, kl, q, out, valid_lens, cache_index, sm_scale, s);
  return after_launch(c, e, s);
}

kvc_status kvc_prefill_attn(kvc_cache* c, int32_t layer, const void* q, const void* k, const void* v, void* out,
                            int32_t start, int32_t t, float sm_scale, void* stream) {
  if (!q || !k || !v || !out || !static_ok(c, layer)) return KVC_ERR_INVALID_ARG;
  if (c->d.attn != KVC_ATTN_GQA || c->d.dtype != KVC_BF16) return KVC_ERR_UNSUPPORTED;
  if (t < 1) return KVC_ERR_INVALID_ARG;
  if (start < 0 || (int64_t)start + t > c->d.max_context) return KVC_ERR_CAPACITY;
  if (!(sm_scale > 0.0f) || sm_scale > 3.0e38f) return KVC_ERR_INVALID_ARG;
  uint8_t* kl;
  uint8_t* vl;
  kvc_layer_ptrs(c, layer, (void**)&kl, (void**)&vl);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = kvc_launch_copy_rows(k, v, kl, vl, c->d.batch, c->d.n_kv_heads, t, c->row_elems * c->elem,
                                      c->d.max_context, nullptr, start, c->err_flag, s);
  if (e == hipSuccess) e = kvc_launch_prefill_attn(c, kl, vl, q, out, start, t, sm_scale, s);
  return after_launch(c, e, s);
}

kvc_status kvc_append_decode_attn(kvc_cache* c, int32_t layer, const void* k_new, const void* v_new,
                                  const void* q, void* out, const int32_t* cache_index, float sm_scale,
                                  void* stream) {
  if (!k_new || !v_new || !q || !out || !cache_index || !static_ok(c, layer)) return KVC_ERR_INVALID_ARG;
  if (c->d.attn != KVC_ATTN_GQA) return KVC_ERR_UNSUPPORTED;
  if (!(sm_scale > 0.0f) || sm_scale > 3.0e38f) return KVC_ERR_INVALID_ARG;
  void* kl;
  void* vl;
  kvc_layer_ptrs(c, layer, &kl, &vl);
  float* ks = nullptr;
  float* vs = nullptr;
  if (c->d.dtype == KVC_I8) kvc_layer_scales(c, layer, (void**)&ks, (void**)&vs);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = kvc_launch_gqa_decode(c, kl, vl, q, out, nullptr, cache_index, sm_scale, s, k_new, v_new, ks, vs);
  return after_launch(c, e, s);
}

kvc_status kvc_mla_decode(kvc_cache* c, int32_t layer, const void* q_nope, const void* q_rope,
                          const void* w_uk, const void* w_uv, void* out, const int32_t* valid_lens,
                          const int32_t* cache_index, float sm_scale, void* stream) {
  if (!q_nope || !q_rope || !w_uk || !w_uv || !out || !static_ok(c, layer))
    return KVC_ERR_INVALID_ARG;
  if (c->d.attn != KVC_ATTN_MLA) return KVC_ERR_INVALID_ARG;
  if (!valid_lens && !cache_index) return KVC_ERR_INVALID_ARG;
  if (!(sm_scale > 0.0f) || sm_scale > 3.0e38f) return KVC_ERR_INVALID_ARG;
  void* kl;
  void* vl;
  kvc_layer_ptrs(c, layer, &kl, &vl);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = kvc_launch_mla_absorb(c, q_nope, q_rope, w_uk, c->ws_qabs, s);
  if (e == hipSuccess)
    e = kvc_launch_mla_attn(c, kl, c->ws_qabs, c->ws_olat, valid_lens, cache_index, sm_scale, s);
  if (e == hipSuccess) e = kvc_launch_mla_uproj(c, c->ws_olat, w_uv, out, s);
  return after_launch(c, e, s);
}

kvc_status kvc_paged_append(kvc_cache* c, int32_t layer, const void* k_new, const void* v_new,
                            const int32_t* block_table, const int32_t* cache_index, int32_t t_new, void* stream) {
  if (!c || !c->paged || !layer_ok(c, layer) || !k_new || !v_new || !block_table || !cache_index)
    return KVC_ERR_INVALID_ARG;
  if (t_new < 1) return KVC_ERR_INVALID_ARG;
  if (t_new > c->d.max_context) return KVC_ERR_CAPACITY;
  uint8_t* kl;
  uint8_t* vl;
  kvc_layer_ptrs(c, layer, (void**)&kl, (void**)&vl);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = kvc_launch_paged_rows(k_new, v_new, kl, vl, block_table, c->d.batch, c->d.n_kv_heads, t_new,
                                       c->row_elems * c->elem, c->block_shift, c->num_blocks, c->table_width,
                                       c->d.max_context, cache_index, c->err_flag, s);
  return after_launch(c, e, s);
}

kvc_status kvc_paged_decode_attn(kvc_cache* c, int32_t layer, const void* q, void* out,
                                 const int32_t* block_table, const int32_t* valid_lens,
                                 const int32_t* cache_index, float sm_scale, void* stream) {
  if (!c || !c->paged || !layer_ok(c, layer) || !q || !out || !block_table) return KVC_ERR_INVALID_ARG;
  if (!valid_lens && !cache_index) return KVC_ERR_INVALID_ARG;
  if (!(sm_scale > 0.0f) || sm_scale > 3.0e38f) return KVC_ERR_INVALID_ARG;
  void* kl;
  void* vl;
  kvc_layer_ptrs(c, layer, &kl, &vl);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = kvc_launch_gqa_decode(c, kl, vl, q, out, valid_lens, cache_index, sm_scale, s, nullptr, nullptr,
                                       nullptr, nullptr, block_table);
  return after_launch(c, e, s);
}

kvc_status kvc_paged_append_decode_attn(kvc_cache* c, int32_t layer, const void* k_new, const void* v_new,
                                        const void* q, void* out, const int32_t* block_table,
                                        const int32_t* cache_index, float sm_scale, void* stream) {
  if (!c || !c->paged || !layer_ok(c, layer) || !k_new || !v_new || !q || !out || !block_table || !cache_index)
    return KVC_ERR_INVALID_ARG;
  if (!(sm_scale > 0.0f) || sm_scale > 3.0e38f) return KVC_ERR_INVALID_ARG;
  void* kl;
  void* vl;
  kvc_layer_ptrs(c, layer, &kl, &vl);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = kvc_launch_gqa_decode(c, kl, vl, q, out, nullptr, cache_index, sm_scale, s, k_new, v_new,
                                       nullptr, nullptr, block_table);
  return after_launch(c, e, s);
}

kvc_status kvc_set_workgroups(kvc_cache* c, int32_t n) {
  if (!c || n < 0 || n > c->max_workgroups) return KVC_ERR_INVALID_ARG;
  c->workgroups_forced = n;
  return KVC_OK;
}

kvc_status kvc_get_workgroups(const kvc_cache* c, int32_t* n, int32_t* max_n) {
  if (!c || !n) return KVC_ERR_INVALID_ARG;
  *n = c->workgroups_forced;
  if (max_n) *max_n = c->max_workgroups;
  return KVC_OK;
}

}  // extern "C"

// ---- decode attention for callers that cannot allocate --------------------
//
// kvc_decode_attn_noalloc runs the decode kernels of kvc_decode_attn with
// their workspace in this static array (one copy on each device, zero when
// the code object is loaded, held until the process ends) instead of the
// one kvc_alloc makes. Layout, from the start: the cached split of the work
// (its size fixed by the device's compute units), a flag word, the arrival
// counters (a fixed region of kNoAllocCounters), then the (m, l) pairs and
// the partial accumulators of the call's shape. The plan and the counters
// therefore never overlap another shape's partials; the counters and the
// plan's arrival count reset themselves at the end of every launch, and the
// plan is keyed by grid, mode, batch, segments per sequence and lengths.
// Calls that overlap on one device race on this memory.
namespace {

constexpr size_t kNoAllocBytes = 16u << 20;
constexpr size_t kNoAllocCounters = 65536;  // (sequence, query head) pairs, at most
__device__ __align__(256) static uint8_t scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};
int g_scratch_cus[kMaxDevices] = {};

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// The device address of `scratch` on the current device (the host-side name
// is not a device address) and its compute-unit count, looked up once per
// device with that device current.
kvc_status scratch_of_device(uint8_t** ptr, int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVC_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVC_ERR_DEVICE;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      return KVC_ERR_DEVICE;
    g_scratch_ptr[dev] = (uint8_t*)p;
    g_scratch_cus[dev] = n;
  }
  *ptr = g_scratch_ptr[dev];
  *cus = g_scratch_cus[dev];
  return KVC_OK;
}

}  // namespace

extern "C" {

kvc_status kvc_decode_attn_noalloc(const kvc_desc* desc, const void* k_layer, const void* v_layer, const void* q,
                                   void* out, const int32_t* valid_lens, const int32_t* cache_index,
                                   float sm_scale, int32_t* err_flag, void* stream) {
  kvc_status st = validate_desc(desc);
  if (st != KVC_OK) return st;
  if (desc->attn != KVC_ATTN_GQA || (desc->dtype != KVC_BF16 && desc->dtype != KVC_F32))
    return KVC_ERR_UNSUPPORTED;
  if (!k_layer || !v_layer || !q || !out || (!valid_lens && !cache_index)) return KVC_ERR_INVALID_ARG;
  if (!(sm_scale > 0.0f) || sm_scale > 3.0e38f) return KVC_ERR_INVALID_ARG;
  const uint64_t pairs = (uint64_t)desc->batch * desc->n_heads;
  if (pairs > kNoAllocCounters) return KVC_ERR_UNSUPPORTED;
  uint8_t* base = nullptr;
  int cus = 0;
  st = scratch_of_device(&base, &cus);
  if (st != KVC_OK) return st;

  // the launch as kvc_decode_attn makes it on a cache of this shape, with the
  // default grid (one workgroup per compute unit for these dtypes)
  kvc_cache c;
  memset(&c, 0, sizeof(c));
  c.d = *desc;
  c.num_cus = cus;
  c.elem = elem_size(desc->dtype);
  c.row_elems = desc->head_dim;
  c.max_workgroups = cus;
  c.ws_entries = ((uint64_t)cus + pairs) * 16;
  size_t off = 0;
  c.ws_plan = (int32_t*)(base + off);
  off += round256(((size_t)KVC_PLAN_HEAD + (size_t)cus * KVC_PLAN_INTS) * 4);
  int32_t* own_flag = (int32_t*)(base + off);
  off += 256;
  c.ws_cnt = (int32_t*)(base + off);
  off += round256(kNoAllocCounters * 4);
  c.ws_ml = (float*)(base + off);
  off += round256(c.ws_entries * 2 * sizeof(float));
  c.ws_acc = (float*)(base + off);
  off += round256(c.ws_entries * desc->head_dim * sizeof(float));
  if (off > kNoAllocBytes) return KVC_ERR_UNSUPPORTED;
  c.err_flag = err_flag ? err_flag : own_flag;
  const hipError_t e = kvc_launch_gqa_decode(&c, k_layer, v_layer, q, out, valid_lens, cache_index, sm_scale,
                                             (hipStream_t)stream);
  return e == hipSuccess ? KVC_OK : KVC_ERR_DEVICE;
}

kvc_status kvc_check(kvc_cache* c, void* stream) {
  if (!c) return KVC_ERR_INVALID_ARG;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return KVC_ERR_DEVICE;
  int32_t flag = 0;
  if (hipMemcpy(&flag, c->err_flag, sizeof(flag), hipMemcpyDeviceToHost) != hipSuccess)
    return KVC_ERR_DEVICE;
  if (flag) {
    if (hipMemset(c->err_flag, 0, sizeof(int32_t)) != hipSuccess) return KVC_ERR_DEVICE;
    if (hipDeviceSynchronize() != hipSuccess) return KVC_ERR_DEVICE;
    return KVC_ERR_DEVICE_RANGE;
  }
  return KVC_OK;
}

const char* kvc_strerror(kvc_status s) {
  switch (s) {
    case KVC_OK: return "ok";
    case KVC_ERR_INVALID_ARG: return "invalid argument";
    case KVC_ERR_CAPACITY: return "rows outside the cache capacity";
    case KVC_ERR_OOM: return "device allocation failed";
    case KVC_ERR_DEVICE: return "HIP runtime error";
    case KVC_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVC_ERR_DEVICE_RANGE: return "device-side index out of range (sequence skipped)";
  }
  return "unknown status";
}

}  // extern "C"
