// Row copies into the cache: the prefill fill (rows [start, start+t) of
// every sequence) and the in-place decode append (rows
// [cache_index[b], cache_index[b] + t_new) of sequence b), into the static
// buffer or through a block table.
//
// "KV Cache Optimization: GQA Audit, In-Place Buffers, Persistent Prompts",
// "#2 In-place KV cache updates", "After": the new rows are slice-assigned
// into the fixed-capacity buffer and nothing else changes. "10.3 - KV cache
// implementation details", section 5 step 2: append k_t, v_t to the layer's
// cache. Both are pure bit copies.
//
// Layout: src is [B][G][t][row] (G = H_kv, or 1 for the latent cache) and
// dst is [B][G][S][row]; for each (b, g) the t source rows are contiguous and
// land on a contiguous block of t rows in dst, so the copy is a set of
// contiguous 16-byte vectors: one thread per vector, fully coalesced on both
// sides. K and V are copied by the same thread.

#include "kvc_internal.h"

namespace {

__global__ __launch_bounds__(256) void copy_rows_kernel(
    const uint4* __restrict__ src_k, const uint4* __restrict__ src_v, uint4* __restrict__ dst_k,
    uint4* __restrict__ dst_v, int groups_per_seq, int t, int row_vecs, int max_context,
    long total_vecs, const int32_t* __restrict__ dev_start, int host_start,
    int32_t* __restrict__ err_flag) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total_vecs) return;
  const long block_vecs = (long)t * row_vecs;   // vectors of one (b, g) block
  const long bg = i / block_vecs;               // flattened (b, g)
  const long off = i - bg * block_vecs;         // vector offset inside the block
  const int b = (int)(bg / groups_per_seq);
  const int start = dev_start ? dev_start[b] : host_start;
  if (start < 0 || (long)start + t > max_context) {
    // skipped sequence: one thread per sequence raises the sticky flag
    if (off == 0 && bg % groups_per_seq == 0) atomicOr(err_flag, 1);
    return;
  }
  const long dst = (bg * max_context + start) * (long)row_vecs + off;
  dst_k[dst] = src_k[i];
  if (src_v) dst_v[dst] = src_v[i];
}

// Append through a block table ("10.3 - KV cache implementation details",
// section 7.2): row r of sequence b goes to row r % block_size of physical
// block table[b][r / block_size], pool layout [num_blocks][G][block_size][row].
// Grid (ceil(G t row_vecs / 256), B): every workgroup of sequence b first
// checks that the rows fit and that every table entry they reach lies in
// the pool (a few entries per thread), so the whole sequence is written or
// skipped; then each thread copies one 16-byte vector of K and of V.
__global__ __launch_bounds__(256) void paged_rows_kernel(
    const uint4* __restrict__ src_k, const uint4* __restrict__ src_v, uint4* __restrict__ pool_k,
    uint4* __restrict__ pool_v, const int32_t* __restrict__ table, int groups, int t, int row_vecs,
    int block_shift, int num_blocks, int table_width, int max_context, const int32_t* __restrict__ dev_start,
    int32_t* __restrict__ err_flag) {
  const int b = blockIdx.y;
  const int start = dev_start[b];
  const int32_t* trow = table + (long)b * table_width;
  bool bad = start < 0 || (long)start + t > max_context;  // the same in every thread
  if (!bad) {
    const int first = start >> block_shift;
    const int last = (start + t - 1) >> block_shift;
    int any = 0;
    for (int i = first + (int)threadIdx.x; i <= last; i += 256) any |= trow[i] < 0 || trow[i] >= num_blocks;
    bad = __syncthreads_or(any) != 0;
  }
  if (bad) {
    if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(err_flag, 1);
    return;
  }
  const long per_seq = (long)groups * t * row_vecs;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= per_seq) return;
  const long per_group = (long)t * row_vecs;
  const int g = (int)(i / per_group);
  const int rem = (int)(i - g * per_group);
  const int row = rem / row_vecs;
  const int vec = rem - row * row_vecs;
  const int r = start + row;
  const long blk = trow[r >> block_shift];
  const long dst = (((blk * groups + g) << block_shift) + (r & ((1 << block_shift) - 1))) * row_vecs + vec;
  const long src = (long)b * per_seq + i;
  pool_k[dst] = src_k[src];
  pool_v[dst] = src_v[src];
}

// Live-prefix image ("KV Cache Optimization: GQA Audit, In-Place Buffers,
// Persistent Prompts", "#3 Persistent KV across sessions": only the live
// prefix is saved). Grid (x chunks, sequence b, layer * kv_parts + kv): the
// n_b rows of every kv head of (b, layer, kv) are one run in the cache per
// head ([S] rows apart) and one packed run in the image, copied as units of
// U (16-byte vectors for rows, 4-byte words for int8 scales).
typedef uint32_t vec4u __attribute__((ext_vector_type(4)));  // 16-byte unit (a vector type for nt loads)

template <typename U>
__global__ __launch_bounds__(256) void prefix_copy_kernel(U* __restrict__ cache, U* __restrict__ image,
                                                          const int32_t* __restrict__ map, bool save,
                                                          long long layer_units, long long kv_units, int kv_parts,
                                                          int groups, int max_context, int row_units,
                                                          long long total_rows) {
  const int b = blockIdx.y;
  const int lk = blockIdx.z;
  const int n = map[2 * b];
  if (n <= 0) return;
  const long long first = map[2 * b + 1];
  const int layer = lk / kv_parts;
  const int kv = lk - layer * kv_parts;
  const long long run = (long long)n * row_units;  // units of one kv head's rows
  const long long units = run * groups;
  U* cb = cache + layer * layer_units + kv * kv_units + (long long)b * groups * max_context * row_units;
  U* ib = image + ((long long)lk * total_rows + first) * groups * row_units;
  // every unit is read once and written once: non-temporal on both sides
  auto move = [&](U* cp, U* ip) {
    if (save)
      __builtin_nontemporal_store(__builtin_nontemporal_load(cp), ip);
    else
      __builtin_nontemporal_store(__builtin_nontemporal_load(ip), cp);
  };
  if (units < (1LL << 31)) {  // 32-bit index arithmetic (the usual case)
    const uint32_t run32 = (uint32_t)run;
    for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < (uint32_t)units; i += gridDim.x * 256u) {
      const uint32_t g = i / run32;
      const uint32_t rem = i - g * run32;
      move(cb + (long long)g * max_context * row_units + rem, ib + (long long)g * run + rem);
    }
    return;
  }
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < units; i += (long long)gridDim.x * 256) {
    const int g = (int)(i / run);
    const long long rem = i - g * run;
    move(cb + (long long)g * max_context * row_units + rem, ib + g * run + rem);
  }
}

}  // namespace

hipError_t kvc_launch_prefix_copy(uint8_t* cache, uint8_t* image, const int32_t* map, bool save,
                                  uint64_t layer_bytes, uint64_t kv_bytes, int n_layers, int kv_parts, int batch,
                                  int max_batch_rows, int groups, int max_context, int row_bytes, int unit_bytes,
                                  int64_t total_rows, hipStream_t stream) {
  if (row_bytes % unit_bytes != 0 || layer_bytes % unit_bytes != 0 || kv_bytes % unit_bytes != 0)
    return hipErrorInvalidValue;
  if (max_batch_rows <= 0) return hipSuccess;  // no rows to copy
  if (batch > 65535 || (long long)n_layers * kv_parts > 65535) return hipErrorInvalidValue;
  const int row_units = row_bytes / unit_bytes;
  const long long units = (long long)max_batch_rows * groups * row_units;
  long long gx = (units + 1023) / 1024;  // about four units per thread
  if (gx > 65535) gx = 65535;
  const dim3 grid((unsigned)gx, (unsigned)batch, (unsigned)(n_layers * kv_parts));
  if (unit_bytes == 16)
    prefix_copy_kernel<vec4u><<<grid, dim3(256), 0, stream>>>(
        (vec4u*)cache, (vec4u*)image, map, save, (long long)(layer_bytes / 16), (long long)(kv_bytes / 16), kv_parts,
        groups, max_context, row_units, total_rows);
  else if (unit_bytes == 4)
    prefix_copy_kernel<uint32_t><<<grid, dim3(256), 0, stream>>>(
        (uint32_t*)cache, (uint32_t*)image, map, save, (long long)(layer_bytes / 4), (long long)(kv_bytes / 4),
        kv_parts, groups, max_context, row_units, total_rows);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t kvc_launch_paged_rows(const void* src_k, const void* src_v, uint8_t* pool_k, uint8_t* pool_v,
                                 const int32_t* table, int batch, int n_kv_heads, int t, int row_bytes,
                                 int block_shift, int num_blocks, int table_width, int max_context,
                                 const int32_t* dev_start, int32_t* err_flag, hipStream_t stream) {
  if (row_bytes % 16 != 0 || !dev_start || !table) return hipErrorInvalidValue;
  const int row_vecs = row_bytes / 16;
  const long per_seq = (long)n_kv_heads * t * row_vecs;
  const long blocks = (per_seq + 255) / 256;
  if (blocks > 0x7fffffffL || batch > 65535) return hipErrorInvalidValue;
  paged_rows_kernel<<<dim3((unsigned)blocks, (unsigned)batch), dim3(256), 0, stream>>>(
      (const uint4*)src_k, (const uint4*)src_v, (uint4*)pool_k, (uint4*)pool_v, table, n_kv_heads, t, row_vecs,
      block_shift, num_blocks, table_width, max_context, dev_start, err_flag);
  return hipGetLastError();
}

hipError_t kvc_launch_copy_rows(const void* src_k, const void* src_v, uint8_t* dst_k, uint8_t* dst_v,
                                int batch, int n_kv_heads, int t, int row_bytes, int max_context,
                                const int32_t* dev_start, int host_start, int32_t* err_flag,
                                hipStream_t stream) {
  if (row_bytes % 16 != 0) return hipErrorInvalidValue;
  const int row_vecs = row_bytes / 16;
  const long total = (long)batch * n_kv_heads * t * row_vecs;
  const int threads = 256;
  const long blocks = (total + threads - 1) / threads;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  copy_rows_kernel<<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(
      (const uint4*)src_k, (const uint4*)src_v, (uint4*)dst_k, (uint4*)dst_v, n_kv_heads, t,
      row_vecs, max_context, total, dev_start, host_start, err_flag);
  return hipGetLastError();
}
