// Row copies into the static cache: the prefill fill (rows [start, start+t)
// of every sequence) and the in-place decode append (rows
// [cache_index[b], cache_index[b] + t_new) of sequence b).
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

}  // namespace

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
