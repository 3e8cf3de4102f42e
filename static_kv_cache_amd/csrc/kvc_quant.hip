// Quantising row copy into an int8 cache: the prefill fill and the in-place
// append of KVC_I8 caches.
//
// "10.3 - KV cache implementation details", section 4.4: the cache stored in
// lower precision (int8, p_cache = 1). "KV Cache Optimization: GQA Audit,
// In-Place Buffers, Persistent Prompts", "#2 ... After" / "Mutual
// exclusion": the new rows are slice-assigned into the fixed buffer, and a
// quantisation composes with that only if no row is ever re-quantised, so
// each row is quantised exactly once, here, when it is written:
//   amax = max_i |x_i|, scale = amax / 127,
//   code_i = round_half_even(x_i * (127 / amax)) clamped to [-127, 127],
// every step in IEEE binary32 (correctly rounded division and product, then
// v_rndne), a row of zeros giving scale 0 and codes 0. Nothing else of the
// cache changes.
//
// Layout: src is bf16 [B][G][t][D]; the codes go to [B][G][S][D] (int8) and
// the scale to [B][G][S] (float32). Sixteen consecutive lanes take one row
// (D / 16 elements each): the row maximum is four xor-shuffles inside the
// sixteen, then every lane writes its D / 16 codes and the first lane the
// scale. K rows come first, then V rows, one grid.

#include "kvc_internal.h"

namespace {

template <int EPL>  // elements per lane: D / 16
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ src_k,
                                                         const uint16_t* __restrict__ src_v, int8_t* __restrict__ dst_k,
                                                         int8_t* __restrict__ dst_v, float* __restrict__ ks,
                                                         float* __restrict__ vs, int groups_per_seq, int t,
                                                         int max_context, long rows_per_tensor,
                                                         const int32_t* __restrict__ dev_start, int host_start,
                                                         int32_t* __restrict__ err_flag) {
  constexpr int D = 16 * EPL;
  const long r = ((long)blockIdx.x * blockDim.x + threadIdx.x) >> 4;  // row of this lane group
  const int sub = threadIdx.x & 15;                                    // lane within the group
  if (r >= 2 * rows_per_tensor) return;                                // whole groups exit together
  const bool is_v = r >= rows_per_tensor;
  const long rr = is_v ? r - rows_per_tensor : r;  // row inside [B][G][t]
  const long bg = rr / t;
  const int i = (int)(rr - bg * t);
  const int b = (int)(bg / groups_per_seq);
  const int start = dev_start ? dev_start[b] : host_start;
  if (start < 0 || (long)start + t > max_context) {
    // skipped sequence: the first lane of the sequence's first K row raises the flag
    if (!is_v && sub == 0 && i == 0 && bg % groups_per_seq == 0) atomicOr(err_flag, 1);
    return;
  }
  const uint16_t* src = (is_v ? src_v : src_k) + rr * D + sub * EPL;
  float x[EPL];
#pragma unroll
  for (int e = 0; e < EPL; e += 2) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(src + e);
    x[e] = __uint_as_float(w << 16);
    x[e + 1] = __uint_as_float(w & 0xFFFF0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
  const bool zero = amax == 0.0f;
  const float inv = zero ? 0.0f : __fdiv_rn(127.0f, amax);  // binary32, correctly rounded
  const long dst_row = bg * max_context + start + i;
  uint32_t words[EPL / 4];
#pragma unroll
  for (int e = 0; e < EPL; e += 4) {
    uint32_t wd = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float c = rintf(__fmul_rn(x[e + k], inv));  // half to even; the product is not fused
      c = fminf(fmaxf(c, -127.0f), 127.0f);
      wd |= ((uint32_t)(int)c & 0xFFu) << (8 * k);
    }
    words[e / 4] = wd;
  }
  int8_t* dst = (is_v ? dst_v : dst_k) + dst_row * D + sub * EPL;
  if constexpr (EPL == 4) {
    *reinterpret_cast<uint32_t*>(dst) = words[0];
  } else if constexpr (EPL == 8) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(words[0], words[1]);
  } else {
#pragma unroll
    for (int k = 0; k < EPL / 16; ++k)
      reinterpret_cast<uint4*>(dst)[k] = make_uint4(words[4 * k], words[4 * k + 1], words[4 * k + 2], words[4 * k + 3]);
  }
  if (sub == 0) (is_v ? vs : ks)[dst_row] = zero ? 0.0f : __fdiv_rn(amax, 127.0f);
}

}  // namespace

hipError_t kvc_launch_quant_rows(const void* src_k, const void* src_v, uint8_t* dst_k, uint8_t* dst_v,
                                 float* ks, float* vs, int batch, int n_kv_heads, int t, int head_dim,
                                 int max_context, const int32_t* dev_start, int host_start,
                                 int32_t* err_flag, hipStream_t stream) {
  const long rows = (long)batch * n_kv_heads * t;  // per tensor
  const long threads_total = 2 * rows * 16;
  const long blocks = (threads_total + 255) / 256;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  const auto* sk = static_cast<const uint16_t*>(src_k);
  const auto* sv = static_cast<const uint16_t*>(src_v);
  auto* dk = reinterpret_cast<int8_t*>(dst_k);
  auto* dv = reinterpret_cast<int8_t*>(dst_v);
  switch (head_dim) {
    case 64:
      quant_rows_kernel<4><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
          sk, sv, dk, dv, ks, vs, n_kv_heads, t, max_context, rows, dev_start, host_start, err_flag);
      break;
    case 128:
      quant_rows_kernel<8><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
          sk, sv, dk, dv, ks, vs, n_kv_heads, t, max_context, rows, dev_start, host_start, err_flag);
      break;
    case 256:
      quant_rows_kernel<16><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
          sk, sv, dk, dv, ks, vs, n_kv_heads, t, max_context, rows, dev_start, host_start, err_flag);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
