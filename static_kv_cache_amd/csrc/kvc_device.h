// Device-side pieces shared by the attention kernels (GQA and latent):
// vector types, bf16 rounding, the row space that the persistent grid splits,
// and the device-coherent accesses used to hand partials between workgroups.
// Internal to libkvc.so.
#pragma once

#include <math.h>
#include <stdint.h>

#include "kvc_internal.h"

namespace kvcd {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBufWord3 = 0x00020000;  // raw buffer resource word 3 (32-bit data format)
// Cache policy of the loads that stream the cache rows: "nt" (non-temporal).
// A decode launch reads each row once, so the rows are not kept in the L2 and
// the Infinity Cache (Llama-3-shaped layer: 36.0 -> 33.9 us; sc0 made no
// difference and sc1 was slower).
constexpr int kStreamLoad = 2;
// Cache policy "sc1" of a raw buffer store (written through to memory) and
// of a raw buffer load (coherent at device scope, as the relaxed agent-scope
// accesses below: reads partials stored by workgroups on other XCDs).
constexpr int kWriteThrough = 16;
constexpr int kCoherentLoad = 16;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Values the caller knows to be the same in every lane (derived from shared
// memory or kernel arguments), taken from the first lane so the compiler
// keeps them in scalar registers: loop bounds become scalar branches, and a
// buffer descriptor built from them stays in SGPRs (a descriptor the
// compiler thinks divergent wraps every load in a waterfall loop).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ const void* uniform(const void* p) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}
// Raw buffer descriptor over [p, p + nbytes) (p and nbytes wave-uniform):
// loads at or past nbytes return zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(uniform(p)), 0, uniform(nbytes), kBufWord3);
}

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ void store_out(uint16_t* p, float f) { *p = bf16_rne(f); }
__device__ __forceinline__ void store_out(float* p, float f) { *p = f; }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Valid rows of sequence b as the kernels use them: lengths outside
// [min_rows, max_context] count as 0 (the sequence is skipped and flagged).
// min_rows is 1 when the launch also appends the row at cache_index[b].
__device__ __forceinline__ int seq_rows(const int32_t* valid_lens, const int32_t* cache_index, int b,
                                        int max_context, int min_rows, bool* bad) {
  const int n = valid_lens ? valid_lens[b] : cache_index[b] + 1;
  *bad = n < min_rows || n > max_context;
  return *bad ? 0 : n;
}

// Partials handed between workgroups of one kernel, which may sit on
// different XCDs (each with its own L2), are written and read with
// device-scope relaxed atomic accesses (global_store/load ... sc1): coherent
// at device scope per location. A writer waits for its stores to complete
// (vmcnt(0)) before it counts itself in, and the last arrival reads them
// back. This avoids the full-L2 writeback/invalidate of a device-scope fence.
__device__ __forceinline__ void put(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// the same for two consecutive floats (8-byte aligned), in one load
__device__ __forceinline__ void get2(const float* p, float& x, float& y) {
  const uint64_t u = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  x = __uint_as_float((uint32_t)u);
  y = __uint_as_float((uint32_t)(u >> 32));
}
// s_waitcnt vmcnt(0) (expcnt, lgkmcnt left alone): this thread's stores are done
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---- the row space ---------------------------------------------------------
//
// A "segment" is the valid rows [0, n_b) of one (sequence, head chunk) pair
// (for GQA the chunk runs over kv heads and query-head chunks; for the
// latent cache over query-head chunks). The HC segments of sequence b are
// laid end to end in one row space, each taking u_b = n_b + seg_rows
// virtual rows (none if n_b = 0) of which the last n_b are real: seg_rows
// stands for the fixed start-up cost of a segment (query load, the first
// tile's latency, the epilogue), so a workgroup whose range crosses into a
// new segment is handed correspondingly fewer real rows. The workgroups
// take consecutive ranges of the row space (Partition below); the part of a
// segment inside one workgroup's range is a "piece".

constexpr int kMaxSpan = 64;               // the longest segment spans <= kMaxSpan + 2 workgroups
constexpr int kMaxMerge = kMaxSpan + 2;    // pieces of one segment, at most
constexpr int kMinRowsPerWorkgroup = 64;   // and every workgroup gets >= 64 rows (no empty ranges)
constexpr int kMaxSegRows = 1024;          // start-up rows allowed (the desc limits keep R < 2^31)

// The split of the row space among the persistent workgroups: workgroup w
// takes [lo(w), lo(w + 1)) with lo(w) = R w / W. The grid is capped so that
// every share has >= kMinRowsPerWorkgroup rows and >= 1/kMaxSpan of the
// longest segment (u_max virtual rows), so a segment is cut into at most
// kMaxMerge pieces.
struct Partition {
  long long R;
  int W;

  __device__ __forceinline__ Partition(long long R_, int n_wg, int u_max) : R(R_), W(1) {
    long long w = n_wg;
    w = min(w, max(1LL, R * kMaxSpan / max(u_max, 1)));
    w = min(w, max(1LL, R / kMinRowsPerWorkgroup));
    W = (int)w;
  }
  __device__ __forceinline__ long long lo(int w) const { return w >= W ? R : R * w / W; }
  // Workgroup whose range contains row x.
  __device__ __forceinline__ int of(long long x) const {
    int w = (int)(x * W / R);
    w = min(max(w, 0), W - 1);
    while (w + 1 < W && lo(w + 1) <= x) ++w;
    while (w > 0 && lo(w) > x) --w;
    return w;
  }
};

// Prefix sums s_prefix[0..B] of u_b and the largest u_b, by the first wave
// (64 sequences per pass, an inclusive shuffle scan within the wave and a
// running offset between passes), written to shared memory without a
// barrier; only the first wave calls it. Out-of-range lengths raise
// *err_flag when flag_errors is set. With `snap`, *s_same tells whether
// every length is non-zero and equal to snap[b].
__device__ __forceinline__ void scan_lengths(const int32_t* valid_lens, const int32_t* cache_index, int B,
                                             int max_context, int seg_rows, int32_t* s_prefix, int32_t* s_umax,
                                             int32_t* err_flag, bool flag_errors, int min_rows,
                                             const int32_t* snap, int32_t* s_same) {
  const int t = threadIdx.x;
  {
    int carry = 0, umax = 0;
    bool same = snap != nullptr;  // every length equal to snap[b] and non-zero
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int b = b0 + t;
      int n = 0;
      if (b < B) {
        bool bad;
        n = seq_rows(valid_lens, cache_index, b, max_context, min_rows, &bad);
        if (bad && flag_errors) atomicOr(err_flag, 1);
        if (snap) same = same && n > 0 && snap[b] == n;
      }
      int x = n > 0 ? n + seg_rows : 0;
      umax = max(umax, x);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        x += (t >= off) ? y : 0;
      }
      if (b < B) s_prefix[b + 1] = carry + x;
      carry += __shfl(x, 63);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) umax = max(umax, __shfl_xor(umax, off));
    if (snap) same = __builtin_amdgcn_ballot_w64(!same) == 0;
    if (t == 0) {
      s_prefix[0] = 0;
      *s_umax = umax;
      if (s_same) *s_same = same ? 1 : 0;
    }
  }
}

// scan_lengths by the first wave, then a barrier that publishes the sums.
// Every thread of the workgroup must call it.
__device__ __forceinline__ void build_row_space(const int32_t* valid_lens, const int32_t* cache_index, int B,
                                                int max_context, int seg_rows, int32_t* s_prefix,
                                                int32_t* s_umax, int32_t* err_flag, bool flag_errors,
                                                int min_rows = 0) {
  if (threadIdx.x < 64)
    scan_lengths(valid_lens, cache_index, B, max_context, seg_rows, s_prefix, s_umax, err_flag, flag_errors,
                 min_rows, nullptr, nullptr);
  __syncthreads();
}

// ---- the cached split of the work ------------------------------------------
//
// The split (each workgroup's pieces) depends only on the valid lengths, the
// grid and the append mode, which the layers of one decode step share. A
// launch that finds the cached plan made for its lengths takes its pieces
// from its entry and starts streaming without the partition and piece
// search (the decode kernel even starts its first piece before the lengths
// have arrived, and confirms them at a barrier after the piece's first
// loads). Otherwise it works the split out,
// records its entry, and the last workgroup to finish publishes the header
// (so no workgroup of that launch can see a header whose entries are not
// written yet). Launches with an empty or out-of-range sequence never
// publish. Layout (KVC_PLAN_* in kvc_internal.h): header [valid, grid, mode
// (min rows + 2 x segments per sequence), batch, arrival count, 0, 0, 0],
// the lengths, then per workgroup a
// piece count (-1: more than kPlanPieces) and kPieceInts ints per piece
// (b, hc, r_begin, r_end, n, w0, np; w0, np = the segment's first workgroup
// and number of pieces, for pieces that are part of a segment).
constexpr int kPlanPieces = 8;
constexpr int kPieceInts = 7;
static_assert(1 + kPlanPieces * kPieceInts <= KVC_PLAN_INTS, "plan entry too small");

struct PlanState {
  int32_t gate;  // the header and the lengths match: the cached plan is for this launch
  int32_t last;  // this workgroup publishes the new header
};

// Whether the header names this launch's grid, mode and batch (the lengths
// are compared by scan_lengths). Uniform: every wave reads it.
__device__ __forceinline__ bool plan_key(const int32_t* plan, int n_wg, int mode, int B) {
  // the four header words in one load, compared without short-circuit
  // branches (which made them four dependent loads at the kernel's start)
  const int4 h = *reinterpret_cast<const int4*>(plan);
  return (h.x == 1) & (h.y == n_wg) & (h.z == mode) & (h.w == B);
}

// This workgroup's cached entry.
__device__ __forceinline__ const int32_t* plan_entry(const int32_t* plan) {
  return plan + KVC_PLAN_HEAD + (size_t)blockIdx.x * KVC_PLAN_INTS;
}

// Records piece k of this workgroup's new entry (thread 0; `recorded` is its count, -1 once full).
__device__ __forceinline__ void plan_record(int32_t* plan, int& recorded, int b, int hc, int r_begin, int r_end,
                                            int n, int w0, int np) {
  if (threadIdx.x != 0 || recorded < 0) return;
  if (recorded == kPlanPieces) {
    recorded = -1;
    return;
  }
  int32_t* pc = plan + KVC_PLAN_HEAD + (size_t)blockIdx.x * KVC_PLAN_INTS + 1 + recorded * kPieceInts;
  pc[0] = b;
  pc[1] = hc;
  pc[2] = r_begin;
  pc[3] = r_end;
  pc[4] = n;
  pc[5] = w0;
  pc[6] = np;
  ++recorded;
}

// End of a launch that worked the split out: every thread calls it. Writes
// the entry's count, counts the workgroup in, and the last workgroup of the
// launch publishes the header for the lengths in s_prefix (u_b = n_b +
// seg_rows per non-empty sequence).
__device__ __forceinline__ void plan_publish(int32_t* plan, PlanState& st, int recorded, const int32_t* s_prefix,
                                             int B, int seg_rows, int n_wg, int mode) {
  const int t = threadIdx.x;
  if (t == 0) {
    plan[KVC_PLAN_HEAD + (size_t)blockIdx.x * KVC_PLAN_INTS] = recorded;
    const int arrived = __hip_atomic_fetch_add(plan + 4, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    st.last = arrived == n_wg - 1;
  }
  __syncthreads();
  if (!st.last) return;
  bool all = true;
  for (int b = t; b < B; b += blockDim.x) {
    const int u = s_prefix[b + 1] - s_prefix[b];
    all = all && u > 0;
    plan[KVC_PLAN_LENS + b] = u > 0 ? u - seg_rows : 0;
  }
  const int usable = __syncthreads_and(all ? 1 : 0);
  if (t == 0) {
    plan[1] = n_wg;
    plan[2] = mode;
    plan[3] = B;
    plan[4] = 0;
    plan[0] = usable ? 1 : 0;
  }
}

// Calls f(b, hc, r_begin, r_end, n, real0) for every piece of the row range
// [x, hi): rows [r_begin, r_end) (r_end > r_begin) of segment (b, hc), whose
// n real rows start at row-space position real0.
template <class F>
__device__ __forceinline__ void for_each_piece(const int32_t* s_prefix, int B, int HC, int seg_rows,
                                               long long x, long long hi, F&& f) {
  // first segment holding row x: sequence by binary search, then head chunk
  int lo_b = 0, hi_b = B - 1;
  while (lo_b < hi_b) {
    const int mid = (lo_b + hi_b + 1) >> 1;
    if ((long long)s_prefix[mid] * HC <= x) lo_b = mid; else hi_b = mid - 1;
  }
  int b = lo_b;
  while ((long long)s_prefix[b + 1] * HC <= x) ++b;  // skip empty sequences
  int u = s_prefix[b + 1] - s_prefix[b];               // virtual rows per segment of b
  int hc = (int)((x - (long long)s_prefix[b] * HC) / u);
  while (x < hi) {
    const long long vs = (long long)s_prefix[b] * HC + (long long)hc * u;
    const long long real0 = vs + seg_rows;
    const long long seg_end = vs + u;
    const long long piece_end = seg_end < hi ? seg_end : hi;
    const int n = u - seg_rows;
    const int r_begin = x > real0 ? (int)(x - real0) : 0;
    const int r_end = piece_end > real0 ? (int)(piece_end - real0) : 0;
    if (r_end > r_begin) f(b, hc, r_begin, r_end, n, real0);  // else only virtual rows
    x = piece_end;
    if (x >= hi) break;
    if (++hc == HC) {  // next sequence with rows
      hc = 0;
      do { ++b; } while (s_prefix[b + 1] == s_prefix[b]);
      u = s_prefix[b + 1] - s_prefix[b];
    }
  }
}

}  // namespace kvcd
