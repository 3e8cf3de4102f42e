// Decode attention over the static cache (MHA / GQA / MQA).
//
// What is computed ("10.3 - KV cache implementation details", section 5
// step 2, and section 4.1-4.2 for shared key/value heads): for every
// sequence b and query head h, with kv head g = h / (H / H_kv) and
// n = n_b valid rows,
//     out[b,h] = softmax(sm_scale * K[b,g,0:n] q[b,h]) V[b,g,0:n].
// Rows at or past n are never loaded ("KV Cache Optimization ...", "#2 ...
// After": reads stop at the valid length).
//
// How (flash-decoding style, exact up to rounding order):
//  - Work space. A "segment" is the valid rows [0, n_b) of one (sequence,
//    kv head, head chunk); segments are laid end to end in one row space
//    (each with a fixed number of start-up rows in front, P::kSegRows).
//    The grid is persistent: one 256-thread workgroup per CU by default, and
//    the workgroups take consecutive equal ranges of that space (stream-K
//    style), so every workgroup streams about the same number of rows
//    whatever the ragged valid lengths are, in one round. The part of a
//    segment inside one workgroup (a "piece") is processed as a unit.
//  - A piece is streamed ONCE and applied to all query heads of its head
//    chunk. bf16 caches (MfmaPiece): each wave takes 16-row tiles in turn;
//    q.k is one v_mfma_f32_16x16x32_bf16 per 32 dims with the 16 K rows as
//    the A operand (static caches: loaded from HBM as whole 1 KB blocks,
//    staged in LDS and read back in the operand's layout; block-table
//    caches: loaded in that layout) and the
//    chunk's query heads, zero-padded to 16, as the B operand; the score
//    tile that comes out is exactly the A operand of p.v
//    (v_mfma_f32_16x16x16_bf16, K = the 16 rows), and V reaches its B
//    operand through a row-major, skewed LDS tile read back with
//    ds_read_b64_tr_b16 (one transpose read per 16 output columns). Each
//    wave keeps its next tile in flight in registers while it uses the
//    current one. fp32 caches (ValuPiece): one row per LPR consecutive
//    lanes, FMA partial dots summed with DPP adds (quad_perm,
//    row_half_mirror, row_mirror) and FMA accumulation. Softmax is the fp32
//    online form in log2 units in both.
//  - The waves (and, for fp32, a wave's row slots) are combined at the end
//    of a piece (cross-lane shuffles, then LDS). A piece that is a whole
//    segment is normalised and written directly. Otherwise it stores its
//    partial (m, l, acc[D]) to slot w + s of the workspace (unique per
//    workgroup w and segment s) with device-coherent stores, waits for them
//    to complete and counts itself in on the segment's counter; the last
//    piece to arrive merges all of them with exp2(m_p - m*) weights and
//    resets the counter (no device-scope fence: see put/get below). One
//    kernel per call.
// Empty sequences (n = 0) give zeros; out-of-range n gives zeros and raises
// the sticky device flag.

#include <math.h>

#include <type_traits>

#include "kvc_device.h"

namespace {

using namespace kvcd;

constexpr float kLazy = 8.0f;  // log2 headroom before the running maximum is moved (VALU piece)
constexpr float kLazyMfma = 64.0f;  // the same for the matrix-core piece (fp32 sums, bf16 P)
constexpr int kWaves = 4;      // waves per workgroup
constexpr int kThreads = 64 * kWaves;

template <typename T>
struct Storage;
template <>
struct Storage<float> {  // fp32: 4 elements per 16-byte vector
  static constexpr int kEPV = 4;
};

// Cross-lane move within a row of 16 lanes. All patterns used here are
// permutations, so every source lane is valid; bound_ctrl lets the compiler
// fold the move into the consuming add (v_add_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of LPR lanes; every lane of a group gets the sum.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (LPR >= 2) x += dpp<0xB1>(x);    // quad_perm(1,0,3,2): lane ^ 1
  if constexpr (LPR >= 4) x += dpp<0x4E>(x);    // quad_perm(2,3,0,1): lane ^ 2
  if constexpr (LPR >= 8) x += dpp<0x141>(x);   // row_half_mirror: other quad of the 8
  if constexpr (LPR >= 16) x += dpp<0x140>(x);  // row_mirror: other half of the 16
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  if constexpr (LPR >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Partial dot product of one 16-byte vector of q with one of k.
__device__ __forceinline__ float vec_dot(const uint4& q, const uint4& k, uint16_t) {
  float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.x),
                                            __builtin_bit_cast(bf16x2_t, k.x), 0.0f, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.y),
                                      __builtin_bit_cast(bf16x2_t, k.y), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.z),
                                      __builtin_bit_cast(bf16x2_t, k.z), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w),
                                      __builtin_bit_cast(bf16x2_t, k.w), s, false);
  return s;
}
__device__ __forceinline__ float vec_dot(const uint4& q, const uint4& k, float) {
  float s = __uint_as_float(q.x) * __uint_as_float(k.x);
  s = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), s);
  s = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), s);
  s = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), s);
  return s;
}

// 16-byte vector -> fp32 elements.
__device__ __forceinline__ void vec_unpack(const uint4& v, float (&f)[8], uint16_t) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void vec_unpack(const uint4& v, float (&f)[4], float) {
  f[0] = __uint_as_float(v.x);
  f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z);
  f[3] = __uint_as_float(v.w);
}

struct DecodeArgs {
  const void* k;               // layer keys   [B][H_kv][S][D]
  const void* v;               // layer values [B][H_kv][S][D]
  const void* q;               // [B][H][D]
  void* out;                   // [B][H][D]
  const int32_t* valid_lens;   // [B] or null
  const int32_t* cache_index;  // [B] or null
  float scale_log2;
  int batch, n_heads, n_kv_heads, max_context;
  int head_chunks;             // chunks per kv head's query group
  int chunk_heads;             // query heads per chunk (group / head_chunks)
  int n_wg;                    // persistent grid size (launched)
  int whole_rows;              // segments of at most this many rows each go whole to one workgroup (0: never)
  float* ws_acc;               // [slot][GC][D]
  float* ws_ml;                // [slot][GC][2]
  int32_t* ws_cnt;             // [B * H_kv * chunks] arrival counters (self-resetting)
  int32_t* err_flag;
  // int8 caches: the layer's row scales [B][H_kv][S] (null otherwise)
  const float* k_scale;
  const float* v_scale;
  // Fused append (null for plain decode): the new rows [B][H_kv][1][D]. Row
  // n_b - 1 = cache_index[b] of every segment is then taken from here, not
  // from the cache, and written into the cache by the piece that ends there.
  const void* k_new;
  const void* v_new;
  int32_t* plan;               // decode plan cache (KVC_PLAN_HEAD + n_wg * KVC_PLAN_INTS ints)
  // Block-table caches (null otherwise): k and v are the layer's pools
  // [num_blocks][H_kv][block_size][D] of pool_bytes bytes each, and row r of
  // sequence b lives in block table[b * table_width + (r >> block_shift)].
  const int32_t* table;
  int block_shift, num_blocks, table_width, pool_bytes;
};

// Fused append: the piece of segment (b, g, chunk) that ends at the
// segment's last row holds the new row (else -1).
__device__ __forceinline__ int fused_row(const DecodeArgs& a, int r_end, int n) {
  return (a.k_new && r_end == n) ? n - 1 : -1;
}

// ... and chunk 0 of that piece writes the new K and V rows into the cache
// (after its tile loop, so the copy does not delay the first loads). No
// piece uses the cache's copy of row n - 1 in this launch (the matrix-core
// piece never loads it; the vector piece may load it and then replaces it
// with the new row), so the write needs no ordering against the readers.
template <typename T, int D>
__device__ __forceinline__ void fused_write(const DecodeArgs& a, int b, int g, int chunk, int fresh) {
  if (fresh < 0 || chunk != 0) return;
  constexpr int kVecs = D * (int)sizeof(T) / 16;  // 16-byte vectors per row
  const size_t src = ((size_t)b * a.n_kv_heads + g) * kVecs;
  const size_t dst = (((size_t)b * a.n_kv_heads + g) * a.max_context + fresh) * kVecs;
  for (int i = threadIdx.x; i < 2 * kVecs; i += 64 * kWaves) {
    const bool kk = i < kVecs;
    const int v = kk ? i : i - kVecs;
    const uint4 x = reinterpret_cast<const uint4*>(kk ? a.k_new : a.v_new)[src + v];
    reinterpret_cast<uint4*>(const_cast<void*>(kk ? a.k : a.v))[dst + v] = x;
  }
}

// Start-up cost of a segment in rows: a workgroup that begins a segment
// pays for its q load, the first tile's latency and the epilogue whatever
// the number of rows. Each segment is given this many virtual rows in front
// of its real ones, so a workgroup whose range crosses into another segment
// is handed correspondingly fewer real rows and all workgroups finish
// together. Virtual rows map to no work. The allowance is the piece's
// (P::kSegRows), measured per piece at the Llama-3 shape.


// A piece that is part of a segment (only a workgroup's first and last
// piece can be) is recorded while the workgroup streams on; at the end the
// workgroup waits once for all of its partial stores, counts its pieces in,
// and for each segment where it arrived last merges all pieces:
//   m* = max_p m_p, l* = sum_p l_p 2^(m_p - m*), out = sum_p acc_p 2^(m_p - m*) / l*,
// writes the chunk's output rows and resets the counter.
struct SplitPiece {
  long long s;
  int n, b, h0;
  int w0, np;  // the segment's first workgroup and number of pieces
};

constexpr int kWideRound = 32;  // pieces per round of partial loads when a segment has more than 8

// Merge of a segment cut into more than 8 pieces (one long sequence over
// the grid) into its output rows o. The first kWideRound pieces' partials
// (four dims per thread, 16-byte loads) and every (m_p, l_p) are requested
// in one round of loads; meanwhile nothing waits. Then each wave works out
// the weights 2^(m_p - m*) and 1 / l* of its heads (one piece per lane,
// wave reductions) into shared memory, and every partial enters with its
// final weight (no rescaling between rounds). Long-context layer (32 pieces
// per segment): 30.4 -> 30.3 us; the merging workgroup spends ~2.7 us
// waiting for the 128 KB of partials, ~1.5 us before that on its count-in.
template <typename T, int D, int SH>
__device__ __forceinline__ void merge_wide(const DecodeArgs& a, long long s, int w0, int np, int gc, T* o) {
  static_assert(kMaxMerge <= 128 && SH <= 4 * kWaves, "two pieces per lane, four heads per wave");
  __shared__ float s_w[kMaxMerge * SH];  // weight of (piece p, head h) at p * SH + h
  __shared__ float s_inv[SH];            // 1 / l* of each head
  constexpr int DV = D / 4;              // four-dim groups per head
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // the segment's partials: pieces 0 .. np - 1, each SH heads of D floats
  const __amdgpu_buffer_rsrc_t ares =
      buffer_rsrc(a.ws_acc + ((size_t)w0 + s) * SH * D, np * SH * D * (int)sizeof(float));
  auto ml = [&](int p, int h) { return a.ws_ml + (((size_t)w0 + p + s) * SH + h) * 2; };
  for (int v0 = 0; v0 < gc * DV; v0 += kThreads) {
    const int vi = min(v0 + (int)threadIdx.x, gc * DV - 1);
    const int h = vi / DV;
    const int d = 4 * (vi - h * DV);
    float x[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int p0 = 0; p0 < np; p0 += kWideRound) {
      u32x4_t acc[kWideRound];  // pieces past np load zeros
#pragma unroll
      for (int i = 0; i < kWideRound; ++i)
        acc[i] = __builtin_amdgcn_raw_buffer_load_b128(ares, (((p0 + i) * SH + h) * D + d) * 4, 0, kCoherentLoad);
      if (v0 == 0 && p0 == 0) {
        // wave w: heads w, w + 4, ...; lane: pieces lane and lane + 64
        float mm[4][2], ll[4][2];
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int hh = wave + kWaves * k, p = lane + 64 * u;
            mm[k][u] = -INFINITY;
            ll[k][u] = 0.0f;
            if (hh < gc && p < np) get2(ml(p, hh), mm[k][u], ll[k][u]);
          }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int hh = wave + kWaves * k;
          if (hh >= gc) break;  // uniform in the wave
          float mx = fmaxf(mm[k][0], mm[k][1]);
#pragma unroll
          for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
          float ls = 0.0f;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int p = lane + 64 * u;
            const float f = (p < np) ? __builtin_amdgcn_exp2f(mm[k][u] - mx) : 0.0f;
            ls = fmaf(ll[k][u], f, ls);
            if (p < np) s_w[p * SH + hh] = f;
          }
#pragma unroll
          for (int off = 32; off >= 1; off >>= 1) ls += __shfl_xor(ls, off);
          if (lane == 0) s_inv[hh] = 1.0f / ls;
        }
        __syncthreads();
      }
#pragma unroll
      for (int i = 0; i < kWideRound; ++i) {
        const float f = (p0 + i < np) ? s_w[min(p0 + i, np - 1) * SH + h] : 0.0f;
        const f32x4_t v = __builtin_bit_cast(f32x4_t, acc[i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = fmaf(v[e], f, x[e]);
      }
    }
    if (v0 + (int)threadIdx.x < gc * DV) {
      const float inv = s_inv[h];
#pragma unroll
      for (int e = 0; e < 4; ++e) store_out(o + h * D + d + e, x[e] * inv);
    }
  }
}

template <typename T, int D, int SH>
__device__ __forceinline__ void finish_splits(const DecodeArgs& a, const SplitPiece* sp, int nsp, int* s_flag) {
  wait_stores();
  __syncthreads();
  if (threadIdx.x < nsp) {
    const SplitPiece& q = sp[threadIdx.x];
    const int old = __hip_atomic_fetch_add(a.ws_cnt + q.s, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_flag[threadIdx.x * 3 + 0] = (old == q.np - 1) ? 1 : 0;
    s_flag[threadIdx.x * 3 + 1] = q.w0;
    s_flag[threadIdx.x * 3 + 2] = q.np;
  }
  __syncthreads();
  // A segment of at most 8 pieces (a decode batch's) is merged in one round
  // of loads: each thread requests (m_p, l_p, acc_p) of its output elements
  // for all pieces at once and folds them into a running (maximum,
  // denominator, sum). A longer segment (one sequence split over the grid)
  // is merged by merge_wide.
  const int gc = a.chunk_heads;
  constexpr int E = 2;  // output elements per thread and pass
  constexpr int K = 8;  // pieces per batch of loads
  // Short segments (at most K pieces), when a chunk's outputs fit one pass
  // of two adjacent dims per thread: the pieces' (m, l) and partial pairs of
  // every segment this workgroup merges are requested in one round of 8-byte
  // loads (only the pieces there are), then folded as below.
  bool short_done = false;
  if (gc * D <= 2 * kThreads) {
    bool merge[2];
    int w0[2], np[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      merge[k] = k < nsp && s_flag[k * 3] && s_flag[k * 3 + 2] <= K;
      w0[k] = s_flag[k * 3 + 1];
      np[k] = s_flag[k * 3 + 2];
    }
    const int e2 = 2 * threadIdx.x;  // this thread's first output element of the chunk
    const bool live = e2 < gc * D;
    const int h = live ? e2 / D : 0;
    const int d = live ? e2 - h * D : 0;
    float mm[2][K], ll[2][K], a0[2][K], a1[2][K];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
#pragma unroll
      for (int i = 0; i < K; ++i) {
        if (merge[k] && i < np[k]) {
          const size_t ent = ((size_t)(w0[k] + i + sp[k].s)) * SH + h;
          get2(a.ws_ml + ent * 2, mm[k][i], ll[k][i]);
          get2(a.ws_acc + ent * D + d, a0[k][i], a1[k][i]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (!merge[k]) continue;
      float bm = -INFINITY;
#pragma unroll
      for (int i = 0; i < K; ++i) bm = (i < np[k]) ? fmaxf(bm, mm[k][i]) : bm;
      float x0 = 0.0f, x1 = 0.0f, ls = 0.0f;
#pragma unroll
      for (int i = 0; i < K; ++i) {
        if (i < np[k]) {
          const float f = __builtin_amdgcn_exp2f(mm[k][i] - bm);
          x0 = fmaf(a0[k][i], f, x0);
          x1 = fmaf(a1[k][i], f, x1);
          ls = fmaf(ll[k][i], f, ls);
        }
      }
      if (live) {
        T* o = reinterpret_cast<T*>(a.out) + ((size_t)sp[k].b * a.n_heads + sp[k].h0) * D + e2;
        store_out(o, x0 / ls);
        store_out(o + 1, x1 / ls);
      }
      if (threadIdx.x == 0) __hip_atomic_store(a.ws_cnt + sp[k].s, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    short_done = true;
  }
  for (int k = 0; k < nsp; ++k) {
    if (!s_flag[k * 3]) continue;
    const SplitPiece& q = sp[k];
    const int w0 = s_flag[k * 3 + 1];
    const int np = s_flag[k * 3 + 2];
    if (short_done && np <= K) continue;  // merged above
    T* o = reinterpret_cast<T*>(a.out) + ((size_t)q.b * a.n_heads + q.h0) * D;
    if (np > K) {
      merge_wide<T, D, SH>(a, q.s, w0, np, gc, o);
    } else {
      for (int base = 0; base < gc * D; base += E * kThreads) {
        int h[E], d[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int idx = min(base + e * kThreads + (int)threadIdx.x, gc * D - 1);
          h[e] = idx / D;
          d[e] = idx - h[e] * D;
        }
        float mm[E][K], ll[E][K], aa[E][K];
#pragma unroll
        for (int e = 0; e < E; ++e)
#pragma unroll
          for (int i = 0; i < K; ++i) {
            const size_t ent = ((size_t)(w0 + min(i, np - 1) + q.s)) * SH + h[e];
            mm[e][i] = get(a.ws_ml + ent * 2);
            ll[e][i] = get(a.ws_ml + ent * 2 + 1);
            aa[e][i] = get(a.ws_acc + ent * D + d[e]);
          }
#pragma unroll
        for (int e = 0; e < E; ++e) {
          float bm = -INFINITY;
#pragma unroll
          for (int i = 0; i < K; ++i) bm = (i < np) ? fmaxf(bm, mm[e][i]) : bm;
          float x = 0.0f, ls = 0.0f;
#pragma unroll
          for (int i = 0; i < K; ++i) {
            const float f = (i < np) ? __builtin_amdgcn_exp2f(mm[e][i] - bm) : 0.0f;
            x = fmaf(aa[e][i], f, x);
            ls = fmaf(ll[e][i], f, ls);
          }
          const int idx = base + e * kThreads + (int)threadIdx.x;
          if (idx < gc * D) store_out(o + idx, x / ls);
        }
      }
    }
    if (threadIdx.x == 0) __hip_atomic_store(a.ws_cnt + q.s, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <typename T, int D, int GC>
struct ValuPiece {
  using Elem = T;
  static constexpr int kD = D;
  static constexpr int kSlotHeads = GC;  // partial entries per workspace slot
  static constexpr int EPV = Storage<T>::kEPV;  // elements per 16-byte vector
  static constexpr int LPR = D / EPV;           // lanes per cached row
  static constexpr int RPI = 64 / LPR;          // rows per wave instruction (row slots)
  static constexpr int U = (GC >= 8) ? 2 : 4;   // row vectors per K (and V) per tile and lane
  static constexpr int TILE = RPI * U;          // rows per wave per tile
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "row must map onto a wave");

  struct Smem {
    float acc[kWaves][GC][D];
    float m[kWaves][GC];
    float l[kWaves][GC];
  };

  // Rows [r_begin, r_end) of segment (b, g, chunk). Writes the normalised
  // output when the piece is the whole segment, else the partial of `slot`.
  static constexpr int kSegRows = 192;  // start-up rows of a segment (see the row space)
  static constexpr bool kSpeculative = true;  // nothing but shared memory is touched before the gate
  static constexpr bool kPair = false;
  struct PieceRef {};
  static constexpr int kWgPerCu = 1;
  static __device__ __forceinline__ bool run(const DecodeArgs& a, Smem& sm, int b, int g, int chunk, int r_begin,
                             int r_end, int n, bool whole, long long slot, const int32_t* gate = nullptr) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rs = lane / LPR;          // row slot of this lane
    const int vec = lane - rs * LPR;    // which 16-byte vector of the row this lane owns
    const int h0 = g * (a.n_heads / a.n_kv_heads) + chunk * GC;
    const float scale_log2 = a.scale_log2;

    uint4 qv[GC];
#pragma unroll
    for (int j = 0; j < GC; ++j)
      qv[j] = reinterpret_cast<const uint4*>(reinterpret_cast<const T*>(a.q) +
                                             ((size_t)b * a.n_heads + h0 + j) * D)[vec];

    float m[GC], l[GC], acc[GC][EPV];
#pragma unroll
    for (int j = 0; j < GC; ++j) {
      m[j] = -INFINITY;
      l[j] = 0.0f;
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[j][e] = 0.0f;
    }

    const size_t row0 = ((size_t)b * a.n_kv_heads + g) * (size_t)a.max_context;
    const uint4* kp = reinterpret_cast<const uint4*>(a.k) + row0 * LPR + vec;
    const uint4* vp = reinterpret_cast<const uint4*>(a.v) + row0 * LPR + vec;
    const int fresh = fused_row(a, r_end, n);  // row taken from the new rows, or -1
    const uint4* knp = reinterpret_cast<const uint4*>(a.k_new) + ((size_t)b * a.n_kv_heads + g) * LPR + vec;
    const uint4* vnp = reinterpret_cast<const uint4*>(a.v_new) + ((size_t)b * a.n_kv_heads + g) * LPR + vec;

    // Tile loads never leave [r_begin, r_end): rows past the end are clamped
    // to the last valid row (and masked in the softmax), so the next tile can
    // be requested unconditionally while the current one is being used.
    auto load_tile = [&](int base, uint4 (&kr)[U], uint4 (&vr)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int rc = min(base + u * RPI + rs, r_end - 1);
        kr[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kp) +
                                                                     (size_t)rc * LPR));
        vr[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vp) +
                                                                     (size_t)rc * LPR));
      }
      // rows at or past `fresh` clamp to it: every such lane takes the new
      // row (the cache row is stale until this launch writes it)
      if (fresh >= 0 && base + TILE > fresh) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (min(base + u * RPI + rs, r_end - 1) == fresh) {
            kr[u] = *knp;
            vr[u] = *vnp;
          }
        }
      }
    };
    // One tile: raw scores q.k, then the online softmax in log2 units with
    // the scale folded into one FMA (scale > 0, so max commutes with it).
    // The running maximum is only moved (and acc, l rescaled) when some
    // lane's tile maximum exceeds it by more than kLazy; otherwise the stale
    // maximum is kept and p <= 2^kLazy. The final division by l makes the
    // result the same for any reference maximum.
    auto use_tile = [&](int base, const uint4 (&kr)[U], const uint4 (&vr)[U], auto full_tag) {
      constexpr bool kFull = decltype(full_tag)::value;  // every row of the tile is live
      float s[U][GC];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < GC; ++j) s[u][j] = group_sum<LPR>(vec_dot(qv[j], kr[u], T()));
      if constexpr (!kFull) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const bool live = base + u * RPI + rs < r_end;
#pragma unroll
          for (int j = 0; j < GC; ++j) s[u][j] = live ? s[u][j] : -INFINITY;
        }
      }
      float nms[GC];  // -(reference maximum), finite
#pragma unroll
      for (int j = 0; j < GC; ++j) {
        float tmax = s[0][j];
#pragma unroll
        for (int u = 1; u < U; ++u) tmax = fmaxf(tmax, s[u][j]);
        const float cand = tmax * scale_log2;
        if (__builtin_amdgcn_ballot_w64(cand > m[j] + kLazy)) {
          const float mn = fmaxf(m[j], cand);
          const float c = __builtin_amdgcn_exp2f(m[j] - ((mn == -INFINITY) ? 0.0f : mn));
          l[j] *= c;
#pragma unroll
          for (int e = 0; e < EPV; ++e) acc[j][e] *= c;
          m[j] = mn;
        }
        nms[j] = (m[j] == -INFINITY) ? 0.0f : -m[j];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float vf[EPV];
        vec_unpack(vr[u], vf, T());
#pragma unroll
        for (int j = 0; j < GC; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[u][j], scale_log2, nms[j]));
          l[j] += p;
#pragma unroll
          for (int e = 0; e < EPV; ++e) acc[j][e] = fmaf(p, vf[e], acc[j][e]);
        }
      }
    };
    using FullTile = std::integral_constant<bool, true>;
    using EdgeTile = std::integral_constant<bool, false>;
    auto use_any = [&](int base, const uint4 (&kr)[U], const uint4 (&vr)[U]) {
      if (base + TILE <= r_end) use_tile(base, kr, vr, FullTile());
      else use_tile(base, kr, vr, EdgeTile());
    };

    // Software pipeline over the wave's tiles: two register buffers, the next
    // tile always in flight while the current one is consumed. Tiles go in
    // pairs; a second tile entirely past r_end is all-masked (clamped loads
    // that contribute p = 0).
    const int stride = kWaves * TILE;
    int base = r_begin + wave * TILE;
    uint4 ka[U], va[U], kb[U], vb[U];
    load_tile(base, ka, va);
    if (gate) {  // the piece was started before its inputs were confirmed
      __syncthreads();
      if (!*gate) return false;
    }
    for (; base < r_end; base += 2 * stride) {
      load_tile(base + stride, kb, vb);
      use_any(base, ka, va);
      load_tile(base + 2 * stride, ka, va);
      use_any(base + stride, kb, vb);
    }

    fused_write<T, D>(a, b, g, chunk, fresh);
    // Combine the wave's row slots (lanes with the same vector index).
#pragma unroll
    for (int j = 0; j < GC; ++j) {
      float mw = m[j];
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) mw = fmaxf(mw, __shfl_xor(mw, off));
      const float f = __builtin_amdgcn_exp2f(m[j] - ((mw == -INFINITY) ? 0.0f : mw));
      float lw = l[j] * f;
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) lw += __shfl_xor(lw, off);
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        float x = acc[j][e] * f;
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) x += __shfl_xor(x, off);
        acc[j][e] = x;
      }
      m[j] = mw;
      l[j] = lw;
    }
    if (rs == 0) {
#pragma unroll
      for (int j = 0; j < GC; ++j)
#pragma unroll
        for (int e = 0; e < EPV; ++e) sm.acc[wave][j][vec * EPV + e] = acc[j][e];
      if (vec == 0) {
#pragma unroll
        for (int j = 0; j < GC; ++j) {
          sm.m[wave][j] = m[j];
          sm.l[wave][j] = l[j];
        }
      }
    }
    __syncthreads();

    // Combine the waves (a wave with no live row has m = -inf, weight 0).
    for (int idx = threadIdx.x; idx < GC * D; idx += kThreads) {
      const int j = idx / D;
      const int d = idx - j * D;
      float mx = sm.m[0][j];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, sm.m[w][j]);
      float x = 0.0f, lsum = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(sm.m[w][j] - mx);  // mx finite: piece non-empty
        x = fmaf(sm.acc[w][j][d], f, x);
        lsum = fmaf(sm.l[w][j], f, lsum);
      }
      if (whole) {
        store_out(reinterpret_cast<T*>(a.out) + ((size_t)b * a.n_heads + h0 + j) * D + d, x / lsum);
      } else {
        const size_t e = (size_t)slot * GC + j;
        put(a.ws_acc + e * D + d, x);
        if (d == 0) {
          put(a.ws_ml + e * 2, mx);
          put(a.ws_ml + e * 2 + 1, lsum);
        }
      }
    }
    __syncthreads();  // the shared buffers are reused by the next piece
    return true;
  }
};



// Byte offset that lies past every pool (pools are < 2^30 bytes): buffer
// loads from it and from anything up to 2^30 beyond return zeros.
constexpr int kNoRow = 1 << 30;

// bf16 piece on the matrix cores (see the file comment). Lane l of a wave is
// (g, j) = (l / 16, l % 16). MFMA 16x16x32: A lane holds A[j][8g..8g+7],
// B lane holds B[8g..8g+7][j], D lane holds D[4g..4g+3][j]; 16x16x16: the
// same with 4g..4g+3 in place of 8g..8g+7.
//
// PAGED: the same piece over a block-table cache ("10.3 - KV cache
// implementation details", section 7.2). At the start of a piece the
// workgroup copies the table entries of the piece's rows into LDS as byte
// offsets of the blocks' (kv head) row groups in the pool (kNoRow for an
// entry outside the pool, which also raises the device flag). A 16-row tile
// spans at most two blocks (block_size >= 16), so each tile reads two
// offsets and every lane forms the offsets of the rows it loads; rows past
// the piece get kNoRow, which reads as zeros as the static piece's tail does.
template <int D, bool PAGED = false>
struct MfmaPiece {
  using Elem = uint16_t;
  static constexpr int kD = D;
  static constexpr int kSlotHeads = 16;        // partial entries per workspace slot
  static constexpr int KS = D / 32;            // q.k steps of 32 dims
  static constexpr int NB = D / 16;            // p.v output column blocks
  static constexpr int TR = 16;                // rows per tile
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int VCH = TR * CPR / 64;    // V chunks per lane per tile
  static constexpr int VSTRIDE = 2 * D + 32;   // bytes per staged V row (skew spreads LDS banks)
  // K staged through LDS (static caches with rows wider than 64 bytes; see
  // stage_k), and the bytes per staged K row: the 16-byte skew puts the 16
  // rows an A-operand read touches (one 16-byte column, lanes of one g) on 16
  // different bank quads
  static constexpr bool kStageK = !PAGED && D > 32;
  static constexpr int KSTRIDE = 2 * D + 16;
  static constexpr int NBUF = D <= 64 ? 3 : 2; // register tiles in the ring (register budget)
  static_assert(D % 32 == 0 && VCH >= 1 && TR * CPR % 64 == 0, "head_dim must be 32..256");
  static constexpr int kTable = PAGED ? KVC_MAX_TABLE : 1;

  struct Smem {
    union {
      struct {
        unsigned char v[kWaves][TR * VSTRIDE];  // per-wave V staging (tile loop)
        unsigned char k[kWaves][kStageK ? TR * KSTRIDE : 16];  // per-wave K staging (tile loop)
        int32_t blk[kTable];                    // block-table caches: block offsets of the piece's rows
      } t;
      struct {
        float acc[kWaves][16][D];
        float m[kWaves][16];
        float l[kWaves][16];
      } c;                                     // per-wave results (end of piece)
    } u;
  };

  // The paged piece raises the device flag for table entries it reads
  // before its first loads, so it is never started ahead of its inputs.
  static constexpr bool kSpeculative = !PAGED;
  // Static caches stream a workgroup's first two pieces as one (run_pair).
  static constexpr bool kPair = !PAGED;
  // One workgroup per CU: measured faster than the two a CU could hold (fewer
  // pieces to merge, no second workgroup competing for issue slots and LDS).
  static constexpr int kWgPerCu = 1;
  // Start-up rows of a segment (see the row space). Llama-3 layer step at
  // 192 / 224 / 256 start-up rows: 32.17 / 31.74 / 31.95 us on one machine,
  // 224 / 256 / 288: 31.48 / 31.75 / 31.70 on a second, 192 / 256 / 320:
  // 31.65 / 31.18 / 31.44 on a third; long context 29.15 / 29.13 / 29.64
  // at 192 / 224 / 256.
  static constexpr int kSegRows = 224;

  // With kStageK, K tiles are loaded like V tiles, as contiguous 16-byte
  // chunks (chunk i of lane l is chunk f % CPR of row f / CPR, f = 64 i + l),
  // so every load instruction reads 1 KB of whole cache lines; a load in the
  // A-operand layout reads 64 bytes of each of 16 rows, which at rows wider
  // than 64 bytes sends twice the requests (Llama-3 layer 32.6 -> 31.6 us,
  // int8 23.6 -> 22.5 us). At d_h = 32 that layout is itself one contiguous
  // 1 KB block, and the staging would only add latency (a 12-layer step at
  // d_h = 32: 86 -> 91 us). The tile is staged in the wave's LDS area ...
  static __device__ __forceinline__ void stage_k(unsigned char* ks, const bf16x8_t (&kr)[KS]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const int f = i * 64 + lane;
      *reinterpret_cast<bf16x8_t*>(ks + (f / CPR) * KSTRIDE + (f % CPR) * 16) = kr[i];
    }
  }
  // ... and read back as the A operand of q.k: lane (g, j) takes row j, dims
  // [32 k + 8 g, 32 k + 8 g + 8) in step k, so s[t] = K[row 4g + t] . q[head
  // column j].
  static __device__ __forceinline__ f32x4_t scores(const unsigned char* ks, const bf16x8_t (&q)[KS]) {
    const int lane = threadIdx.x & 63;
    const unsigned char* row = ks + (lane & 15) * KSTRIDE + 16 * (lane >> 4);
    bf16x8_t av[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) av[k] = *reinterpret_cast<const bf16x8_t*>(row + 64 * k);
    f32x4_t s = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < KS; ++k) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[k], q[k], s, 0, 0, 0);
    return s;
  }
  static __device__ __forceinline__ bool run(const DecodeArgs& a, Smem& sm, int b, int kvg, int chunk,
                                             int r_begin, int r_end, int n, bool whole, long long slot,
                                             const int32_t* gate = nullptr) {
    if constexpr (!PAGED) {
      const PieceRef A{b, kvg, chunk, r_begin, r_end, n, whole, slot};
      return run_pair(a, sm, A, A, false, gate);
    }
    b = uniform(b);
    kvg = uniform(kvg);
    chunk = uniform(chunk);
    r_begin = uniform(r_begin);
    r_end = uniform(r_end);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int j = lane & 15;
    const int gc = a.chunk_heads;

    const int h0 = kvg * (a.n_heads / a.n_kv_heads) + chunk * gc;
    const float scale_log2 = a.scale_log2;

    // q as the B operand: column j is head h0 + j, zero past the chunk
    // (loaded after the first tiles are requested, so the two latencies overlap)
    bf16x8_t qb[KS];

    f32x4_t o[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY;  // reference maximum of head column j (log2 units)
    float l = 0.0f;       // this lane's share of the softmax denominator of column j

    const size_t row0 = ((size_t)b * a.n_kv_heads + kvg) * (size_t)a.max_context;
    const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k) + row0 * D;
    const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v) + row0 * D;
    unsigned char* vs = sm.u.t.v[wave];

    // Buffer resources spanning exactly the valid rows [0, r_end) of this
    // (sequence, kv head): loads of rows past the end (the tail of the last
    // tile, prefetches past the piece) return zeros without touching memory,
    // and their scores are masked below.
    // Fused append: the new row `fresh` lies outside the resources (it reads
    // as zeros) and is taken from k_new / v_new by the lanes that hold it.
    const int fresh = uniform(fused_row(a, r_end, n));
    const int r_cache = fresh >= 0 ? fresh : r_end;  // rows read from the cache
    const __amdgpu_buffer_rsrc_t kres = PAGED ? buffer_rsrc(a.k, a.pool_bytes) : buffer_rsrc(kbase, r_cache * (2 * D));
    const __amdgpu_buffer_rsrc_t vres = PAGED ? buffer_rsrc(a.v, a.pool_bytes) : buffer_rsrc(vbase, r_cache * (2 * D));
    // K in the A-operand layout (row j, dims 8g.. of each 32-dim step: one
    // table lookup per lane; contiguous chunks measured 0.2 us slower here),
    // V as contiguous 16-byte chunks
    const int koff = j * (2 * D) + 16 * g;
    const int voff = lane * 16;
    const uint16_t* knew = reinterpret_cast<const uint16_t*>(a.k_new) + ((size_t)b * a.n_kv_heads + kvg) * D;
    const uint16_t* vnew = reinterpret_cast<const uint16_t*>(a.v_new) + ((size_t)b * a.n_kv_heads + kvg) * D;

    // Block-table caches: the piece's table slice, as block offsets in LDS.
    const int shift = PAGED ? uniform(a.block_shift) : 0;
    const int blk0 = r_begin >> shift;
    const int nblk = ((r_end - 1) >> shift) - blk0 + 1;
    if constexpr (PAGED) {
      const int32_t* trow = a.table + (size_t)b * a.table_width + blk0;
      const int grp_bytes = (2 * D) << shift;  // one kv head's rows of one block
      for (int i = threadIdx.x; i < nblk; i += kThreads) {
        const int e = trow[i];
        const bool ok = e >= 0 && e < a.num_blocks;
        if (!ok) atomicOr(a.err_flag, 1);
        sm.u.t.blk[i] = ok ? (e * a.n_kv_heads + kvg) * grp_bytes : kNoRow;
      }
      __syncthreads();
    }
    // Fused append through the table: the new row is attended from k_new /
    // v_new and written after the loop, if its block's entry is valid; if
    // not, it reads as zeros (the block's other rows too), as after
    // kvc_paged_append (which skips such a sequence) and kvc_paged_decode_attn.
    const int fresh_off =
        (PAGED && fresh >= 0) ? uniform(sm.u.t.blk[(fresh >> shift) - blk0]) : kNoRow;  // pool byte offset
    const bool patch = fresh >= 0 && (!PAGED || fresh_off != kNoRow);
    // Byte offset of row r of the tile at `base` (r < base + TR), given the
    // offsets of the tile's first and second block. (The new row's stale pool
    // copy may be loaded; patch_tile replaces it before it is used.)
    auto paged_row = [&](int base, int r, int off0, int off1) {
      const int off = ((r >> shift) == (base >> shift)) ? off0 : off1;
      return r < r_end ? off + ((r & ((1 << shift) - 1)) * (2 * D)) : kNoRow;
    };
    // the lanes that hold the new row take it from k_new / v_new
    auto patch_tile = [&](int base, bf16x8_t (&kr)[KS], u32x4_t (&vr)[VCH]) {
      if (patch && fresh >= base && fresh < base + TR) {  // this tile holds the new row
        if (base + j == fresh) {
#pragma unroll
          for (int k = 0; k < KS; ++k) kr[k] = *reinterpret_cast<const bf16x8_t*>(knew + 32 * k + 8 * g);
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
          const int f = i * 64 + lane;
          if (base + f / CPR == fresh) vr[i] = *reinterpret_cast<const u32x4_t*>(vnew + 8 * (f % CPR));
        }
      }
    };

    auto load_tile = [&](int base, bf16x8_t (&kr)[KS], u32x4_t (&vr)[VCH]) {
      if constexpr (PAGED) {
        // base >= r_begin; a tile past the piece reads clamped entries and
        // all its rows get kNoRow
        const int off0 = sm.u.t.blk[min((base >> shift) - blk0, nblk - 1)];
        const int off1 = sm.u.t.blk[min(((base + TR - 1) >> shift) - blk0, nblk - 1)];
        const int kb = paged_row(base, base + j, off0, off1) + 16 * g;
#pragma unroll
        for (int k = 0; k < KS; ++k)
          kr[k] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(kres, kb + 64 * k, 0, kStreamLoad));
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
          const int f = i * 64 + lane;
          const int vb = paged_row(base, base + f / CPR, off0, off1) + (f % CPR) * 16;
          vr[i] = __builtin_amdgcn_raw_buffer_load_b128(vres, vb, 0, kStreamLoad);
        }
        patch_tile(base, kr, vr);
        return;
      }
      const int kb = base * (2 * D) + koff;
#pragma unroll
      for (int k = 0; k < KS; ++k)
        kr[k] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(kres, kb + 64 * k, 0, kStreamLoad));
      const int vb = base * (2 * D) + voff;
#pragma unroll
      for (int i = 0; i < VCH; ++i) vr[i] = __builtin_amdgcn_raw_buffer_load_b128(vres, vb + 1024 * i, 0, kStreamLoad);
      patch_tile(base, kr, vr);
    };
    auto use_tile = [&](int base, const bf16x8_t (&kr)[KS], const u32x4_t (&vr)[VCH]) {
      // stage V row-major in LDS
#pragma unroll
      for (int i = 0; i < VCH; ++i) {
        const int f = i * 64 + lane;
        *reinterpret_cast<u32x4_t*>(vs + (f / CPR) * VSTRIDE + (f % CPR) * 16) = vr[i];
      }
      // scores: s[t] = K[row base + 4g + t] . q[head column j]
      f32x4_t s = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < KS; ++k) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[k], qb[k], s, 0, 0, 0);
      if (base + TR > r_end) {
#pragma unroll
        for (int t = 0; t < 4; ++t) s[t] = (base + 4 * g + t < r_end) ? s[t] : -INFINITY;
      }
      // online softmax with a lazily moved reference maximum: p and the bf16
      // P operand keep full relative precision up to 2^kLazyMfma, so the
      // reference is only moved (and o rescaled) when a score exceeds it by
      // that much, which in practice happens only on a wave's first tile
      const float cand = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])) * scale_log2;
      if (__builtin_amdgcn_ballot_w64(cand > m + kLazyMfma)) {
        float mt = fmaxf(cand, __shfl_xor(cand, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m, mt);
        const float c = __builtin_amdgcn_exp2f(m - ((mn == -INFINITY) ? 0.0f : mn));
        l *= c;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float ct = __shfl(c, 4 * g + t);  // factor of output row (head column) 4g + t
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) o[nb][t] *= ct;
        }
        m = mn;
      }
      const float nm = (m == -INFINITY) ? 0.0f : -m;
      // P rounded to bf16 for the product; the denominator sums the same
      // rounded weights, so the output is a convex combination of V rows
      s16x4_t pa;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const __bf16 pb = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[t], scale_log2, nm));
        pa[t] = __builtin_bit_cast(short, pb);
        l += (float)pb;
      }
      // p.v: B operand = V[base + 4g + t][16 nb + j] by one transpose read
      const unsigned char* vrow = vs + (4 * g + (j >> 2)) * VSTRIDE + 8 * (j & 3);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const s16x4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(vrow + 32 * nb));
        o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, o[nb], 0, 0, 0);
      }
    };

    // Software pipeline: a ring of NBUF register tiles, NBUF - 1 of them in
    // flight while one is used. Loads are unconditional (rows past r_end read
    // as zeros), and tiles past r_end are skipped, so every wave keeps its
    // prefetch going.
    const int stride = kWaves * TR;
    int base = r_begin + wave * TR;
    bf16x8_t kbuf[NBUF][KS];
    u32x4_t vbuf[NBUF][VCH];
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) load_tile(base + i * stride, kbuf[i], vbuf[i]);
    {
      const bool real = j < gc;
      const uint16_t* qh =
          reinterpret_cast<const uint16_t*>(a.q) + ((size_t)b * a.n_heads + h0 + (real ? j : 0)) * D;
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        u32x4_t v = *reinterpret_cast<const u32x4_t*>(qh + 32 * k + 8 * g);
        v = real ? v : u32x4_t{0u, 0u, 0u, 0u};
        qb[k] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
    if (gate) {  // the piece was started before its inputs were confirmed
      __syncthreads();
      if (!*gate) return false;
    }
    for (; base < r_end; base += NBUF * stride) {
#pragma unroll
      for (int i = 0; i < NBUF; ++i) {
        load_tile(base + (i + NBUF - 1) * stride, kbuf[(i + NBUF - 1) % NBUF], vbuf[(i + NBUF - 1) % NBUF]);
        if (base + i * stride < r_end) use_tile(base + i * stride, kbuf[i], vbuf[i]);
      }
    }

    if constexpr (!PAGED) {
      fused_write<uint16_t, D>(a, b, kvg, chunk, fresh);
    } else if (patch && chunk == 0) {  // the new row into its block
      uint8_t* kdst = reinterpret_cast<uint8_t*>(const_cast<void*>(a.k)) + fresh_off +
                      (fresh & ((1 << shift) - 1)) * (2 * D);
      uint8_t* vdst = reinterpret_cast<uint8_t*>(const_cast<void*>(a.v)) + fresh_off +
                      (fresh & ((1 << shift) - 1)) * (2 * D);
      for (int i = threadIdx.x; i < 2 * CPR; i += kThreads) {
        const bool kk = i < CPR;
        const int c = kk ? i : i - CPR;
        const uint4 x = reinterpret_cast<const uint4*>(kk ? knew : vnew)[c];
        reinterpret_cast<uint4*>(kk ? kdst : vdst)[c] = x;
      }
    }
    combine(a, sm, o, m, l, b, h0, whole, slot);
    return true;
  }


  // One piece's fields.
  struct PieceRef {
    int b, kvg, chunk, r_begin, r_end, n;
    bool whole;
    long long slot;
  };

  // Static cache: a workgroup's pieces A and (hasB) B as one stream of tiles.
  // Each wave takes its tiles of A, then its tiles of B, in one loop; one
  // load sequence serves every tile (the piece's rows are chosen by uniform
  // selects), so the ring keeps B's first tiles in flight while the last
  // tiles of A are used and A is combined: the second piece starts without
  // waiting for a first load. Same arithmetic, tile for tile, as one piece at
  // a time. (The code is shaped for the compiler's wait counts: every round
  // issues the same loads, and the rare branches, A's combine and the fused
  // append's row write, only add memory operations.)
  static __device__ __forceinline__ bool run_pair(const DecodeArgs& a, Smem& sm, const PieceRef& A,
                                                  const PieceRef& Bp, bool hasB, const int32_t* gate) {
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int j = lane & 15;
    const int gc = a.chunk_heads;
    const int group = a.n_heads / a.n_kv_heads;
    const float scale_log2 = a.scale_log2;
    const int stride = kWaves * TR;

    const int a_b = uniform(A.b), a_kvg = uniform(A.kvg), a_rb = uniform(A.r_begin), a_re = uniform(A.r_end);
    const int a_fresh = uniform(fused_row(a, a_re, A.n));
    const int a_cache = a_fresh >= 0 ? a_fresh : a_re;  // rows read from the cache
    const int a_h0 = a_kvg * group + uniform(A.chunk) * gc;
    // B's fields (an empty piece when there is none: no rows, no tiles)
    const int b_b = hasB ? uniform(Bp.b) : a_b, b_kvg = hasB ? uniform(Bp.kvg) : a_kvg;
    const int b_rb = hasB ? uniform(Bp.r_begin) : 0, b_re = hasB ? uniform(Bp.r_end) : 0;
    const int b_fresh = hasB ? uniform(fused_row(a, b_re, Bp.n)) : -1;
    const int b_cache = b_fresh >= 0 ? b_fresh : b_re;
    const int b_h0 = hasB ? b_kvg * group + uniform(Bp.chunk) * gc : a_h0;

    // this wave's tiles: A's at a_rb + wave TR + t stride (t < TA), then B's
    // at b_rb + wave TR + (t - TA) stride (t < total)
    const int a_first = a_rb + wave * TR, b_first = b_rb + wave * TR;
    const int TA = a_first < a_re ? (a_re - a_first + stride - 1) / stride : 0;
    const int TB = b_first < b_re ? (b_re - b_first + stride - 1) / stride : 0;
    const int total = TA + TB;

    const int voff = lane * 16;  // V tiles as contiguous 16-byte chunks
    unsigned char* vs = sm.u.t.v[wave];
    unsigned char* ks = sm.u.t.k[wave];
    // K chunk i of this lane: contiguous as V (kStageK), else in the A-operand
    // layout (row j, dims [32 i + 8 g, 32 i + 8 g + 8)); its row in the tile,
    // its first dim, and its byte offset koff + kstep i in the tile
    auto krow = [&](int i) { return kStageK ? (i * 64 + lane) / CPR : j; };
    auto kdim = [&](int i) { return kStageK ? 8 * ((i * 64 + lane) % CPR) : 32 * i + 8 * g; };
    const int koff = kStageK ? voff : j * (2 * D) + 16 * g;
    constexpr int kstep = kStageK ? 1024 : 64;

    // Rows [base, base + TR) of tile t. Buffer resources span exactly the rows
    // [0, cache) of the piece's (sequence, kv head); loads past them (the tail
    // of the last tile, prefetches past the last tile) return zeros, and
    // their scores are masked. The new row of a fused append lies outside
    // them and is taken from k_new / v_new by the lanes that hold it.
    auto load = [&](int t, bf16x8_t (&kr)[KS], u32x4_t (&vr)[VCH]) {
      const bool inA = t < TA;
      const int sb = inA ? a_b : b_b, skvg = inA ? a_kvg : b_kvg;
      const int rows = inA ? a_cache : b_cache;
      const int base = inA ? a_first + t * stride : b_first + (t - TA) * stride;
      const int fresh = inA ? a_fresh : b_fresh;
      const size_t row0 = ((size_t)sb * a.n_kv_heads + skvg) * (size_t)a.max_context;
      const __amdgpu_buffer_rsrc_t kres =
          buffer_rsrc(reinterpret_cast<const uint16_t*>(a.k) + row0 * D, rows * (2 * D));
      const __amdgpu_buffer_rsrc_t vres =
          buffer_rsrc(reinterpret_cast<const uint16_t*>(a.v) + row0 * D, rows * (2 * D));
      const int kb = base * (2 * D) + koff;
#pragma unroll
      for (int i = 0; i < KS; ++i)
        kr[i] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(kres, kb + kstep * i, 0, kStreamLoad));
      const int vb = base * (2 * D) + voff;
#pragma unroll
      for (int i = 0; i < VCH; ++i) vr[i] = __builtin_amdgcn_raw_buffer_load_b128(vres, vb + 1024 * i, 0, kStreamLoad);
      if (fresh >= base && fresh < base + TR) {  // this tile holds the new row
        const size_t src = ((size_t)sb * a.n_kv_heads + skvg) * D;
        const uint16_t* knew = reinterpret_cast<const uint16_t*>(a.k_new) + src;
        const uint16_t* vnew = reinterpret_cast<const uint16_t*>(a.v_new) + src;
#pragma unroll
        for (int i = 0; i < KS; ++i) {
          if (base + krow(i) == fresh) kr[i] = *reinterpret_cast<const bf16x8_t*>(knew + kdim(i));
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
          const int f = i * 64 + lane;
          if (base + f / CPR == fresh) vr[i] = *reinterpret_cast<const u32x4_t*>(vnew + 8 * (f % CPR));
        }
      }
    };

    bf16x8_t qa[KS], qn[KS];  // the current piece's queries, and B's
    f32x4_t o[NB];
    float m, l;
    auto reset = [&]() {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      m = -INFINITY;  // reference maximum of head column j (log2 units)
      l = 0.0f;       // this lane's share of the softmax denominator of column j
    };
    reset();
    // q as the B operand: column j is head h0 + j, zero past the chunk (a
    // buffer resource over the chunk's gc heads returns zeros for those
    // columns, so no select waits for the data)
    auto load_q = [&](bf16x8_t (&q)[KS], int sb, int h0) {
      const __amdgpu_buffer_rsrc_t qres =
          buffer_rsrc(reinterpret_cast<const uint16_t*>(a.q) + ((size_t)sb * a.n_heads + h0) * D, gc * (2 * D));
#pragma unroll
      for (int k = 0; k < KS; ++k)
        q[k] = __builtin_bit_cast(bf16x8_t,
                                  __builtin_amdgcn_raw_buffer_load_b128(qres, j * (2 * D) + 64 * k + 16 * g, 0, 0));
    };

    // Tile t < total: raw scores q.k, the online softmax, p.v; the fused
    // append's new row is written into the cache by chunk 0 from the
    // registers that hold it (no piece reads the cache's copy of that row in
    // this launch, so the write needs no ordering).
    auto use = [&](int t, const bf16x8_t (&kr)[KS], const u32x4_t (&vr)[VCH]) {
      const bool inA = t < TA;
      const int base = inA ? a_first + t * stride : b_first + (t - TA) * stride;
      const int r_end = inA ? a_re : b_re;
      const int fresh = inA ? a_fresh : b_fresh;
      // stage V and K row-major in LDS
#pragma unroll
      for (int i = 0; i < VCH; ++i) {
        const int f = i * 64 + lane;
        *reinterpret_cast<u32x4_t*>(vs + (f / CPR) * VSTRIDE + (f % CPR) * 16) = vr[i];
      }
      if constexpr (kStageK) stage_k(ks, kr);
      if (fresh >= base && fresh < base + TR && (inA ? A.chunk : Bp.chunk) == 0) {
        const int sb = inA ? a_b : b_b, skvg = inA ? a_kvg : b_kvg;
        const size_t row = ((size_t)sb * a.n_kv_heads + skvg) * (size_t)a.max_context + fresh;
        uint16_t* kd = reinterpret_cast<uint16_t*>(const_cast<void*>(a.k)) + row * D;
        uint16_t* vd = reinterpret_cast<uint16_t*>(const_cast<void*>(a.v)) + row * D;
#pragma unroll
        for (int i = 0; i < KS; ++i) {
          if (base + krow(i) == fresh) *reinterpret_cast<bf16x8_t*>(kd + kdim(i)) = kr[i];
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
          const int f = i * 64 + lane;
          if (base + f / CPR == fresh) *reinterpret_cast<u32x4_t*>(vd + 8 * (f % CPR)) = vr[i];
        }
      }
      // scores: s[u] = K[row base + 4g + u] . q[head column j]
      f32x4_t s = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (kStageK) {
        s = scores(ks, qa);
      } else {
#pragma unroll
        for (int k = 0; k < KS; ++k) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[k], qa[k], s, 0, 0, 0);
      }
      if (base + TR > r_end) {
#pragma unroll
        for (int u = 0; u < 4; ++u) s[u] = (base + 4 * g + u < r_end) ? s[u] : -INFINITY;
      }
      // online softmax with a lazily moved reference maximum: p and the bf16
      // P operand keep full relative precision up to 2^kLazyMfma, so the
      // reference is only moved (and o rescaled) when a score exceeds it by
      // that much, which in practice happens only on a wave's first tile
      const float cand = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])) * scale_log2;
      if (__builtin_amdgcn_ballot_w64(cand > m + kLazyMfma)) {
        float mt = fmaxf(cand, __shfl_xor(cand, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m, mt);
        const float c = __builtin_amdgcn_exp2f(m - ((mn == -INFINITY) ? 0.0f : mn));
        l *= c;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float ct = __shfl(c, 4 * g + u);  // factor of output row (head column) 4g + u
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) o[nb][u] *= ct;
        }
        m = mn;
      }
      const float nm = (m == -INFINITY) ? 0.0f : -m;
      // P rounded to bf16 for the product; the denominator sums the same
      // rounded weights, so the output is a convex combination of V rows
      s16x4_t pa;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const __bf16 pb = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[u], scale_log2, nm));
        pa[u] = __builtin_bit_cast(short, pb);
        l += (float)pb;
      }
      // p.v: B operand = V[base + 4g + u][16 nb + j] by one transpose read
      const unsigned char* vrow = vs + (4 * g + (j >> 2)) * VSTRIDE + 8 * (j & 3);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const s16x4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(vrow + 32 * nb));
        o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, o[nb], 0, 0, 0);
      }
    };
    // A's end: combine it, then start B with its queries (every wave does
    // this once, in order, before its first tile of B or after its last tile)
    bool switched = false;
    auto finish_a = [&]() {
      combine(a, sm, o, m, l, a_b, a_h0, A.whole, A.slot);
      reset();
#pragma unroll
      for (int k = 0; k < KS; ++k) qa[k] = qn[k];
      switched = true;
    };

    // Software pipeline: a ring of NBUF register tiles, NBUF - 1 of them in
    // flight while one is used. The first tile, then the queries of B and A
    // (their latencies overlap), then the rest of the ring; the first use is
    // taken out of the loop, so both queries are known to have arrived after
    // it (loads complete in issue order; the loop then never waits for them).
    bf16x8_t kbuf[NBUF][KS];
    u32x4_t vbuf[NBUF][VCH];
    load(0, kbuf[0], vbuf[0]);
    load_q(qn, b_b, b_h0);
    load_q(qa, a_b, a_h0);
#pragma unroll
    for (int i = 1; i < NBUF; ++i) load(i, kbuf[i], vbuf[i]);
    if (gate) {  // the pieces were started before their inputs were confirmed
      __syncthreads();
      if (!*gate) return false;
    }
    if (total > 0) {
      if (TA == 0) finish_a();
      use(0, kbuf[0], vbuf[0]);
    }
    // tile t in buffer t mod NBUF; round t0 (= 1 mod NBUF) uses tiles t0 ..
    // t0 + NBUF - 1 and loads tiles t0 + NBUF - 1 .. t0 + 2 NBUF - 2
    for (int t0 = 1; t0 < total; t0 += NBUF) {
#pragma unroll
      for (int i = 0; i < NBUF; ++i) {
        const int t = t0 + i;
        load(t + NBUF - 1, kbuf[(1 + i + NBUF - 1) % NBUF], vbuf[(1 + i + NBUF - 1) % NBUF]);
        if (t < total) {
          if (t == TA) finish_a();
          use(t, kbuf[(1 + i) % NBUF], vbuf[(1 + i) % NBUF]);
        }
      }
    }
    if (!switched) finish_a();
    if (hasB) combine(a, sm, o, m, l, b_b, b_h0, Bp.whole, Bp.slot);
    return true;
  }

  // End of a piece: combine the waves' (o, m, l) and write the output (whole
  // segment) or the partial of `slot`. Every thread of the workgroup calls it.
  static __device__ __forceinline__ void combine(const DecodeArgs& a, Smem& sm, const f32x4_t (&o)[NB], float m,
                                                 float l, int b, int h0, bool whole, long long slot) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int j = lane & 15;
    const int gc = a.chunk_heads;
    // denominators: sum the lane shares of each head column
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    __syncthreads();  // every wave is done with its V staging area
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = 4 * g + t;
      if (i < gc) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sm.u.c.acc[wave][i][16 * nb + j] = o[nb][t];
      }
    }
    if (g == 0 && j < gc) {
      sm.u.c.m[wave][j] = m;
      sm.u.c.l[wave][j] = l;
    }
    __syncthreads();

    // Combine the waves (a wave with no live row has m = -inf, weight 0).
    for (int idx = threadIdx.x; idx < gc * D; idx += kThreads) {
      const int h = idx / D;
      const int d = idx - h * D;
      float mx = sm.u.c.m[0][h];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) mx = fmaxf(mx, sm.u.c.m[w][h]);
      float x = 0.0f, lsum = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(sm.u.c.m[w][h] - mx);
        x = fmaf(sm.u.c.acc[w][h][d], f, x);
        lsum = fmaf(sm.u.c.l[w][h], f, lsum);
      }
      if (whole) {
        store_out(reinterpret_cast<uint16_t*>(a.out) + ((size_t)b * a.n_heads + h0 + h) * D + d, x / lsum);
      } else {
        const size_t e = (size_t)slot * kSlotHeads + h;
        put(a.ws_acc + e * D + d, x);
        if (d == 0) {
          put(a.ws_ml + e * 2, mx);
          put(a.ws_ml + e * 2 + 1, lsum);
        }
      }
    }
    __syncthreads();  // shared memory is reused by the next piece
  }
};

// 16 int8 codes (one 16-byte vector) -> 16 bf16 values, as two 8-element
// vectors. Exact: |code| <= 127 needs 7 significant bits; the bf16 is the
// upper half of the code's binary32 value.
__device__ __forceinline__ void codes_to_bf16(const u32x4_t& w, u32x4_t& lo, u32x4_t& hi) {
  uint32_t r[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t x = w[q];
    const float f0 = (float)(int)(int8_t)(x & 0xFFu);
    const float f1 = (float)(int)(int8_t)((x >> 8) & 0xFFu);
    const float f2 = (float)(int)(int8_t)((x >> 16) & 0xFFu);
    const float f3 = (float)(int)(int8_t)(x >> 24);
    r[2 * q] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
    r[2 * q + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
  }
  lo = u32x4_t{r[0], r[1], r[2], r[3]};
  hi = u32x4_t{r[4], r[5], r[6], r[7]};
}

// int8 pieces ("10.3 - KV cache implementation details", section 4.4): the
// matrix-core piece over int8 codes with a float32 scale per row. K row r
// stands for code * sk[r] and V row r for code * sv[r], so
//   score_r = sk[r] * (codes_r . q)   and   o = sum_r (p_r sv[r]) codes_r,
// with l = sum_r p_r. Lane (g, j) takes the A operand of q.k from row j's
// codes [g D/4, (g+1) D/4) (16-byte vectors), converted to bf16 in registers
// (exact), and the query's B operand uses the same assignment of dims to
// (lane, step); a dot product does not depend on the order of its dims. The
// score tile is scaled by the rows' K scales. V codes are converted the same
// way and staged in LDS as bf16 for the transpose read, and each row's V
// scale is folded into the bf16 P operand. Rows past the piece read as zero
// codes with zero scales and are masked. Half the bytes of the bf16 piece
// per row, plus 8 bytes of scales.
template <int D>
struct I8Piece {
  using Base = MfmaPiece<D>;
  using Elem = uint16_t;                      // q, out and partials as for bf16
  static constexpr int kD = D;
  static constexpr int kSlotHeads = Base::kSlotHeads;
  static constexpr int KS = D / 32;           // q.k steps of 32 dims
  static constexpr int NB = D / 16;           // p.v output column blocks
  static constexpr int TR = 16;               // rows per tile
  static constexpr int CPR = D / 16;          // 16-byte code vectors per row
  static constexpr int KL = D / 64;           // K code vectors per lane per tile (D / 4 codes)
  static constexpr int VL = TR * CPR / 64;    // V code vectors per lane per tile
  static constexpr int VSTRIDE = Base::VSTRIDE;
  // K code tiles staged through LDS where a row is wider than 64 bytes (see
  // MfmaPiece::stage_k), and the bytes per staged K code row (in the bf16
  // piece's K area, which is larger); the skew spreads the 16 rows of an
  // A-operand read over the banks
  static constexpr bool kStageK = D > 64;
  static constexpr int KSTRIDE = D + 16;
  static_assert(!kStageK || (Base::kStageK && KSTRIDE <= Base::KSTRIDE), "K codes fit the K staging area");
  static constexpr int NBUF = Base::NBUF;  // (three tiles measured the same, four slower)
  // Two workgroups per CU where the registers allow (d_h <= 128): the int8
  // tile's conversions make each wave's chain long enough that a second
  // wave per SIMD pays, above all in the fused launch, whose piece with the
  // new row quantises it behind a barrier (layer step 26.2 -> 24.4 us; the
  // decode alone 25.0 -> 24.9 us).
  static constexpr int kWgPerCu = D <= 128 ? 2 : 1;
  static_assert(D >= 64 && D % 64 == 0 && VL >= 1, "int8 head_dim must be 64, 128 or 256");
  struct Smem : Base::Smem {
    __attribute__((aligned(16))) int8_t nq[2][D];  // fused append: the new K and V rows' codes
    float ns[2];                                   // and their scales
  };

  struct Tile {
    u32x4_t k[KL];
    u32x4_t v[VL];
    f32x4_t sk, sv;  // scales of rows 4g .. 4g + 3 of the tile
  };

  static constexpr bool kSpeculative = true;  // nothing but shared memory is touched before the gate
  static constexpr bool kPair = false;
  // Start-up rows of a segment. Decode alone, 192 / 224 / 256 / 384 / 448 /
  // 512: 22.52 / 22.42 / 21.74 / 21.80 / 21.79 / 22.06 us; the fused layer
  // step (its piece holding the new row quantises it behind a barrier
  // before its tiles), 256 / 384 / 448 / 512: 23.43 / 22.49 / 22.07 / 21.94.
  // One value serves both modes, so that a fused launch and append + decode
  // split the rows alike and give the same bits.
  static constexpr int kSegRows = 448;
  struct PieceRef {};
  static __device__ __forceinline__ bool run(const DecodeArgs& a, Smem& sm, int b, int kvg, int chunk,
                                             int r_begin, int r_end, int n, bool whole, long long slot,
                                             const int32_t* gate = nullptr) {
    b = uniform(b);
    kvg = uniform(kvg);
    chunk = uniform(chunk);
    r_begin = uniform(r_begin);
    r_end = uniform(r_end);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int j = lane & 15;
    const int gc = a.chunk_heads;
    const int h0 = kvg * (a.n_heads / a.n_kv_heads) + chunk * gc;
    const float scale_log2 = a.scale_log2;

    bf16x8_t qb[KS];
    f32x4_t o[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m = -INFINITY;
    float l = 0.0f;

    // resources spanning exactly rows [0, r_end) of the (sequence, kv head)
    // Fused append: the new row `fresh` lies outside the resources (its cache
    // row is stale until this launch writes it) and is quantised here, with
    // the append kernel's arithmetic, into shared memory; the lanes that hold
    // it take it from there when the tile is used.
    const int fresh = uniform(fused_row(a, r_end, n));
    const int r_cache = fresh >= 0 ? fresh : r_end;
    const size_t row0 = ((size_t)b * a.n_kv_heads + kvg) * (size_t)a.max_context;
    const __amdgpu_buffer_rsrc_t kres = buffer_rsrc(reinterpret_cast<const int8_t*>(a.k) + row0 * D, r_cache * D);
    const __amdgpu_buffer_rsrc_t vres = buffer_rsrc(reinterpret_cast<const int8_t*>(a.v) + row0 * D, r_cache * D);
    const __amdgpu_buffer_rsrc_t ksres = buffer_rsrc(a.k_scale + row0, r_cache * 4);
    const __amdgpu_buffer_rsrc_t vsres = buffer_rsrc(a.v_scale + row0, r_cache * 4);
    if (fresh >= 0) {
      if (wave < 2) quantize_new_row(a, sm, b, kvg, wave);
      __syncthreads();
    }
    // V code tiles as contiguous 16-byte vectors; K code vector i of this
    // lane: contiguous too with kStageK (staged in LDS and read back in the
    // A-operand layout, as in the bf16 piece), else row j's codes
    // [g D/4 + 16 i, g D/4 + 16 i + 16). krow: its row in the tile; kcol: its
    // first code.
    const int voff = lane * 16;
    unsigned char* vs = sm.u.t.v[wave];
    unsigned char* ks = sm.u.t.k[wave];
    auto krow = [&](int i) { return kStageK ? (i * 64 + lane) / CPR : j; };
    auto kcol = [&](int i) { return kStageK ? 16 * ((i * 64 + lane) % CPR) : g * (D / 4) + 16 * i; };

    auto load_tile = [&](int base, Tile& tl) {
#pragma unroll
      for (int i = 0; i < KL; ++i)
        tl.k[i] = __builtin_amdgcn_raw_buffer_load_b128(kres, (base + krow(i)) * D + kcol(i), 0, kStreamLoad);
      const int vb = base * D + voff;
#pragma unroll
      for (int i = 0; i < VL; ++i) tl.v[i] = __builtin_amdgcn_raw_buffer_load_b128(vres, vb + 1024 * i, 0, kStreamLoad);
      tl.sk = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ksres, (base + 4 * g) * 4, 0, kStreamLoad));
      tl.sv = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vsres, (base + 4 * g) * 4, 0, kStreamLoad));
    };
    auto use_tile = [&](int base, const Tile& tile, auto patch_tag) {
      constexpr bool kPatch = decltype(patch_tag)::value;  // the piece holds the new row
      Tile tl = tile;
      if (kPatch && fresh >= base && fresh < base + TR) {  // this tile holds the new row
#pragma unroll
        for (int i = 0; i < KL; ++i) {
          if (base + krow(i) == fresh) tl.k[i] = *reinterpret_cast<const u32x4_t*>(sm.nq[0] + kcol(i));
        }
#pragma unroll
        for (int i = 0; i < VL; ++i) {
          const int f = i * 64 + lane;
          if (base + f / CPR == fresh) tl.v[i] = *reinterpret_cast<const u32x4_t*>(sm.nq[1] + (f % CPR) * 16);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (base + 4 * g + t == fresh) {
            tl.sk[t] = sm.ns[0];
            tl.sv[t] = sm.ns[1];
          }
        }
      }
      // V codes -> bf16, staged row-major in LDS
#pragma unroll
      for (int i = 0; i < VL; ++i) {
        const int f = i * 64 + lane;
        u32x4_t lo, hi;
        codes_to_bf16(tl.v[i], lo, hi);
        unsigned char* dst = vs + (f / CPR) * VSTRIDE + (f % CPR) * 32;
        *reinterpret_cast<u32x4_t*>(dst) = lo;
        *reinterpret_cast<u32x4_t*>(dst + 16) = hi;
      }
      // K codes in the A-operand layout (row j's codes [g D/4, (g + 1) D/4)):
      // with kStageK, staged row-major and read back
      u32x4_t kc[KL];
      if constexpr (kStageK) {
#pragma unroll
        for (int i = 0; i < KL; ++i)
          *reinterpret_cast<u32x4_t*>(ks + krow(i) * KSTRIDE + kcol(i)) = tl.k[i];
#pragma unroll
        for (int i = 0; i < KL; ++i)
          kc[i] = *reinterpret_cast<const u32x4_t*>(ks + j * KSTRIDE + g * (D / 4) + 16 * i);
      } else {
#pragma unroll
        for (int i = 0; i < KL; ++i) kc[i] = tl.k[i];
      }
      // scores: codes . q on the matrix cores, then the rows' K scales
      f32x4_t sc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < KL; ++i) {
        u32x4_t lo, hi;
        codes_to_bf16(kc[i], lo, hi);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, lo), qb[2 * i], sc, 0, 0, 0);
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, hi), qb[2 * i + 1], sc, 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) sc[t] *= tl.sk[t];
      if (base + TR > r_end) {
#pragma unroll
        for (int t = 0; t < 4; ++t) sc[t] = (base + 4 * g + t < r_end) ? sc[t] : -INFINITY;
      }
      // online softmax with a lazily moved reference maximum (as the bf16 piece)
      const float cand = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])) * scale_log2;
      if (__builtin_amdgcn_ballot_w64(cand > m + kLazyMfma)) {
        float mt = fmaxf(cand, __shfl_xor(cand, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m, mt);
        const float c = __builtin_amdgcn_exp2f(m - ((mn == -INFINITY) ? 0.0f : mn));
        l *= c;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float ct = __shfl(c, 4 * g + t);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) o[nb][t] *= ct;
        }
        m = mn;
      }
      const float nm = (m == -INFINITY) ? 0.0f : -m;
      s16x4_t pa;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sc[t], scale_log2, nm));
        l += p;
        pa[t] = __builtin_bit_cast(short, (__bf16)(p * tl.sv[t]));
      }
      // p.v: B operand = V[base + 4g + t][16 nb + j] by one transpose read
      const unsigned char* vrow = vs + (4 * g + (j >> 2)) * VSTRIDE + 8 * (j & 3);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const s16x4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(vrow + 32 * nb));
        o[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, o[nb], 0, 0, 0);
      }
    };

    // Ring of NBUF register tiles as in the bf16 piece: loads past r_end are
    // unconditional (zeros), tiles past r_end are skipped.
    const int stride = kWaves * TR;
    int base = r_begin + wave * TR;
    Tile buf[NBUF];
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) load_tile(base + i * stride, buf[i]);
    {
      const bool real = j < gc;
      const uint16_t* qh =
          reinterpret_cast<const uint16_t*>(a.q) + ((size_t)b * a.n_heads + h0 + (real ? j : 0)) * D + g * (D / 4);
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        u32x4_t v = *reinterpret_cast<const u32x4_t*>(qh + 8 * k);
        v = real ? v : u32x4_t{0u, 0u, 0u, 0u};
        qb[k] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
    if (gate) {  // the piece was started before its inputs were confirmed
      __syncthreads();
      if (!*gate) return false;
    }
    // the loop is instantiated twice so that only the piece holding the new
    // row pays for the check
    auto stream = [&](auto patch_tag) {
      for (; base < r_end; base += NBUF * stride) {
#pragma unroll
        for (int i = 0; i < NBUF; ++i) {
          load_tile(base + (i + NBUF - 1) * stride, buf[(i + NBUF - 1) % NBUF]);
          if (base + i * stride < r_end) use_tile(base + i * stride, buf[i], patch_tag);
        }
      }
    };
    if (fresh >= 0) stream(std::integral_constant<bool, true>());
    else stream(std::integral_constant<bool, false>());
    if (fresh >= 0 && chunk == 0) write_new_row(a, sm, b, kvg, fresh);
    Base::combine(a, sm, o, m, l, b, h0, whole, slot);
    return true;
  }

  // One wave quantises the new row of (b, g) from k_new (kv = 0) or v_new
  // (kv = 1) exactly as the append kernel does: row maximum (exact in any
  // order), 127 / amax and amax / 127 correctly rounded, codes
  // rint(x * (127 / amax)) clamped to [-127, 127]; a zero row gives zeros.
  static __device__ __forceinline__ void quantize_new_row(const DecodeArgs& a, Smem& sm, int b, int g, int kv) {
    constexpr int EPL = D / 64;  // elements per lane
    const int lane = threadIdx.x & 63;
    const uint16_t* src = reinterpret_cast<const uint16_t*>(kv == 0 ? a.k_new : a.v_new) +
                          ((size_t)b * a.n_kv_heads + g) * D + lane * EPL;
    float x[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] = __uint_as_float((uint32_t)src[e] << 16);
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const bool zero = amax == 0.0f;
    const float inv = zero ? 0.0f : __fdiv_rn(127.0f, amax);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float c = rintf(__fmul_rn(x[e], inv));
      c = fminf(fmaxf(c, -127.0f), 127.0f);
      sm.nq[kv][lane * EPL + e] = (int8_t)(int)c;
    }
    if (lane == 0) sm.ns[kv] = zero ? 0.0f : __fdiv_rn(amax, 127.0f);
  }

  // ... and writes it into the cache (codes and scales), after the tile loop.
  static __device__ __forceinline__ void write_new_row(const DecodeArgs& a, Smem& sm, int b, int g, int fresh) {
    const size_t row = ((size_t)b * a.n_kv_heads + g) * (size_t)a.max_context + fresh;
    const int t = threadIdx.x;
    if (t < 2 * (D / 16)) {
      const int kv = t / (D / 16);
      const int v = t - kv * (D / 16);
      int8_t* dst = reinterpret_cast<int8_t*>(const_cast<void*>(kv == 0 ? a.k : a.v)) + row * D + 16 * v;
      *reinterpret_cast<u32x4_t*>(dst) = *reinterpret_cast<const u32x4_t*>(sm.nq[kv] + 16 * v);
    } else if (t < 2 * (D / 16) + 2) {
      const int kv = t - 2 * (D / 16);
      const_cast<float*>(kv == 0 ? a.k_scale : a.v_scale)[row] = sm.ns[kv];
    }
  }
};

// Persistent decode kernel: grid = W workgroups of 256 threads.
template <class P>
__global__ __launch_bounds__(kThreads) void gqa_decode_kernel(DecodeArgs a) {
  static_assert(P::kSegRows >= 0 && P::kSegRows <= kMaxSegRows, "row space must stay below 2^31");
  __shared__ typename P::Smem sm;
  __shared__ int32_t s_prefix[KVC_MAX_BATCH + 1];
  __shared__ int32_t s_umax;  // longest segment in virtual rows
  __shared__ PlanState st;    // the cached split of the work (kvc_device.h)
  __shared__ int s_flag[6];
  __shared__ SplitPiece split[2];  // a workgroup's first and last piece may be parts of segments

  const int B = a.batch;
  const int t = threadIdx.x;
  const int w = blockIdx.x;
  const int min_rows = a.k_new ? 1 : 0;
  const int HC = a.n_kv_heads * a.head_chunks;  // segments per sequence
  const int32_t* entry = plan_entry(a.plan);
  // the plan's mode: append or not, and the segments per sequence (a cache's
  // workspace serves one shape, a shared one may serve several)
  const int plan_mode = min_rows + 2 * HC;
  const bool key = plan_key(a.plan, a.n_wg, plan_mode, B);
  const int entry_count = entry[0];  // requested with the header, whatever the key
  const int count = uniform(key ? entry_count : -1);  // pieces in this workgroup's cached entry
  // The first two cached pieces' fields, requested now so that their
  // latency overlaps the length scan below (read before it, the first loads
  // of wave 0, and with them every wave's gate, waited for both in turn).
  int first[kPieceInts], second[kPieceInts];
#pragma unroll
  for (int i = 0; i < kPieceInts; ++i) {
    first[i] = entry[1 + i];
    second[i] = entry[1 + kPieceInts + i];
  }
  if (t < 64) {
    scan_lengths(a.valid_lens, a.cache_index, B, a.max_context, P::kSegRows, s_prefix, &s_umax, a.err_flag,
                 blockIdx.x == 0, min_rows, a.plan + KVC_PLAN_LENS, &st.gate);
    if (t == 0) st.gate = st.gate && key;
  }
  // With a cached entry the first piece starts at once, before the lengths
  // are confirmed: its loads stay inside the cache whatever they are, and it
  // touches nothing but shared memory before its gate (a barrier after its
  // first loads) confirms them. Otherwise the barrier comes first.
  const bool speculate = P::kSpeculative && count >= 1;
  if (!speculate) __syncthreads();  // publishes the prefix sums and the gate
  int nsplit = 0;
  if (speculate || (st.gate && count >= 1)) {
    bool planned = true;
    int k0 = 0;
    if constexpr (P::kPair) {
      // the first two pieces as one stream (the second's first tiles are
      // loaded while the first ends)
      if (count >= 2) {
        typename P::PieceRef pr[2];
        int fs[2][kPieceInts];
#pragma unroll
        for (int i = 0; i < kPieceInts; ++i) {
          fs[0][i] = uniform(first[i]);
          fs[1][i] = uniform(second[i]);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int hc = fs[q][1];
          const long long s = (long long)fs[q][0] * HC + hc;
          pr[q] = typename P::PieceRef{fs[q][0], hc / a.head_chunks, hc % a.head_chunks, fs[q][2], fs[q][3], fs[q][4],
                                       fs[q][2] == 0 && fs[q][3] == fs[q][4], (long long)w + s};
        }
        if (!P::run_pair(a, sm, pr[0], pr[1], true, speculate ? &st.gate : nullptr)) {
          planned = false;  // not this launch's plan: the gate's barrier published the prefix sums
        } else {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            if (!pr[q].whole && nsplit < 2) {
              if (threadIdx.x == 0) {  // read after the barriers in finish_splits
                split[nsplit].s = pr[q].slot - w;
                split[nsplit].n = fs[q][4];
                split[nsplit].b = fs[q][0];
                split[nsplit].h0 = pr[q].kvg * (a.n_heads / a.n_kv_heads) + pr[q].chunk * a.chunk_heads;
                split[nsplit].w0 = fs[q][5];
                split[nsplit].np = fs[q][6];
              }
              ++nsplit;
            }
          }
          k0 = 2;
        }
      }
    }
    for (int k = k0; planned && k < count; ++k) {
      const int32_t* pc = entry + 1 + k * kPieceInts;
      int f[kPieceInts];
#pragma unroll
      for (int i = 0; i < kPieceInts; ++i) f[i] = k == 0 ? first[i] : pc[i];
      const int b = uniform(f[0]), hc = uniform(f[1]), r_begin = uniform(f[2]), r_end = uniform(f[3]);
      const int n = uniform(f[4]);
      const long long s = (long long)b * HC + hc;
      const bool whole = r_begin == 0 && r_end == n;
      const int kvg = hc / a.head_chunks;
      const int chunk = hc % a.head_chunks;
      if (!P::run(a, sm, b, kvg, chunk, r_begin, r_end, n, whole, (long long)w + s,
                  (k == 0 && speculate) ? &st.gate : nullptr)) {
        planned = false;  // not this launch's plan: the gate's barrier published the prefix sums
        break;
      }
      if (!whole && nsplit < 2) {
        if (threadIdx.x == 0) {  // read after the barriers in finish_splits
          split[nsplit].s = s;
          split[nsplit].n = n;
          split[nsplit].b = b;
          split[nsplit].h0 = kvg * (a.n_heads / a.n_kv_heads) + chunk * a.chunk_heads;
          split[nsplit].w0 = f[5];
          split[nsplit].np = f[6];
        }
        ++nsplit;
      }
    }
    if (planned) {
      if (nsplit > 0) finish_splits<typename P::Elem, P::kD, P::kSlotHeads>(a, split, nsplit, s_flag);
      return;
    }
  }
  const bool fresh = !st.gate;  // no plan for these lengths: work it out and record it
  if (!fresh && count == 0) return;  // the plan gives this workgroup nothing

  const long long R = (long long)s_prefix[B] * HC;
  // Empty (or out-of-range) sequences get zero outputs, spread over the grid.
  for (int bz = w; bz < B; bz += a.n_wg) {
    if (s_prefix[bz + 1] == s_prefix[bz]) {
      using T = typename P::Elem;
      T* o = reinterpret_cast<T*>(a.out) + (size_t)bz * a.n_heads * P::kD;
      for (int i = t; i < a.n_heads * P::kD; i += kThreads) store_out(o + i, 0.0f);
    }
  }

  const Partition part(R, a.n_wg, s_umax);
  // Short segments are not split: when every segment has at most
  // a.whole_rows rows and the grid has a workgroup for each, workgroup w
  // takes segment w whole (sequence w / HC, chunk w % HC) and nothing is
  // merged. A split then costs more (partial stores, count-in, merge) than
  // it saves on so few rows.
  const int nseg = B * HC;
  const bool whole_mode = nseg <= a.n_wg && s_umax - P::kSegRows <= a.whole_rows;
  int recorded = 0;  // pieces in this workgroup's new entry (thread 0)
  if (w < (whole_mode ? nseg : part.W)) {
    long long x, hi;
    if (whole_mode) {
      const int sb = w / HC;
      const long long u = s_prefix[sb + 1] - s_prefix[sb];
      x = (long long)s_prefix[sb] * HC + (long long)(w - sb * HC) * u;
      hi = x + u;  // x = hi for an empty sequence
    } else {
      x = part.lo(w);
      hi = part.lo(w + 1);
    }
    if (x < hi) for_each_piece(s_prefix, B, HC, P::kSegRows, x, hi,
                   [&](int b, int hc, int r_begin, int r_end, int n, long long real0) {
      const long long s = (long long)b * HC + hc;
      const bool whole = r_begin == 0 && r_end == n;
      const int kvg = hc / a.head_chunks;
      const int chunk = hc % a.head_chunks;
      P::run(a, sm, b, kvg, chunk, r_begin, r_end, n, whole, (long long)w + s);
      const int w0 = whole ? w : part.of(real0);
      const int np = whole ? 1 : part.of(real0 + n - 1) - w0 + 1;
      if (!whole && nsplit < 2) {
        if (threadIdx.x == 0) {  // read after the barriers in finish_splits
          split[nsplit].s = s;
          split[nsplit].n = n;
          split[nsplit].b = b;
          split[nsplit].h0 = kvg * (a.n_heads / a.n_kv_heads) + chunk * a.chunk_heads;
          split[nsplit].w0 = w0;
          split[nsplit].np = np;
        }
        ++nsplit;
      }
      if (fresh) plan_record(a.plan, recorded, b, hc, r_begin, r_end, n, w0, np);
    });
    if (nsplit > 0) finish_splits<typename P::Elem, P::kD, P::kSlotHeads>(a, split, nsplit, s_flag);
  }
  if (fresh) plan_publish(a.plan, st, recorded, s_prefix, B, P::kSegRows, a.n_wg, plan_mode);
}

template <class P, typename T, int D>
hipError_t launch_piece(const kvc_cache* c, DecodeArgs a, int chunk_heads, hipStream_t stream) {
  const int group = c->d.n_heads / c->d.n_kv_heads;
  a.chunk_heads = chunk_heads;
  a.head_chunks = group / chunk_heads;
  // P::kWgPerCu workgroups per CU by default (one for the bf16 and fp32
  // pieces, two for the int8 piece where its registers allow; see there).
  a.n_wg = c->workgroups_forced > 0 ? c->workgroups_forced : c->num_cus * P::kWgPerCu;
  if (a.n_wg > c->max_workgroups) a.n_wg = c->max_workgroups;
  // Default grid: a segment of at most 512 rows and 128 KB of cache rows
  // (K, V and any scales) is streamed whole by one workgroup; measured per
  // layer at 512 rows, d_h = 32, B = 8, H_kv = 8: 7.3 us whole against 8.7
  // split over 256 workgroups, and whole stops paying at 256 KB per segment
  // (d_h = 128: 11.5 against 9.5). A forced grid always splits.
  const int row_bytes = 2 * D * c->elem + (c->d.dtype == KVC_I8 ? 2 * (int)sizeof(float) : 0);
  const int whole_rows = (128 << 10) / row_bytes;
  a.whole_rows = c->workgroups_forced > 0 ? 0 : (whole_rows < 512 ? whole_rows : 512);
  gqa_decode_kernel<P><<<dim3(a.n_wg), dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

// bf16: matrix-core piece; the group is cut into chunks of at most 16 heads.
template <int D>
hipError_t launch_bf16(const kvc_cache* c, const DecodeArgs& a, hipStream_t st) {
  const int group = c->d.n_heads / c->d.n_kv_heads;
  int gc = group <= 16 ? group : 16;
  while (group % gc != 0) --gc;
  return launch_piece<MfmaPiece<D>, uint16_t, D>(c, a, gc, st);
}

// bf16 block-table cache: the paged matrix-core piece, chunks as for bf16.
template <int D>
hipError_t launch_paged(const kvc_cache* c, const DecodeArgs& a, hipStream_t st) {
  const int group = c->d.n_heads / c->d.n_kv_heads;
  int gc = group <= 16 ? group : 16;
  while (group % gc != 0) --gc;
  return launch_piece<MfmaPiece<D, true>, uint16_t, D>(c, a, gc, st);
}

// int8: matrix-core piece over codes; chunks of at most 16 heads as bf16.
template <int D>
hipError_t launch_i8(const kvc_cache* c, const DecodeArgs& a, hipStream_t st) {
  const int group = c->d.n_heads / c->d.n_kv_heads;
  int gc = group <= 16 ? group : 16;
  while (group % gc != 0) --gc;
  return launch_piece<I8Piece<D>, uint16_t, D>(c, a, gc, st);
}

// fp32: VALU piece with GC heads per chunk.
template <int D>
hipError_t launch_f32(const kvc_cache* c, const DecodeArgs& a, hipStream_t st) {
  const int group = c->d.n_heads / c->d.n_kv_heads;
  if (group % 8 == 0) return launch_piece<ValuPiece<float, D, 8>, float, D>(c, a, 8, st);
  if (group % 4 == 0) return launch_piece<ValuPiece<float, D, 4>, float, D>(c, a, 4, st);
  if (group % 2 == 0) return launch_piece<ValuPiece<float, D, 2>, float, D>(c, a, 2, st);
  return launch_piece<ValuPiece<float, D, 1>, float, D>(c, a, 1, st);
}

}  // namespace

hipError_t kvc_launch_gqa_decode(const kvc_cache* c, const void* k_layer, const void* v_layer,
                                 const void* q, void* out, const int32_t* valid_lens,
                                 const int32_t* cache_index, float sm_scale, hipStream_t stream,
                                 const void* k_new, const void* v_new, const float* k_scale,
                                 const float* v_scale, const int32_t* block_table) {
  if (c->d.batch > KVC_MAX_BATCH || (long long)c->d.batch * c->d.n_heads > 0x7fffffffLL)
    return hipErrorInvalidValue;
  DecodeArgs a;
  a.k = k_layer;
  a.v = v_layer;
  a.q = q;
  a.out = out;
  a.valid_lens = valid_lens;
  a.cache_index = cache_index;
  a.scale_log2 = sm_scale * kLog2e;
  a.batch = c->d.batch;
  a.n_heads = c->d.n_heads;
  a.n_kv_heads = c->d.n_kv_heads;
  a.head_chunks = 1;
  a.chunk_heads = 1;
  a.max_context = c->d.max_context;
  a.n_wg = 1;
  a.whole_rows = 0;
  a.ws_acc = c->ws_acc;
  a.ws_ml = c->ws_ml;
  a.ws_cnt = c->ws_cnt;
  a.err_flag = c->err_flag;
  a.k_new = k_new;
  a.v_new = v_new;
  a.plan = c->ws_plan;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.table = block_table;
  a.block_shift = c->block_shift;
  a.num_blocks = c->num_blocks;
  a.table_width = c->table_width;
  a.pool_bytes = (int)c->kv_bytes;
  if (c->paged) {
    if (!block_table || c->d.dtype != KVC_BF16 || c->table_width > KVC_MAX_TABLE ||
        c->kv_bytes >= (1ull << 30))
      return hipErrorInvalidValue;
    switch (c->d.head_dim) {
      case 32: return launch_paged<32>(c, a, stream);
      case 64: return launch_paged<64>(c, a, stream);
      case 128: return launch_paged<128>(c, a, stream);
      case 256: return launch_paged<256>(c, a, stream);
    }
    return hipErrorInvalidValue;
  }
  if (c->d.dtype == KVC_I8) {
    if (!k_scale || !v_scale) return hipErrorInvalidValue;
    switch (c->d.head_dim) {
      case 64: return launch_i8<64>(c, a, stream);
      case 128: return launch_i8<128>(c, a, stream);
      case 256: return launch_i8<256>(c, a, stream);
    }
    return hipErrorInvalidValue;
  }
  const bool bf16 = c->d.dtype == KVC_BF16;
  switch (c->d.head_dim) {
    case 32: return bf16 ? launch_bf16<32>(c, a, stream) : launch_f32<32>(c, a, stream);
    case 64: return bf16 ? launch_bf16<64>(c, a, stream) : launch_f32<64>(c, a, stream);
    case 128: return bf16 ? launch_bf16<128>(c, a, stream) : launch_f32<128>(c, a, stream);
    case 256: return bf16 ? launch_bf16<256>(c, a, stream) : launch_f32<256>(c, a, stream);
  }
  return hipErrorInvalidValue;
}
