// Latent (MLA) decode over the static latent cache.
//
// What is computed ("10.3 - KV cache implementation details", section 4.3;
// "KV-Cache Mechanics", the MHA / GQA / MLA comparison and its "absorb"
// overhead): every cached row holds the latent c_j (d_c = 512) followed by
// the rotary key kR_j (d_R = 64), shared by all query heads. For query head
// h of sequence b with n = n_b valid rows,
//     q~[b,h]  = [ W_UK[h]^T q_nope[b,h] ; q_rope[b,h] ]          (absorb)
//     o~[b,h]  = softmax(sm_scale * R[b,0:n] q~[b,h]) R[b,0:n,0:d_c]  (latent attention)
//     out[b,h] = W_UV[h]^T o~[b,h]                                  (up-projection)
// which equals attention with per-head keys [W_UK[h] c_j ; kR_j] and values
// W_UV[h]^T c_j (associativity). Rows at or past n are never loaded.
//
// How:
//  - Latent attention is the part that reads the cache, and it is a dense
//    contraction (16 heads x 576 dims per row against every row), so it runs
//    on the matrix cores. Work space as for GQA (row space of segments =
//    (sequence, chunk of up to 16 heads), persistent grid, pieces). A
//    workgroup streams its rows in tiles of 32 rows (36 KB, one contiguous
//    block) staged through two skewed LDS tiles used in turn (one barrier per
//    tile besides the score exchange); the next two tiles are in flight in
//    registers while the current one is used. The latent rows are read from
//    HBM once for all heads of the chunk.
//  - The score tile S = R_tile q~^T is split over the 576 dims: each wave
//    takes a quarter (144 dims: four v_mfma_f32_16x16x32_bf16 steps and one
//    v_mfma_f32_16x16x16_bf16 step, with the rows as the A operand read from
//    LDS and the heads as the B operand held in registers); the four partial
//    tiles are summed through LDS in the same order by every wave, so all
//    waves hold identical softmax state. Then each wave applies P to its own
//    quarter (128) of the 512 latent columns with one 32-row
//    v_mfma_f32_16x16x32_bf16 per 16 columns (lane (g, j) takes rows
//    4g .. 4g + 3 of both 16-row blocks, in the same order in P and in V,
//    which reaches the B operand through one ds_read_b64_tr_b16 per block).
//    The 32-dim form does twice the work per instruction of the 16-dim one
//    and measured 1.7x its rate.
//  - Every piece writes its partial (o~ / l as bf16, m and l as fp32) to
//    slot w + s; a second kernel merges the pieces of each (sequence, head)
//    with weights 2^(m_p - m*) l_p / l*. A latent partial is 16 x 512 wide,
//    too wide for one workgroup to merge at the end of the streaming kernel.
//  - The absorb and up-projection are small batched products over the
//    weights (2 MB each), on the matrix cores with the weight block staged
//    in LDS.

#include "kvc_device.h"

namespace {

using namespace kvcd;

constexpr int kDc = 512;                     // latent width
constexpr int kDr = 64;                      // rotary key width
constexpr int kRow = kDc + kDr;              // elements per cached row
constexpr int kRowBytes = 2 * kRow;          // 1152
constexpr int kTok = 32;                     // rows per tile
constexpr int kStride = kRowBytes + 16;      // LDS bytes per staged row (skew: conflict-free reads)
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kCols = kDc / kWaves;          // latent columns per wave in p.v (128)
constexpr int kNB = kCols / 16;              // output column blocks per wave
constexpr int kQDims = kRow / kWaves;        // q.k dims per wave (144)
constexpr int kQS = kQDims / 32;             // q.k steps of 32 dims per wave (4) ...
constexpr int kQT = kQDims - 32 * kQS;       // ... and a last step of 16 dims
static_assert(kQT == 16, "a wave's q.k dims are 32 kQS + 16");
constexpr int kVec = kTok * kRowBytes / 16 / kThreads;  // staged 16-byte vectors per thread per tile
constexpr int kRowVecs = kRowBytes / 16;     // 72
constexpr int kSlotHeads = 16;               // partial entries per workspace slot
// Start-up rows of a segment (see kvc_device.h): none. A segment's first
// piece costs little beyond its rows here, and with 8 workgroups per segment
// (B = 32, 4096 rows) any allowance lands on the same eighth of the grid
// (the workgroups of one XCD): 160 rows made them finish 9 us before the
// rest (latent attention 37.6 -> 36.3 us without).
constexpr int kSegRowsMla = 0;
constexpr float kLazyMfma = 64.0f;           // log2 headroom before the reference maximum moves
static_assert(kTok * kRowBytes % (16 * kThreads) == 0, "tile must split evenly over the threads");
static_assert(kSegRowsMla <= kMaxSegRows, "row space must stay below 2^31");

struct MlaArgs {
  const uint16_t* rows;        // layer rows [B][S][576]
  const uint16_t* q_abs;       // absorbed queries [B][H][576]
  uint16_t* part;              // [slot][16][512] partial o~ / l (bf16)
  float* ml;                   // [slot][16][2]  m (log2 units), l
  uint16_t* out;               // merged latent output [B][H][512]
  const int32_t* valid_lens;   // [B] or null
  const int32_t* cache_index;  // [B] or null
  float scale_log2;
  int batch, n_heads, max_context;
  int head_chunks, chunk_heads;  // H = head_chunks * chunk_heads, chunk_heads <= 16
  int n_wg;
  int32_t* err_flag;
  int32_t* seg_info;           // [B * head_chunks][2]: first workgroup and pieces of each non-empty segment
};

// Rows [r_begin, r_end) of sequence b against heads [hc * gc, (hc + 1) * gc).
// tiles: two staged tiles used in turn; sred: 8 KB of LDS for the per-wave
// partial score tiles.
__device__ __forceinline__ void mla_piece(const MlaArgs& a, unsigned char* tiles, f32x4_t* sred, int b, int hc,
                                          int r_begin, int r_end, long long slot) {
  b = uniform(b);
  hc = uniform(hc);
  r_begin = uniform(r_begin);
  r_end = uniform(r_end);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int j = lane & 15;
  const int gc = a.chunk_heads;
  const int h0 = hc * gc;
  const float scale_log2 = a.scale_log2;

  // q~ as the B operand of this wave's quarter of the 576 dims (k steps of
  // 16): column j is head h0 + j, zero past the chunk (loaded after the
  // first tiles are requested, so the two latencies overlap)
  bf16x8_t qb[kQS];
  s16x4_t qt;

  f32x4_t o[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) o[nb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m = -INFINITY;  // reference maximum of head column j (log2 units)
  float l = 0.0f;       // this lane's share of column j's denominator

  // The resource spans exactly rows [0, r_end) of the sequence: loads past
  // the end (the tail of the last tile, prefetches after it) return zeros
  // without touching memory, and their scores are masked.
  const uint16_t* seq = a.rows + (size_t)b * a.max_context * kRow;
  const __amdgpu_buffer_rsrc_t res = buffer_rsrc(seq, r_end * kRowBytes);
  auto load = [&](u32x4_t (&st)[kVec], int t0) {
    const int off = t0 * kRowBytes + (int)threadIdx.x * 16;
#pragma unroll
    for (int i = 0; i < kVec; ++i) st[i] = __builtin_amdgcn_raw_buffer_load_b128(res, off + i * 16 * kThreads, 0, kStreamLoad);
  };
  auto stage = [&](unsigned char* tile, const u32x4_t (&st)[kVec]) {
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
      const int f = (int)threadIdx.x + i * kThreads;
      *reinterpret_cast<u32x4_t*>(tile + (f / kRowVecs) * kStride + (f % kRowVecs) * 16) = st[i];
    }
  };
  // One tile whose rows start at t0 (rows at or past r_end are masked; a
  // tile wholly past the end changes nothing).
  auto use_tile = [&](const unsigned char* tile, int t0) {
    // this wave's partial scores over its 144 dims, two 16-row blocks:
    // four steps of 32 dims (lane (g, j): row j, dims 32k + 8g ..) and one of 16
    f32x4_t sp[2];
    // all A fragments of the tile are requested before the first product
    bf16x8_t av[2][kQS];
    s16x4_t at[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const unsigned char* arow = tile + (16 * tb + j) * kStride + 2 * kQDims * wave;  // tile: this tile's rows
#pragma unroll
      for (int k = 0; k < kQS; ++k) av[tb][k] = *reinterpret_cast<const bf16x8_t*>(arow + 64 * k + 16 * g);
      at[tb] = *reinterpret_cast<const s16x4_t*>(arow + 64 * kQS + 8 * g);
    }
    // keep the reads ahead of the products (the scheduler would otherwise
    // pair each read with its product and wait out every LDS latency)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      sp[tb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < kQS; ++k) sp[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[tb][k], qb[k], sp[tb], 0, 0, 0);
      sp[tb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(at[tb], qt, sp[tb], 0, 0, 0);
      sred[(wave * 2 + tb) * 64 + lane] = sp[tb];
    }
    __syncthreads();  // partial scores visible
    // full scores, summed in the same order by every wave (identical softmax
    // state in all waves): s[tb][t] = R[t0 + 16 tb + 4g + t] . q~[head j]
    f32x4_t s[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      s[tb] = sred[tb * 64 + lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) s[tb] += sred[(w * 2 + tb) * 64 + lane];
    }
    if (t0 + kTok > r_end) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int t = 0; t < 4; ++t) s[tb][t] = (t0 + 16 * tb + 4 * g + t < r_end) ? s[tb][t] : -INFINITY;
    }
    // online softmax with a lazily moved reference maximum (p <= 2^kLazyMfma)
    const float cand = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                             fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3]))) * scale_log2;
    if (__builtin_amdgcn_ballot_w64(cand > m + kLazyMfma)) {
      float mt = fmaxf(cand, __shfl_xor(cand, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mn = fmaxf(m, mt);
      const float c = __builtin_amdgcn_exp2f(m - ((mn == -INFINITY) ? 0.0f : mn));
      l *= c;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float ct = __shfl(c, 4 * g + t);  // factor of output row (head) 4g + t
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) o[nb][t] *= ct;
      }
      m = mn;
    }
    const float nm = (m == -INFINITY) ? 0.0f : -m;
    // P as the A operand of one 32-row p.v: lane (g, j) takes rows 4g .. 4g + 3
    // of both blocks (the summed rows are in the same order in A and B, so the
    // order does not matter)
    bf16x8_t pa;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // the denominator sums the bf16 weights that enter the product
      pa[u] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[u >> 2][u & 3], scale_log2, nm));
      l += (float)pa[u];
    }
    // p.v over this wave's latent columns [128 wave, 128 wave + 128): B = the
    // rows 4g + t of both blocks by one transpose read per block
    const unsigned char* vrow = tile + (4 * g + (j >> 2)) * kStride + 2 * kCols * wave + 8 * (j & 3);
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(vrow + 32 * nb));
      const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(vrow + 16 * kStride + 32 * nb));
      const bf16x8_t vb = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o[nb], 0, 0, 0);
    }
  };

  // Two register tiles in flight: the body is straight-line over a pair of
  // tiles, so the wait before staging one leaves the other's loads pending.
  u32x4_t st0[kVec], st1[kVec];
  load(st0, r_begin);
  load(st1, r_begin + kTok);
  {
    const bool real = j < gc;
    const uint16_t* qh = a.q_abs + ((size_t)b * a.n_heads + h0 + (real ? j : 0)) * kRow + kQDims * wave;
#pragma unroll
    for (int k = 0; k < kQS; ++k) {
      u32x4_t v = *reinterpret_cast<const u32x4_t*>(qh + 32 * k + 8 * g);
      qb[k] = __builtin_bit_cast(bf16x8_t, real ? v : u32x4_t{0u, 0u, 0u, 0u});
    }
    const s16x4_t vt = *reinterpret_cast<const s16x4_t*>(qh + 32 * kQS + 4 * g);
    qt = real ? vt : s16x4_t{0, 0, 0, 0};
  }
  // Two LDS tiles in turn: a wave stages tile i into buffer i % 2 only after
  // the barrier of tile i - 1, which every wave reaches after it is done
  // with tile i - 2 (the buffer's previous tile) and with its score
  // exchange, so one barrier per tile (plus the exchange's) suffices.
  unsigned char* const tile0 = tiles;
  unsigned char* const tile1 = tiles + kTok * kStride;
  for (int t0 = r_begin; t0 < r_end; t0 += 2 * kTok) {
    stage(tile0, st0);
    load(st0, t0 + 2 * kTok);
    __syncthreads();  // the tile is visible
    use_tile(tile0, t0);
    stage(tile1, st1);
    load(st1, t0 + 3 * kTok);
    __syncthreads();
    use_tile(tile1, t0 + kTok);
  }

  // denominators of the head columns, then the partial o~ / l (bf16, put
  // together in LDS as [head][column] and stored 16 bytes per lane, written
  // through to memory), m and l. Against one 2-byte store per element this
  // took the latent attention from 35.0 to 34.1 us (B = 32, 4096 rows).
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  __syncthreads();  // every wave is done with the tiles
  uint16_t* const po = reinterpret_cast<uint16_t*>(tiles);  // [16][512] bf16 (16 KB)
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int hr = 4 * g + t;
    const float inv = 1.0f / __shfl(l, hr);  // l >= 1: the piece has a live row
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) po[hr * kDc + kCols * wave + 16 * nb + j] = bf16_rne(o[nb][t] * inv);
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t pres = buffer_rsrc(a.part + (size_t)slot * kSlotHeads * kDc, gc * kDc * 2);
#pragma unroll
  for (int i = 0; i < kSlotHeads * kDc / 8 / kThreads; ++i) {
    const int v = (int)threadIdx.x + kThreads * i;  // 16-byte vector v: head v / 64, columns 8 (v % 64) ..
    __builtin_amdgcn_raw_buffer_store_b128(reinterpret_cast<const u32x4_t*>(po)[v], pres, 16 * v, 0, kWriteThrough);
  }
  if (wave == 0 && g == 0 && j < gc) {
    put(a.ml + ((size_t)slot * kSlotHeads + j) * 2, m);
    put(a.ml + ((size_t)slot * kSlotHeads + j) * 2 + 1, l);
  }
  __syncthreads();  // the tiles are reused by the next piece
}

// Persistent latent attention: grid = W workgroups of 256 threads, one per
// CU by default, so each wave may use a whole SIMD's register file.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void mla_split_kernel(MlaArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char tile[2 * kTok * kStride];
  __shared__ f32x4_t sred[kWaves * 2 * 64];
  __shared__ int32_t s_prefix[KVC_MAX_BATCH + 1];
  __shared__ int32_t s_umax;
  const int B = a.batch;
  build_row_space(a.valid_lens, a.cache_index, B, a.max_context, kSegRowsMla, s_prefix, &s_umax, a.err_flag,
                  blockIdx.x == 0);
  const int HC = a.head_chunks;
  const long long R = (long long)s_prefix[B] * HC;
  const Partition part(R, a.n_wg, s_umax);
  const int w = blockIdx.x;
  if (w >= part.W) return;
  const long long x = part.lo(w);
  const long long hi = part.lo(w + 1);
  if (x >= hi) return;
  for_each_piece(s_prefix, B, HC, kSegRowsMla, x, hi,
                 [&](int b, int hc, int r_begin, int r_end, int n, long long real0) {
                   const long long s = (long long)b * HC + hc;
                   mla_piece(a, tile, sred, b, hc, r_begin, r_end, (long long)w + s);
                   if (r_begin == 0 && threadIdx.x == 0) {  // the segment's first piece: tell the merge
                     a.seg_info[2 * s] = w;
                     a.seg_info[2 * s + 1] = part.of(real0 + n - 1) - w + 1;
                   }
                 });
}

// Merge of the pieces of segment (b, hc) for latent columns [64 y, 64 y + 64):
// grid (B * HC, 8), 256 threads = 16 heads x 16 threads of 4 columns. The
// segment's first workgroup and number of pieces come from the split kernel
// (written by the workgroup that held the segment's first piece), requested
// together with the sequence's length.
constexpr int kMergeCols = 64;
__global__ __launch_bounds__(kThreads) void mla_merge_kernel(MlaArgs a) {
  __shared__ float s_m[kMaxMerge * kSlotHeads];  // m_p of (piece p, head), head-minor
  __shared__ float s_l[kMaxMerge * kSlotHeads];  // l_p
  __shared__ float s_w[kMaxMerge * kSlotHeads];  // weight of the normalised partial
  const int HC = a.head_chunks;
  const int gc = a.chunk_heads;
  const int seg = blockIdx.x;
  const int b = seg / HC;
  const int hc = seg - b * HC;
  const int h = threadIdx.x >> 4;
  const int col = kMergeCols * blockIdx.y + 4 * (threadIdx.x & 15);
  uint16_t* o = a.out + ((size_t)b * a.n_heads + hc * gc + h) * kDc + col;
  bool bad;
  const int n = seq_rows(a.valid_lens, a.cache_index, b, a.max_context, 0, &bad);
  const int w0 = uniform(a.seg_info[2 * seg]);
  const int np = uniform(a.seg_info[2 * seg + 1]);
  if (n == 0) {  // empty or out-of-range sequence: zeros (the split kernel wrote no pieces)
    if (h < gc) *reinterpret_cast<uint2*>(o) = make_uint2(0u, 0u);
    return;
  }
  const long long slot0 = (long long)w0 + seg;
  // This thread's partial columns for the first K pieces are requested
  // before the weights are worked out, so both loads overlap.
  constexpr int K = 16;
  const uint16_t* pc = a.part + (slot0 * kSlotHeads + (h < gc ? h : 0)) * kDc + col;
  uint2 v[K];
#pragma unroll
  for (int i = 0; i < K; ++i) v[i] = *reinterpret_cast<const uint2*>(pc + (size_t)min(i, np - 1) * kSlotHeads * kDc);
  for (int t = threadIdx.x; t < np * gc; t += kThreads) {
    const int p = t / gc, hh = t - p * gc;
    s_m[t] = a.ml[((slot0 + p) * kSlotHeads + hh) * 2];
    s_l[t] = a.ml[((slot0 + p) * kSlotHeads + hh) * 2 + 1];
  }
  __syncthreads();
  // weight of (piece p, head hh), one per thread: 2^(m_p - m*) l_p / l*
  for (int t = threadIdx.x; t < np * gc; t += kThreads) {
    const int hh = t % gc;
    float mx = -INFINITY;
    for (int p = 0; p < np; ++p) mx = fmaxf(mx, s_m[p * gc + hh]);
    float lsum = 0.0f;
    for (int p = 0; p < np; ++p) lsum += __builtin_amdgcn_exp2f(s_m[p * gc + hh] - mx) * s_l[p * gc + hh];
    s_w[t] = __builtin_amdgcn_exp2f(s_m[t] - mx) * s_l[t] / lsum;
  }
  __syncthreads();
  if (h >= gc) return;
  float x[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int p0 = 0; p0 < np; p0 += K) {
    if (p0 > 0) {
#pragma unroll
      for (int i = 0; i < K; ++i)
        v[i] = *reinterpret_cast<const uint2*>(pc + (size_t)min(p0 + i, np - 1) * kSlotHeads * kDc);
    }
#pragma unroll
    for (int i = 0; i < K; ++i) {
      if (p0 + i < np) {
        const float wt = s_w[(p0 + i) * gc + h];
        x[0] = fmaf(__uint_as_float(v[i].x << 16), wt, x[0]);
        x[1] = fmaf(__uint_as_float(v[i].x & 0xFFFF0000u), wt, x[1]);
        x[2] = fmaf(__uint_as_float(v[i].y << 16), wt, x[2]);
        x[3] = fmaf(__uint_as_float(v[i].y & 0xFFFF0000u), wt, x[3]);
      }
    }
  }
  *reinterpret_cast<uint2*>(o) = make_uint2((uint32_t)bf16_rne(x[0]) | ((uint32_t)bf16_rne(x[1]) << 16),
                                            (uint32_t)bf16_rne(x[2]) | ((uint32_t)bf16_rne(x[3]) << 16));
}

// ---- absorb and up-projection ---------------------------------------------
//
// Both are batched products over the heads with the batch as M:
//   absorb:  q~[:, h, 0:512] = q_nope[:, h, :] (B x 128)  . W_UK[h] (128 x 512)
//   up-proj: out[:, h, :]     = o~[:, h, :]    (B x 512)  . W_UV[h] (512 x 128)
// They are small and latency-bound, so the reduction is split over the
// waves: a workgroup takes 16 output columns n0 .. n0 + 16 of one head (grid
// H x N / 16), wave w multiplies the k range [K/4 w, K/4 (w + 1)) with a
// chain of K/64 products per 16-row batch block, and the four partial
// tiles are summed in LDS in a fixed order. The weight slice W[h][:,
// n0:n0+16] is staged row-major in LDS (32 bytes per k row + skew) and
// reaches the B operand of v_mfma_f32_16x16x16_bf16 through
// ds_read_b64_tr_b16 (the weights are stored K-major, so this is the
// transpose the operand needs). The A operand (4 consecutive k of one batch
// row) is read straight from global memory, a whole 16-row batch block at a
// time, requested before the block before it is multiplied (the first
// together with the weights). fp32 sums, bf16 out. Splitting the 512-long
// up-projection reduction this way took it from 10.8 to 4.9 us (B = 32,
// H = 16): the column-split form ran one 32-long dependent chain per wave
// on 32 workgroups.
constexpr int kGemmCols = 16;                   // output columns per workgroup
constexpr int kGemmStride = 2 * kGemmCols + 16;  // LDS bytes per staged weight row (skew)

template <int K>
__global__ __launch_bounds__(256) void mla_gemm_kernel(const uint16_t* __restrict__ a, long long a_head,
                                                       long long lda, const uint16_t* __restrict__ w,
                                                       int n_total, uint16_t* __restrict__ c, long long c_head,
                                                       long long ldc, int m_total,
                                                       const uint16_t* __restrict__ rope, int n_heads) {
  constexpr int KW = K / 4;   // k range per wave
  constexpr int KS = KW / 16;  // k steps per wave
  static_assert(KS >= 1 && KW % 16 == 0, "reduction must split into 16-steps per wave");
  __shared__ __attribute__((aligned(16))) unsigned char wt[K * kGemmStride];
  __shared__ f32x4_t red[4][64];  // partial tiles of one batch block
  const int h = blockIdx.x;
  const int n0 = blockIdx.y * kGemmCols;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int j = lane & 15;
  // lane (g, j): batch row m0 + j, k = KW wave + 16 s + 4g .. +3 (rows past
  // the batch are clamped to the last one and never stored)
  const uint16_t* ah = a + (size_t)h * a_head + KW * wave + 4 * g;
  auto load_a = [&](int m0, s16x4_t (&ab)[KS]) {
    const uint16_t* arow = ah + (size_t)min(m0 + j, m_total - 1) * lda;
#pragma unroll
    for (int s = 0; s < KS; ++s) ab[s] = *reinterpret_cast<const s16x4_t*>(arow + 16 * s);
  };
  // stage W[h][0:K][n0:n0+16]: two 16-byte vectors per k row
  constexpr int kPer = K * 2 / 256;
  static_assert(K * 2 % 256 == 0, "weight slice must split evenly over the threads");
  const uint16_t* wh = w + (size_t)h * K * n_total + n0;
  u32x4_t wv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int f = (int)threadIdx.x + 256 * i;
    wv[i] = *reinterpret_cast<const u32x4_t*>(wh + (size_t)(f >> 1) * n_total + 8 * (f & 1));
  }
  s16x4_t ab0[KS], ab1[KS];
  load_a(0, ab0);
  // absorb only: the first column block of each head also copies q_rope
  // into columns [512, 576) of q~ (16-byte vectors, 8 per row)
  if (rope && blockIdx.y == 0) {
    for (int i = threadIdx.x; i < m_total * (kDr / 8); i += 256) {
      const int b = i / (kDr / 8), r = 8 * (i - b * (kDr / 8));
      *reinterpret_cast<u32x4_t*>(c + (size_t)h * c_head + (size_t)b * ldc + kDc + r) =
          *reinterpret_cast<const u32x4_t*>(rope + ((size_t)b * n_heads + h) * kDr + r);
    }
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int f = (int)threadIdx.x + 256 * i;
    *reinterpret_cast<u32x4_t*>(wt + (f >> 1) * kGemmStride + 16 * (f & 1)) = wv[i];
  }
  __syncthreads();
  // B operand: rows 4g + t of each 16-row k step of this wave's range, column j
  const unsigned char* brow = wt + (KW * wave + 4 * g + (j >> 2)) * kGemmStride + 8 * (j & 3);
  uint16_t* ch = c + (size_t)h * c_head + n0 + j;
  auto block = [&](int m0, const s16x4_t (&ab)[KS]) {
    f32x4_t acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const s16x4_t bv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(brow + 16 * s * kGemmStride));
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ab[s], bv, acc, 0, 0, 0);
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {  // D row 4g + t is batch row m0 + 4g + t, column j
      const f32x4_t x = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int m = m0 + 4 * g + t;
        if (m < m_total) ch[(size_t)m * ldc] = bf16_rne(x[t]);
      }
    }
    __syncthreads();  // red is reused by the next block
  };
  // batch blocks in pairs: the next block's A fragments are in flight while
  // the current block's chain runs
  for (int m0 = 0; m0 < m_total; m0 += 32) {
    load_a(m0 + 16, ab1);
    block(m0, ab0);
    if (m0 + 16 >= m_total) break;
    load_a(m0 + 32, ab0);
    block(m0 + 16, ab1);
  }
}

}  // namespace

hipError_t kvc_launch_mla_attn(const kvc_cache* c, const void* rows_layer, const void* q_abs, void* out_lat,
                               const int32_t* valid_lens, const int32_t* cache_index, float sm_scale,
                               hipStream_t stream) {
  MlaArgs a;
  a.rows = static_cast<const uint16_t*>(rows_layer);
  a.q_abs = static_cast<const uint16_t*>(q_abs);
  a.part = reinterpret_cast<uint16_t*>(c->ws_acc);
  a.ml = c->ws_ml;
  a.out = static_cast<uint16_t*>(out_lat);
  a.valid_lens = valid_lens;
  a.cache_index = cache_index;
  a.scale_log2 = sm_scale * kLog2e;
  a.batch = c->d.batch;
  a.n_heads = c->d.n_heads;
  a.max_context = c->d.max_context;
  a.chunk_heads = c->d.n_heads <= kSlotHeads ? c->d.n_heads : kSlotHeads;
  a.head_chunks = c->d.n_heads / a.chunk_heads;
  a.n_wg = c->workgroups_forced > 0 ? c->workgroups_forced : c->num_cus;  // one per CU (measured best)
  if (a.n_wg > c->max_workgroups) a.n_wg = c->max_workgroups;
  a.err_flag = c->err_flag;
  a.seg_info = c->ws_seg;
  mla_split_kernel<<<dim3(a.n_wg), dim3(kThreads), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  mla_merge_kernel<<<dim3(a.batch * a.head_chunks, kDc / kMergeCols), dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t kvc_launch_mla_absorb(const kvc_cache* c, const void* q_nope, const void* q_rope, const void* w_uk,
                                 uint16_t* q_abs, hipStream_t stream) {
  const int B = c->d.batch, H = c->d.n_heads, dn = c->d.head_dim;
  if (dn != 128) return hipErrorInvalidValue;
  mla_gemm_kernel<128><<<dim3(H, kDc / kGemmCols), dim3(256), 0, stream>>>(
      static_cast<const uint16_t*>(q_nope), dn, (long long)H * dn, static_cast<const uint16_t*>(w_uk), kDc, q_abs,
      kRow, (long long)H * kRow, B, static_cast<const uint16_t*>(q_rope), H);
  return hipGetLastError();
}

hipError_t kvc_launch_mla_uproj(const kvc_cache* c, const uint16_t* o_lat, const void* w_uv, void* out,
                                hipStream_t stream) {
  const int B = c->d.batch, H = c->d.n_heads, dv = c->d.head_dim;
  if (dv != 128) return hipErrorInvalidValue;
  mla_gemm_kernel<kDc><<<dim3(H, dv / kGemmCols), dim3(256), 0, stream>>>(
      o_lat, kDc, (long long)H * kDc, static_cast<const uint16_t*>(w_uv), dv, static_cast<uint16_t*>(out), dv,
      (long long)H * dv, B, nullptr, H);
  return hipGetLastError();
}
