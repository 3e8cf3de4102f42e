// Causal prefill attention over the static cache (bf16).
//
// What is computed ("KV-Cache Mechanics", "AR Static KV-Cache": the prompt's
// forward pass fills the cache from cache_index 0, a later chunk continues
// at cache_index = start; "10.3 - KV cache implementation details", section
// 3, causal attention, and section 4.2 for shared key/value heads): after
// the chunk's rows [start, start + t) are in the cache, query i of the chunk
// (position start + i) of head h attends the cache rows 0 .. start + i of
// kv head g = h / (H / H_kv):
//     out[b,h,i] = softmax(sm_scale * K[b,g,0:start+i+1] q[b,h,i]) V[b,g,0:start+i+1].
//
// How (matrix cores, the decode piece's layout with query positions in
// place of heads):
//  - A workgroup of four waves takes hpw = min(G, 4) heads of one kv head
//    (G = H / H_kv; 1 if G is not a power of two) and 16 QG 4 / hpw
//    positions; wave w takes head hpw0 + w % hpw and QG groups of 16
//    positions. The K/V tiles of the kv head are therefore shared by all
//    heads of the group the workgroup holds, and every K and V operand read
//    from LDS feeds the products of QG query groups (two at d_h <= 128: the
//    loop's LDS reads and copies per product halve, 166 -> 137 us per layer
//    at a 4096-token prompt; three groups take 232 registers, two waves per
//    SIMD, 151 us).
//  - Keys go in tiles of 32 rows, K and V each copied from memory straight
//    into LDS by the waves' buffer loads (no registers, no LDS write
//    instructions), into two buffers used in turn: the next tile's copy is
//    issued right after the barrier that opens the current one, so one
//    barrier per tile suffices and a whole tile of work hides the copy's
//    latency (a third buffer, copies two tiles ahead, measured the same).
//    Each buffer is an array of its own and the loop is unrolled twice, so
//    the compiler sees which buffer every LDS read touches and does not
//    make the reads of one buffer wait for the copy into the other. Rows
//    are stored unpadded with their 16-byte chunks XOR-swizzled (per row,
//    differently for K and V), so both the A-operand reads of K and the
//    transposed reads of V touch every bank once; the lane part of every
//    LDS address is worked out once, the buffer and block parts are
//    constant offsets.
//  - Scores: S[key][query] on v_mfma_f32_16x16x32_bf16, 16 keys (A, from LDS)
//    against 16 queries (B, in registers), per 16-key block. Causal mask per
//    (key, query). fp32 online softmax in log2 units with a lazily moved
//    reference maximum per query group, moved once per tile.
//  - p.v on v_mfma_f32_16x16x32_bf16, two 16-key blocks per product, with V
//    read back transposed from LDS by ds_read_b64_tr_b16; each wave keeps its
//    own (o, m, l), so no cross-wave merge: the output rows are normalised
//    and written by the wave. The denominators are the product of P with a
//    block of ones, so they sum the same bf16 weights p.v uses.
//  - Tiles whose keys all lie past a wave's last query are skipped by that
//    wave; the query blocks with the most keys are launched first, for every
//    head group.

#include <type_traits>

#include "kvc_device.h"

namespace {

using namespace kvcd;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLazy = 64.0f;            // log2 headroom before the reference maximum moves

struct PrefillArgs {
  const uint16_t* k;      // layer keys [B][H_kv][S][D]
  const uint16_t* v;      // layer values
  const uint16_t* q;      // [B][H][t][D]
  uint16_t* out;          // [B][H][t][D]
  float scale_log2;
  int n_heads, n_kv_heads, max_context, start, t;
  int hpw;                // heads per workgroup (1, 2 or 4)
  int n_qblocks;          // position blocks of 64 QG / hpw per (b, head group)
};

template <int D>
struct Prefill {
  static constexpr int KS = D / 32;                 // q.k steps of 32 dims
  static constexpr int NB = D / 16;                 // output column blocks
  // keys per tile: 32 (a 64-key tile doubles the LDS per workgroup and
  // halves the workgroups a CU holds: 188 vs 215 us at a 4096-token prompt)
  static constexpr int TK = 32;
  static constexpr int NKB = TK / 16;               // 16-key blocks per tile
  static constexpr int ROW = 2 * D;                 // bytes per staged row
  static constexpr int CPR = ROW / 16;              // 16-byte chunks per row
  static constexpr int SWM = (CPR < 16 ? CPR : 16) - 1;  // chunk bits the swizzle changes
  static constexpr int TILE = TK * ROW;             // bytes of a K (or V) tile
  static constexpr int DMA = TILE / 1024 / kWaves;  // 1 KB copy instructions per wave per tile (K and V each)
  static_assert(TILE % (1024 * kWaves) == 0 && NKB % 2 == 0, "tile must split into 1 KB copies per wave");
};

// Chunk c of staged row r sits at chunk c ^ swizzle(r) of its LDS row.
// K: 16 consecutive rows give 16 different swizzles (A-operand reads of one
// chunk of 16 rows). V: rows r and r + 8 differ in the lowest bit and 8
// consecutive rows in the others (transposed reads of two chunks of 8 rows).
__device__ __forceinline__ int swz_k(int r, int mask) { return r & mask; }
// 16 bytes per lane from the buffer at voffset into LDS at dst + 16 lane
// (dst wave-uniform), not through registers.
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t res, unsigned char* dst, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (__attribute__((address_space(3))) void*)dst, 16, voffset, 0, 0, 0);
}
__device__ __forceinline__ int swz_v(int r, int mask) { return ((r << 1) | ((r >> 3) & 1)) & mask; }

template <int D, int QG>
__global__ __launch_bounds__(kThreads) void prefill_attn_kernel(PrefillArgs a) {
  using P = Prefill<D>;
  // K tile t and V tile t are staged in buffer t % 2: four arrays of their
  // own (see the header)
  __shared__ __attribute__((aligned(1024))) unsigned char lk0[P::TILE], lk1[P::TILE], lv0[P::TILE], lv1[P::TILE];
  auto kbuf = [&](int bf) { return bf ? lk1 : lk0; };
  auto vbuf = [&](int bf) { return bf ? lv1 : lv0; };

  const int lane = threadIdx.x & 63;
  const int wave = uniform((int)threadIdx.x >> 6);
  const int g = lane >> 4;
  const int j = lane & 15;
  const int hpw = a.hpw;
  const int span = 64 * QG / hpw;                   // positions per workgroup
  const int qb = a.n_qblocks - 1 - (int)blockIdx.y;
  const int groups = a.n_heads / hpw;
  const int b = (int)blockIdx.x / groups;
  const int hg = (int)blockIdx.x - b * groups;
  const int h = uniform(hg * hpw + wave % hpw);
  const int p0 = uniform(qb * span + 16 * QG * (wave / hpw));  // wave's first position; group qg adds 16 qg
  const int kvh = (hg * hpw) / (a.n_heads / a.n_kv_heads);
  const int last = min(qb * span + span, a.t) - 1;  // last position of the workgroup
  const int kend = a.start + last + 1;              // keys [0, kend) are needed
  const int qp0 = a.start + p0;                     // the wave's first absolute position

  const size_t row0 = ((size_t)b * a.n_kv_heads + kvh) * (size_t)a.max_context;
  const int rows = a.start + a.t;

  // the wave's QG x 16 queries as B operands: column j of group qg is
  // position p0 + 16 qg + j (positions past the chunk load zeros)
  bf16x8_t qv[QG][P::KS];
  {
    const __amdgpu_buffer_rsrc_t qres = buffer_rsrc(a.q + ((size_t)b * a.n_heads + h) * a.t * D, a.t * P::ROW);
#pragma unroll
    for (int qg = 0; qg < QG; ++qg)
#pragma unroll
      for (int k = 0; k < P::KS; ++k)
        qv[qg][k] = __builtin_bit_cast(
            bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(qres, (p0 + 16 * qg + j) * P::ROW + 64 * k + 16 * g, 0, 0));
  }

  // o, and in lsum the denominators: the product of P with a block of ones,
  // so lsum[qg][w] is the sum of the bf16 weights of output row (query) 4g + w
  f32x4_t o[QG][P::NB], lsum[QG];
  float m[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
#pragma unroll
    for (int nb = 0; nb < P::NB; ++nb) o[qg][nb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    lsum[qg] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m[qg] = -INFINITY;
  }
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  const float scale_log2 = a.scale_log2;

  // Lane parts of the addresses, fixed for the whole loop:
  //  - copies: wave w's copy i fills bytes [1024 I, 1024 I + 1024) of a K (V)
  //    tile, I = w DMA + i, 16 bytes per lane, with the chunk that position
  //    holds after the swizzle (from the tile's first row)
  int dk[P::DMA], dv[P::DMA];
#pragma unroll
  for (int i = 0; i < P::DMA; ++i) {
    const int pos = 64 * (wave * P::DMA + i) + lane;
    const int r = pos / P::CPR, cp = pos - r * P::CPR;
    dk[i] = r * P::ROW + 16 * (cp ^ swz_k(r, P::SWM));
    dv[i] = r * P::ROW + 16 * (cp ^ swz_v(r, P::SWM));
  }
  //  - K as the A operand: row 16 kb + j (its swizzle is that of row j), dims
  //    [32 k + 8 g, 32 k + 8 g + 8)
  int ka[P::KS];
#pragma unroll
  for (int k = 0; k < P::KS; ++k) ka[k] = j * P::ROW + 16 * ((4 * k + g) ^ swz_k(j, P::SWM));
  //  - V by transposed reads: row 32 pp + 16 e + r0 (its swizzle is that of
  //    row r0), the two chunks of column block nb; blocks nb and nb + 8 are
  //    256 bytes apart
  constexpr int NV = P::NB < 8 ? P::NB : 8;
  int va[NV];
  {
    const int r0 = 4 * g + (j >> 2);
    const int sv = swz_v(r0, P::SWM);
#pragma unroll
    for (int n = 0; n < NV; ++n) va[n] = r0 * P::ROW + 16 * ((2 * n + ((j & 3) >> 1)) ^ sv) + 8 * (j & 1);
  }

  // copies of tile t into buffer bf (the resource starts at the tile, so
  // rows past start + t read zeros)
  auto copy_k = [&](int bf, int t) {
    const __amdgpu_buffer_rsrc_t res = buffer_rsrc(a.k + (row0 + (size_t)t * P::TK) * D, (rows - t * P::TK) * P::ROW);
#pragma unroll
    for (int i = 0; i < P::DMA; ++i) copy_to_lds(res, kbuf(bf) + 1024 * (wave * P::DMA + i), dk[i]);
  };
  auto copy_v = [&](int bf, int t) {
    const __amdgpu_buffer_rsrc_t res = buffer_rsrc(a.v + (row0 + (size_t)t * P::TK) * D, (rows - t * P::TK) * P::ROW);
#pragma unroll
    for (int i = 0; i < P::DMA; ++i) copy_to_lds(res, vbuf(bf) + 1024 * (wave * P::DMA + i), dv[i]);
  };
  // scores of the tile in buffer BF: sc[qg][kb][w] = K[16 kb + 4g + w] . q[16 qg + j]
  auto qk = [&](auto bf_c, f32x4_t (&sc)[QG][P::NKB]) {
    constexpr int BF = decltype(bf_c)::value;
#pragma unroll
    for (int kb = 0; kb < P::NKB; ++kb) {
      bf16x8_t av[P::KS];
#pragma unroll
      for (int k = 0; k < P::KS; ++k)
        av[k] = *reinterpret_cast<const bf16x8_t*>(kbuf(BF) + 16 * kb * P::ROW + ka[k]);
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        sc[qg][kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < P::KS; ++k)
          sc[qg][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[k], qv[qg][k], sc[qg][kb], 0, 0, 0);
      }
    }
  };

  const int ntiles = (kend + P::TK - 1) / P::TK;
  // tiles with a key some query of the wave sees
  const int nlive = min(ntiles, (qp0 + 16 * QG - 1) / P::TK + 1);

  f32x4_t cur[QG][P::NKB];
  // Tile `it` from buffer PAR (known at compile time: the loop is unrolled
  // twice): this wave's copies of the tile have landed; the barrier makes
  // every wave's copies visible and confirms every wave is done with tile
  // it - 1, whose buffer the next copy overwrites. Then the scores of all
  // its blocks, one update of the reference maximum per query group, and
  // p.v over the pair of blocks.
  auto step = [&](auto par_c, int it) {
    constexpr int PAR = decltype(par_c)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (it + 1 < ntiles) {
      copy_k(PAR ^ 1, it + 1);
      copy_v(PAR ^ 1, it + 1);
    }
    if (it >= nlive) return;
    const int k0 = it * P::TK;
    qk(std::integral_constant<int, PAR>{}, cur);
    float nm[QG];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
      const int qq = qp0 + 16 * qg;
      if (k0 + P::TK - 1 > qq) {
#pragma unroll
        for (int kb = 0; kb < P::NKB; ++kb)
#pragma unroll
          for (int w = 0; w < 4; ++w)
            cur[qg][kb][w] = (k0 + 16 * kb + 4 * g + w <= qq + j) ? cur[qg][kb][w] : -INFINITY;
      }
      float cand = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < P::NKB; ++kb)
        cand = fmaxf(cand, fmaxf(fmaxf(cur[qg][kb][0], cur[qg][kb][1]), fmaxf(cur[qg][kb][2], cur[qg][kb][3])));
      cand *= scale_log2;
      if (__builtin_amdgcn_ballot_w64(cand > m[qg] + kLazy)) {
        float mt = fmaxf(cand, __shfl_xor(cand, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m[qg], mt);
        const float c = __builtin_amdgcn_exp2f(m[qg] - ((mn == -INFINITY) ? 0.0f : mn));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float cw = __shfl(c, 4 * g + w);
#pragma unroll
          for (int nb = 0; nb < P::NB; ++nb) o[qg][nb][w] *= cw;
          lsum[qg][w] *= cw;
        }
        m[qg] = mn;
      }
      nm[qg] = (m[qg] == -INFINITY) ? 0.0f : -m[qg];
    }
    // P as the A operand of 32-key products: lane (g, j) takes keys
    // 4g .. 4g + 3 of both blocks of a pair (the order of the transposed V
    // reads); the denominator sums the same bf16 weights, on the matrix cores
    bf16x8_t pa[QG][P::NKB / 2];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg)
#pragma unroll
      for (int pp = 0; pp < P::NKB / 2; ++pp) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pa[qg][pp][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(cur[qg][2 * pp + (e >> 2)][e & 3], scale_log2, nm[qg]));
        lsum[qg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[qg][pp], ones, lsum[qg], 0, 0, 0);
      }
    // p.v: B operand = V[k0 + 16 kb + 4g + w][16 nb + j] of both blocks of a
    // pair by one transposed read each, shared by the query groups
#pragma unroll
    for (int pp = 0; pp < P::NKB / 2; ++pp) {
#pragma unroll
      for (int nb = 0; nb < P::NB; ++nb) {
        s16x4_t vh[2];
#pragma unroll
        for (int e = 0; e < 2; ++e)
          vh[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(
              vbuf(PAR) + (32 * pp + 16 * e) * P::ROW + 256 * (nb / 8) + va[nb % 8]));
        const bf16x8_t vb = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(vh[0], vh[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qg = 0; qg < QG; ++qg)
          o[qg][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[qg][pp], vb, o[qg][nb], 0, 0, 0);
      }
    }
  };

  copy_k(0, 0);
  copy_v(0, 0);
  for (int it = 0; it < ntiles; it += 2) {
    step(std::integral_constant<int, 0>{}, it);
    if (it + 1 < ntiles) step(std::integral_constant<int, 1>{}, it + 1);
  }

  // normalise and write: lane (g, j) holds output rows (queries) 16 qg + 4g + w, columns 16 nb + j

#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int qi = p0 + 16 * qg + 4 * g + w;
      if (qi < a.t) {
        uint16_t* dst = a.out + (((size_t)b * a.n_heads + h) * a.t + qi) * D + j;
        const float inv = 1.0f / lsum[qg][w];  // lsum >= 1: the query attends at least its own key
#pragma unroll
        for (int nb = 0; nb < P::NB; ++nb) dst[16 * nb] = bf16_rne(o[qg][nb][w] * inv);
      }
    }
  }
}

}  // namespace

hipError_t kvc_launch_prefill_attn(const kvc_cache* c, const void* k_layer, const void* v_layer, const void* q,
                                   void* out, int start, int t, float sm_scale, hipStream_t stream) {
  PrefillArgs a;
  a.k = static_cast<const uint16_t*>(k_layer);
  a.v = static_cast<const uint16_t*>(v_layer);
  a.q = static_cast<const uint16_t*>(q);
  a.out = static_cast<uint16_t*>(out);
  a.scale_log2 = sm_scale * kLog2e;
  a.n_heads = c->d.n_heads;
  a.n_kv_heads = c->d.n_kv_heads;
  a.max_context = c->d.max_context;
  a.start = start;
  a.t = t;
  const int G = a.n_heads / a.n_kv_heads;
  a.hpw = G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1);
  // query groups of 16 per wave (one at d_h = 256, where the registers
  // allow no more)
  const int QG = c->d.head_dim == 256 ? 1 : 2;
  const int span = 64 * QG / a.hpw;
  a.n_qblocks = (t + span - 1) / span;
  const long long nx = (long long)c->d.batch * (a.n_heads / a.hpw);
  if (nx > 0x7fffffff || a.n_qblocks > 65535) return hipErrorInvalidValue;
  dim3 grid((unsigned)nx, (unsigned)a.n_qblocks);
  switch (c->d.head_dim) {
    case 64: prefill_attn_kernel<64, 2><<<grid, dim3(kThreads), 0, stream>>>(a); break;
    case 128: prefill_attn_kernel<128, 2><<<grid, dim3(kThreads), 0, stream>>>(a); break;
    case 256: prefill_attn_kernel<256, 1><<<grid, dim3(kThreads), 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
