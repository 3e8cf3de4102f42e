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
//    (G = H / H_kv; 1 if G is not a power of two) and 64 / hpw positions;
//    wave w takes head hpw0 + w % hpw and 16 positions. The K/V tiles of the
//    kv head are therefore shared by all heads of the group the workgroup
//    holds.
//  - Keys go in tiles of 32 rows, K and V each copied
//    from memory straight into LDS by the waves' buffer loads (no registers,
//    no LDS write instructions), into two buffers used in turn: the next
//    tile's copy is issued right after the barrier that opens the current
//    one, so one barrier per tile suffices and a whole tile of work hides the
//    copy's latency. Rows are stored unpadded with their 16-byte chunks
//    XOR-swizzled (per row, differently for K and V), so both the A-operand
//    reads of K and the transposed reads of V touch every bank once.
//  - Scores: S[key][query] on v_mfma_f32_16x16x32_bf16, 16 keys (A, from LDS)
//    against the wave's 16 queries (B, in registers), per 16-key block.
//    Causal mask per (key, query). fp32 online softmax in log2 units with a
//    lazily moved reference maximum per query column, moved once per tile.
//  - p.v on v_mfma_f32_16x16x32_bf16, two 16-key blocks per product, with V
//    read back transposed from LDS by ds_read_b64_tr_b16; each wave keeps its
//    own (o, m, l), so no cross-wave merge: the output rows are normalised
//    and written by the wave.
//  - Tiles whose keys all lie past a wave's last query are skipped by that
//    wave; the query blocks with the most keys are launched first, for every
//    head group.

#include "kvc_device.h"

namespace {

using namespace kvcd;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLazy = 64.0f;            // log2 headroom before the reference maximum moves
constexpr int kQueryGroups = 1;           // query groups of 16 per wave (2 measured within noise of 1)

struct PrefillArgs {
  const uint16_t* k;      // layer keys [B][H_kv][S][D]
  const uint16_t* v;      // layer values
  const uint16_t* q;      // [B][H][t][D]
  uint16_t* out;          // [B][H][t][D]
  float scale_log2;
  int n_heads, n_kv_heads, max_context, start, t;
  int hpw;                // heads per workgroup (1, 2 or 4)
  int n_qblocks;          // position blocks of 64 / hpw per (b, head group)
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
  // [buffer][K, V][tile]
  __shared__ __attribute__((aligned(1024))) unsigned char lds[2][2][P::TILE];

  const int lane = threadIdx.x & 63;
  const int wave = uniform((int)threadIdx.x >> 6);
  const int g = lane >> 4;
  const int j = lane & 15;
  const int hpw = a.hpw;
  const int span = 64 * QG / hpw;                   // positions per workgroup
  // x (dispatched fastest) runs over (sequence, head group), y over position
  // blocks with the most keys first, so every head group's heavy blocks go first
  const int qb = a.n_qblocks - 1 - (int)blockIdx.y;
  const int groups = a.n_heads / hpw;
  const int b = (int)blockIdx.x / groups;
  const int hg = (int)blockIdx.x - b * groups;
  const int h = uniform(hg * hpw + wave % hpw);
  const int p0 = uniform(qb * span + 16 * QG * (wave / hpw));  // wave's first position; group qg adds 16 qg
  const int kvh = (hg * hpw) / (a.n_heads / a.n_kv_heads);
  const int last = min(qb * span + span, a.t) - 1;  // last position of the workgroup
  const int kend = a.start + last + 1;              // keys [0, kend) are needed

  // the kv head's rows [0, start + t) as resources (loads past them read zeros)
  const size_t row0 = ((size_t)b * a.n_kv_heads + kvh) * (size_t)a.max_context;
  const int rows = a.start + a.t;
  const __amdgpu_buffer_rsrc_t kres = buffer_rsrc(a.k + row0 * D, rows * P::ROW);
  const __amdgpu_buffer_rsrc_t vres = buffer_rsrc(a.v + row0 * D, rows * P::ROW);

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

  // Copy of the tile at key k0 into buffer u: wave w's copy i fills bytes
  // [1024 I, 1024 I + 1024) of the K and V tiles, I = w DMA + i, lane by lane
  // (16 bytes each) with the chunk each position holds.
  auto copy = [&](int u, int k0) {
#pragma unroll
    for (int i = 0; i < P::DMA; ++i) {
      const int I = wave * P::DMA + i;
      const int pos = 64 * I + lane;  // 16-byte position in the tile
      const int r = pos / P::CPR, cp = pos - r * P::CPR;
      const int off = (k0 + r) * P::ROW;
      copy_to_lds(kres, &lds[u][0][1024 * I], off + 16 * (cp ^ swz_k(r, P::SWM)));
      copy_to_lds(vres, &lds[u][1][1024 * I], off + 16 * (cp ^ swz_v(r, P::SWM)));
    }
  };

  // One tile from buffer u: the scores of all its blocks, one update of the
  // reference maximum, then p.v over pairs of blocks.
  auto use = [&](int u, int k0) {
    const unsigned char* kt = lds[u][0];
    const unsigned char* vt = lds[u][1];
    bf16x8_t pa[QG][P::NKB / 2];
    bool live[QG];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
      const int qp0 = a.start + p0 + 16 * qg;  // first absolute position of the group
      live[qg] = k0 <= qp0 + 15;                // uniform: some key of the tile is visible to the group
      if (!live[qg]) continue;
      // sc[kb][w] = K[k0 + 16 kb + 4g + w] . q[query j]
      f32x4_t sc[P::NKB];
#pragma unroll
      for (int kb = 0; kb < P::NKB; ++kb) {
        const int r = 16 * kb + j;
        const unsigned char* arow = kt + r * P::ROW;
        const int sw = swz_k(r, P::SWM);
        bf16x8_t av[P::KS];
#pragma unroll
        for (int k = 0; k < P::KS; ++k) av[k] = *reinterpret_cast<const bf16x8_t*>(arow + 16 * ((4 * k + g) ^ sw));
        sc[kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < P::KS; ++k) sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[k], qv[qg][k], sc[kb], 0, 0, 0);
      }
      if (k0 + P::TK - 1 > qp0) {  // the tile reaches past some query of the group: causal mask
#pragma unroll
        for (int kb = 0; kb < P::NKB; ++kb)
#pragma unroll
          for (int w = 0; w < 4; ++w) sc[kb][w] = (k0 + 16 * kb + 4 * g + w <= qp0 + j) ? sc[kb][w] : -INFINITY;
      }
      float cand = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < P::NKB; ++kb)
        cand = fmaxf(cand, fmaxf(fmaxf(sc[kb][0], sc[kb][1]), fmaxf(sc[kb][2], sc[kb][3])));
      cand *= scale_log2;
      if (__builtin_amdgcn_ballot_w64(cand > m[qg] + kLazy)) {
        float mt = fmaxf(cand, __shfl_xor(cand, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m[qg], mt);
        const float c = __builtin_amdgcn_exp2f(m[qg] - ((mn == -INFINITY) ? 0.0f : mn));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float cw = __shfl(c, 4 * g + w);  // factor of output row (query) 4g + w
#pragma unroll
          for (int nb = 0; nb < P::NB; ++nb) o[qg][nb][w] *= cw;
          lsum[qg][w] *= cw;
        }
        m[qg] = mn;
      }
      const float nm = (m[qg] == -INFINITY) ? 0.0f : -m[qg];
      // P as the A operand of 32-key products: lane (g, j) takes keys
      // 4g .. 4g + 3 of both blocks of a pair (the order of the transposed V
      // reads); the denominator sums the same bf16 weights, on the matrix cores
#pragma unroll
      for (int pp = 0; pp < P::NKB / 2; ++pp) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pa[qg][pp][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[2 * pp + (e >> 2)][e & 3], scale_log2, nm));
        lsum[qg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[qg][pp], ones, lsum[qg], 0, 0, 0);
      }
    }
    // p.v: B operand = V[k0 + 16 kb + 4g + w][16 nb + j] of both blocks of a
    // pair by one transposed read each, shared by the query groups
#pragma unroll
    for (int pp = 0; pp < P::NKB / 2; ++pp) {
#pragma unroll
      for (int nb = 0; nb < P::NB; ++nb) {
        s16x4_t vh[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 16 * (2 * pp + e) + 4 * g + (j >> 2);
          const int c = (2 * nb + ((j & 3) >> 1)) ^ swz_v(r, P::SWM);
          vh[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4_t*)(vt + r * P::ROW + 16 * c + 8 * (j & 1)));
        }
        const bf16x8_t vb = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(vh[0], vh[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qg = 0; qg < QG; ++qg)
          if (live[qg]) o[qg][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[qg][pp], vb, o[qg][nb], 0, 0, 0);
      }
    }
  };

  const int ntiles = (kend + P::TK - 1) / P::TK;
  copy(0, 0);
  for (int it = 0; it < ntiles; ++it) {
    const int u = it & 1;
    const int k0 = it * P::TK;
    // this wave's copies of tile `it` (and the queries) have landed; the
    // barrier makes every wave's copies visible and confirms every wave is
    // done with tile it - 1, whose buffer the next copy overwrites
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (it + 1 < ntiles) copy(u ^ 1, k0 + P::TK);
    if (k0 > a.start + p0 + 16 * QG - 1) continue;  // all keys past this wave's queries
    use(u, k0);
  }

  // normalise and write: lane (g, j) holds output rows (queries) 4g + w, columns 16 nb + j
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int qi = p0 + 16 * qg + 4 * g + w;
      const float lr = lsum[qg][w];
      if (qi < a.t) {
        uint16_t* dst = a.out + (((size_t)b * a.n_heads + h) * a.t + qi) * D + j;
        const float inv = 1.0f / lr;  // lr >= 1: the query attends at least its own key
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
  // query groups of 16 per wave: each K/V read from LDS feeds QG x the products
  constexpr int QG = kQueryGroups;
  const int span = 64 * QG / a.hpw;
  a.n_qblocks = (t + span - 1) / span;
  const long long nx = (long long)c->d.batch * (a.n_heads / a.hpw);
  if (nx > 0x7fffffff || a.n_qblocks > 65535) return hipErrorInvalidValue;
  dim3 grid((unsigned)nx, (unsigned)a.n_qblocks);
  switch (c->d.head_dim) {
    case 64: prefill_attn_kernel<64, QG><<<grid, dim3(kThreads), 0, stream>>>(a); break;
    case 128: prefill_attn_kernel<128, QG><<<grid, dim3(kThreads), 0, stream>>>(a); break;
    case 256: prefill_attn_kernel<256, (QG > 2 ? 2 : QG)><<<grid, dim3(kThreads), 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
