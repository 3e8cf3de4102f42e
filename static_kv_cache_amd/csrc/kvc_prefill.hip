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
//  - Keys go in tiles of 32 rows, staged row-major in LDS (skewed rows) by
//    the whole workgroup, with the next tile in flight in registers. (Two
//    or four query groups of 16 per wave, or two to four tiles in flight,
//    measured slower at a 4096-token prompt: fewer workgroups for the causal
//    load balance and lower occupancy cost more than the LDS reads and load
//    latency they save.)
//  - Scores: S[key][query] on v_mfma_f32_16x16x32_bf16, 16 keys (A, from LDS)
//    against the wave's 16 queries (B, in registers), per 16-key block.
//    Causal mask per (key, query). fp32 online softmax in log2 units with a
//    lazily moved reference maximum per query column.
//  - p.v on v_mfma_f32_16x16x16_bf16 with V read back transposed from LDS by
//    ds_read_b64_tr_b16; each wave keeps its own (o, m, l), so no cross-wave
//    merge: the output rows are normalised and written by the wave.
//  - Blocks whose keys all lie past a wave's last query are skipped by that
//    wave; the query blocks with the most keys are launched first, for every
//    head group.

#include "kvc_device.h"

namespace {

using namespace kvcd;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeys = 32;                 // keys per tile
constexpr float kLazy = 64.0f;            // log2 headroom before the reference maximum moves
constexpr int kQueryGroups = 1;           // query groups of 16 per wave (1 measured best)
constexpr int kTilesInFlight = 1;         // K/V tiles in flight in registers (1 measured best)

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
  static constexpr int KSTRIDE = 2 * D + 16;        // bytes per staged K row
  static constexpr int VSTRIDE = 2 * D + 32;        // bytes per staged V row
  static constexpr int VEC = kKeys * 2 * D / 16 / kThreads;  // 16-byte vectors per thread per tile (K, and V)
  static_assert(VEC >= 1 && kKeys * 2 * D % (16 * kThreads) == 0, "tile must split evenly");
};

template <int D, int QG>
__global__ __launch_bounds__(kThreads) void prefill_attn_kernel(PrefillArgs a) {
  using P = Prefill<D>;
  __shared__ __attribute__((aligned(16))) unsigned char ks[kKeys * P::KSTRIDE];
  __shared__ __attribute__((aligned(16))) unsigned char vsm[kKeys * P::VSTRIDE];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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
  const __amdgpu_buffer_rsrc_t kres = buffer_rsrc(a.k + row0 * D, rows * (2 * D));
  const __amdgpu_buffer_rsrc_t vres = buffer_rsrc(a.v + row0 * D, rows * (2 * D));

  // the wave's QG x 16 queries as B operands: column j of group qg is position p0 + 16 qg + j
  bf16x8_t qv[QG][P::KS];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const int pos = p0 + 16 * qg + j;
    const bool real = pos < a.t;
    const uint16_t* qh = a.q + (((size_t)b * a.n_heads + h) * a.t + (real ? pos : 0)) * D + 8 * g;
#pragma unroll
    for (int k = 0; k < P::KS; ++k) {
      u32x4_t x = *reinterpret_cast<const u32x4_t*>(qh + 32 * k);
      x = real ? x : u32x4_t{0u, 0u, 0u, 0u};
      qv[qg][k] = __builtin_bit_cast(bf16x8_t, x);
    }
  }

  f32x4_t o[QG][P::NB];
  float m[QG], l[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
#pragma unroll
    for (int nb = 0; nb < P::NB; ++nb) o[qg][nb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m[qg] = -INFINITY;
    l[qg] = 0.0f;
  }
  const float scale_log2 = a.scale_log2;

  // tile staging: thread t moves 16-byte vectors t + 256 i of the K and V
  // tiles; a ring of NPF register tiles keeps the next NPF tiles in flight
  constexpr int NPF = kTilesInFlight;
  u32x4_t kr[NPF][P::VEC], vr[NPF][P::VEC];
  auto load = [&](int k0, u32x4_t (&kd)[P::VEC], u32x4_t (&vd)[P::VEC]) {
#pragma unroll
    for (int i = 0; i < P::VEC; ++i) {
      const int f = (int)threadIdx.x + i * kThreads;
      kd[i] = __builtin_amdgcn_raw_buffer_load_b128(kres, k0 * (2 * D) + f * 16, 0, 0);
      vd[i] = __builtin_amdgcn_raw_buffer_load_b128(vres, k0 * (2 * D) + f * 16, 0, 0);
    }
  };
  auto stage = [&](const u32x4_t (&kd)[P::VEC], const u32x4_t (&vd)[P::VEC]) {
#pragma unroll
    for (int i = 0; i < P::VEC; ++i) {
      const int f = (int)threadIdx.x + i * kThreads;
      const int r = f / (D / 8), c = f % (D / 8);
      *reinterpret_cast<u32x4_t*>(ks + r * P::KSTRIDE + c * 16) = kd[i];
      *reinterpret_cast<u32x4_t*>(vsm + r * P::VSTRIDE + c * 16) = vd[i];
    }
  };

#pragma unroll
  for (int s = 0; s < NPF; ++s) load(kKeys * s, kr[s], vr[s]);  // loads past the rows read zeros
  for (int kbase = 0; kbase < kend; kbase += NPF * kKeys) {
#pragma unroll
  for (int s = 0; s < NPF; ++s) {
    const int k0 = kbase + kKeys * s;
    if (k0 >= kend) break;
    __syncthreads();  // every wave is done with the previous tile
    stage(kr[s], vr[s]);
    if (k0 + NPF * kKeys < kend) load(k0 + NPF * kKeys, kr[s], vr[s]);
    __syncthreads();  // the tile is visible
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int kb0 = k0 + 16 * blk;
      if (kb0 > a.start + p0 + 16 * QG - 1) continue;  // all keys past this wave's queries
      // the block's 16 keys as A operands, read from LDS once for all query groups
      const unsigned char* arow = ks + (16 * blk + j) * P::KSTRIDE + 16 * g;
      bf16x8_t av[P::KS];
#pragma unroll
      for (int k = 0; k < P::KS; ++k) av[k] = *reinterpret_cast<const bf16x8_t*>(arow + 64 * k);
      s16x4_t pa[QG];
      bool live[QG];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        const int qp0 = a.start + p0 + 16 * qg;  // first absolute position of the group
        live[qg] = kb0 <= qp0 + 15;               // uniform: some key of the block is visible to the group
        if (!live[qg]) continue;
        f32x4_t sc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < P::KS; ++k) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[k], qv[qg][k], sc, 0, 0, 0);
        if (kb0 + 15 > qp0) {  // the block reaches past some query of the group: causal mask
#pragma unroll
          for (int u = 0; u < 4; ++u) sc[u] = (kb0 + 4 * g + u <= qp0 + j) ? sc[u] : -INFINITY;
        }
        const float cand = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])) * scale_log2;
        if (__builtin_amdgcn_ballot_w64(cand > m[qg] + kLazy)) {
          float mt = fmaxf(cand, __shfl_xor(cand, 16));
          mt = fmaxf(mt, __shfl_xor(mt, 32));
          const float mn = fmaxf(m[qg], mt);
          const float c = __builtin_amdgcn_exp2f(m[qg] - ((mn == -INFINITY) ? 0.0f : mn));
          l[qg] *= c;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float cu = __shfl(c, 4 * g + u);  // factor of output row (query) 4g + u
#pragma unroll
            for (int nb = 0; nb < P::NB; ++nb) o[qg][nb][u] *= cu;
          }
          m[qg] = mn;
        }
        const float nm = (m[qg] == -INFINITY) ? 0.0f : -m[qg];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          // the denominator sums the bf16 weights that enter the product
          const __bf16 pb = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[u], scale_log2, nm));
          l[qg] += (float)pb;
          pa[qg][u] = __builtin_bit_cast(short, pb);
        }
      }
      // p.v: B operand = V[kb0 + 4g + u][16 nb + j] by one transpose read, shared by the groups
      const unsigned char* vrow = vsm + (16 * blk + 4 * g + (j >> 2)) * P::VSTRIDE + 8 * (j & 3);
#pragma unroll
      for (int nb = 0; nb < P::NB; ++nb) {
        const s16x4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(vrow + 32 * nb));
#pragma unroll
        for (int qg = 0; qg < QG; ++qg)
          if (live[qg]) o[qg][nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa[qg], vb, o[qg][nb], 0, 0, 0);
      }
    }
  }
  }

  // normalise and write: lane (g, j) holds output rows (queries) 4g + u, columns 16 nb + j
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    float lq = l[qg];
    lq += __shfl_xor(lq, 16);
    lq += __shfl_xor(lq, 32);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int qi = p0 + 16 * qg + 4 * g + u;
      const float lr = __shfl(lq, 4 * g + u);
      if (qi < a.t) {
        uint16_t* dst = a.out + (((size_t)b * a.n_heads + h) * a.t + qi) * D + j;
        const float inv = 1.0f / lr;  // lr >= 1: the query attends at least its own key
#pragma unroll
        for (int nb = 0; nb < P::NB; ++nb) dst[16 * nb] = bf16_rne(o[qg][nb][u] * inv);
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
