// Internal declarations shared by the host library and the kernels of
// libkvc.so. Nothing here is part of the C ABI (include/kvc.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc.h"

// Largest batch the attention kernels accept (their prefix sums of the
// valid lengths live in LDS).
#define KVC_MAX_BATCH 2048
// Most persistent workgroups per CU the workspace is sized for.
#define KVC_MAX_WG_PER_CU 8

struct kvc_cache {
  kvc_desc d;
  int device;
  int num_cus;
  uint8_t* base;          // cache region (one allocation, lives until kvc_free)
  bool owns_base;
  uint64_t bytes;         // physical bytes of the region
  int elem;               // bytes per stored element (4 fp32, 2 bf16, 1 int8)
  uint64_t layer_bytes;   // bytes per layer (K and V together for GQA)
  uint64_t kv_bytes;      // offset of V from K inside a layer (GQA)
  int row_elems;          // elements per cached row: head_dim (GQA) or d_c + d_R (MLA)
  uint64_t scale_layer_bytes;  // int8: bytes of one layer's K and V scales (0 otherwise)
  uint64_t scale_kv_bytes;     // int8: offset of the V scales from the K scales in a layer
  uint8_t* scales;        // int8: [L][2][B][H_kv][S] float32 scales (after the codes), else NULL
  int32_t* ws_map;        // [B][2]: rows and first image row of each sequence's run (prefix save/load)
  int32_t* ws_plan;       // decode plan cache: KVC_PLAN_HEAD ints, then KVC_PLAN_INTS per workgroup
  int32_t* ws_seg;        // latent cache: [B][head chunks][2] first workgroup and pieces of each segment
  bool paged;             // block-table cache: layer = [K|V][num_blocks][H_kv][block_size][d_h]
  int block_size, block_shift, num_blocks, table_width;  // table_width = max_context / block_size

  // fixed workspace (allocated once by kvc_alloc)
  int max_workgroups;     // num_cus * KVC_MAX_WG_PER_CU
  uint64_t ws_entries;    // partial entries: (max_workgroups + batch * n_heads) * 16
  float* ws_acc;          // [entry][acc_width] unnormalised partial outputs
  float* ws_ml;           // [entry][2]  (reference maximum in log2 units, sum)
  int32_t* ws_cnt;        // [batch * n_heads] per-segment arrival counters (zeroed once, self-resetting)
  uint16_t* ws_qabs;      // MLA: absorbed queries [B][H][d_c + d_R] (bf16)
  uint16_t* ws_olat;      // MLA: latent outputs   [B][H][d_c] (bf16)
  int32_t* err_flag;      // sticky device-range flag
  int32_t workgroups_forced;  // 0 = as many as the chip keeps resident
  bool sync_check;        // KVC_SYNC_CHECK=1
};

// ---- launchers (defined in the kernel translation units) -------------------

// Row copy into the cache: for each (b, g) of B*H_kv row groups, rows
// [start_b, start_b + t) get src[b][g][0..t). start_b = dev_start ?
// dev_start[b] : host_start. Sequences out of range are skipped and raise
// *err_flag. row_bytes must be a multiple of 16.
hipError_t kvc_launch_copy_rows(const void* src_k, const void* src_v, uint8_t* dst_k, uint8_t* dst_v,
                                int batch, int n_kv_heads, int t, int row_bytes, int max_context,
                                const int32_t* dev_start, int host_start, int32_t* err_flag,
                                hipStream_t stream);

// Decode plan cache (kvc_decode.hip): header [valid, grid, min rows, batch,
// arrival count, 0, 0, 0], the KVC_MAX_BATCH lengths the plan was made for,
// then one entry of KVC_PLAN_INTS ints per workgroup.
#define KVC_PLAN_LENS 8
#define KVC_PLAN_HEAD (KVC_PLAN_LENS + KVC_MAX_BATCH)
#define KVC_PLAN_INTS 64

// Largest block table slice one decode piece keeps in LDS (blocks per sequence).
#define KVC_MAX_TABLE 4096

// Row copy into a paged cache: rows [start_b, start_b + t) of sequence b
// through table[b] (table_width entries per sequence); a sequence whose rows
// leave [0, max_context) or reach an entry outside [0, num_blocks) is skipped
// and raises *err_flag.
hipError_t kvc_launch_paged_rows(const void* src_k, const void* src_v, uint8_t* pool_k, uint8_t* pool_v,
                                 const int32_t* table, int batch, int n_kv_heads, int t, int row_bytes,
                                 int block_shift, int num_blocks, int table_width, int max_context,
                                 const int32_t* dev_start, int32_t* err_flag, hipStream_t stream);

// Live-prefix copy between the cache and an image payload (save: cache ->
// image, load: image -> cache). map[2b] rows of sequence b (<= 0: nothing),
// starting at image row map[2b + 1] of each (layer, K|V) section of
// total_rows * n_kv_heads rows. unit_bytes is 16 (rows) or 4 (int8 scales).
hipError_t kvc_launch_prefix_copy(uint8_t* cache, uint8_t* image, const int32_t* map, bool save,
                                  uint64_t layer_bytes, uint64_t kv_bytes, int n_layers, int kv_parts, int batch,
                                  int max_batch_rows, int groups, int max_context, int row_bytes, int unit_bytes,
                                  int64_t total_rows, hipStream_t stream);

// Quantising row copy into an int8 cache: as kvc_launch_copy_rows for bf16
// source rows [B][H_kv][t][d] (d = head_dim), writing each row's int8 codes
// to dst_k / dst_v ([B][H_kv][S][d]) and its float32 scale to ks / vs
// ([B][H_kv][S]).
hipError_t kvc_launch_quant_rows(const void* src_k, const void* src_v, uint8_t* dst_k, uint8_t* dst_v,
                                 float* ks, float* vs, int batch, int n_kv_heads, int t, int head_dim,
                                 int max_context, const int32_t* dev_start, int host_start,
                                 int32_t* err_flag, hipStream_t stream);

// Persistent split-context GQA decode (pieces merged in the same kernel).
// With k_new / v_new (and valid_lens null) the launch also appends the new
// row at cache_index and attends it from k_new / v_new (not for int8). On an
// int8 cache k_scale / v_scale are the layer's row scales.
hipError_t kvc_launch_gqa_decode(const kvc_cache* c, const void* k_layer, const void* v_layer,
                                 const void* q, void* out, const int32_t* valid_lens,
                                 const int32_t* cache_index, float sm_scale, hipStream_t stream,
                                 const void* k_new = nullptr, const void* v_new = nullptr,
                                 const float* k_scale = nullptr, const float* v_scale = nullptr,
                                 const int32_t* block_table = nullptr);

// Causal prefill attention of a chunk [start, start + t) whose rows are
// already in the cache (bf16 GQA): q, out = [B][H][t][D].
hipError_t kvc_launch_prefill_attn(const kvc_cache* c, const void* k_layer, const void* v_layer, const void* q,
                                   void* out, int start, int t, float sm_scale, hipStream_t stream);

// Latent (MLA) decode over absorbed queries q_abs [B][H][d_c + d_R] (bf16)
// into out_lat [B][H][d_c] (bf16).
hipError_t kvc_launch_mla_attn(const kvc_cache* c, const void* rows_layer, const void* q_abs,
                               void* out_lat, const int32_t* valid_lens, const int32_t* cache_index,
                               float sm_scale, hipStream_t stream);

// MLA query absorption q~ = [W_UK^T q_nope ; q_rope] and output up-projection
// out = W_UV^T o~ (bf16 in/out, fp32 accumulation).
hipError_t kvc_launch_mla_absorb(const kvc_cache* c, const void* q_nope, const void* q_rope,
                                 const void* w_uk, uint16_t* q_abs, hipStream_t stream);
hipError_t kvc_launch_mla_uproj(const kvc_cache* c, const uint16_t* o_lat, const void* w_uv,
                                void* out, hipStream_t stream);
