// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vattn {

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* cu_q;
  const int32_t* cu_kv;
  uint16_t* out;
  float* lse;
  float* part_o;    // [B_max, Hq, nsplit, D] unnormalised partial outputs
  float4* part_ml;  // [B_max, Hq, nsplit] (m in log2 units, l, lt, unused): l sums the
                    // weights in fp32, lt as they entered P V (bf16 on the MFMA path)
  int32_t* err;
  int32_t* counters;  // [n_units] arrival counters of the fused merge (kept at 0 between launches)
  // Gathered keys (null: contiguous): key j of sequence b is K/V row
  // kv_idx[cu_kv[b] + j], clamped into [0, kv_bound); cu_kv then indexes the
  // list and kv_rows is the list's capacity.
  const int32_t* kv_idx;
  int64_t kv_bound;
  int B, Hq, Hkv, G, D;
  int head_blocks;  // workgroups per (b, hk) along the head dimension
  int nsplit, chunk_keys;
  int s_max_q, s_max_kv;
  int64_t q_rows, kv_rows;
  int64_t q_rs, k_rs, v_rs, o_rs;  // row (token) strides of q, k, v, out in elements
  float c;          // softmax scale * log2(e)
  int direct;       // 1: normalise and write out/lse; 0: write partials
  int fused;        // with direct == 0: 1 = last split workgroup merges, 0 = combine kernel
  int fused_local;  // fused merge with every split of a unit on one XCD: plain loads/stores
};

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* cu_q;
  const int32_t* cu_kv;
  uint16_t* out;
  float* lse;
  int32_t* err;
  // Live-tile list, entries (b << 16) | q_tile: the caller's host-built map
  // (exact-grid comparator, n_map entries, one workgroup per entry and KV
  // head) or the device-built schedule (sched_count != null: the entry count
  // is read on the device and a persistent grid strides over the list).
  const int32_t* tile_map;
  int n_map;
  const int32_t* sched_count;
  int B, B_max, Hq, Hkv, G;
  int tq;        // query tokens per workgroup (rows = G * tq)
  int n_qtiles;  // ceil(s_max_q / tq)
  int s_max_q, s_max_kv;
  int64_t q_rows, kv_rows;
  int64_t q_rs, k_rs, v_rs, o_rs;  // row (token) strides of q, k, v, out in elements
  float c;
  int causal;
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* out;
  const uint16_t* dout;
  const float* lse;
  const int32_t* cu_q;
  const int32_t* cu_kv;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;  // [B_max, s_max_q, Hq] row-wise <dO, O>, written by the dq kernel
  int32_t* err;
  int B, B_max, Hq, Hkv, G;
  int tq;        // dq kernel: query tokens per workgroup (rows = G * tq = 128)
  int n_qtiles;  // ceil(s_max_q / tq)
  int n_ktiles;  // dk/dv kernel: ceil(s_max_kv / 128)
  int s_max_q, s_max_kv;
  int64_t q_rows, kv_rows;
  // row (token) strides in elements
  int64_t q_rs, k_rs, v_rs, o_rs, do_rs, dq_rs, dk_rs, dv_rs;
  float c;       // scale * log2(e)
  float scale;
  int causal;
};

// ev0 / ev1 (may be null): measurement events stamped with the start / end
// of the split (or direct) kernel's dispatch; the combine kernel is not timed.
hipError_t launch_decode(const DecodeArgs& a, int path, int nw, int grid, int combine_grid,
                         hipStream_t st, hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
hipError_t launch_clear_words(int32_t* words, int n, hipStream_t st);
hipError_t launch_prefill(const PrefillArgs& a, int D, int grid, hipStream_t st,
                          hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);
// Builds the live-tile list of a prefill pass into list / *count (one
// workgroup); reads cu_seqlens_q (and cu_seqlens_kv, for the error word).
hipError_t launch_prefill_schedule(const PrefillArgs& a, int32_t* list, int32_t* count,
                                   hipStream_t st);
hipError_t launch_padding_mask(const int32_t* cu, int B, int max_seqlen, uint8_t* mask,
                               hipStream_t st);
hipError_t launch_cross_padding_mask(const int32_t* cu_q, const int32_t* cu_kv, int B,
                                     int max_q, int max_kv, uint8_t* mask_q, uint8_t* mask_kv,
                                     hipStream_t st);
hipError_t launch_clear_word(int32_t* word, hipStream_t st);
// dq kernel (grid_dq workgroups) then dk/dv kernel (grid_dkdv), both > 0;
// ev0 / ev1 (may be null) are stamped at the start of the first and the end
// of the second.
hipError_t launch_backward(const BwdArgs& a, int D, int grid_dq, int grid_dkdv, hipStream_t st,
                           hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr);

}  // namespace vattn
