// C ABI of the library: plan creation (the only allocation), execute (enqueue
// only: no host read of device data, no allocation, no synchronisation), the
// padding mask, and plan queries. See include/vattn.h for the contract.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <cmath>
#include <new>

#include "../../include/vattn.h"
#include "launch.hpp"
#include "plan.hpp"
#include "plan_state.hpp"

namespace {

vattn_status device_cu_count(int* n_cu, int* dev) {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess) return VATTN_ERR_HIP;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess)
    return VATTN_ERR_HIP;
  *n_cu = n;
  if (dev) *dev = d;
  return VATTN_OK;
}

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline uintptr_t align_up(uintptr_t x, uintptr_t a) { return (x + a - 1) & ~(a - 1); }

}  // namespace

namespace vattn {

uint64_t scratch_layout(const vattn_plan_info& info, uint8_t* base, vattn_plan_s* p) {
  const uint64_t n_cnt = info.direct || !info.is_decode ? 0 : (uint64_t)info.n_units;
  const uint64_t off_cnt = 256;
  const uint64_t off_ml = align_up(off_cnt + n_cnt * sizeof(int32_t), 256);
  const uint64_t n_part =
      info.direct || !info.is_decode ? 0 : (uint64_t)info.B_max * info.Hq * info.nsplit;
  const uint64_t off_o = align_up(off_ml + n_part * sizeof(float4), 256);
  uint64_t total = off_o + n_part * (uint64_t)info.D * sizeof(float);
  if (info.prefill_persistent)
    total = 512 + (uint64_t)info.B_max * info.n_qtiles * sizeof(int32_t);
  const uint64_t off_delta = align_up(total, 256);
  if (info.backward)
    total = off_delta + (uint64_t)info.B_max * info.s_max_q * info.Hq * sizeof(float);
  if (base && p) {
    p->scratch = base;
    p->err = (int32_t*)base;
    p->counters = n_cnt ? (int32_t*)(base + off_cnt) : nullptr;
    p->part_ml = n_part ? (float4*)(base + off_ml) : nullptr;
    p->part_o = n_part ? (float*)(base + off_o) : nullptr;
    p->sched_count = info.prefill_persistent ? (int32_t*)(base + 256) : nullptr;
    p->sched_list = info.prefill_persistent ? (int32_t*)(base + 512) : nullptr;
    p->delta = info.backward ? (float*)(base + off_delta) : nullptr;
  }
  return total;
}

}  // namespace vattn

extern "C" {

const char* vattn_status_string(vattn_status s) {
  switch (s) {
    case VATTN_OK: return "ok";
    case VATTN_ERR_INVALID_ARG: return "invalid argument";
    case VATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case VATTN_ERR_HIP: return "HIP runtime error";
    case VATTN_ERR_OOM: return "out of device memory";
    case VATTN_ERR_TOO_LARGE:
      return "the plan's scratch exceeds the static array of vattn_execute_noalloc";
  }
  return "unknown status";
}

int vattn_abi_version(void) { return VATTN_ABI_VERSION; }

vattn_status vattn_plan_describe(int B_max, int s_max_q, int s_max_kv, int Hq, int Hkv, int D,
                                 int causal, const vattn_plan_opts* opts,
                                 vattn_plan_info* info) {
  int n_cu = (opts && opts->n_cu_override > 0) ? opts->n_cu_override : 0;
  if (n_cu == 0) {
    vattn_status st = device_cu_count(&n_cu, nullptr);
    if (st != VATTN_OK) return st;
  }
  return vattn::plan_compute(B_max, s_max_q, s_max_kv, Hq, Hkv, D, causal, opts, n_cu, info);
}

vattn_status vattn_plan_ex(vattn_plan_t* out, int B_max, int s_max_q, int s_max_kv, int Hq,
                           int Hkv, int D, int causal, const vattn_plan_opts* opts) {
  if (!out) return VATTN_ERR_INVALID_ARG;
  *out = nullptr;
  int n_cu = 0, dev = 0;
  vattn_status st = device_cu_count(&n_cu, &dev);
  if (st != VATTN_OK) return st;
  if (opts && opts->n_cu_override > 0) n_cu = opts->n_cu_override;
  vattn_plan_info info;
  st = vattn::plan_compute(B_max, s_max_q, s_max_kv, Hq, Hkv, D, causal, opts, n_cu, &info);
  if (st != VATTN_OK) return st;

  vattn_plan_s* p = new (std::nothrow) vattn_plan_s();
  if (!p) return VATTN_ERR_OOM;
  p->info = info;
  p->device = dev;
  const uint64_t total = vattn::scratch_layout(info, nullptr, nullptr);
  p->info.scratch_bytes = (long long)total;
  void* mem = nullptr;
  hipError_t e = hipMalloc(&mem, total);
  if (e != hipSuccess || !mem) {
    (void)hipGetLastError();
    delete p;
    return e == hipErrorOutOfMemory ? VATTN_ERR_OOM : VATTN_ERR_HIP;
  }
  vattn::scratch_layout(info, (uint8_t*)mem, p);
  const int n_cnt = p->counters ? info.n_units : 0;
  // plan creation may synchronise (it is not on the hot path): zero the
  // error word and the merge counters once with kernels, then wait for them.
  if (vattn::launch_clear_word(p->err, nullptr) != hipSuccess ||
      vattn::launch_clear_words(p->counters, n_cnt, nullptr) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(mem);
    delete p;
    return VATTN_ERR_HIP;
  }
  *out = p;
  return VATTN_OK;
}

vattn_status vattn_plan(vattn_plan_t* out, int B_max, int s_max_q, int s_max_kv, int Hq, int Hkv,
                        int D, int causal) {
  return vattn_plan_ex(out, B_max, s_max_q, s_max_kv, Hq, Hkv, D, causal, nullptr);
}

vattn_status vattn_plan_query(vattn_plan_t p, vattn_plan_info* info) {
  if (!p || !info) return VATTN_ERR_INVALID_ARG;
  *info = p->info;
  return VATTN_OK;
}

static vattn_status check_exec(vattn_plan_t p, int B, const void* q, const void* k, const void* v,
                               const int32_t* cu_q, const int32_t* cu_kv, void* out, float* lse,
                               int64_t q_rows, int64_t kv_rows) {
  if (!p) return VATTN_ERR_INVALID_ARG;
  if (B < 0 || B > p->info.B_max) return VATTN_ERR_INVALID_ARG;
  if (q_rows < 0 || kv_rows < 0) return VATTN_ERR_INVALID_ARG;
  if (q_rows > INT32_MAX || kv_rows > INT32_MAX) return VATTN_ERR_UNSUPPORTED;
  if (B == 0) return VATTN_OK;
  if (!q || !k || !v || !cu_q || !cu_kv || !out || !lse) return VATTN_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return VATTN_ERR_INVALID_ARG;
  if (!aligned(lse, 4) || !aligned(cu_q, 4) || !aligned(cu_kv, 4)) return VATTN_ERR_INVALID_ARG;
  return VATTN_OK;
}

// Row (token) strides in elements of q, k, v and out.
struct Strides {
  int64_t q, k, v, o;
};

static Strides packed_strides(const vattn_plan_info& in) {
  return Strides{(int64_t)in.Hq * in.D, (int64_t)in.Hkv * in.D, (int64_t)in.Hkv * in.D,
                 (int64_t)in.Hq * in.D};
}

// Gathered keys for decode: the index list and the K/V row count (null: none).
struct Gather {
  const int32_t* idx;
  int64_t bound;
};

static vattn_status run(vattn_plan_t p, int B, const void* q, const void* k, const void* v,
                        const int32_t* cu_q, const int32_t* cu_kv, void* out, float* lse,
                        int64_t q_rows, int64_t kv_rows, const int32_t* tile_map, int n_map,
                        const Strides& rs, vattn_stream_t stream,
                        const Gather& gather = Gather{nullptr, 0}) {
  const vattn_plan_info& in = p->info;
  const float c = (float)(1.0 / std::sqrt((double)in.D) * 1.4426950408889634);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (p->ev_start) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) return VATTN_ERR_HIP;
    if (cs != hipStreamCaptureStatusNone) return VATTN_ERR_INVALID_ARG;
  }
  if (in.is_decode) {
    vattn::DecodeArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.cu_q = cu_q;
    a.cu_kv = cu_kv;
    a.out = (uint16_t*)out;
    a.lse = lse;
    a.part_o = p->part_o;
    a.part_ml = p->part_ml;
    a.err = p->err;
    a.counters = p->counters;
    a.B = B;
    a.Hq = in.Hq;
    a.Hkv = in.Hkv;
    a.G = in.Hq / in.Hkv;
    a.D = in.D;
    a.head_blocks = in.head_blocks;
    a.nsplit = in.nsplit;
    a.chunk_keys = in.chunk_keys;
    a.s_max_q = in.s_max_q;
    a.s_max_kv = in.s_max_kv;
    a.q_rows = q_rows;
    a.kv_rows = kv_rows;
    a.q_rs = rs.q;
    a.k_rs = rs.k;
    a.v_rs = rs.v;
    a.o_rs = rs.o;
    a.c = c;
    a.direct = in.direct;
    a.fused = in.fused_combine;
    // the split-major grid puts unit u's splits on XCD u % 8 when the unit
    // count is a multiple of the 8 XCDs (workgroups go round-robin to XCDs)
    a.fused_local = in.fused_combine && (in.n_units % 8 == 0) ? 1 : 0;
    a.kv_idx = gather.idx;
    a.kv_bound = gather.bound;
    int combine_grid = in.combine_grid;
    if (gather.idx && in.fused_combine) {  // gathered keys merge in the combine kernel
      a.fused = 0;
      const int heads = in.D == 256 ? 1 : 2;  // query heads per combine workgroup
      combine_grid = in.B_max * ((in.Hq + heads - 1) / heads);
    }
    e = vattn::launch_decode(a, in.decode_path, in.threads / 64, in.grid, combine_grid,
                             st, p->ev_start, p->ev_stop);
  } else {
    // the prefill kernel addresses a K or V tile with 32-bit offsets from
    // its first row: rows below 2^25 elements apart
    if (rs.k >= (int64_t(1) << 25) || rs.v >= (int64_t(1) << 25)) return VATTN_ERR_INVALID_ARG;
    vattn::PrefillArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.cu_q = cu_q;
    a.cu_kv = cu_kv;
    a.out = (uint16_t*)out;
    a.lse = lse;
    a.err = p->err;
    a.tile_map = tile_map;
    a.n_map = n_map;
    a.sched_count = nullptr;
    a.B = B;
    a.B_max = in.B_max;
    a.Hq = in.Hq;
    a.Hkv = in.Hkv;
    a.G = in.Hq / in.Hkv;
    a.tq = in.q_tokens_per_tile;
    a.n_qtiles = in.n_qtiles;
    a.s_max_q = in.s_max_q;
    a.s_max_kv = in.s_max_kv;
    a.q_rows = q_rows;
    a.kv_rows = kv_rows;
    a.q_rs = rs.q;
    a.k_rs = rs.k;
    a.v_rs = rs.v;
    a.o_rs = rs.o;
    a.c = c;
    a.causal = in.causal;
    const int64_t grid = tile_map ? (int64_t)n_map * in.Hkv : in.grid;
    if (grid == 0) return VATTN_OK;
    if (grid > INT32_MAX) return VATTN_ERR_UNSUPPORTED;
    if (!tile_map && in.prefill_persistent) {
      // the schedule kernel lists the live tiles; the persistent grid walks them
      e = vattn::launch_prefill_schedule(a, p->sched_list, p->sched_count, st);
      if (e != hipSuccess) return VATTN_ERR_HIP;
      a.tile_map = p->sched_list;
      a.sched_count = p->sched_count;
    }
    e = vattn::launch_prefill(a, in.D, (int)grid, st, p->ev_start, p->ev_stop);
  }
  return e == hipSuccess ? VATTN_OK : VATTN_ERR_HIP;
}

}  // extern "C"

vattn_status vattn::execute_packed(vattn_plan_s* p, int B, const void* q, const void* k,
                                   const void* v, const int32_t* cu_q, const int32_t* cu_kv,
                                   void* out, float* lse, int64_t q_rows, int64_t kv_rows,
                                   vattn_stream_t stream) {
  vattn_status st = check_exec(p, B, q, k, v, cu_q, cu_kv, out, lse, q_rows, kv_rows);
  if (st != VATTN_OK || B == 0) return st;
  return run(p, B, q, k, v, cu_q, cu_kv, out, lse, q_rows, kv_rows, nullptr, 0,
             packed_strides(p->info), stream);
}

extern "C" {

vattn_status vattn_execute(vattn_plan_t p, int B, const void* q, const void* k, const void* v,
                           const int32_t* cu_q, const int32_t* cu_kv, void* out, float* lse,
                           int64_t q_rows, int64_t kv_rows, vattn_stream_t stream) {
  return vattn::execute_packed(p, B, q, k, v, cu_q, cu_kv, out, lse, q_rows, kv_rows, stream);
}

vattn_status vattn_execute_gathered(vattn_plan_t p, int B, const void* q, const void* k,
                                    const void* v, const int32_t* cu_q, const int32_t* cu_idx,
                                    const int32_t* kv_idx, void* out, float* lse, int64_t q_rows,
                                    int64_t kv_rows, int64_t n_idx, vattn_stream_t stream) {
  // row-capacity checks apply to q (q_rows) and to the index list (n_idx)
  vattn_status st = check_exec(p, B, q, k, v, cu_q, cu_idx, out, lse, q_rows, n_idx);
  if (st != VATTN_OK) return st;
  if (!p->info.is_decode) return VATTN_ERR_UNSUPPORTED;
  if (kv_rows < 1 || kv_rows > INT32_MAX) return VATTN_ERR_INVALID_ARG;
  if (B == 0) return VATTN_OK;
  if (!kv_idx || !aligned(kv_idx, 4)) return VATTN_ERR_INVALID_ARG;
  return run(p, B, q, k, v, cu_q, cu_idx, out, lse, q_rows, n_idx, nullptr, 0,
             packed_strides(p->info), stream, Gather{kv_idx, kv_rows});
}

vattn_status vattn_execute_strided(vattn_plan_t p, int B, const void* q, int64_t q_row_stride,
                                   const void* k, int64_t k_row_stride, const void* v,
                                   int64_t v_row_stride, const int32_t* cu_q,
                                   const int32_t* cu_kv, void* out, int64_t out_row_stride,
                                   float* lse, int64_t q_rows, int64_t kv_rows,
                                   vattn_stream_t stream) {
  vattn_status st = check_exec(p, B, q, k, v, cu_q, cu_kv, out, lse, q_rows, kv_rows);
  if (st != VATTN_OK) return st;
  const vattn_plan_info& in = p->info;
  const Strides packed = packed_strides(in);
  const Strides rs{q_row_stride ? q_row_stride : packed.q, k_row_stride ? k_row_stride : packed.k,
                   v_row_stride ? v_row_stride : packed.v,
                   out_row_stride ? out_row_stride : packed.o};
  // every row holds its heads contiguously (head stride D); rows keep the
  // 16-byte alignment of the base pointers and do not overlap
  if (rs.q < packed.q || rs.k < packed.k || rs.v < packed.v || rs.o < packed.o)
    return VATTN_ERR_INVALID_ARG;
  if ((rs.q | rs.k | rs.v | rs.o) & 7) return VATTN_ERR_INVALID_ARG;
  if (B == 0) return VATTN_OK;
  return run(p, B, q, k, v, cu_q, cu_kv, out, lse, q_rows, kv_rows, nullptr, 0, rs, stream);
}

vattn_status vattn_execute_exact_grid(vattn_plan_t p, int B, const void* q, const void* k,
                                      const void* v, const int32_t* cu_q, const int32_t* cu_kv,
                                      void* out, float* lse, int64_t q_rows, int64_t kv_rows,
                                      const int32_t* tile_map, int n_tiles,
                                      vattn_stream_t stream) {
  vattn_status st = check_exec(p, B, q, k, v, cu_q, cu_kv, out, lse, q_rows, kv_rows);
  if (st != VATTN_OK) return st;
  if (p->info.is_decode) return VATTN_ERR_UNSUPPORTED;
  if (n_tiles < 0 || (n_tiles > 0 && !tile_map) || !aligned(tile_map, 4))
    return VATTN_ERR_INVALID_ARG;
  if (B == 0 || n_tiles == 0) return VATTN_OK;
  return run(p, B, q, k, v, cu_q, cu_kv, out, lse, q_rows, kv_rows, tile_map, n_tiles,
             packed_strides(p->info), stream);
}

vattn_status vattn_backward(vattn_plan_t p, int B, const void* q, int64_t q_row_stride,
                            const void* k, int64_t k_row_stride, const void* v,
                            int64_t v_row_stride, const void* out, int64_t out_row_stride,
                            const void* dout, int64_t dout_row_stride, const float* lse,
                            const int32_t* cu_q, const int32_t* cu_kv, void* dq,
                            int64_t dq_row_stride, void* dk, int64_t dk_row_stride, void* dv,
                            int64_t dv_row_stride, int64_t q_rows, int64_t kv_rows,
                            vattn_stream_t stream) {
  if (!p) return VATTN_ERR_INVALID_ARG;
  if (!p->info.backward) return VATTN_ERR_UNSUPPORTED;
  vattn_status st =
      check_exec(p, B, q, k, v, cu_q, cu_kv, const_cast<void*>(out), const_cast<float*>(lse),
                 q_rows, kv_rows);
  if (st != VATTN_OK) return st;
  const vattn_plan_info& in = p->info;
  const int64_t pq = (int64_t)in.Hq * in.D, pk = (int64_t)in.Hkv * in.D;
  const int64_t rs[8] = {q_row_stride,   k_row_stride,  v_row_stride,  out_row_stride,
                         dout_row_stride, dq_row_stride, dk_row_stride, dv_row_stride};
  const int64_t packed[8] = {pq, pk, pk, pq, pq, pq, pk, pk};
  int64_t r[8];
  for (int i = 0; i < 8; ++i) {
    r[i] = rs[i] ? rs[i] : packed[i];
    // the dk/dv kernel forms in-step row offsets with 24-bit multiplies
    if (r[i] < packed[i] || (r[i] & 7) || r[i] >= (int64_t(1) << 24)) return VATTN_ERR_INVALID_ARG;
  }
  if (B == 0) return VATTN_OK;
  if (!dout || !dq || !dk || !dv) return VATTN_ERR_INVALID_ARG;
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return VATTN_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  if (p->ev_start) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(hs, &cs) != hipSuccess) return VATTN_ERR_HIP;
    if (cs != hipStreamCaptureStatusNone) return VATTN_ERR_INVALID_ARG;
  }
  vattn::BwdArgs a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.out = (const uint16_t*)out;
  a.dout = (const uint16_t*)dout;
  a.lse = lse;
  a.cu_q = cu_q;
  a.cu_kv = cu_kv;
  a.dq = (uint16_t*)dq;
  a.dk = (uint16_t*)dk;
  a.dv = (uint16_t*)dv;
  a.delta = p->delta;
  a.err = p->err;
  a.B = B;
  a.B_max = in.B_max;
  a.Hq = in.Hq;
  a.Hkv = in.Hkv;
  a.G = in.Hq / in.Hkv;
  a.tq = in.bwd_q_tokens_per_tile;
  a.n_qtiles = (in.s_max_q + a.tq - 1) / a.tq;
  a.n_ktiles = (in.s_max_kv + vattn::kBwdKeys - 1) / vattn::kBwdKeys;
  a.s_max_q = in.s_max_q;
  a.s_max_kv = in.s_max_kv;
  a.q_rows = q_rows;
  a.kv_rows = kv_rows;
  a.q_rs = r[0];
  a.k_rs = r[1];
  a.v_rs = r[2];
  a.o_rs = r[3];
  a.do_rs = r[4];
  a.dq_rs = r[5];
  a.dk_rs = r[6];
  a.dv_rs = r[7];
  a.scale = (float)(1.0 / std::sqrt((double)in.D));
  a.c = (float)(1.0 / std::sqrt((double)in.D) * 1.4426950408889634);
  a.causal = in.causal;
  hipError_t e = vattn::launch_backward(a, in.D, in.bwd_grid_dq, in.bwd_grid_dkdv, hs,
                                        p->ev_start, p->ev_stop);
  return e == hipSuccess ? VATTN_OK : VATTN_ERR_HIP;
}

vattn_status vattn_padding_mask(const int32_t* cu_seqlens, int B, int max_seqlen, uint8_t* mask,
                                vattn_stream_t stream) {
  if (B < 0 || max_seqlen < 0) return VATTN_ERR_INVALID_ARG;
  if (B == 0 || max_seqlen == 0) return VATTN_OK;
  if (!cu_seqlens || !mask || !aligned(cu_seqlens, 4)) return VATTN_ERR_INVALID_ARG;
  hipError_t e = vattn::launch_padding_mask(cu_seqlens, B, max_seqlen, mask, (hipStream_t)stream);
  return e == hipSuccess ? VATTN_OK : VATTN_ERR_HIP;
}

vattn_status vattn_plan_set_kernel_events(vattn_plan_t p, void* start, void* stop) {
  if (!p || (!start) != (!stop)) return VATTN_ERR_INVALID_ARG;
  p->ev_start = (hipEvent_t)start;
  p->ev_stop = (hipEvent_t)stop;
  return VATTN_OK;
}

vattn_status vattn_cross_padding_mask(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                      int B, int max_seqlen_q, int max_seqlen_kv,
                                      uint8_t* mask_q, uint8_t* mask_kv, vattn_stream_t stream) {
  if (B < 0 || max_seqlen_q < 0 || max_seqlen_kv < 0) return VATTN_ERR_INVALID_ARG;
  if (B == 0 || (max_seqlen_q == 0 && max_seqlen_kv == 0)) return VATTN_OK;
  if (!cu_seqlens_q || !cu_seqlens_kv || !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_kv, 4))
    return VATTN_ERR_INVALID_ARG;
  if ((max_seqlen_q > 0 && !mask_q) || (max_seqlen_kv > 0 && !mask_kv))
    return VATTN_ERR_INVALID_ARG;
  hipError_t e = vattn::launch_cross_padding_mask(cu_seqlens_q, cu_seqlens_kv, B, max_seqlen_q,
                                                  max_seqlen_kv, mask_q, mask_kv,
                                                  (hipStream_t)stream);
  return e == hipSuccess ? VATTN_OK : VATTN_ERR_HIP;
}

const int32_t* vattn_plan_error_word(vattn_plan_t p) { return p ? p->err : nullptr; }

vattn_status vattn_plan_read_error(vattn_plan_t p, int32_t* value) {
  if (!p || !value) return VATTN_ERR_INVALID_ARG;
  if (hipDeviceSynchronize() != hipSuccess) return VATTN_ERR_HIP;
  if (hipMemcpy(value, p->err, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
    return VATTN_ERR_HIP;
  return VATTN_OK;
}

vattn_status vattn_plan_clear_error(vattn_plan_t p, vattn_stream_t stream) {
  if (!p) return VATTN_ERR_INVALID_ARG;
  return vattn::launch_clear_word(p->err, (hipStream_t)stream) == hipSuccess ? VATTN_OK
                                                                              : VATTN_ERR_HIP;
}

void vattn_plan_destroy(vattn_plan_t p) {
  if (!p) return;
  if (p->scratch) (void)hipFree(p->scratch);
  delete p;
}

}  // extern "C"
