// Internal: the state behind a vattn_plan_t, the layout of a plan's scratch
// memory, and the packed-layout enqueue path, shared by the plan-based entry
// points (api.cpp) and the entry point that works on static device memory
// (noalloc.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vattn.h"

struct vattn_plan_s {
  vattn_plan_info info;
  int device;
  uint8_t* scratch;  // error word | merge counters | (m, l) partials | O partials
  int32_t* err;
  int32_t* counters;
  float4* part_ml;
  float* part_o;
  int32_t* sched_count;  // prefill schedule: live-tile count, then the list
  int32_t* sched_list;
  float* delta;          // backward: [B_max, s_max_q, Hq] row-wise <dout, out>
  hipEvent_t ev_start, ev_stop;  // measurement hook (caller-owned), or null
};

namespace vattn {

// Bytes of scratch a plan with this info needs. With base != null, also
// points p's scratch sections into [base, base + size): error word at 0;
// decode merge counters, (m, l) pairs and O partials (split plans); for a
// scheduled prefill the live-tile count at 256 and the list from 512; the
// backward's row-wise <dout, out> buffer last. Sections are 256-byte aligned.
uint64_t scratch_layout(const vattn_plan_info& info, uint8_t* base, vattn_plan_s* p);

// Argument checks of vattn_execute, then its enqueue on packed tensors.
vattn_status execute_packed(vattn_plan_s* p, int B, const void* q, const void* k,
                            const void* v, const int32_t* cu_q, const int32_t* cu_kv, void* out,
                            float* lse, int64_t q_rows, int64_t kv_rows, vattn_stream_t stream);

}  // namespace vattn
