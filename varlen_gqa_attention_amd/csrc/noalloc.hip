// vattn_execute_noalloc: one attention pass with no allocation at all, for
// callers that cannot allocate device memory (code under graph capture that
// must not call hipMalloc, tight serving loops, harnesses that forbid it).
//
// The plan is computed on the host for each call (the same chooser as
// vattn_plan, default options, no device call beyond reading the CU count),
// and the plan's scratch (error word, merge counters, split partials) lives
// in `scratch`, a file-scope device array of fixed size. Each GPU holds its
// own copy of the array for the life of the process; its device address is
// looked up once per device (hipGetSymbolAddress) and only that address is
// ever handed to kernels. Every call on a GPU shares that GPU's array, so
// calls that overlap on one GPU (two streams, or two host threads) race on
// it. The split kernel writes every partial slot the merge reads in the same
// call; the merge counters of the in-kernel merge (which the default plan
// selects when all split workgroups fit the device at once: at most 256
// units, 1 KiB of counters) must be zero when a call starts: the array is
// zero when the code object is loaded, the first call on a device also
// clears the error word and counters with a kernel (unless its stream is
// being captured), and every merge resets the counters it used.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/vattn.h"
#include "launch.hpp"
#include "plan.hpp"
#include "plan_state.hpp"

namespace {

constexpr uint64_t kScratchBytes = VATTN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_mu;
uint8_t* g_ptr[kMaxDevices];  // device address of `scratch` per device (null: not looked up)

constexpr int kClearWords = 1024;  // error word + merge counters of any plan that uses them

// Device address of this device's `scratch`, looked up on first use with the
// device current (then, if `st` is not capturing, its first words are
// cleared on `st`). Returns null on failure.
uint8_t* scratch_ptr(int dev, hipStream_t st) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) return nullptr;
    if (cs == hipStreamCaptureStatusNone &&
        vattn::launch_clear_words(static_cast<int32_t*>(ptr), kClearWords, st) != hipSuccess)
      return nullptr;
    g_ptr[dev] = static_cast<uint8_t*>(ptr);
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" vattn_status vattn_execute_noalloc(int B_max, int s_max_q, int s_max_kv, int Hq,
                                              int Hkv, int D, int causal, int B, const void* q,
                                              const void* k, const void* v,
                                              const int32_t* cu_seqlens_q,
                                              const int32_t* cu_seqlens_kv, void* out, float* lse,
                                              int64_t q_rows, int64_t kv_rows, int32_t* err_word,
                                              vattn_stream_t stream) {
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return VATTN_ERR_HIP;
  if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return VATTN_ERR_HIP;
  vattn_plan_s p = {};
  vattn_status st =
      vattn::plan_compute(B_max, s_max_q, s_max_kv, Hq, Hkv, D, causal, nullptr, n_cu, &p.info);
  if (st != VATTN_OK) return st;
  const uint64_t need = vattn::scratch_layout(p.info, nullptr, nullptr);
  if (need > kScratchBytes) return VATTN_ERR_TOO_LARGE;
  if (err_word && ((uintptr_t)err_word & 3)) return VATTN_ERR_INVALID_ARG;
  uint8_t* base = scratch_ptr(dev, (hipStream_t)stream);
  if (!base) return VATTN_ERR_HIP;
  p.device = dev;
  p.info.scratch_bytes = (long long)need;
  vattn::scratch_layout(p.info, base, &p);
  if (err_word) p.err = err_word;  // else flags go to the array's own (unread) word
  return vattn::execute_packed(&p, B, q, k, v, cu_seqlens_q, cu_seqlens_kv, out, lse, q_rows,
                               kv_rows, stream);
}
