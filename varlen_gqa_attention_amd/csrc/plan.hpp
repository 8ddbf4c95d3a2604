// Plan-time chooser: pure host arithmetic, no HIP calls (unit-testable on a
// machine without a GPU).
#pragma once
#include "../../include/vattn.h"

namespace vattn {

// Geometry fixed by the kernels.
constexpr int kDecodeBlockN = 64;     // decode KV tile used by the split rule (keys)
constexpr int kDecodeMfmaHeads = 16;  // heads per workgroup on the MFMA decode path
constexpr int kDecodeWaveHeads = 4;   // heads per workgroup on the wave decode path
constexpr int kWaveMaxG = 3;          // auto: G <= this uses the wave path (MFMA measured
                                      // faster from G = 4 on)
// split rule: workgroups per CU to aim for at D = 128 (scaled by 128 / D)
constexpr int kDecodeTargetPerCu = VATTN_DEFAULT_TARGET;
constexpr int kMinChunkTiles = VATTN_DEFAULT_MIN_CHUNK;   // split rule: fewest KV tiles per split
// query rows (heads x tokens) per prefill workgroup: 8 waves (4 for D = 256)
// of 32 rows; threads per prefill workgroup
constexpr int prefill_rows(int D) { return D <= 128 ? 256 : 128; }
constexpr int prefill_threads(int D) { return D <= 128 ? 512 : 256; }
// backward: query rows (heads x tokens) per dq workgroup (8 waves of 32, 4
// at D = 256), keys per dk/dv workgroup (4 waves of 32) and dk/dv workgroups
// per key tile (two 128-column slices at D = 256)
constexpr int bwd_rows(int D) { return D <= 128 ? 256 : 128; }
constexpr int kBwdKeys = 128;
constexpr int bwd_slices(int D) { return D <= 128 ? 1 : D / 128; }
// largest query-tile count per sequence the on-device prefill schedule handles
constexpr int kSchedMaxQtiles = 8192;

// Fills *info (sizes only; no allocation). n_cu must be > 0.
vattn_status plan_compute(int B_max, int s_max_q, int s_max_kv, int Hq, int Hkv, int D,
                          int causal, const vattn_plan_opts* opts, int n_cu,
                          vattn_plan_info* info);

}  // namespace vattn
