// Device helpers shared by the gfx950 kernels: vector types, bf16 packing,
// cross-lane reductions, the per-sequence prologue and LDS swizzles.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegInf = -__builtin_inff();

// Error-word bits (mirrors VATTN_ERRBIT_* in the public header).
constexpr int kErrQLen = 0x1;
constexpr int kErrKvLen = 0x2;
constexpr int kErrRows = 0x4;
constexpr int kErrIndex = 0x8;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (nearest-even) and pack them, low half first
// (one v_cvt_pk_bf16_f32).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// DPP row-local exchanges (16-lane rows). Control codes from the GCN/CDNA DPP
// encoding: quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E, row_half_mirror
// = 0x141, row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Full-wave xor exchange through the LDS crossbar (no LDS memory used).
__device__ __forceinline__ float xor_lane(float x, int mask) {
  int lane = __lane_id();
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
      (lane ^ mask) << 2, __builtin_bit_cast(int, x)));
}

// Lanes 32 (or 16) apart through the gfx950 lane-swap instructions
// (v_permlane32_swap / v_permlane16_swap): with both operands x, each lane
// ends up holding the pair {x[lane], x[lane ^ 32]} (or ^ 16) across the two
// registers, so a max or a sum of the two is the exchange-and-combine step of
// a reduction without the LDS round trip of ds_bpermute. Written as inline
// asm (a VALU op, no memory access) with two distinct read-write operands:
// this hipcc's builtin for these instructions returns the second result from
// the wrong register. The s_nop gives the wait states a swap needs after a
// VALU write of its operands.
__device__ __forceinline__ void lane_swap32(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void lane_swap16(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float max_xor32(float x) {
  float a = x, b = x;
  lane_swap32(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_xor32(float x) {
  float a = x, b = x;
  lane_swap32(a, b);
  return a + b;
}
__device__ __forceinline__ float max_xor16(float x) {
  float a = x, b = x;
  lane_swap16(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_xor16(float x) {
  float a = x, b = x;
  lane_swap16(a, b);
  return a + b;
}

// Sum over aligned groups of N lanes (N in 1..64); every lane of the group
// receives the group total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<0xB1>(x);
  if constexpr (N >= 4) x += dpp<0x4E>(x);
  if constexpr (N >= 8) x += dpp<0x141>(x);
  if constexpr (N >= 16) x += dpp<0x140>(x);
  if constexpr (N >= 32) x = sum_xor16(x);
  if constexpr (N >= 64) x = sum_xor32(x);
  return x;
}

// Max over aligned groups of N lanes (N in 1..64), as group_sum.
template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp<0xB1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp<0x4E>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<0x141>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<0x140>(x));
  if constexpr (N >= 32) x = max_xor16(x);
  if constexpr (N >= 64) x = max_xor32(x);
  return x;
}

// Max / sum across lanes that differ only in the bits of [FROM, 64): combines
// the aligned groups of FROM lanes that hold the same element.
template <int FROM>
__device__ __forceinline__ float across_groups_max(float x) {
  if constexpr (FROM <= 1) x = fmaxf(x, dpp<0xB1>(x));
  if constexpr (FROM <= 2) x = fmaxf(x, xor_lane(x, 2));
  if constexpr (FROM <= 4) x = fmaxf(x, xor_lane(x, 4));
  if constexpr (FROM <= 8) x = fmaxf(x, xor_lane(x, 8));
  if constexpr (FROM <= 16) x = max_xor16(x);
  if constexpr (FROM <= 32) x = max_xor32(x);
  return x;
}
template <int FROM>
__device__ __forceinline__ float across_groups_sum(float x) {
  if constexpr (FROM <= 1) x += dpp<0xB1>(x);
  if constexpr (FROM <= 2) x += xor_lane(x, 2);
  if constexpr (FROM <= 4) x += xor_lane(x, 4);
  if constexpr (FROM <= 8) x += xor_lane(x, 8);
  if constexpr (FROM <= 16) x = sum_xor16(x);
  if constexpr (FROM <= 32) x = sum_xor32(x);
  return x;
}

// 16-byte global load / store of raw bits.
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// ---------------------------------------------------------------------------
// Sequence prologue: offsets and lengths read on the device from cu_seqlens
// entries b and b+1 only. Lengths are int32 differences; anything outside
// [0, s_max] is clamped and flagged, and a sequence is cut so that it stays
// inside the caller's row capacity. No read ever leaves [0, rows).
// ---------------------------------------------------------------------------
struct Span {
  int start;
  int len;
  int flags;
};

__device__ __forceinline__ Span read_span(const int32_t* cu, int b, int s_max, int64_t rows,
                                          int len_bit) {
  uint32_t a = (uint32_t)cu[b], e = (uint32_t)cu[b + 1];
  int len = (int)(e - a);
  int start = (int)a;
  int flags = 0;
  if (len < 0 || len > s_max) {
    flags |= len_bit;
    len = len < 0 ? 0 : s_max;
  }
  if (start < 0 || (int64_t)start > rows) {
    if (len > 0) flags |= kErrRows;
    start = 0;
    len = 0;
  } else if ((int64_t)start + len > rows) {
    flags |= kErrRows;
    len = (int)(rows - start);
  }
  return Span{start, len, flags};
}

__device__ __forceinline__ void report(int32_t* err, int flags) {
  if (flags) atomicOr(err, flags);
}

// ---------------------------------------------------------------------------
// LDS tile swizzles. Tiles hold rows of D bf16 (D/8 chunks of 16 bytes); the
// 16-byte chunk index is XOR-permuted per row. The XOR operand is always kept
// below the chunk count of a row, so every permuted chunk stays inside its row
// (the failure mode the HEAD_DIM=32 commit of the AstrAI decode kernel fixed).
// ---------------------------------------------------------------------------

// Row pattern for reads where consecutive lanes read the same chunk of
// consecutive rows (K operand of QK^T): rows that share a 256-byte bank line
// window land on different 16-byte bank groups.
template <int D>
__device__ __forceinline__ int swz_rows(int row, int chunk) {
  constexpr int CPR = D / 8;                  // chunks per row
  constexpr int RPL = CPR >= 16 ? 1 : 16 / CPR;  // rows per 256-byte line
  return chunk ^ ((row / RPL) & (CPR - 1));
}

// Pattern for V tiles read with the 16-lane transposed read of the
// 16x16x32 MFMA operand (decode): each 16-lane group reads 4 consecutive rows
// x 2 consecutive chunks, and a half-wave covers 16 consecutive rows.
template <int D>
__device__ __forceinline__ int swz_tr16(int row, int chunk) {
  constexpr int CPR = D / 8;
  if constexpr (CPR >= 16) return chunk ^ ((2 * row) & (CPR - 1));
  else if constexpr (CPR == 8) return chunk ^ (row & 7);
  else return chunk ^ ((row >> 1) & 3);
}

// Pattern for V tiles read with the transposed read of the 32x32x16 MFMA
// operand (prefill): a half-wave reads 4 consecutive rows x 4 consecutive
// chunks.
template <int D>
__device__ __forceinline__ int swz_tr32(int row, int chunk) {
  constexpr int CPR = D / 8;
  if constexpr (CPR >= 16) return chunk ^ ((4 * row) & (CPR - 1));
  else if constexpr (CPR == 8) return chunk ^ ((2 * row) & 7);
  else return chunk;
}

// Pattern for tiles read both ways: row reads as the 32x32x16 MFMA operand
// (16 lanes on 16 consecutive rows, one 16-byte chunk) and the transposed
// read of the same tile (a half-wave on 4 consecutive rows x 4 consecutive
// chunks). The XOR operand puts the low two row bits above the next two, so
// any 16 consecutive rows and any 4 consecutive rows x 4 chunks land on
// distinct 16-byte bank groups (checked by enumeration of both patterns).
template <int D>
__device__ __forceinline__ int swz_dual(int row, int chunk) {
  constexpr int CPR = D / 8;
  if constexpr (CPR >= 16) return chunk ^ (4 * (row & 3) + ((row >> 2) & 3));
  else if constexpr (CPR == 8) return chunk ^ ((2 * (row & 3) + ((row >> 1) & 7)) & 7);
  else return chunk ^ ((row >> 2) & 3);
}

}  // namespace vattn
