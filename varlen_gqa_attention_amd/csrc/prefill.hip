// Causal varlen prefill for GQA on gfx950 (online softmax, bf16 MFMA).
//
// A workgroup owns one query tile of one sequence for one KV head: the G query
// heads of that KV head are folded into the 128 rows of the tile (rows =
// heads x tq tokens, tq = 128 / G; kernbench ADR commit page, "GQA via M-fold"
// finding), so every K/V tile brought into LDS serves all G heads. Its 4 waves
// own 32 rows each. The grid is sized at plan time from B_max and s_max_q;
// each workgroup reads its sequence's offsets from cu_seqlens on the device
// and exits at once when its tile lies past the real length (cudnn-frontend
// issue #552, How the other backends avoid this: tiles read device lengths
// and early-exit).
//
// Per 64-key tile: S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from a
// swizzled LDS tile as the A operand, Q^T held in registers as B), online
// softmax in base 2 with per-lane row state (a lane's scores all belong to
// one query row), then O^T += V^T P^T where P^T is the S^T accumulator
// rounded to bf16 in place and V^T comes from the transposed LDS read. Only
// tiles that cross the causal diagonal or the end of the keys are masked.
//
// Workgroup order is XCD-aware: workgroup i runs on XCD i % 8, so the grid is
// arranged such that each XCD walks whole (sequence, KV head) units, largest
// query tiles first, keeping a unit's K/V in that XCD's L2 while its tiles run.
#include "device.hpp"
#include "launch.hpp"

namespace vattn {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

__device__ __forceinline__ bf16x4 lds_read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
}

template <int D>
struct PrefillCfg {
  static constexpr int BN = 64;        // keys per tile
  static constexpr int CPR = D / 8;    // 16-byte chunks per row
  static constexpr int KS = D / 16;    // k-steps of 16 for Q K^T
  static constexpr int DBLK = D / 32;  // 32-wide d blocks of P V
  static constexpr int LPT = BN * CPR / 256;  // 16-byte loads per thread per tile (K or V)
  static constexpr int TILE_BYTES = BN * D * 2;
  static constexpr int OCC = D <= 128 ? 2 : 1;
};

template <int D>
__global__ __launch_bounds__(256, PrefillCfg<D>::OCC) void prefill_kernel(PrefillArgs a) {
  using C = PrefillCfg<D>;
  constexpr int BN = C::BN, CPR = C::CPR, KS = C::KS, DBLK = C::DBLK, LPT = C::LPT;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::TILE_BYTES];
  uint8_t* lk = lds;
  uint8_t* lv = lds + C::TILE_BYTES;

  // ---- which (sequence, kv head, query tile)
  int b, hk, qt;
  if (a.tile_map) {
    const int e = blockIdx.x / a.Hkv;
    hk = blockIdx.x % a.Hkv;
    if (e >= a.n_map) return;
    const int entry = a.tile_map[e];
    b = entry >> 16;
    qt = entry & 0xffff;
    if (b < 0 || qt >= a.n_qtiles) return;
  } else {
    const int x = blockIdx.x & 7, p = blockIdx.x >> 3;
    const int u = x + 8 * (p / a.n_qtiles);
    qt = a.n_qtiles - 1 - p % a.n_qtiles;
    if (u >= a.B_max * a.Hkv) return;
    b = u / a.Hkv;
    hk = u % a.Hkv;
  }
  if (b >= a.B) return;
  const Span sq = read_span(a.cu_q, b, a.s_max_q, a.q_rows, kErrQLen);
  const Span sk = read_span(a.cu_kv, b, a.s_max_kv, a.kv_rows, kErrKvLen);
  if (qt == 0 && hk == 0 && threadIdx.x == 0) report(a.err, sq.flags | sk.flags);
  const int Lq = sq.len, Lk = sk.len;
  const int t0 = qt * a.tq;
  if (t0 >= Lq) return;  // dead tile

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = 32 * w + (lane & 31);
  const int hl = row / a.tq;
  const int tok = t0 + row % a.tq;
  const bool row_ok = hl < a.G && tok < Lq;
  const int hq = hk * a.G + hl;
  const int shift = Lk - Lq;  // bottom-right causal alignment
  const int row_lim = a.causal ? tok + shift : Lk - 1;  // last visible key of this row
  const int t_last = min(t0 + a.tq - 1, Lq - 1);
  const int kend = a.causal ? max(0, min(Lk, t_last + shift + 1)) : Lk;
  const int kfull = a.causal ? max(0, min(Lk, t0 + shift + 1)) : Lk;  // keys seen by all rows

  // ---- Q^T operand: lane holds Q[row][16 ks + 8 (lane >> 5) .. +8]
  bf16x8 qv[KS];
  {
    const uint16_t* qp = a.q + ((int64_t)(sq.start + tok) * a.Hq + hq) * D + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = {0, 0, 0, 0};
      if (row_ok) x = ld16(qp + 16 * ks);
      qv[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  float m = kNegInf, l = 0.f;
  f32x16 o[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[i][j] = 0.f;

  const int64_t kvstride = (int64_t)a.Hkv * D;
  const uint16_t* kbase = a.k + ((int64_t)sk.start * a.Hkv + hk) * D;
  const uint16_t* vbase = a.v + ((int64_t)sk.start * a.Hkv + hk) * D;
  const int ntiles = (kend + BN - 1) / BN;

  auto load_tile = [&](int jt, u32x4 (&kr)[LPT], u32x4 (&vr)[LPT]) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int qi = i * 256 + threadIdx.x;
      const int key = min(jt * BN + qi / CPR, kend - 1);
      const int64_t off = key * kvstride + 8 * (qi % CPR);
      kr[i] = ld16(kbase + off);
      vr[i] = ld16(vbase + off);
    }
  };

  u32x4 kr[LPT], vr[LPT];
  if (ntiles > 0) load_tile(0, kr, vr);
  for (int jt = 0; jt < ntiles; ++jt) {
    if (jt > 0) __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int qi = i * 256 + threadIdx.x;
      const int r = qi / CPR, c = qi % CPR;
      *reinterpret_cast<u32x4*>(lk + r * D * 2 + swz_rows<D>(r, c) * 16) = kr[i];
      *reinterpret_cast<u32x4*>(lv + r * D * 2 + swz_tr32<D>(r, c) * 16) = vr[i];
    }
    __syncthreads();
    if (jt + 1 < ntiles) load_tile(jt + 1, kr, vr);

    const int key0 = jt * BN;
    // ---- S^T = K Q^T: two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) sacc[kb][j] = 0.f;
      const int r = 32 * kb + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = 2 * ks + (lane >> 5);
        const u32x4 kx = *reinterpret_cast<const u32x4*>(lk + r * D * 2 + swz_rows<D>(r, c) * 16);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kx), qv[ks],
                                                           sacc[kb], 0, 0, 0);
      }
    }
    // ---- online softmax (lane: row `row`, keys key0 + 32 kb + 8 (i/4) + 4 (lane>>5) + i%4)
    const bool need_mask = key0 + BN > kfull;
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = sacc[kb][i] * a.c;
        if (need_mask) {
          const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          if (key > row_lim || key >= Lk) x = kNegInf;
        }
        sacc[kb][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, xor_lane(mx, 32));
    const float mnew = fmaxf(m, mx);
    const float msub = (mnew == kNegInf) ? 0.f : mnew;
    const float alpha = fast_exp2(m - msub);
    m = mnew;
    float psum = 0.f;
    u32x4 pk[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = fast_exp2(sacc[kb][8 * h + 2 * j] - msub);
          const float p1 = fast_exp2(sacc[kb][8 * h + 2 * j + 1] - msub);
          psum += p0 + p1;
          pk[kb][h][j] = pack_bf16x2(p0, p1);
        }
    l = l * alpha + psum;
#pragma unroll
    for (int i = 0; i < DBLK; ++i) o[i] *= alpha;

    // ---- O^T += V^T P^T: k-steps (kb, h) of 16 keys each
    const int g = lane >> 4, m16 = lane & 15;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8 pt = __builtin_bit_cast(bf16x8, pk[kb][h]);
        const int r1 = 32 * kb + 16 * h + 4 * (g >> 1) + (m16 >> 2);
        const int r2 = r1 + 8;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          const int col = 32 * db + 16 * (g & 1) + 4 * (m16 & 3);
          const int ch = col >> 3, half = (col >> 2) & 1;
          const bf16x4 x1 = lds_read_tr(lv + r1 * D * 2 + swz_tr32<D>(r1, ch) * 16 + half * 8);
          const bf16x4 x2 = lds_read_tr(lv + r2 * D * 2 + swz_tr32<D>(r2, ch) * 16 + half * 8);
          const bf16x8 vt = __builtin_shufflevector(x1, x2, 0, 1, 2, 3, 4, 5, 6, 7);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt, pt, o[db], 0, 0, 0);
        }
      }
  }

  // ---- epilogue: lane holds O^T[d = 32 db + 8 (i/4) + 4 (lane>>5) + i%4][row]
  l += xor_lane(l, 32);
  if (!row_ok) return;
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  uint16_t* op = a.out + ((int64_t)(sq.start + tok) * a.Hq + hq) * D + 4 * (lane >> 5);
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      u32x2 wv;
      wv[0] = pack_bf16x2(o[db][4 * i4 + 0] * inv, o[db][4 * i4 + 1] * inv);
      wv[1] = pack_bf16x2(o[db][4 * i4 + 2] * inv, o[db][4 * i4 + 3] * inv);
      *reinterpret_cast<u32x2*>(op + 32 * db + 8 * i4) = wv;
    }
  if ((lane >> 5) == 0)
    a.lse[(int64_t)(sq.start + tok) * a.Hq + hq] = (l > 0.f) ? (m + fast_log2(l)) * kLn2 : kNegInf;
}

template <int D>
static hipError_t launch_prefill_d(const PrefillArgs& a, int grid, hipStream_t st) {
  prefill_kernel<D><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, int D, int grid, hipStream_t st) {
  switch (D) {
    case 32: return launch_prefill_d<32>(a, grid, st);
    case 64: return launch_prefill_d<64>(a, grid, st);
    case 128: return launch_prefill_d<128>(a, grid, st);
    case 256: return launch_prefill_d<256>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vattn
