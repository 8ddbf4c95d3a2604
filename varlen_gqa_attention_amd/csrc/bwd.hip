// Backward of causal varlen GQA attention on gfx950: dq, dk, dv (bf16) from
// q, k, v, the forward's out and lse, and the output gradient dout.
//
// The pages name a THD backward under the forward's contract (cudnn-frontend
// issue #552, Related: the THD backward contract): packed or row-strided
// views, device-read cu_seqlens, dead tiles exiting, no host round trip. The
// arithmetic is the derivative of the forward through the softmax, with the
// softmax weights recomputed from the stored log-sum-exp:
//   p_ij = exp(s_ij - LSE_i), dp_ij = <dO_i, v_j>, delta_i = <dO_i, O_i>,
//   ds_ij = p_ij (dp_ij - delta_i), dq_i = scale sum_j ds_ij k_j,
//   dk_j = scale sum_i ds_ij q_i, dv_j = sum_i p_ij dO_i
// (dk, dv summed over the G query heads that read KV head j's head).
//
// Two kernels, no atomics (results do not depend on scheduling):
//  * dq kernel: workgroup = (sequence, KV head, query tile) with the G heads
//    folded into 256 rows, 8 waves of 32 rows (two per SIMD), as in the
//    forward. Per 64-key tile, one 32-key half after the other: S^T = K Q^T
//    and dP^T = V dO^T (Q^T and dO^T in registers, K and V rows from LDS),
//    P and dS in registers (one row per lane), dQ^T += K^T dS^T with K^T from
//    the transposed LDS read. Its prologue also computes delta_i from dO and
//    O and stores it for the second kernel.
//  * dk/dv kernel: workgroup = (sequence, KV head, 128-key tile), 32 keys per
//    wave (one wave per SIMD) with K and V of those keys in registers. It
//    walks the query rows that can see its keys (64 tokens of one query head
//    per step, all G heads): S = Q K^T and dP = dO V^T with Q and dO rows
//    from LDS, P and dS (one key per lane), then dV^T += dO^T P and
//    dK^T += Q^T dS with dO^T and Q^T from the transposed LDS read; the two
//    32-row halves of a step are software-pipelined.
//  * At D = 256 each workgroup of either kernel produces one 128-column slice
//    of its output (recomputing S and dP over the full D), the dq kernel runs
//    4 waves and the dk/dv kernel steps over 32 rows, to fit the registers.
// Every contraction is v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and
// dS are rounded to bf16 as MFMA operands. Tiles pass through a two-stage
// LDS ring with one barrier per step, filled by direct-to-LDS loads one
// step ahead (the dq kernel's K/V tiles, the dk/dv kernel's Q/dO tiles).
#include <hip/hip_ext.h>

#include "device.hpp"
#include "launch.hpp"

namespace vattn {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

__device__ __forceinline__ bf16x4 bwd_read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Direct global -> LDS load of 16 bytes per lane through a buffer resource
// (raw, byte offset voff from the resource's base): lane l's bytes land at
// lds_base + 16 l (lds_base must be the same for the whole wave). Completion
// is counted by vmcnt like any vector-memory load. (With the global-address
// form in flight the compiler would make every LDS read wait for all earlier
// ones; with buffer loads it counts them.)
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// Resource over the bytes from `base` on (no size limit: the kernel forms
// in-range offsets only), 32-bit data format (gfx9).
__device__ __forceinline__ rsrc_t raw_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, 0x00020000);
}
__device__ __forceinline__ void lds_dma16(rsrc_t r, uint32_t voff, uint8_t* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_base, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ void bwd_wait_vmem() {
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
}

template <int D, int WAVES = 4>
struct BwdCfg {
  static constexpr int NW = WAVES;             // waves per workgroup
  static constexpr int THREADS = NW * 64;
  static constexpr int BN = 64;                // keys (dq) or query rows (dk/dv) per step
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int KS = D / 16;            // k-steps of 16 over d
  static constexpr int DBLK = D / 32;          // 32-wide d blocks
  static constexpr int TILE_BYTES = BN * D * 2;
  static constexpr int CH = (BN * CPR + THREADS - 1) / THREADS;  // 16-byte chunks per thread
};

// A-operand fragment of a 32-row block of a row-major LDS tile (rows of D
// bf16, swz_dual layout): lane holds row 32 blk + lane % 32, elements
// 16 ks + 8 (lane / 32) .. + 8.
template <int D>
__device__ __forceinline__ bf16x8 frag_rows(const uint8_t* t, int blk, int ks, int lane) {
  const int r = 32 * blk + (lane & 31);
  const int c = 2 * ks + (lane >> 5);
  return __builtin_bit_cast(bf16x8,
                            *reinterpret_cast<const u32x4*>(t + r * D * 2 + swz_dual<D>(r, c) * 16));
}

// A-operand fragment of the transpose of a 64-row LDS tile (swz_dual layout)
// for k-step `step` (16 rows) and d block db: lane holds column
// d = 32 db + lane % 32 at the 8 rows that the bf16 packing of a 32x32 MFMA
// accumulator (see pack_acc) puts in lane / 32's half of that k-step.
template <int D>
__device__ __forceinline__ bf16x8 frag_tr(const uint8_t* t, int step, int db, int lane) {
  const int g = lane >> 4, m16 = lane & 15;
  const int blk = step >> 1, h = step & 1;
  const int r1 = 32 * blk + 16 * h + 4 * (g >> 1) + (m16 >> 2);
  const int r2 = r1 + 8;
  const int col = 32 * db + 16 * (g & 1) + 4 * (m16 & 3);
  const int ch = col >> 3, half = (col >> 2) & 1;
  const bf16x4 x1 = bwd_read_tr(t + r1 * D * 2 + swz_dual<D>(r1, ch) * 16 + half * 8);
  const bf16x4 x2 = bwd_read_tr(t + r2 * D * 2 + swz_dual<D>(r2, ch) * 16 + half * 8);
  return __builtin_shufflevector(x1, x2, 0, 1, 2, 3, 4, 5, 6, 7);
}

// bf16 B operand for k-step (blk, h) from a 32x32 accumulator block: lane
// holds accumulator entries 8 h .. 8 h + 7 (rows 16 h + 4 (lane / 32) + 0..3
// and + 8..11 of the block).
__device__ __forceinline__ bf16x8 pack_acc(const f32x16& x, int h) {
  u32x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(x[8 * h + 2 * j], x[8 * h + 2 * j + 1]);
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ float dot8(u32x4 a, u32x4 b) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    s = fmaf(bf16_lo(a[j]), bf16_lo(b[j]), s);
    s = fmaf(bf16_hi(a[j]), bf16_hi(b[j]), s);
  }
  return s;
}

// ---------------------------------------------------------------------------
// dq kernel (also writes delta)
// ---------------------------------------------------------------------------
// Waves of the dq kernel: 8 (two per SIMD) up to D = 128; at D = 256 a wave
// needs a SIMD's whole register file.
template <int D>
constexpr int dq_waves() { return D <= 128 ? 8 : 4; }

template <int D>
__global__ __launch_bounds__((BwdCfg<D, dq_waves<D>()>::THREADS)) void bwd_dq_kernel(BwdArgs a) {
  using C = BwdCfg<D, dq_waves<D>()>;  // waves of 32 rows
  constexpr int BN = C::BN, CPR = C::CPR, KS = C::KS, CH = C::CH;
  constexpr int PF = KS < 2 ? KS : 2;  // k-steps of LDS reads in flight
  // At D = 256 a workgroup accumulates one 128-column slice of dQ (two
  // workgroups per query tile, each recomputing S and dP over the full D),
  // so that Q, dO and the dQ accumulators fit one wave's registers.
  constexpr int DS = D <= 128 ? D : 128;  // dQ columns per workgroup
  constexpr int NSL = D / DS;
  constexpr int DBLK = DS / 32;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * 2 * C::TILE_BYTES];

  const int x = blockIdx.x & 7, p = blockIdx.x >> 3;
  const int per_unit = a.n_qtiles * NSL;
  const int u = x + 8 * (p / per_unit);
  if (u >= a.B_max * a.Hkv) return;
  const int b = u / a.Hkv, hk = u % a.Hkv;
  const int qt = a.n_qtiles - 1 - (p % per_unit) / NSL, sl = (p % per_unit) % NSL;
  if (b >= a.B) return;
  const Span sq = read_span(a.cu_q, b, a.s_max_q, a.q_rows, kErrQLen);
  const Span sk = read_span(a.cu_kv, b, a.s_max_kv, a.kv_rows, kErrKvLen);
  if (qt == 0 && hk == 0 && sl == 0 && threadIdx.x == 0) report(a.err, sq.flags | sk.flags);
  const int Lq = sq.len, Lk = sk.len;
  const int t0 = qt * a.tq;
  if (t0 >= Lq) return;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int shift = Lk - Lq;
  const int t_last = min(t0 + a.tq - 1, Lq - 1);
  const int kend = a.causal ? max(0, min(Lk, t_last + shift + 1)) : Lk;
  const int kfull = a.causal ? max(0, min(Lk, t0 + shift + 1)) : Lk;

  const int row = 32 * w + (lane & 31);
  const int hl = row / a.tq;
  const int tok = t0 + row % a.tq;
  const bool row_ok = hl < a.G && tok < Lq;
  const int hq = hk * a.G + hl;
  const int row_lim = a.causal ? tok + shift : Lk - 1;
  const int64_t qrow = (int64_t)sq.start + tok;

  // Q^T, dO^T operands and O (for delta): lane holds row's elements
  // 16 ks + 8 (lane / 32) .. + 8
  bf16x8 qv[KS], dov[KS];
  float delta = 0.f, lse = kNegInf;
  {
    const int off = hq * D + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 xq = {0, 0, 0, 0}, xd = {0, 0, 0, 0}, xo = {0, 0, 0, 0};
      if (row_ok) {
        xq = ld16(a.q + qrow * a.q_rs + off + 16 * ks);
        xd = ld16(a.dout + qrow * a.do_rs + off + 16 * ks);
        xo = ld16(a.out + qrow * a.o_rs + off + 16 * ks);
      }
      qv[ks] = __builtin_bit_cast(bf16x8, xq);
      dov[ks] = __builtin_bit_cast(bf16x8, xd);
      delta += dot8(xd, xo);
    }
    if (row_ok) lse = a.lse[qrow * a.Hq + hq];
  }

  const int64_t krs = a.k_rs, vrs = a.v_rs;
  const uint16_t* kbase = a.k + (int64_t)sk.start * krs + hk * D;
  const uint16_t* vbase = a.v + (int64_t)sk.start * vrs + hk * D;
  const int ntiles = (kend + BN - 1) / BN;
  // K and V tiles go straight into a two-stage LDS ring (buffer-resource
  // loads, one resource per tile at its first key row; byte offsets below
  // 2^31: rows < 64 apart, row strides < 2^24 elements): the lane that fills
  // slot (row r, position c') loads chunk swz_dual(r, c') of the row (the
  // swizzle is an XOR, its own inverse). Rows past the keys are clamped to
  // the last key (masked later). Tile jt + 1 is issued at the start of
  // iteration jt, into the stage that tile jt - 1 used.
  const int wave0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * 64;
  auto issue_tile = [&](int jt, uint8_t* dst) {
    const int key0 = jt * BN;
    const rsrc_t rk = raw_rsrc(kbase + (int64_t)key0 * krs);
    const rsrc_t rv = raw_rsrc(vbase + (int64_t)key0 * vrs);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int q = threadIdx.x + i * C::THREADS;
      if (BN * CPR % C::THREADS != 0 && q >= BN * CPR) break;  // whole waves
      const int r = q / CPR, c = q % CPR;
      const uint32_t rr = (uint32_t)(min(key0 + r, kend - 1) - key0);
      const uint32_t c16 = 16 * swz_dual<D>(r, c);
      uint8_t* base = dst + (wave0 + i * C::THREADS) * 16;
      lds_dma16(rk, rr * (uint32_t)(krs * 2) + c16, base);
      lds_dma16(rv, rr * (uint32_t)(vrs * 2) + c16, base + C::TILE_BYTES);
    }
  };
  // tile 0's loads share the Q / dO / O loads' round trip
  if (ntiles > 0) issue_tile(0, lds);
  bwd_wait_vmem();

  delta = sum_xor32(delta);
  if (row_ok && lane < 32 && sl == 0)
    a.delta[((int64_t)b * a.s_max_q + tok) * a.Hq + hq] = delta;
  // exponent offset in base 2; a row without visible keys (lse = -inf) gets
  // +inf so that every weight is exp2(-inf) = 0
  const float lse2 = (lse == kNegInf) ? __builtin_inff() : lse * kLog2e;

  f32x16 dq[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) dq[i][j] = 0.f;

  // One tile: issue tile jt + 1 into the other stage, then compute tile jt.
  // The stages are disjoint (restrict), which lets the compiler read `lk`
  // while the direct loads into `nxt` are in flight.
  auto tile = [&](int jt, const uint8_t* __restrict__ lk, uint8_t* __restrict__ nxt) {
    if (jt + 1 < ntiles) issue_tile(jt + 1, nxt);
    const uint8_t* lv = lk + C::TILE_BYTES;
    const int key0 = jt * BN;
    const bool need_mask = key0 + BN > kfull;
    // the two 32-key halves one after the other (one S^T / dP^T block pair
    // in registers at a time, which keeps a wave within the 256 registers of
    // two waves per SIMD)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T = K Q^T and dP^T = V dO^T; K and V row fragments stream from LDS
      // PF k-steps ahead of their MFMAs (the scheduling barriers keep the
      // reads from sinking next to their use)
      f32x16 s, dp;
#pragma unroll
      for (int j = 0; j < 16; ++j) s[j] = dp[j] = 0.f;
      bf16x8 kf[KS], vf[KS];
      auto rd = [&](int ks) {
        kf[ks] = frag_rows<D>(lk, kb, ks, lane);
        vf[ks] = frag_rows<D>(lv, kb, ks, lane);
      };
#pragma unroll
      for (int ks = 0; ks < PF; ++ks) rd(ks);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + PF < KS) rd(ks + PF);
        __builtin_amdgcn_sched_barrier(0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qv[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[ks], dov[ks], dp, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // K^T fragments of the half's two 16-key k-steps, read while the VALU works
      bf16x8 kt[2][DBLK];
      auto rdt = [&](int h) {
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
          kt[h][db] = frag_tr<D>(lk, 2 * kb + h, sl * DBLK + db, lane);
      };
      rdt(0);
      // P and dS (lane: one row; keys key0 + 32 kb + 8 (i/4) + 4 (lane/32) + i%4)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pv = fast_exp2(fmaf(s[i], a.c, -lse2));
        if (need_mask) {
          const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          if (key > row_lim || key >= Lk) pv = 0.f;
        }
        s[i] = pv * (dp[i] - delta);
      }
      // dQ^T += K^T dS^T over the half's two k-steps, K^T read one step ahead
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h == 0) rdt(1);
        const bf16x8 bds = pack_acc(s, h);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[h][db], bds, dq[db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // The barrier also waits for this wave's loads of tile jt (the compiler
  // completes loads to LDS before a workgroup barrier), so after it every
  // wave's part of tile jt is in LDS and no wave still reads the other stage.
  for (int jt = 0; jt < ntiles; ++jt) {
    bwd_wait_vmem();
    __syncthreads();
    tile(jt, lds + (jt & 1) * 2 * C::TILE_BYTES, lds + ((jt + 1) & 1) * 2 * C::TILE_BYTES);
  }

  // epilogue: lane holds dQ^T[d = 32 db + 8 (i/4) + 4 (lane/32) + i%4][row]
  if (!row_ok) return;
  uint16_t* op = a.dq + qrow * a.dq_rs + hq * D + sl * DS + 4 * (lane >> 5);
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      u32x2 wv;
      wv[0] = pack_bf16x2(dq[db][4 * i4 + 0] * a.scale, dq[db][4 * i4 + 1] * a.scale);
      wv[1] = pack_bf16x2(dq[db][4 * i4 + 2] * a.scale, dq[db][4 * i4 + 3] * a.scale);
      *reinterpret_cast<u32x2*>(op + 32 * db + 8 * i4) = wv;
    }
}

// ---------------------------------------------------------------------------
// dk / dv kernel
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(BwdCfg<D>::THREADS, 1) void bwd_dkdv_kernel(BwdArgs a) {
  using C = BwdCfg<D>;
  constexpr int CPR = C::CPR, KS = C::KS;
  constexpr int KEYS = 32 * C::NW;                  // keys per workgroup
  constexpr int PF = KS < 2 ? KS : 2;                // k-steps of LDS reads in flight
  // Up to D = 128 a step covers 64 query rows as two pipelined 32-row
  // halves and a workgroup accumulates all of D. At D = 256 the registers of
  // K, V, dK and dV do not fit beside that: a workgroup accumulates one
  // 128-wide slice of dK, dV (two workgroups per key tile, each recomputing
  // S and dP over the full D) and a step covers 32 rows.
  constexpr int RBS = D <= 128 ? 2 : 1;              // 32-row blocks per step
  constexpr int BN = 32 * RBS;                        // query rows per step
  constexpr int DS = D <= 128 ? D : 128;              // dK / dV columns per workgroup
  constexpr int NSL = D / DS;                         // column slices
  constexpr int DBLK = DS / 32;                       // 32-wide blocks of the slice
  constexpr int TILE = BN * D * 2;                    // one staged Q (or dO) tile
  constexpr int CH = (BN * CPR + C::THREADS - 1) / C::THREADS;
  constexpr int STAGE = 2 * TILE + 2 * BN * 4;       // Q, dO tiles + lse2, delta rows
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE];

  const int x = blockIdx.x & 7, p = blockIdx.x >> 3;
  const int per_unit = a.n_ktiles * NSL;
  const int u = x + 8 * (p / per_unit);
  if (u >= a.B_max * a.Hkv) return;
  const int b = u / a.Hkv, hk = u % a.Hkv;
  const int kt = (p % per_unit) / NSL, sl = (p % per_unit) % NSL;
  if (b >= a.B) return;
  const Span sq = read_span(a.cu_q, b, a.s_max_q, a.q_rows, kErrQLen);
  const Span sk = read_span(a.cu_kv, b, a.s_max_kv, a.kv_rows, kErrKvLen);
  const int Lq = sq.len, Lk = sk.len;
  const int j0 = kt * KEYS;
  if (j0 >= Lk) return;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int shift = Lk - Lq;
  const int key = j0 + 32 * w + (lane & 31);
  const bool key_ok = key < Lk;
  const int64_t krow = (int64_t)sk.start + key;

  // K^T, V^T operands: lane holds key's elements 16 ks + 8 (lane / 32) .. + 8
  bf16x8 kv_[KS], vv[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 xk = {0, 0, 0, 0}, xv = {0, 0, 0, 0};
    if (key_ok) {
      xk = ld16(a.k + krow * a.k_rs + hk * D + 8 * (lane >> 5) + 16 * ks);
      xv = ld16(a.v + krow * a.v_rs + hk * D + 8 * (lane >> 5) + 16 * ks);
    }
    kv_[ks] = __builtin_bit_cast(bf16x8, xk);
    vv[ks] = __builtin_bit_cast(bf16x8, xv);
  }

  // query rows that can see a key of this tile: tokens from t_first (causal:
  // key j0 needs token >= j0 - shift), BN tokens of one query head per step
  const int t_first = a.causal ? max(0, j0 - shift) : 0;
  const int n_tb = Lq > t_first ? (Lq - t_first + BN - 1) / BN : 0;
  const int n_it = n_tb * a.G;
  // Step it covers row block tb_of(it), last block first: the key tiles of a
  // sequence start at different rows (causal) but all end at its last one,
  // so walking down from there keeps the workgroups of a sequence and KV
  // head (one XCD) on the same Q and dO rows at the same time, which then
  // come from that XCD's L2.
  auto tb_of = [&](int it) { return n_tb - 1 - it / a.G; };

  // Staging: the Q and dO tiles of a step go straight from global memory to
  // LDS (lds_dma16); the lane that fills slot (row r, position c') of the
  // swizzled tile loads chunk swz_dual(r, c') of the row (the swizzle is an
  // XOR, its own inverse). Rows past the sequence are clamped to its last
  // row; they get lse = +inf below, so they carry weight 0. lse and delta of
  // the step's rows come through registers and are written (lse in base 2)
  // one step later, so their latency is not waited on at issue.
  float st_lse = 0.f, st_dl = 0.f;
  bool st_dead = false;
  // Per-step addressing (uniform), then the loads in parts: part i = chunk i
  // of the Q and dO tiles, spread over the step's first MFMA region.
  rsrc_t st_rq = raw_rsrc(a.q), st_rd = raw_rsrc(a.dout);
  int st_rlim = 0;
  auto issue_begin = [&](int it) {
    const int tb = tb_of(it), hq = hk * a.G + it % a.G;
    const int tbase = t_first + tb * BN;
    const int rlim = Lq - 1 - tbase;
    const int64_t t0 = (int64_t)sq.start + tbase;
    st_rq = raw_rsrc(a.q + t0 * a.q_rs + hq * D);
    st_rd = raw_rsrc(a.dout + t0 * a.do_rs + hq * D);
    st_rlim = rlim;
    if (threadIdx.x < BN) {
      const uint32_t rr = (uint32_t)min((int)threadIdx.x, rlim);
      st_dead = (int)threadIdx.x > rlim;
      st_lse = a.lse[t0 * a.Hq + hq + __umul24(rr, (uint32_t)a.Hq)];
      st_dl = a.delta[((int64_t)b * a.s_max_q + tbase) * a.Hq + hq + __umul24(rr, (uint32_t)a.Hq)];
    }
  };
  auto issue_part = [&](int i, uint8_t* dst) {
    const int q = threadIdx.x + i * C::THREADS;
    if (BN * CPR % C::THREADS != 0 && q >= BN * CPR) return;  // whole waves
    const int r = q / CPR;
    const uint32_t rr = (uint32_t)min(r, st_rlim);
    const uint32_t c8 = 8 * swz_dual<D>(r, q % CPR);
    uint8_t* base = dst + (q - lane) * 16;
    // byte offsets below 2^31: rows < 64 apart, row strides < 2^24 elements
    lds_dma16(st_rq, 2 * (__umul24(rr, (uint32_t)a.q_rs) + c8), base);
    lds_dma16(st_rd, 2 * (__umul24(rr, (uint32_t)a.do_rs) + c8), base + TILE);
  };
  auto issue_step = [&](int it, uint8_t* dst) {
    issue_begin(it);
#pragma unroll
    for (int i = 0; i < CH; ++i) issue_part(i, dst);
  };
  auto put_rows = [&](uint8_t* dst) {
    if (threadIdx.x < BN) {
      float* rows = reinterpret_cast<float*>(dst + 2 * TILE);
      // rows past the sequence, or without visible keys, get weight 0
      rows[threadIdx.x] = (st_dead || st_lse == kNegInf) ? __builtin_inff() : st_lse * kLog2e;
      rows[BN + threadIdx.x] = st_dl;
    }
  };

  f32x16 dk[DBLK], dv[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) dk[i][j] = dv[i][j] = 0.f;

  // One step: compute from stage `lq` while the next step's tile loads go to
  // stage `nxt` (its lse / delta loads first, its tile loads spread between
  // the first region's MFMAs). The two stages are disjoint (restrict), which
  // lets the compiler read `lq` while the direct loads into `nxt` are in
  // flight.
  auto step = [&](int it, const uint8_t* __restrict__ lq, uint8_t* __restrict__ nxt) {
    const bool more = it + 1 < n_it;
    if (more) issue_begin(it + 1);
    const uint8_t* ldo = lq + TILE;
    const float* lrow = reinterpret_cast<const float*>(lq + 2 * TILE);
    const int tbase = t_first + tb_of(it) * BN;
    // Per step, two 32-row halves in a software pipeline, so that each
    // half's softmax-gradient VALU work runs under the other half's MFMAs:
    //   A: S, dP of rows 0-31
    //   B: S, dP of rows 32-63      | P, dS of rows 0-31
    //   C: dV, dK from rows 0-31    | P, dS of rows 32-63
    //   D: dV, dK from rows 32-63
    // (S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS). Fragment
    // reads for a region are issued during the region before it.
    f32x16 s[2], dp[2], pp[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int j = 0; j < 16; ++j) s[rb][j] = dp[rb][j] = 0.f;
    bf16x8 qf[2][KS], df[2][KS];
    auto rd = [&](int rb, int ks) {
      qf[rb][ks] = frag_rows<D>(lq, rb, ks, lane);
      df[rb][ks] = frag_rows<D>(ldo, rb, ks, lane);
    };
    auto mm = [&](int rb, int ks) {
      s[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[rb][ks], kv_[ks], s[rb], 0, 0, 0);
      dp[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(df[rb][ks], vv[ks], dp[rb], 0, 0, 0);
    };
    bf16x8 dt[4][DBLK], qt[4][DBLK];
    auto rdt = [&](int step) {
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        dt[step][db] = frag_tr<D>(ldo, step, sl * DBLK + db, lane);
        qt[step][db] = frag_tr<D>(lq, step, sl * DBLK + db, lane);
      }
    };
    auto mmt = [&](int step) {
      const bf16x8 bp = pack_acc(pp[step >> 1], step & 1);
      const bf16x8 bds = pack_acc(s[step >> 1], step & 1);
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dt[step][db], bp, dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt[step][db], bds, dk[db], 0, 0, 0);
      }
    };
    // P and dS of one half (lane: one key; rows 32 rb + 8 g + 4 (lane/32)
    // + 0..3); visible iff key < Lk and (not causal or key <= token + shift);
    // rows past the sequence carry lse2 = +inf. grad(rb, i0) does entries
    // i0, i0 + 1 of the half, whose lse2 / delta were read into l4 / d4.
    f32x4 l4[4], d4[4];
    auto rows_of = [&](int rb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = 32 * rb + 8 * g + 4 * (lane >> 5);
        l4[g] = *reinterpret_cast<const f32x4*>(lrow + r0);
        d4[g] = *reinterpret_cast<const f32x4*>(lrow + BN + r0);
      }
    };
    // visible iff key <= min(Lk - 1, vlim + rr) with rr = row - 4 (lane / 32):
    // one compare, and the exponent of a hidden entry is -inf (no branch)
    const int vlim = a.causal ? tbase + shift + 4 * (lane >> 5) : Lk;
    auto grad = [&](int rb, int i0) {
#pragma unroll
      for (int i = i0; i < i0 + 2; ++i) {
        const int g = i >> 2, e = i & 3;
        const bool vis = key <= min(Lk - 1, vlim + 32 * rb + 8 * g + e);
        const float pv = fast_exp2(vis ? fmaf(s[rb][i], a.c, -l4[g][e]) : kNegInf);
        pp[rb][i] = pv;
        s[rb][i] = pv * (dp[rb][i] - d4[g][e]);
      }
    };
    if constexpr (RBS == 2) {
      // A
#pragma unroll
      for (int ks = 0; ks < PF; ++ks) rd(0, ks);
      rows_of(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + PF < KS) rd(0, ks + PF);
        else rd(1, ks + PF - KS);
        __builtin_amdgcn_sched_barrier(0);
        mm(0, ks);
        if (ks < CH && more) issue_part(ks, nxt);
        __builtin_amdgcn_sched_barrier(0);
      }
      // B: two entries of rows 0-31 per k-step of rows 32-63 (the order of
      // the source is kept by the scheduling barriers)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + PF < KS) rd(1, ks + PF);
        if (ks == KS - 2) rdt(0);
        if (ks == KS - 1) rdt(1);
        mm(1, ks);
#pragma unroll
        for (int i0 = 16 * ks / KS; i0 < 16 * (ks + 1) / KS; i0 += 2) grad(0, i0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // C: two entries of rows 32-63 per d block of the rows 0-31 products
      rows_of(1);
#pragma unroll
      for (int step = 0; step < 2; ++step) {
        const bf16x8 bp = pack_acc(pp[0], step);
        const bf16x8 bds = pack_acc(s[0], step);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          if (step == 1 && db == 0) rdt(2);
          if (step == 1 && db == DBLK - 1) rdt(3);
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dt[step][db], bp, dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt[step][db], bds, dk[db], 0, 0, 0);
          const int j = step * DBLK + db;
#pragma unroll
          for (int i0 = 16 * j / (2 * DBLK); i0 < 16 * (j + 1) / (2 * DBLK); i0 += 2) grad(1, i0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // D
      mmt(2);
      mmt(3);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      // one 32-row block per step: S, dP, then P, dS, then dV, dK
#pragma unroll
      for (int ks = 0; ks < PF; ++ks) rd(0, ks);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + PF < KS) rd(0, ks + PF);
        __builtin_amdgcn_sched_barrier(0);
        mm(0, ks);
        if (ks < CH && more) issue_part(ks, nxt);
        __builtin_amdgcn_sched_barrier(0);
      }
      rdt(0);
      rows_of(0);
#pragma unroll
      for (int i0 = 0; i0 < 16; i0 += 2) grad(0, i0);
      rdt(1);
      __builtin_amdgcn_sched_barrier(0);
      mmt(0);
      mmt(1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (n_it > 0) issue_step(0, lds);
  for (int it = 0; it < n_it; ++it) {
    uint8_t* cur = lds + (it & 1) * STAGE;
    bwd_wait_vmem();       // this wave's loads of step it have landed
    put_rows(cur);
    __syncthreads();       // every wave's have; stage (it + 1) & 1 is free
    step(it, cur, lds + ((it + 1) & 1) * STAGE);
  }

  // epilogue: lane holds dK^T / dV^T[d = 32 db + 8 (i/4) + 4 (lane/32) + i%4][key]
  if (!key_ok) return;
  uint16_t* kp = a.dk + krow * a.dk_rs + hk * D + sl * DS + 4 * (lane >> 5);
  uint16_t* vp = a.dv + krow * a.dv_rs + hk * D + sl * DS + 4 * (lane >> 5);
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      u32x2 wk, wv;
      wk[0] = pack_bf16x2(dk[db][4 * i4 + 0] * a.scale, dk[db][4 * i4 + 1] * a.scale);
      wk[1] = pack_bf16x2(dk[db][4 * i4 + 2] * a.scale, dk[db][4 * i4 + 3] * a.scale);
      wv[0] = pack_bf16x2(dv[db][4 * i4 + 0], dv[db][4 * i4 + 1]);
      wv[1] = pack_bf16x2(dv[db][4 * i4 + 2], dv[db][4 * i4 + 3]);
      *reinterpret_cast<u32x2*>(kp + 32 * db + 8 * i4) = wk;
      *reinterpret_cast<u32x2*>(vp + 32 * db + 8 * i4) = wv;
    }
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a, int grid_dq, int grid_dkdv, hipStream_t st,
                               hipEvent_t ev0, hipEvent_t ev1) {
  using C = BwdCfg<D>;
  // with measurement events, ev0 is stamped at the dq kernel's start and ev1
  // at the dk/dv kernel's end (the whole backward)
  constexpr int DQ_THREADS = BwdCfg<D, dq_waves<D>()>::THREADS;
  if (ev0)
    hipExtLaunchKernelGGL(bwd_dq_kernel<D>, dim3(grid_dq), dim3(DQ_THREADS), 0, st, ev0, nullptr,
                          0, a);
  else
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3(grid_dq), dim3(DQ_THREADS), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev0)
    hipExtLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3(grid_dkdv), dim3(C::THREADS), 0, st, nullptr,
                          ev1, 0, a);
  else
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3(grid_dkdv), dim3(C::THREADS), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_backward(const BwdArgs& a, int D, int grid_dq, int grid_dkdv, hipStream_t st,
                           hipEvent_t ev0, hipEvent_t ev1) {
  switch (D) {
    case 32: return launch_bwd_d<32>(a, grid_dq, grid_dkdv, st, ev0, ev1);
    case 64: return launch_bwd_d<64>(a, grid_dq, grid_dkdv, st, ev0, ev1);
    case 128: return launch_bwd_d<128>(a, grid_dq, grid_dkdv, st, ev0, ev1);
    case 256: return launch_bwd_d<256>(a, grid_dq, grid_dkdv, st, ev0, ev1);
  }
  return hipErrorInvalidValue;
}

}  // namespace vattn
