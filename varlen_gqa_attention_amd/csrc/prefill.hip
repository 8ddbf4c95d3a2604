// Causal varlen prefill for GQA on gfx950 (online softmax, bf16 MFMA).
//
// A workgroup owns one query tile of one sequence for one KV head: the G query
// heads of that KV head are folded into the rows of the tile (rows = heads x
// tq tokens; kernbench ADR commit page, "GQA via M-fold" finding), so every
// K/V tile brought into LDS serves all G heads. The grid is sized at plan time
// from B_max and s_max_q; each workgroup reads its sequence's offsets from
// cu_seqlens on the device and exits at once when its tile lies past the real
// length (cudnn-frontend issue #552, How the other backends avoid this: tiles
// read device lengths and early-exit).
//
// Layout of the work: 8 waves (4 at D = 256), each owning one block of 32
// rows. Per 64-key tile, S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (K from
// LDS as the A operand; Q^T held in registers), online softmax in base 2 with
// per-lane row state (all of a lane's scores belong to one query row), then
// O^T += V^T P^T where P^T is the S^T accumulator rounded to bf16 in place and
// V^T comes from the gfx950 transposed LDS read. K/V tiles go straight from
// global memory into a two-stage LDS ring (direct-to-LDS loads, swizzled on
// the global side, conflict-free): tile jt + 1 is in flight while tile jt is
// computed; one workgroup barrier per tile. LDS fragment
// reads run a few k-steps ahead of the MFMAs that consume them. The softmax
// scale folds into the exponent's FMA; the running max used for the exponent
// is only raised when a row's max grows by more than 2^8, so the O accumulator
// is rescaled rarely (exact: l uses the same reference), and once every row
// of a wave has a reference a tile skips the row max unless its weights grew
// past 2^30.
// Only tiles that cross the causal diagonal or the end of the keys are masked.
// When a row of the query tile sees fewer than 64 keys (all of them in the
// first key tile), that tile takes P V with P split into its bf16 rounding
// and the bf16 remainder, so such rows' weights are not rounded to 8 bits.
//
// Workgroup order is XCD-aware: workgroup i runs on XCD i % 8, so the grid is
// arranged such that each XCD walks whole (sequence, KV head) units, largest
// query tiles first, keeping a unit's K/V in that XCD's L2 while its tiles run.
#include <hip/hip_ext.h>

#include "device.hpp"
#include "launch.hpp"
#include "plan.hpp"

namespace vattn {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

__device__ __forceinline__ bf16x4 lds_read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Direct global -> LDS load of 16 bytes per lane through a buffer resource
// (raw, byte offset voff from the resource's base): lane l's bytes land at
// lds_base + 16 l (lds_base must be the same for the whole wave). Completion
// is counted by vmcnt like any vector-memory load. The buffer form rather
// than the global-address form: while a global-address load to LDS is in
// flight the compiler makes every LDS read wait for all earlier ones
// (lgkmcnt(0)), so the K and V fragment reads of a tile could not run ahead
// of the MFMAs that consume them; with buffer loads it counts them.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// Resource over the bytes from `base` on: no size limit (every offset the
// kernel forms is in range by construction), 32-bit data format (gfx9).
__device__ __forceinline__ rsrc_t raw_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, 0x00020000);
}
__device__ __forceinline__ void lds_dma16(rsrc_t r, uint32_t voff, uint8_t* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_base, 16, voff, 0, 0, 0);
}

// s_waitcnt vmcnt(0) with the other counters untouched (gfx9 encoding).
__device__ __forceinline__ void wait_vmem_all() {
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
}

template <int D>
struct PrefillCfg {
  // 8 waves (two per SIMD) of one 32-row block each for D <= 128; at D = 256
  // a wave's registers need a SIMD to itself: 4 waves.
  static constexpr int NW = D <= 128 ? 8 : 4;
  static constexpr int RB = 1;                   // 32-row blocks per wave
  static constexpr int ROWS = NW * RB * 32;      // rows per workgroup
  static constexpr int BN = 64;                  // keys per tile
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int KS = D / 16;              // k-steps of 16 for Q K^T
  static constexpr int DBLK = D / 32;            // 32-wide d blocks of P V
  static constexpr int TILE_BYTES = BN * D * 2;  // one K (or V) tile
  static constexpr int NSTAGE = 2;               // LDS ring depth (K + V per stage)
  static constexpr int THREADS = NW * 64;
};

// One query tile (sequence b, KV head hk, query tile qt) of the pass; the
// whole workgroup calls it with the same arguments (every exit is uniform).
template <int D>
__device__ __forceinline__ void prefill_tile(const PrefillArgs& a, uint8_t* lds, int b, int hk,
                                             int qt) {
  using C = PrefillCfg<D>;
  constexpr int RB = C::RB, BN = C::BN, CPR = C::CPR, KS = C::KS, DBLK = C::DBLK;
  if (b < 0 || b >= a.B || qt >= a.n_qtiles) return;
  const Span sq = read_span(a.cu_q, b, a.s_max_q, a.q_rows, kErrQLen);
  const Span sk = read_span(a.cu_kv, b, a.s_max_kv, a.kv_rows, kErrKvLen);
  if (qt == 0 && hk == 0 && threadIdx.x == 0) report(a.err, sq.flags | sk.flags);
  const int Lq = sq.len, Lk = sk.len;
  const int t0 = qt * a.tq;
  if (t0 >= Lq) return;  // dead tile

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int shift = Lk - Lq;  // bottom-right causal alignment
  const int t_last = min(t0 + a.tq - 1, Lq - 1);
  const int kend = a.causal ? max(0, min(Lk, t_last + shift + 1)) : Lk;
  const int kfull = a.causal ? max(0, min(Lk, t0 + shift + 1)) : Lk;  // keys seen by all rows

  // ---- per row block: this lane's query row
  int tok[RB], hq[RB], row_lim[RB];
  bool row_ok[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = 32 * (RB * w + rb) + (lane & 31);
    const int hl = row / a.tq;
    tok[rb] = t0 + row % a.tq;
    row_ok[rb] = hl < a.G && tok[rb] < Lq;
    hq[rb] = hk * a.G + hl;
    row_lim[rb] = a.causal ? tok[rb] + shift : Lk - 1;
  }

  // ---- Q^T operands: lane holds Q[row][16 ks + 8 (lane >> 5) .. +8]
  bf16x8 qv[RB][KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const uint16_t* qp =
        a.q + (int64_t)(sq.start + tok[rb]) * a.q_rs + hq[rb] * D + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = {0, 0, 0, 0};
      if (row_ok[rb]) x = ld16(qp + 16 * ks);
      qv[rb][ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const int64_t krs = a.k_rs, vrs = a.v_rs;
  const uint16_t* kbase = a.k + (int64_t)sk.start * krs + hk * D;
  const uint16_t* vbase = a.v + (int64_t)sk.start * vrs + hk * D;
  const int ntiles = (kend + BN - 1) / BN;

  // Tiles go straight from global memory into a two-stage LDS ring (16
  // bytes per lane; lane l of a wave lands at the wave's base + 16 l), the
  // swizzle applied on the global side: the lane that fills slot (row r,
  // position c') loads chunk swz(r, c') of the row (each swizzle is an XOR,
  // its own inverse). Tile jt + 1 is issued at the start of iteration jt,
  // into the stage that tile jt - 1 used. Rows past the keys are clamped to
  // the last key (masked later).
  constexpr int CH = (BN * CPR + C::THREADS - 1) / C::THREADS;  // chunks per thread (K or V)
  const int wave0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * 64;
  // One buffer resource per tile (its first key row) and 32-bit byte offsets
  // inside it: 63 rows of a stride below 2^25 elements (the host rejects
  // wider K and V rows) plus one row stay below 2^32 bytes. A full tile's
  // offsets do not change from tile to tile: computed once (up to D = 128,
  // two chunks per thread; at D = 256, eight, whose offsets would cost the
  // registers the kernel does not have: computed per tile).
  constexpr bool kHoist = CH <= 2;
  uint32_t koff[kHoist ? CH : 1], voff[kHoist ? CH : 1];
  if constexpr (kHoist) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int q = threadIdx.x + i * C::THREADS;
      const int r = q / CPR, cp = q % CPR;
      koff[i] = (uint32_t)(r * krs * 2 + swz_rows<D>(r, cp) * 16);
      voff[i] = (uint32_t)(r * vrs * 2 + swz_tr32<D>(r, cp) * 16);
    }
  }
  auto issue_tile = [&](int jt, uint8_t* dst) {
    const int key0 = jt * BN;
    const rsrc_t rk = raw_rsrc(kbase + (int64_t)key0 * krs);
    const rsrc_t rv = raw_rsrc(vbase + (int64_t)key0 * vrs);
    if (kHoist && key0 + BN <= kend) {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        if (BN * CPR % C::THREADS != 0 && threadIdx.x + i * C::THREADS >= BN * CPR) break;
        uint8_t* base = dst + (wave0 + i * C::THREADS) * 16;
        lds_dma16(rk, koff[kHoist ? i : 0], base);
        lds_dma16(rv, voff[kHoist ? i : 0], base + C::TILE_BYTES);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int q = threadIdx.x + i * C::THREADS;
      if (BN * CPR % C::THREADS != 0 && q >= BN * CPR) break;  // whole waves
      const int r = q / CPR, cp = q % CPR;
      const uint32_t rr = (uint32_t)(min(key0 + r, kend - 1) - key0);
      uint8_t* base = dst + (wave0 + i * C::THREADS) * 16;
      lds_dma16(rk, rr * (uint32_t)(krs * 2) + 16 * swz_rows<D>(r, cp), base);
      lds_dma16(rv, rr * (uint32_t)(vrs * 2) + 16 * swz_tr32<D>(r, cp), base + C::TILE_BYTES);
    }
  };

  // Tile 0's loads share the Q loads' round trip. Q must be in registers
  // before the loop: an explicit wait here tells the compiler's counter
  // tracking so.
  if (ntiles > 0) issue_tile(0, lds);
  wait_vmem_all();

  // l: sum of the fp32 weights (for the LSE); lt: sum of the same weights
  // rounded to bf16 as they enter the P V product (normalises O, so the
  // output is a weighted mean of V rows with exactly the weights used)
  float m[RB], l[RB], lt[RB];
  bool settled[RB];  // every row of the wave has a reference max (wave-uniform)
  f32x16 o[RB][DBLK];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = kNegInf;
    l[rb] = 0.f;
    lt[rb] = 0.f;
    settled[rb] = false;
#pragma unroll
    for (int i = 0; i < DBLK; ++i)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[rb][i][j] = 0.f;
  }

  // The two halves of tile jt: h1 = S^T = K Q^T + online softmax (leaves
  // bf16 P in pk), h2 = O^T += V^T P^T. With `lo` (the first key tile, when
  // some row of the query tile sees fewer than 64 keys: then all of that
  // row's keys are in it) P enters P V as two bf16 operands, its rounding pk
  // and the remainder p - bf16(p) in pkl, one more MFMA per step: with bf16
  // weights alone, a row whose few comparable weights multiply V rows far
  // apart misses the output's rounding by up to 2^-8 max|v - O|; over 64 or
  // more keys the weights' rounding errors average out.
  u32x4 pk[RB][2][2], pkl[RB][2][2];
  auto h1 = [&](int jt, const uint8_t* lk, bool lo) {
    const int key0 = jt * BN;
    // ---- S^T = K Q^T: two 32-key blocks x RB row blocks (K read once)
    f32x16 sacc[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[rb][kb][j] = 0.f;
    // K fragments stream from LDS PF k-steps ahead of the MFMAs that use
    // them (the scheduling barriers keep the compiler from pulling the reads
    // back next to their MFMAs, which would expose the LDS latency each step)
    constexpr int PF = KS < 4 ? KS : 4;
    bf16x8 kx[2][KS];
    auto read_k = [&](int ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int r = 32 * kb + (lane & 31);
        const int c = 2 * ks + (lane >> 5);
        kx[kb][ks] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(lk + r * D * 2 + swz_rows<D>(r, c) * 16));
      }
    };
#pragma unroll
    for (int ks = 0; ks < PF; ++ks) read_k(ks);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + PF < KS) read_k(ks + PF);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          sacc[rb][kb] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(kx[kb][ks], qv[rb][ks], sacc[rb][kb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- online softmax per row block (lane: one row; keys
    //      key0 + 32 kb + 8 (i/4) + 4 (lane>>5) + i%4)
    const bool need_mask = key0 + BN > kfull;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
            if (key > row_lim[rb] || key >= Lk) sacc[rb][kb][i] = kNegInf;
          }
      }
      // P = exp2(S c - msub) rounded to bf16 into pk; psum / ptsum: the
      // lane's sums of the fp32 and of the bf16-rounded weights
      float psum = 0.f, ptsum = 0.f;
      auto exps = [&](float msub) __attribute__((always_inline)) {
        psum = 0.f;
        ptsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float p0 = fast_exp2(fmaf(sacc[rb][kb][8 * h + 2 * j], a.c, -msub));
              const float p1 = fast_exp2(fmaf(sacc[rb][kb][8 * h + 2 * j + 1], a.c, -msub));
              psum += p0 + p1;
              const uint32_t w2 = pack_bf16x2(p0, p1);
              pk[rb][kb][h][j] = w2;
              ptsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2),
                                                      __builtin_bit_cast(bf16x2, 0x3F803F80u),
                                                      ptsum, false);
              if (lo) {
                const uint32_t r2 = pack_bf16x2(p0 - bf16_lo(w2), p1 - bf16_hi(w2));
                pkl[rb][kb][h][j] = r2;
                ptsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, r2),
                                                        __builtin_bit_cast(bf16x2, 0x3F803F80u),
                                                        ptsum, false);
              }
            }
      };
      // Once every row of the wave has a reference, the tile's weights are
      // taken against it without a row max; only if some weight may have
      // grown past 2^30 (a lane's sum says so: the sum of 32 weights bounds
      // each) is the tile redone with the max below. Weights up to 2^35 keep
      // l, lt and O far from the fp32 range, and the reference cancels in O
      // and in the LSE.
      bool redo = true;
      if (settled[rb]) {
        exps(m[rb]);
        redo = __builtin_amdgcn_ballot_w64(!(psum <= 0x1p30f)) != 0;
      }
      if (redo) {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[rb][kb][i]);
        mx = max_xor32(mx) * a.c;   // row max in base-2 units
        // raise the reference max when the row max grew by more than 2^8
        // (or the row had no reference yet); rescale O and l when it moves
        const bool grow = mx > m[rb] + 8.f;
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float mnew = grow ? mx : m[rb];
          const float alpha = fast_exp2(m[rb] - mnew);  // m = -inf -> 0
          if (grow) {
            m[rb] = mnew;
            l[rb] *= alpha;
            lt[rb] *= alpha;
#pragma unroll
            for (int i = 0; i < DBLK; ++i) o[rb][i] *= alpha;
          }
        }
        exps((m[rb] == kNegInf) ? 0.f : m[rb]);
        settled[rb] = __builtin_amdgcn_ballot_w64(m[rb] == kNegInf) == 0;
      }
      l[rb] += psum;
      lt[rb] += ptsum;
    }

  };
  auto h2 = [&](const uint8_t* lv, bool lo) {
    // ---- O^T += V^T P^T: k-steps (kb, h) of 16 keys; V^T read once for all
    //      row blocks
    // V^T fragments for the 4 k-steps (kb, h) stream from LDS one k-step
    // ahead of their MFMAs
    const int g = lane >> 4, m16 = lane & 15;
    bf16x8 vt[4][DBLK];
    auto read_v = [&](int step) {
      const int kb = step >> 1, h = step & 1;
      const int r1 = 32 * kb + 16 * h + 4 * (g >> 1) + (m16 >> 2);
      const int r2 = r1 + 8;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const int col = 32 * db + 16 * (g & 1) + 4 * (m16 & 3);
        const int ch = col >> 3, half = (col >> 2) & 1;
        const bf16x4 x1 = lds_read_tr(lv + r1 * D * 2 + swz_tr32<D>(r1, ch) * 16 + half * 8);
        const bf16x4 x2 = lds_read_tr(lv + r2 * D * 2 + swz_tr32<D>(r2, ch) * 16 + half * 8);
        vt[step][db] = __builtin_shufflevector(x1, x2, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    };
    read_v(0);
#pragma unroll
    for (int step = 0; step < 4; ++step) {
      if (step + 1 < 4) read_v(step + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          o[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              vt[step][db], __builtin_bit_cast(bf16x8, pk[rb][step >> 1][step & 1]), o[rb][db],
              0, 0, 0);
          if (lo)
            o[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                vt[step][db], __builtin_bit_cast(bf16x8, pkl[rb][step >> 1][step & 1]),
                o[rb][db], 0, 0, 0);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One tile: issue tile jt + 1 into the other stage, then compute tile jt.
  // The stages are disjoint (restrict), which lets the compiler read `cur`
  // while the direct loads into `nxt` are in flight.
  auto tile = [&](int jt, const uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt, bool lo) {
    if (jt + 1 < ntiles) issue_tile(jt + 1, nxt);
    h1(jt, cur, lo);
    h2(cur + C::TILE_BYTES, lo);
  };
  // The barrier also waits for this wave's loads of tile jt (the compiler
  // completes direct-to-LDS loads before a workgroup barrier), so after it
  // every wave's part of tile jt is in LDS and no wave still reads the stage
  // that tile jt + 1 goes to. The first tile runs outside the loop, the only
  // one that may take the remainder of P, so the loop's code is without it.
  if (ntiles > 0) {
    wait_vmem_all();
    __syncthreads();
    tile(0, lds, lds + 2 * C::TILE_BYTES, kfull < BN);
  }
  for (int jt = 1; jt < ntiles; ++jt) {
    wait_vmem_all();
    __syncthreads();
    tile(jt, lds + (jt & 1) * 2 * C::TILE_BYTES, lds + ((jt + 1) & 1) * 2 * C::TILE_BYTES, false);
  }

  // ---- epilogue: lane holds O^T[d = 32 db + 8 (i/4) + 4 (lane>>5) + i%4][row]
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float ls = sum_xor32(l[rb]), lts = sum_xor32(lt[rb]);
    if (!row_ok[rb]) continue;
    const float inv = (lts > 0.f) ? 1.f / lts : 0.f;
    uint16_t* op = a.out + (int64_t)(sq.start + tok[rb]) * a.o_rs + hq[rb] * D + 4 * (lane >> 5);
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        u32x2 wv;
        wv[0] = pack_bf16x2(o[rb][db][4 * i4 + 0] * inv, o[rb][db][4 * i4 + 1] * inv);
        wv[1] = pack_bf16x2(o[rb][db][4 * i4 + 2] * inv, o[rb][db][4 * i4 + 3] * inv);
        *reinterpret_cast<u32x2*>(op + 32 * db + 8 * i4) = wv;
      }
    if ((lane >> 5) == 0)
      a.lse[(int64_t)(sq.start + tok[rb]) * a.Hq + hq[rb]] =
          (ls > 0.f) ? (m[rb] + fast_log2(ls)) * kLn2 : kNegInf;
  }
}

// Work distribution of a prefill launch; each form is its own kernel, so
// that each holds one inlined copy of the tile code.
enum PrefillGrid { kGridSmax = 0, kGridMap = 1, kGridList = 2 };

template <int D, int GRID>
__global__ __launch_bounds__(PrefillCfg<D>::THREADS, 1) void prefill_kernel(PrefillArgs a) {
  using C = PrefillCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::NSTAGE * 2 * C::TILE_BYTES];
  if constexpr (GRID == kGridList) {
    // persistent: stride over (list entry, KV head) pairs; the list is
    // ordered longest query tiles first, so each round of the stride holds
    // tiles of similar cost
    const int total = *a.sched_count * a.Hkv;
    for (int f = blockIdx.x; f < total; f += gridDim.x) {
      const int entry = a.tile_map[f / a.Hkv];
      prefill_tile<D>(a, lds, entry >> 16, f % a.Hkv, entry & 0xffff);
      __syncthreads();  // the next tile reuses the LDS ring
    }
  } else if constexpr (GRID == kGridMap) {
    const int e = blockIdx.x / a.Hkv;
    if (e >= a.n_map) return;
    const int entry = a.tile_map[e];
    prefill_tile<D>(a, lds, entry >> 16, blockIdx.x % a.Hkv, entry & 0xffff);
  } else {
    // grid from B_max and s_max_q: workgroup i runs on XCD i % 8, and each
    // XCD walks whole (sequence, KV head) units, longest query tiles first
    const int x = blockIdx.x & 7, p = blockIdx.x >> 3;
    const int u = x + 8 * (p / a.n_qtiles);
    if (u >= a.B_max * a.Hkv) return;
    prefill_tile<D>(a, lds, u / a.Hkv, u % a.Hkv, a.n_qtiles - 1 - p % a.n_qtiles);
  }
}

// ---------------------------------------------------------------------------
// Device-built schedule of live query tiles (one workgroup). With n(b) =
// ceil(Lq_b / tq) live tiles for sequence b, the list holds level qt =
// n_qtiles - 1 down to 0, and within a level the sequences with n(b) > qt in
// order of decreasing n(b) (a counting sort): entry position =
// off(qt) + rank(b), where rank(b) = #{b' : n(b') > n(b)} + (place among
// equal n), and off(qt) = sum over levels above qt of their sizes.
// ---------------------------------------------------------------------------
constexpr int kSchedThreads = 1024;

// out[i] = sum of v[j] for j > i (exclusive suffix sum), i < n, in place.
__device__ void block_suffix_sum(int* v, int n, int* part) {
  const int t = threadIdx.x;
  const int per = (n + kSchedThreads - 1) / kSchedThreads;
  const int lo = min(n, t * per), hi = min(n, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += v[i];
  part[t] = sum;
  __syncthreads();
  // suffix scan of the per-thread sums (Hillis-Steele)
  for (int d = 1; d < kSchedThreads; d <<= 1) {
    const int add = (t + d < kSchedThreads) ? part[t + d] : 0;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  int acc = (t + 1 < kSchedThreads) ? part[t + 1] : 0;  // sum of chunks after this one
  for (int i = hi - 1; i >= lo; --i) {
    const int x = v[i];
    v[i] = acc;
    acc += x;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kSchedThreads) void prefill_schedule_kernel(PrefillArgs a,
                                                                        int32_t* list,
                                                                        int32_t* count) {
  __shared__ int hist[kSchedMaxQtiles + 1];  // sequences per live-tile count
  __shared__ int lvl[kSchedMaxQtiles + 1];   // per level: its offset in the list
  __shared__ int part[kSchedThreads];
  const int NQ = a.n_qtiles, t = threadIdx.x;
  for (int i = t; i <= NQ; i += kSchedThreads) hist[i] = 0;
  __syncthreads();
  int flags = 0;
  for (int b = t; b < a.B; b += kSchedThreads) {
    const Span sq = read_span(a.cu_q, b, a.s_max_q, a.q_rows, kErrQLen);
    const Span sk = read_span(a.cu_kv, b, a.s_max_kv, a.kv_rows, kErrKvLen);
    flags |= sq.flags | sk.flags;
    atomicAdd(&hist[(sq.len + a.tq - 1) / a.tq], 1);
  }
  report(a.err, flags);
  __syncthreads();
  // hist[n] -> #{b : n(b) > n} (the first rank of count n, and the size of
  // level n), then the level sizes -> level offsets
  block_suffix_sum(hist, NQ + 1, part);
  for (int i = t; i < NQ; i += kSchedThreads) lvl[i] = hist[i];
  __syncthreads();
  block_suffix_sum(lvl, NQ, part);
  if (t == 0) *count = NQ > 0 ? lvl[0] + hist[0] : 0;
  // ranks: the rank counter of count n starts at hist[n] (sequences with
  // more live tiles come first) and is bumped per sequence
  for (int b = t; b < a.B; b += kSchedThreads) {
    const Span sq = read_span(a.cu_q, b, a.s_max_q, a.q_rows, kErrQLen);
    const int n = (sq.len + a.tq - 1) / a.tq;
    if (n == 0) continue;
    const int r = atomicAdd(&hist[n], 1);
    for (int qt = 0; qt < n; ++qt) list[lvl[qt] + r] = (b << 16) | qt;
  }
}

// With a measurement event pair the kernel is launched through
// hipExtLaunchKernelGGL, which stamps the events with the dispatch's own start
// and end.
template <int D, int GRID>
static hipError_t launch_prefill_g(const PrefillArgs& a, int grid, hipStream_t st, hipEvent_t ev0,
                                   hipEvent_t ev1) {
  if (ev0)
    hipExtLaunchKernelGGL(prefill_kernel<D, GRID>, dim3(grid), dim3(PrefillCfg<D>::THREADS), 0, st,
                          ev0, ev1, 0, a);
  else
    prefill_kernel<D, GRID><<<grid, PrefillCfg<D>::THREADS, 0, st>>>(a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_prefill_d(const PrefillArgs& a, int grid, hipStream_t st, hipEvent_t ev0,
                                   hipEvent_t ev1) {
  if (a.sched_count) return launch_prefill_g<D, kGridList>(a, grid, st, ev0, ev1);
  if (a.tile_map) return launch_prefill_g<D, kGridMap>(a, grid, st, ev0, ev1);
  return launch_prefill_g<D, kGridSmax>(a, grid, st, ev0, ev1);
}

static_assert(PrefillCfg<32>::ROWS == prefill_rows(32) && PrefillCfg<64>::ROWS == prefill_rows(64) &&
                  PrefillCfg<128>::ROWS == prefill_rows(128) &&
                  PrefillCfg<256>::ROWS == prefill_rows(256),
              "plan and kernel disagree on the prefill tile");

hipError_t launch_prefill_schedule(const PrefillArgs& a, int32_t* list, int32_t* count,
                                   hipStream_t st) {
  if (a.n_qtiles > kSchedMaxQtiles) return hipErrorInvalidValue;
  prefill_schedule_kernel<<<1, kSchedThreads, 0, st>>>(a, list, count);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, int D, int grid, hipStream_t st, hipEvent_t ev0,
                          hipEvent_t ev1) {
  switch (D) {
    case 32: return launch_prefill_d<32>(a, grid, st, ev0, ev1);
    case 64: return launch_prefill_d<64>(a, grid, st, ev0, ev1);
    case 128: return launch_prefill_d<128>(a, grid, st, ev0, ev1);
    case 256: return launch_prefill_d<256>(a, grid, st, ev0, ev1);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vattn
