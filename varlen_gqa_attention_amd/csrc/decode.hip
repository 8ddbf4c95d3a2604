// Split-KV decode for varlen GQA on gfx950, plus the log-sum-exp merge.
//
// Method (AstrAI commit log for csrc/kernels/gqa_decode_attn.cu, split-KV
// commit; split-K blog post, The Context: Why Split-K Matters): the KV range
// of each (sequence, kv head) is cut into `nsplit` contiguous chunks that run
// on separate workgroups; each emits an unnormalised partial (O, m, l) and a
// log-sum-exp merge combines them. With one split the same workgroup
// normalises and writes the output directly. By default the merge is a
// separate combine kernel. A plan option moves it into the split kernel: the
// last split workgroup of a unit to finish (a system-scope counter, reset by
// that workgroup so the next launch or graph replay starts from zero) merges
// the unit's partials, which saves a launch but needs write-through partial
// stores and cache-bypassing reads; it measures no faster on gfx950.
//
// Workgroup = (sequence b, kv head hk, head block hb, split s). Its waves take
// the 32-key tiles of the chunk round-robin, keep their own running
// (m, l, O) state, and merge through LDS at the end, so the tile loop itself
// has no workgroup barrier. Each wave double-buffers its tiles in registers
// (two tiles in flight, ping-pong without register copies, so the wait for a
// tile never covers the tile issued after it). Softmax works in base 2 on
// t = s * scale * log2(e) (the scale folds into the exponent in fp32; Q is not
// rounded after scaling); outputs convert back with ln 2.
//
// Two compute paths (dispatch between an MMA and a scalar kernel by G, as in
// the AstrAI "dispatch_decode" commit):
//  * MFMA: the G query heads of a KV head are the 16-wide N dimension of
//    v_mfma_f32_16x16x32_bf16 (heads folded into the matmul dimension, the
//    kernbench "GQA via M-fold" finding). S^T = K Q^T takes K straight from
//    global memory as the A operand (16 contiguous bytes per lane); its
//    output layout is reused unchanged as the P^T operand of O^T = V^T P^T,
//    and V^T comes from a wave-private, swizzled LDS tile through the
//    gfx950 transposed LDS read.
//  * Wave: for small G (GEMV-shaped work) each 16-byte load lane holds 8
//    d-values of one key; dot products use v_dot2_f32_bf16 and DPP row
//    reductions; P V is plain FMAs.
#include <hip/hip_ext.h>

#include "device.hpp"
#include "launch.hpp"

namespace vattn {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
typedef bf16x2 bf16x2_t;

// Reinterpret one 32-bit word as two bf16. The word is taken by value: this
// hipcc miscompiles __builtin_bit_cast applied directly to an ext-vector
// element expression (it reads element 0 whatever the index).
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2_t, w); }

constexpr uint32_t kBf16One2 = 0x3F803F80u;  // two bf16 ones

__device__ __forceinline__ bf16x4 lds_read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
}

// Orders a wave's LDS writes before its later LDS reads (and vice versa).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct UnitCoords {
  int b, hk, hb, s, unit;
};

// Workgroup i = split s = i / n_units of the unit at position i % n_units:
// consecutive workgroups are different units at the same split, so with
// workgroups dispatched round-robin over the 8 XCDs each XCD streams whole
// units (for 8 units, one KV head per XCD) rather than a slice of every head.
// Position p of split s holds unit (p + 8 s) mod n_units: a unit keeps its
// XCD (p mod 8) when n_units is a multiple of 8, while its successive splits
// move 8 positions, i.e. one step of an XCD's own dispatch order. Within an
// XCD, workgroups go to its shader engines in turn by dispatch position, and
// a workgroup waits for a free CU in its engine even when others are idle;
// without the shift all splits of a unit share one engine, and a few long
// sequences can queue on one engine while the rest of the XCD idles.
// Unit r = (b Hkv + j) head_blocks + hb takes KV head (j + b) mod Hkv of
// sequence b: over a batch the unit slot j, and with it the XCD, cycles
// through all KV heads instead of always holding the same one (the heads'
// rows sit at fixed offsets inside each token's row, so a fixed head per XCD
// keeps each XCD on the same slice of every row).
__device__ __forceinline__ UnitCoords unit_of_block(const DecodeArgs& a) {
  int bid = blockIdx.x;
  UnitCoords u;
  const int n_units = gridDim.x / a.nsplit;
  u.s = bid / n_units;
  bid = (int)(((int64_t)(bid % n_units) + 8 * (int64_t)u.s) % n_units);
  u.unit = bid;
  u.hb = bid % a.head_blocks;
  bid /= a.head_blocks;
  u.b = bid / a.Hkv;
  u.hk = (bid % a.Hkv + u.b) % a.Hkv;
  return u;
}

// Drives one wave's tiles w, w + NW, ... (fewer than ntiles in all) through
// two register buffers, A holding tile t and B tile t + NW, so two tiles are
// in flight. Every load in the steady-state loop is unconditional, so the
// number of loads outstanding at each wait is the same on all paths and a
// wait covers only the tile it needs; the last one to three tiles run in
// straight-line tails that issue no further loads (B re-reads tile w only
// when the wave has a single tile).
template <int NW, typename Buf, typename Load, typename Proc>
__device__ __forceinline__ void pipeline_tiles(int w, int ntiles, Buf& A, Buf& B, Load load,
                                               Proc proc) {
  if (w >= ntiles) return;
  const int nt = (ntiles - 1 - w) / NW + 1;
  load(w, A);
  load(w + (nt > 1 ? NW : 0), B);
  int t = w, left = nt;
  for (; left > 3; left -= 2, t += 2 * NW) {
    proc(t, A);
    load(t + 2 * NW, A);
    proc(t + NW, B);
    load(t + 3 * NW, B);
  }
  if (left == 3) {
    proc(t, A);
    load(t + 2 * NW, A);
    proc(t + NW, B);
    proc(t + 2 * NW, A);
  } else {
    proc(t, A);
    if (left == 2) proc(t + NW, B);
  }
}

__device__ __forceinline__ void store_out(const DecodeArgs& a, int qrow, int hq, int d, float val) {
  __bf16 ob = (__bf16)val;
  a.out[(int64_t)qrow * a.o_rs + (int64_t)hq * a.D + d] = __builtin_bit_cast(uint16_t, ob);
}

// Writes O = 0, LSE = -inf (no visible key) for heads [h0, h0 + nh).
__device__ __forceinline__ void store_empty(const DecodeArgs& a, int qrow, int h0, int nh) {
  for (int idx = threadIdx.x; idx < nh * a.D; idx += blockDim.x) {
    const int h = idx / a.D, d = idx % a.D;
    store_out(a, qrow, h0 + h, d, 0.f);
    if (d == 0) a.lse[(int64_t)qrow * a.Hq + h0 + h] = kNegInf;
  }
}

// Partial loads. In the fused merge the partials of other workgroups (other
// XCDs, other L2s) are read with system-scope loads, which bypass the caches;
// they were written with system-scope (write-through) stores.
template <bool COHERENT>
__device__ __forceinline__ float ld_part(const float* p) {
  if constexpr (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  else return *p;
}
template <bool COHERENT>
__device__ __forceinline__ void st_part(float* p, float v) {
  if constexpr (COHERENT) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  else *p = v;
}

// LSE merge of split partials of heads [h0, h0 + nh) of sequence b, written
// as bf16 out and fp32 LSE. A partial is (O, m, l, lt): lt sums the weights
// as they entered the P V product (rounded to bf16 on the MFMA path, equal to
// l on the wave path); O is normalised by the merged lt, so that the output
// is a weighted mean of V rows with exactly the weights used, and the LSE is
// taken from l. Used by the combine kernel and by the in-kernel merge, with
// the same arithmetic in both.
//
// Each head takes kMergeTph(D) = max(32, D / 4) threads, each of which owns 4
// consecutive d (threads past D / 4 only help with the slot loads), so a
// 32-lane half never spans two heads; nh * kMergeTph(D) <= blockDim.x. Slots
// are taken in chunks of 32: lane j of each 32-lane half loads slot s0 + j's
// (m, l, lt), the chunk max and the weighted sums are half-wave reductions,
// and the weights reach every lane of the half by readlane for the O sum
// (16-byte partial loads). The first chunk's loads (slots clamped to the
// allocated nsplit) are issued before `lens()` runs, so the combine kernel
// reads cu_seqlens while its partials are in flight; lens() returns
// {query row, n_live}, or n_live < 0 to write nothing. Slots at or past
// n_live may hold stale values from another launch and are excluded with
// selects (never multiplied by a zero weight, which would keep a NaN). Chunks
// after the first merge online (running max, rescaled sums).
struct MergeTarget {
  int qrow, n_live;
};

template <int D>
constexpr int kMergeTph = D / 4 > 32 ? D / 4 : 32;

template <bool COHERENT>
__device__ __forceinline__ f32x4 ld_part4(const float* p) {
  if constexpr (COHERENT) {
    return f32x4{ld_part<true>(p), ld_part<true>(p + 1), ld_part<true>(p + 2), ld_part<true>(p + 3)};
  } else {
    return *reinterpret_cast<const f32x4*>(p);
  }
}

template <int D, bool COHERENT, typename Lens>
__device__ __forceinline__ void merge_partials(const DecodeArgs& a, int b, int h0, int nh, Lens lens) {
  constexpr int TPH = kMergeTph<D>;
  constexpr int CH = 32;
  const float* pml = reinterpret_cast<const float*>(a.part_ml);
  const int idx = threadIdx.x;
  const int lane = idx & 63, sl = lane & 31;
  const int h = idx / TPH, dq = idx % TPH;
  const bool own_d = dq < D / 4;
  const int d = own_d ? 4 * dq : 0;
  const int hq = h0 + min(h, nh - 1);
  const int64_t base = (int64_t)(b * a.Hq + hq) * a.nsplit;
  f32x4 ml, po[CH];
  auto load_chunk = [&](int s0, int n_slots) {
    ml = ld_part4<COHERENT>(pml + 4 * (base + min(s0 + sl, n_slots - 1)));
#pragma unroll
    for (int j = 0; j < CH; ++j)
      po[j] = ld_part4<COHERENT>(a.part_o + (base + min(s0 + j, n_slots - 1)) * D + d);
  };
  load_chunk(0, a.nsplit);
  const MergeTarget tg = lens();
  if (tg.n_live < 0 || h >= nh) return;  // uniform per 32-lane half
  float M = kNegInf, L = 0.f, Lt = 0.f;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < tg.n_live; s0 += CH) {
    if (s0 > 0) load_chunk(s0, tg.n_live);
    const bool live = s0 + sl < tg.n_live;
    const float Mn = fmaxf(M, group_max<32>(live ? ml[0] : kNegInf));
    const float Ms = (Mn == kNegInf) ? 0.f : Mn;
    const float r = fast_exp2(M - Ms);
    const float wl = live ? fast_exp2(ml[0] - Ms) : 0.f;
    L = L * r + group_sum<32>(live ? wl * ml[1] : 0.f);
    Lt = Lt * r + group_sum<32>(live ? wl * ml[2] : 0.f);
    O *= r;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const float w0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), j));
      const float w1 =
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), 32 + j));
      const float wj = (lane & 32) ? w1 : w0;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      O += (s0 + j < tg.n_live) ? wj * po[j] : z;
    }
    M = Mn;
  }
  if (!own_d) return;
  const float inv = (Lt > 0.f) ? 1.f / Lt : 0.f;
  u32x2 ov;
  ov[0] = pack_bf16x2(O[0] * inv, O[1] * inv);
  ov[1] = pack_bf16x2(O[2] * inv, O[3] * inv);
  *reinterpret_cast<u32x2*>(a.out + (int64_t)tg.qrow * a.o_rs + (int64_t)hq * D + d) = ov;
  if (dq == 0) a.lse[(int64_t)tg.qrow * a.Hq + hq] = (L > 0.f) ? (M + fast_log2(L)) * kLn2 : kNegInf;
}

// Cross-wave merge of per-wave (m, l, O) states held in LDS, then the
// epilogue: direct (normalised bf16 out + LSE) or split partial; in fused
// mode the last split workgroup of the unit then merges all partials.
// mo: [NW][HPB][D] floats, mml: [NW][HPB] (m, l, lt, -). One thread per
// (head, 4 consecutive d), so LDS reads and global stores are 8-16 bytes.
template <int D, int NW, int HPB, bool FUSED>
__device__ __forceinline__ void finish_workgroup(const DecodeArgs& a, const UnitCoords& u, int Lk,
                                                 int qrow, int h0, int nh, const float* mo,
                                                 const float4* mml, int* flag) {
  constexpr int D4 = D / 4;
  for (int idx = threadIdx.x; idx < nh * D4; idx += NW * 64) {
    const int h = idx / D4, d = 4 * (idx % D4);
    float4 ml[NW];
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      ml[w] = mml[w * HPB + h];
      M = fmaxf(M, ml[w].x);
    }
    const float Ms = (M == kNegInf) ? 0.f : M;
    float L = 0.f, Lt = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = fast_exp2(ml[w].x - Ms);
      L += wt * ml[w].y;
      Lt += wt * ml[w].z;
      O += wt * *reinterpret_cast<const f32x4*>(mo + (w * HPB + h) * D + d);
    }
    const int hq = h0 + h;
    if (a.direct) {
      const float inv = (Lt > 0.f) ? 1.f / Lt : 0.f;
      u32x2 ov;
      ov[0] = pack_bf16x2(O[0] * inv, O[1] * inv);
      ov[1] = pack_bf16x2(O[2] * inv, O[3] * inv);
      *reinterpret_cast<u32x2*>(a.out + (int64_t)qrow * a.o_rs + hq * D + d) = ov;
      if (d == 0)
        a.lse[(int64_t)qrow * a.Hq + hq] = (L > 0.f) ? (M + fast_log2(L)) * kLn2 : kNegInf;
    } else {
      const int64_t pidx = ((int64_t)(u.b * a.Hq + hq) * a.nsplit + u.s);
      float* pml = reinterpret_cast<float*>(a.part_ml);
      if (FUSED && !a.fused_local) {
#pragma unroll
        for (int i = 0; i < 4; ++i) st_part<true>(a.part_o + pidx * D + d + i, O[i]);
        if (d == 0) {
          st_part<true>(pml + 4 * pidx, M);
          st_part<true>(pml + 4 * pidx + 1, L);
          st_part<true>(pml + 4 * pidx + 2, Lt);
        }
      } else {
        *reinterpret_cast<f32x4*>(a.part_o + pidx * D + d) = O;
        if (d == 0) a.part_ml[pidx] = float4{M, L, Lt, 0.f};
      }
    }
  }
  if (!FUSED || a.direct) return;
  // In-kernel merge. Once every thread's partial stores have completed (the
  // wait below) the workgroup counts itself in with an atomic, and the last
  // live split of the unit reads all of the unit's partials and merges them.
  // Two forms. XCD-local (fused_local): the plan made every split of a unit
  // land on one XCD (workgroups go round-robin to the 8 XCDs and the unit
  // count is a multiple of 8), so plain stores reach that XCD's L2 and plain
  // loads from another CU of it, whose L1 holds no copy of lines it has not
  // read in this launch, see them. Otherwise the partials are written through
  // to memory and read with cache-bypassing loads. Neither needs an L2
  // write-back or invalidation, unlike a device-scope fence.
  const int n_live = (Lk + a.chunk_keys - 1) / a.chunk_keys;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev =
        __hip_atomic_fetch_add(&a.counters[u.unit], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    const int last = (prev == n_live - 1);
    if (last) __hip_atomic_store(&a.counters[u.unit], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    *flag = last;
  }
  __syncthreads();
  if (!*flag) return;
  constexpr int HPP = NW * 64 / kMergeTph<D>;  // heads per pass
  for (int hc = 0; hc < nh; hc += HPP) {
    auto lens = [&] { return MergeTarget{qrow, n_live}; };
    if (a.fused_local) merge_partials<D, false>(a, u.b, h0 + hc, min(HPP, nh - hc), lens);
    else merge_partials<D, true>(a, u.b, h0 + hc, min(HPP, nh - hc), lens);
  }
}

// ---------------------------------------------------------------------------
// MFMA path
// ---------------------------------------------------------------------------
template <int D, int NW, bool FUSED, bool GATHER>
__global__ __launch_bounds__(NW * 64, D == 128 ? 2 : 1) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int KS = D / 32;     // 32-wide k-steps of Q K^T
  constexpr int DB = D / 16;     // 16-wide d blocks of P V
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  // keys per wave iteration: 32 (P V on 16x16x32 MFMAs) at D <= 64; 16 (P V on
  // 16x16x16 MFMAs) at D >= 128, so that two tiles in flight fit the
  // registers of two waves per SIMD at D = 128 (two workgroups per CU) and of
  // one at D = 256
  constexpr int TILE = D >= 128 ? 16 : 32;
  constexpr int KB = TILE / 16;  // 16-key blocks of Q K^T per tile
  constexpr int DV = TILE * D / 512;  // 16-byte V loads per lane per tile
  constexpr int HPB = 16;        // heads per workgroup
  constexpr int STAGE_BYTES = NW * TILE * D * 2;
  constexpr int MERGE_BYTES = NW * HPB * D * 4 + 4 * NW * HPB * 4;
  constexpr int LDS_BYTES = STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES : MERGE_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  __shared__ int s_flag;

  const UnitCoords u = unit_of_block(a);
  if (u.b >= a.B) return;
  const Span sq = read_span(a.cu_q, u.b, a.s_max_q, a.q_rows, kErrQLen);
  const Span sk = read_span(a.cu_kv, u.b, a.s_max_kv, a.kv_rows, kErrKvLen);
  if (u.s == 0 && u.hb == 0 && u.hk == 0 && threadIdx.x == 0) report(a.err, sq.flags | sk.flags);
  if (sq.len == 0) return;
  const int Lk = sk.len;
  const int qrow = sq.start;
  const int h0 = u.hk * a.G + u.hb * HPB;
  const int nh = min(HPB, a.G - u.hb * HPB);
  const int kbeg = u.s * a.chunk_keys;
  if (!a.direct && kbeg >= Lk) {  // empty split: never merged
    if (FUSED && Lk == 0 && u.s == 0) store_empty(a, qrow, h0, nh);
    return;
  }
  const int kend = min(kbeg + a.chunk_keys, Lk);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int hl = lane & 15, g4 = lane >> 4;

  // Q^T operand: lane holds Q[head hl][32 ks + 8 g4 .. +8]; absent heads are 0.
  bf16x8 qv[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 x = {0, 0, 0, 0};
    if (hl < nh) x = ld16(a.q + (int64_t)qrow * a.q_rs + (h0 + hl) * D + 32 * ks + 8 * g4);
    qv[ks] = __builtin_bit_cast(bf16x8, x);
  }

  // l: sum of the fp32 weights (for the LSE); lt: sum of the same weights
  // rounded to bf16 as they enter the P V product (normalises O)
  float m = kNegInf, l = 0.f, lt = 0.f;
  f32x4 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint8_t* vst = lds + w * TILE * D * 2;
  const int64_t krs = a.k_rs, vrs = a.v_rs;
  // contiguous keys: row = key (bases offset to the sequence); gathered keys:
  // row = kv_idx[sk.start + key]
  const int64_t seq_row = GATHER ? 0 : sk.start;
  const uint16_t* kbase = a.k + seq_row * krs + u.hk * D;
  const uint16_t* vbase = a.v + seq_row * vrs + u.hk * D;
  const int ntiles = (kend > kbeg) ? (kend - kbeg + TILE - 1) / TILE : 0;
  int gflags = 0;
  auto row_of = [&](int idx_or_key) -> int64_t {
    if constexpr (GATHER) {
      int r = idx_or_key;
      if (r < 0 || r >= a.kv_bound) {
        gflags = kErrIndex;
        r = r < 0 ? 0 : (int)(a.kv_bound - 1);
      }
      return r;
    } else {
      return idx_or_key;
    }
  };

  // Gathered keys: each register buffer also holds the row indices of the
  // tile it loads next (fetched when it issues its current tile, 2 NW tiles
  // ahead), so no K/V load waits on an index load issued after other tiles.
  struct TileRegs {
    u32x4 k[KB][KS], v[DV];
    int rk[GATHER ? KB : 1], rv[GATHER ? DV : 1];
  } A, B;
  auto fetch_rows = [&](int t, TileRegs& r) {
    if constexpr (GATHER) {
      const int key0 = kbeg + t * TILE;
#pragma unroll
      for (int kb2 = 0; kb2 < KB; ++kb2)
        r.rk[kb2] = a.kv_idx[sk.start + min(key0 + 16 * kb2 + hl, kend - 1)];
#pragma unroll
      for (int i = 0; i < DV; ++i)
        r.rv[i] = a.kv_idx[sk.start + min(key0 + (i * 64 + lane) / CPR, kend - 1)];
    }
  };
  auto load_tile = [&](int t, TileRegs& r) {
    const int key0 = kbeg + t * TILE;
#pragma unroll
    for (int kb2 = 0; kb2 < KB; ++kb2) {
      const int64_t row = row_of(GATHER ? r.rk[kb2] : min(key0 + 16 * kb2 + hl, kend - 1));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) r.k[kb2][ks] = ld16(kbase + row * krs + 32 * ks + 8 * g4);
    }
#pragma unroll
    for (int i = 0; i < DV; ++i) {
      const int qi = i * 64 + lane;
      const int64_t row = row_of(GATHER ? r.rv[i] : min(key0 + qi / CPR, kend - 1));
      r.v[i] = ld16(vbase + row * vrs + 8 * (qi % CPR));
    }
    fetch_rows(t + 2 * NW, r);
  };

  auto process_tile = [&](int t, const u32x4 (&kr)[KB][KS], const u32x4 (&vr)[DV], auto lo_tag) {
    constexpr bool lo = decltype(lo_tag)::value;
    const int key0 = kbeg + t * TILE;
    // stage V (row-major [key][d], swizzled) in this wave's LDS slice
#pragma unroll
    for (int i = 0; i < DV; ++i) {
      const int qi = i * 64 + lane;
      const int row = qi / CPR, c = qi % CPR;
      *reinterpret_cast<u32x4*>(vst + row * D * 2 + swz_tr16<D>(row, c) * 16) = vr[i];
    }
    // S^T = K Q^T for keys [16 kb2, 16 kb2 + 16)
    f32x4 sacc[KB];
#pragma unroll
    for (int kb2 = 0; kb2 < KB; ++kb2) {
      sacc[kb2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sacc[kb2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, kr[kb2][ks]), qv[ks], sacc[kb2], 0, 0, 0);
    }
    // online softmax; lane holds keys 16 kb2 + 4 g4 + i of head hl
    float sc[4 * KB];
    float mx = kNegInf;
#pragma unroll
    for (int kb2 = 0; kb2 < KB; ++kb2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key0 + 16 * kb2 + 4 * g4 + i;
        const float x = (key < kend) ? sacc[kb2][i] * a.c : kNegInf;
        sc[kb2 * 4 + i] = x;
        mx = fmaxf(mx, x);
      }
    mx = max_xor32(max_xor16(mx));
    const float mnew = fmaxf(m, mx);
    const float msub = (mnew == kNegInf) ? 0.f : mnew;
    const float alpha = fast_exp2(m - msub);
    float psum = 0.f;
    float p[4 * KB];
#pragma unroll
    for (int i = 0; i < 4 * KB; ++i) {
      p[i] = fast_exp2(sc[i] - msub);
      psum += p[i];
    }
    l = l * alpha + psum;
    m = mnew;
#pragma unroll
    for (int i = 0; i < DB; ++i) o[i] *= alpha;
    // For sequences of fewer than 256 keys (lo) P enters P V as two bf16
    // operands, its rounding and the remainder p - bf16(p) rounded again (one
    // more MFMA per d block), so the weights are exact to about 2^-17: with
    // bf16 weights alone, a row whose few comparable weights multiply V rows
    // far apart misses the output's rounding by up to 2^-8 max|v - O|; over
    // more keys the weights' rounding errors average out.
    uint32_t pw[2 * KB], pwl[2 * KB];
    float ptsum = 0.f;
#pragma unroll
    for (int j = 0; j < 2 * KB; ++j) {
      pw[j] = pack_bf16x2(p[2 * j], p[2 * j + 1]);
      ptsum = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pw[j]), as_bf16x2(kBf16One2), ptsum, false);
    }
    if constexpr (lo) {
#pragma unroll
      for (int j = 0; j < 2 * KB; ++j) {
        pwl[j] = pack_bf16x2(p[2 * j] - bf16_lo(pw[j]), p[2 * j + 1] - bf16_hi(pw[j]));
        ptsum =
            __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pwl[j]), as_bf16x2(kBf16One2), ptsum, false);
      }
    }
    lt = lt * alpha + ptsum;

    wave_lds_sync();
    // O^T += V^T P^T; V^T operand lane: d = 16 db + hl, keys 4 g4 + j (and
    // 16 + 4 g4 + j for 32-key tiles: the key order of the P^T operand above)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = 16 * db + 4 * (hl & 3);
      const int r1 = 4 * g4 + (hl >> 2);
      const int ch = col >> 3, half = (col >> 2) & 1;
      const bf16x4 x1 = lds_read_tr(vst + r1 * D * 2 + swz_tr16<D>(r1, ch) * 16 + half * 8);
      if constexpr (KB == 2) {
        const int r2 = r1 + 16;
        const bf16x4 x2 = lds_read_tr(vst + r2 * D * 2 + swz_tr16<D>(r2, ch) * 16 + half * 8);
        const bf16x8 vt = __builtin_shufflevector(x1, x2, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 pt = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
        const bf16x8 ptl = __builtin_bit_cast(bf16x8, u32x4{pwl[0], pwl[1], pwl[2], pwl[3]});
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pt, o[db], 0, 0, 0);
        if constexpr (lo) o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, ptl, o[db], 0, 0, 0);
      } else {
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        const s16x4 pt = __builtin_bit_cast(s16x4, u32x2{pw[0], pw[1]});
        const s16x4 ptl = __builtin_bit_cast(s16x4, u32x2{pwl[0], pwl[1]});
        o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, x1), pt, o[db],
                                                         0, 0, 0);
        if constexpr (lo)
          o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, x1), ptl,
                                                           o[db], 0, 0, 0);
      }
    }
    wave_lds_sync();
  };

  if (w < ntiles) {
    fetch_rows(w, A);
    fetch_rows(w + (w + NW < ntiles ? NW : 0), B);
  }
  // sequences of fewer than 256 keys take P V with the remainder of P (see
  // process_tile); each form is its own copy of the tile loop
  if (Lk < 256)
    pipeline_tiles<NW>(w, ntiles, A, B, [&](int t, TileRegs& r) { load_tile(t, r); },
                       [&](int t, TileRegs& r) {
                         process_tile(t, r.k, r.v, std::integral_constant<bool, true>{});
                       });
  else
    pipeline_tiles<NW>(w, ntiles, A, B, [&](int t, TileRegs& r) { load_tile(t, r); },
                       [&](int t, TileRegs& r) {
                         process_tile(t, r.k, r.v, std::integral_constant<bool, false>{});
                       });
  if constexpr (GATHER) report(a.err, gflags);
  // l: each lane summed its own 8 keys per tile; add the four key groups
  l = sum_xor32(sum_xor16(l));
  lt = sum_xor32(sum_xor16(lt));

  __syncthreads();  // staging area becomes the merge area
  float* mo = reinterpret_cast<float*>(lds);
  float4* mml = reinterpret_cast<float4*>(mo + NW * HPB * D);
#pragma unroll
  for (int db = 0; db < DB; ++db)
    *reinterpret_cast<f32x4*>(mo + (w * HPB + hl) * D + 16 * db + 4 * g4) = o[db];
  if (g4 == 0) mml[w * HPB + hl] = float4{m, l, lt, 0.f};
  __syncthreads();
  finish_workgroup<D, NW, HPB, FUSED>(a, u, Lk, qrow, h0, nh, mo, mml, &s_flag);
}

// ---------------------------------------------------------------------------
// Wave (VALU) path for small G
// ---------------------------------------------------------------------------
template <int D, int NW, int GM, bool FUSED, bool GATHER>
__global__ __launch_bounds__(NW * 64) void decode_wave_kernel(DecodeArgs a) {
  constexpr int LPR = D / 8;             // lanes per key row (8 d-values each)
  constexpr int RPI = 64 / LPR;          // key rows per load instruction
  constexpr int TILE = (D <= 64) ? 32 : 16;  // keys per wave iteration (two tiles in flight)
  constexpr int NI = TILE / RPI;         // loads per tile for K and for V
  constexpr int MERGE_FLOATS = NW * GM * D + 4 * NW * GM;
  __shared__ __attribute__((aligned(16))) float lds[MERGE_FLOATS];
  __shared__ int s_flag;

  const UnitCoords u = unit_of_block(a);
  if (u.b >= a.B) return;
  const Span sq = read_span(a.cu_q, u.b, a.s_max_q, a.q_rows, kErrQLen);
  const Span sk = read_span(a.cu_kv, u.b, a.s_max_kv, a.kv_rows, kErrKvLen);
  if (u.s == 0 && u.hb == 0 && u.hk == 0 && threadIdx.x == 0) report(a.err, sq.flags | sk.flags);
  if (sq.len == 0) return;
  const int Lk = sk.len;
  const int qrow = sq.start;
  const int h0 = u.hk * a.G + u.hb * GM;
  const int nh = min(GM, a.G - u.hb * GM);
  const int kbeg = u.s * a.chunk_keys;
  if (!a.direct && kbeg >= Lk) {
    if (FUSED && Lk == 0 && u.s == 0) store_empty(a, qrow, h0, nh);
    return;
  }
  const int kend = min(kbeg + a.chunk_keys, Lk);

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane / LPR, c = lane % LPR;

  u32x4 qw[GM];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    qw[g] = u32x4{0, 0, 0, 0};
    if (g < nh) qw[g] = ld16(a.q + (int64_t)qrow * a.q_rs + (h0 + g) * D + 8 * c);
  }
  float m[GM], l[GM], o[GM][8];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[g][j] = 0.f;
  }
  const int64_t krs = a.k_rs, vrs = a.v_rs;
  const int64_t seq_row = GATHER ? 0 : sk.start;  // gathered: rows come from kv_idx
  const uint16_t* kbase = a.k + seq_row * krs + u.hk * D + 8 * c;
  const uint16_t* vbase = a.v + seq_row * vrs + u.hk * D + 8 * c;
  const int ntiles = (kend > kbeg) ? (kend - kbeg + TILE - 1) / TILE : 0;
  int gflags = 0;

  // gathered keys: the row indices of a buffer's next tile are fetched when
  // it issues its current one (as in the MFMA path)
  auto fetch_rows = [&](int t, int (&ix)[NI]) {
    if constexpr (GATHER) {
      const int key0 = kbeg + t * TILE;
#pragma unroll
      for (int i = 0; i < NI; ++i) ix[i] = a.kv_idx[sk.start + min(key0 + i * RPI + r, kend - 1)];
    }
  };
  auto load_tile = [&](int t, u32x4 (&kr)[NI], u32x4 (&vr)[NI], int (&ix)[NI], int t_next) {
    const int key0 = kbeg + t * TILE;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      int64_t row = min(key0 + i * RPI + r, kend - 1);
      if constexpr (GATHER) {
        int rr = ix[i];
        if (rr < 0 || rr >= a.kv_bound) {
          gflags = kErrIndex;
          rr = rr < 0 ? 0 : (int)(a.kv_bound - 1);
        }
        row = rr;
      }
      kr[i] = ld16(kbase + row * krs);
      vr[i] = ld16(vbase + row * vrs);
    }
    fetch_rows(t_next, ix);
  };

  auto process_tile = [&](int t, const u32x4 (&kr)[NI], const u32x4 (&vr)[NI]) {
    const int key0 = kbeg + t * TILE;
    float s[NI][GM];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int g = 0; g < GM; ++g) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qw[g][j]), as_bf16x2(kr[i][j]), acc,
                                                false);
        s[i][g] = acc;
      }
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int g = 0; g < GM; ++g) s[i][g] = group_sum<LPR>(s[i][g]);

#pragma unroll
    for (int g = 0; g < GM; ++g) {
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const bool ok = key0 + i * RPI + r < kend;
        s[i][g] = ok ? s[i][g] * a.c : kNegInf;
        mx = fmaxf(mx, s[i][g]);
      }
      mx = across_groups_max<LPR>(mx);
      const float mnew = fmaxf(m[g], mx);
      const float msub = (mnew == kNegInf) ? 0.f : mnew;
      const float alpha = fast_exp2(m[g] - msub);
      m[g] = mnew;
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        s[i][g] = fast_exp2(s[i][g] - msub);
        psum += s[i][g];
      }
      l[g] = l[g] * alpha + psum;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[g][j] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float vf[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vf[2 * j] = bf16_lo(vr[i][j]);
        vf[2 * j + 1] = bf16_hi(vr[i][j]);
      }
#pragma unroll
      for (int g = 0; g < GM; ++g)
#pragma unroll
        for (int j = 0; j < 8; ++j) o[g][j] = fmaf(s[i][g], vf[j], o[g][j]);
    }
  };

  u32x4 kA[NI], vA[NI], kB[NI], vB[NI];
  int ixA[NI], ixB[NI];
  // Two tiles in flight with unconditional loads, as in pipeline_tiles, but
  // one loop: past the wave's last tile the loads re-read that tile (cached).
  // This path runs long sequences (many tiles per wave), where the re-reads
  // are negligible, and the compact loop keeps register use low.
  if (w < ntiles) {
    const int tl = w + NW * ((ntiles - 1 - w) / NW);
    fetch_rows(w, ixA);
    fetch_rows(min(w + NW, tl), ixB);
    load_tile(w, kA, vA, ixA, min(w + 2 * NW, tl));
    load_tile(min(w + NW, tl), kB, vB, ixB, min(w + 3 * NW, tl));
    for (int t = w; t < ntiles; t += 2 * NW) {
      process_tile(t, kA, vA);
      load_tile(min(t + 2 * NW, tl), kA, vA, ixA, min(t + 4 * NW, tl));
      if (t + NW < ntiles) process_tile(t + NW, kB, vB);
      load_tile(min(t + 3 * NW, tl), kB, vB, ixB, min(t + 5 * NW, tl));
    }
  }
  if constexpr (GATHER) report(a.err, gflags);
  // add the row groups' partial sums (their m are identical)
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    l[g] = across_groups_sum<LPR>(l[g]);
#pragma unroll
    for (int j = 0; j < 8; ++j) o[g][j] = across_groups_sum<LPR>(o[g][j]);
  }
  float* mo = lds;
  float4* mml = reinterpret_cast<float4*>(mo + NW * GM * D);
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      *reinterpret_cast<f32x4*>(mo + (w * GM + g) * D + 8 * c) =
          f32x4{o[g][0], o[g][1], o[g][2], o[g][3]};
      *reinterpret_cast<f32x4*>(mo + (w * GM + g) * D + 8 * c + 4) =
          f32x4{o[g][4], o[g][5], o[g][6], o[g][7]};
    }
  }
  if (lane == 0) {
#pragma unroll
    // P V runs in fp32 here: the weights are used unrounded (lt = l)
    for (int g = 0; g < GM; ++g) mml[w * GM + g] = float4{m[g], l[g], l[g], 0.f};
  }
  __syncthreads();
  finish_workgroup<D, NW, GM, FUSED>(a, u, Lk, qrow, h0, nh, mo, mml, &s_flag);
}

// ---------------------------------------------------------------------------
// LSE combine kernel: one workgroup per (sequence, query head)
// ---------------------------------------------------------------------------
// One 64-thread workgroup per (sequence, 64 / kMergeTph(D) consecutive query
// heads): two heads at D <= 128, one at D = 256.
template <int D>
constexpr int kCombineHeads = 64 / kMergeTph<D>;

template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
  constexpr int HPW = kCombineHeads<D>;
  const int hblocks = (a.Hq + HPW - 1) / HPW;
  const int h0 = (blockIdx.x % hblocks) * HPW, b = blockIdx.x / hblocks;
  if (b >= a.B) return;
  merge_partials<D, false>(a, b, h0, min(HPW, a.Hq - h0), [&] {
    const Span sq = read_span(a.cu_q, b, a.s_max_q, a.q_rows, kErrQLen);
    const Span sk = read_span(a.cu_kv, b, a.s_max_kv, a.kv_rows, kErrKvLen);
    return MergeTarget{sq.start, sq.len == 0 ? -1 : (sk.len + a.chunk_keys - 1) / a.chunk_keys};
  });
}

__global__ void clear_words_kernel(int32_t* w, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) w[i] = 0;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
// With a measurement event pair the kernel is launched through
// hipExtLaunchKernelGGL, which stamps the events with the dispatch's own start
// and end (no separate event packets around it).
template <typename Kern>
static void launch_timed(Kern kern, int grid, int threads, hipStream_t st, hipEvent_t ev0,
                         hipEvent_t ev1, const DecodeArgs& a) {
  if (ev0) hipExtLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, st, ev0, ev1, 0, a);
  else kern<<<grid, threads, 0, st>>>(a);
}

template <int D, bool FUSED, bool GATHER>
static void launch_split(const DecodeArgs& a, int path, int nw, int grid, hipStream_t st,
                         hipEvent_t ev0, hipEvent_t ev1) {
  // 8-wave workgroups only for D <= 128 (the plan never picks them above)
  if constexpr (D <= 128) {
    if (nw == 8) {
      if (path == 2) launch_timed(decode_mfma_kernel<D, 8, FUSED, GATHER>, grid, 512, st, ev0, ev1, a);
      else launch_timed(decode_wave_kernel<D, 8, 4, FUSED, GATHER>, grid, 512, st, ev0, ev1, a);
      return;
    }
  }
  if (path == 2) launch_timed(decode_mfma_kernel<D, 4, FUSED, GATHER>, grid, 256, st, ev0, ev1, a);
  else launch_timed(decode_wave_kernel<D, 4, 4, FUSED, GATHER>, grid, 256, st, ev0, ev1, a);
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs& a, int path, int nw, int grid, int combine_grid,
                                  hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  // the fused-merge and gathered-key code is compiled only into the kernels
  // that use it (gathered keys always merge in the combine kernel)
  if (a.kv_idx) launch_split<D, false, true>(a, path, nw, grid, st, ev0, ev1);
  else if (a.fused && !a.direct) launch_split<D, true, false>(a, path, nw, grid, st, ev0, ev1);
  else launch_split<D, false, false>(a, path, nw, grid, st, ev0, ev1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.direct || a.fused) return e;
  decode_combine_kernel<D><<<combine_grid, 64, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int path, int nw, int grid, int combine_grid,
                         hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  switch (a.D) {
    case 32: return launch_decode_d<32>(a, path, nw, grid, combine_grid, st, ev0, ev1);
    case 64: return launch_decode_d<64>(a, path, nw, grid, combine_grid, st, ev0, ev1);
    case 128: return launch_decode_d<128>(a, path, nw, grid, combine_grid, st, ev0, ev1);
    case 256: return launch_decode_d<256>(a, path, nw, grid, combine_grid, st, ev0, ev1);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_clear_words(int32_t* w, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
  clear_words_kernel<<<blocks, 256, 0, st>>>(w, n);
  return hipGetLastError();
}

}  // namespace vattn
