// Plan-time chooser (host only).
//
// Split rule (AstrAI commit log for csrc/kernels/gqa_decode_attn.cu,
// split-KV commit): choose the split count to fill the device with about two
// workgroups per CU, capped by the KV tile count and by 32; when
// batch * kv_heads already fills the device the rule yields one split and the
// kernel writes the output directly with no combine pass. The count depends
// only on plan-time values (B_max, s_max_kv, heads, CU count), so it is fixed
// inside a captured graph (split-K blog post, The Thinking Process;
// Assumptions and Their Validity). Grids are sized from the declared B_max
// and s_max (cudnn-frontend issue #552, Proposal to evaluate).
//
// Readings where the pages leave the rule open: "about two per CU" is
// ceil(target * n_cu / n_units) with n_units the decode workgroups per split;
// "tile count" is ceil(s_max_kv / 64); splits are contiguous chunks of whole
// tiles and the count is recomputed from the chunk size so that no split is
// empty at s_max_kv. The pages' rule is a plan option (target 2 workgroups
// per CU, no work floor). The default is tuned for this chip: 16 workgroups
// per CU at D = 128, scaled by 128 / D (a CU holds several decode
// workgroups at once, each of which streams at a rate set by the bytes it
// keeps in flight, and finer splits even out batches whose lengths vary,
// where the longest sequence's workgroup would otherwise set the step time;
// at larger D a split's bytes grow, at smaller D they shrink); the rule's
// form, caps and direct-write fallback are unchanged. One bound is added by
// default: a split keeps at least 16 tiles (1024 keys) at s_max_kv, below
// which the per-workgroup start and merge cost more than the parallelism
// returns (measured on 2048-key gathered lists and 8192-key batches).
#include "plan.hpp"

#include <stdint.h>

namespace vattn {

static inline int cdiv(int a, int b) { return (a + b - 1) / b; }

vattn_status plan_compute(int B_max, int s_max_q, int s_max_kv, int Hq, int Hkv, int D,
                          int causal, const vattn_plan_opts* opts, int n_cu,
                          vattn_plan_info* info) {
  if (!info) return VATTN_ERR_INVALID_ARG;
  if (B_max < 1 || s_max_q < 1 || s_max_kv < 1 || Hq < 1 || Hkv < 1 || n_cu < 1)
    return VATTN_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return VATTN_ERR_INVALID_ARG;
  if (s_max_q > 65535 * 128 || B_max > (1 << 15)) return VATTN_ERR_UNSUPPORTED;
  if (D != 32 && D != 64 && D != 128 && D != 256) return VATTN_ERR_UNSUPPORTED;
  vattn_plan_opts o = {};
  if (opts) o = *opts;
  const int target =
      o.target_blocks_per_cu > 0 ? o.target_blocks_per_cu : kDecodeTargetPerCu * 128 / D;
  const int cap = o.nsplit_cap > 0 ? o.nsplit_cap : 32;
  const int min_chunk = o.min_chunk_tiles > 0 ? o.min_chunk_tiles : kMinChunkTiles;
  const int G = Hq / Hkv;

  vattn_plan_info in = {};
  in.B_max = B_max;
  in.s_max_q = s_max_q;
  in.s_max_kv = s_max_kv;
  in.Hq = Hq;
  in.Hkv = Hkv;
  in.D = D;
  in.causal = causal ? 1 : 0;
  in.n_cu = n_cu;
  in.is_decode = (s_max_q == 1);

  if (in.is_decode) {
    int path = o.force_decode_path;
    if (path != VATTN_DECODE_WAVE && path != VATTN_DECODE_MFMA)
      path = (G <= kWaveMaxG) ? VATTN_DECODE_WAVE : VATTN_DECODE_MFMA;
    in.decode_path = path;
    const int hpb = (path == VATTN_DECODE_MFMA) ? kDecodeMfmaHeads : kDecodeWaveHeads;
    in.head_blocks = cdiv(G, hpb);
    const int64_t units = (int64_t)B_max * Hkv * in.head_blocks;
    if (units > (1 << 30)) return VATTN_ERR_UNSUPPORTED;
    in.n_units = (int)units;
    in.block_n = kDecodeBlockN;
    in.n_tiles = cdiv(s_max_kv, kDecodeBlockN);
    int nsplit;
    if (o.force_nsplit > 0) {
      nsplit = o.force_nsplit < in.n_tiles ? o.force_nsplit : in.n_tiles;
    } else {
      const int64_t want = ((int64_t)target * n_cu + in.n_units - 1) / in.n_units;
      int64_t ns = want;
      if (ns > in.n_tiles) ns = in.n_tiles;
      if (ns > cap) ns = cap;
      // each split keeps at least min_chunk tiles of work at s_max_kv
      const int64_t by_work = cdiv(in.n_tiles, min_chunk);
      if (ns > by_work) ns = by_work;
      nsplit = ns < 1 ? 1 : (int)ns;
    }
    const int chunk_tiles = cdiv(in.n_tiles, nsplit);
    nsplit = cdiv(in.n_tiles, chunk_tiles);
    in.nsplit = nsplit;
    in.chunk_keys = chunk_tiles * kDecodeBlockN;
    in.direct = (nsplit == 1);
    const int64_t grid = (int64_t)in.n_units * nsplit;
    if (grid > (1LL << 31) - 1) return VATTN_ERR_UNSUPPORTED;
    in.grid = (int)grid;
    // 4 waves per workgroup. The wave path takes 8 when at most one
    // workgroup lands on each CU, so that a lone workgroup keeps enough bytes
    // in flight; the MFMA path measured faster with 4 in that case too (its
    // waves hold two 32-key tiles each, and the cross-wave merge halves).
    // (D = 256 stays at 4 waves: 8 would exceed the register file.)
    in.threads = (in.grid <= n_cu && D <= 128 && in.decode_path == 1) ? 512 : 256;
    if (o.decode_waves == 4 || (o.decode_waves == 8 && D <= 128)) in.threads = 64 * o.decode_waves;
    // Where the merge runs. By default in the split kernel (the last split
    // workgroup of a unit merges) when every split workgroup is resident at
    // once (grid <= CUs) and each unit's splits share an XCD (units a
    // multiple of the 8 XCDs, so the partials stay in that XCD's L2): the
    // merge then overlaps other units' streaming and saves the second
    // launch (long decode: 32.6 vs 33.7 us/step). Otherwise a separate
    // combine kernel (with several rounds of workgroups it measured faster).
    // Option 1 forces the in-kernel merge, 2 the combine kernel.
    const bool auto_fuse = in.n_units % 8 == 0 && (int64_t)in.n_units * nsplit <= n_cu;
    in.fused_combine =
        (!in.direct && (o.fuse_combine == 1 || (o.fuse_combine == 0 && auto_fuse))) ? 1 : 0;
    // combine: one 64-thread workgroup per (sequence, two query heads), one
    // head at D = 256
    in.combine_grid = (in.direct || in.fused_combine) ? 0 : B_max * cdiv(Hq, D == 256 ? 1 : 2);
    in.scratch_bytes = 256;  // error word, aligned
    if (!in.direct)
      in.scratch_bytes += (int64_t)in.n_units * 4 + 256 +
                          (int64_t)B_max * Hq * nsplit * ((int64_t)D * 4 + 16) + 256;
  } else {
    if (G > prefill_rows(D)) return VATTN_ERR_UNSUPPORTED;
    in.q_tokens_per_tile = prefill_rows(D) / G;
    in.n_qtiles = cdiv(s_max_q, in.q_tokens_per_tile);
    if (in.n_qtiles > 65535) return VATTN_ERR_UNSUPPORTED;
    const int64_t units = (int64_t)B_max * Hkv;
    const int64_t grid = 8 * ((units + 7) / 8) * (int64_t)in.n_qtiles;
    if (grid > (1LL << 31) - 1) return VATTN_ERR_UNSUPPORTED;
    in.n_units = (int)units;
    in.threads = prefill_threads(D);
    in.block_n = 64;
    in.n_tiles = cdiv(s_max_kv, 64);
    in.nsplit = 1;
    in.direct = 1;
    // Default: the grid covers B_max x n_qtiles tiles and workgroups on dead
    // tiles exit (measured as fast as the alternatives on this chip: a dead
    // workgroup costs well under a microsecond, and the unit-major order keeps
    // a unit's K/V in its XCD's L2). Option 1: a schedule kernel lists the
    // live tiles on the device, longest first, and a persistent grid (one
    // workgroup per CU) walks the list; not available when the schedule's
    // per-level table would not fit in LDS.
    in.prefill_persistent = (o.prefill_grid == 1 && in.n_qtiles <= kSchedMaxQtiles) ? 1 : 0;
    if (in.prefill_persistent) {
      in.grid = n_cu;
      in.scratch_bytes = 512 + (int64_t)B_max * in.n_qtiles * 4;
    } else {
      in.grid = (int)grid;
      in.scratch_bytes = 256;
    }
  }
  if (o.backward == 1) {
    // backward kernels: dq workgroups of bwd_rows(D) rows (G heads folded),
    // dk/dv workgroups of 128 keys, each of both over one 128-column slice of
    // its output at D = 256; the grids cover B_max x s_max like the forward
    if (G > bwd_rows(D)) return VATTN_ERR_UNSUPPORTED;
    in.backward = 1;
    in.bwd_q_tokens_per_tile = bwd_rows(D) / G;
    const int64_t units8 = 8 * (((int64_t)B_max * Hkv + 7) / 8);
    const int64_t g_dq = units8 * cdiv(s_max_q, in.bwd_q_tokens_per_tile) * bwd_slices(D);
    const int64_t g_kv = units8 * cdiv(s_max_kv, kBwdKeys) * bwd_slices(D);
    if (g_dq > (1LL << 31) - 1 || g_kv > (1LL << 31) - 1) return VATTN_ERR_UNSUPPORTED;
    in.bwd_grid_dq = (int)g_dq;
    in.bwd_grid_dkdv = (int)g_kv;
    in.scratch_bytes += 256 + (int64_t)B_max * s_max_q * Hq * 4;
  }
  *info = in;
  return VATTN_OK;
}

}  // namespace vattn
