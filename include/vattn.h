/*
 * vattn.h — varlen grouped-query attention for MI355X (gfx950), C ABI.
 *
 * The library computes scaled-dot-product attention over ragged, THD-packed
 * sequences with grouped-query heads: query head h reads KV head h / G,
 * G = Hq / Hkv (the contiguous grouping that makes [T, Hq, D] ->
 * [T, Hkv, G, D] a byte-conserving reshape; kernbench2 ADR commit page,
 * "GQA via M-fold" finding). Scale is 1/sqrt(D). Causal visibility is
 * bottom-right aligned: query i of a sequence sees key j iff
 * j <= i + (Lk - Lq). A query row with no visible key gets O = 0 and
 * LSE = -inf.
 *
 * Design points taken from the pages:
 *  - Plan/execute split (cudnn-frontend issue #552 "frost(sdpa): THD execute
 *    host round-trip", Proposal to evaluate; How the other backends avoid
 *    this): the grid is sized at plan time from the declared B_max and s_max;
 *    execute reads the exact cu_seqlens on the device, exits dead tiles early,
 *    and never reads device data on the host, so a step can be captured into a
 *    graph and nothing recompiles when lengths change.
 *  - Split-KV decode (AstrAI commit log for csrc/kernels/gqa_decode_attn.cu,
 *    split-KV commit): KV is partitioned across extra workgroups that emit
 *    unnormalised (O, m, l) partials, merged by a log-sum-exp combine kernel;
 *    the split count fills the device with about two workgroups per compute
 *    unit, capped by the KV tile count and by 32, and falls back to one direct
 *    write pass when batch * kv_heads already saturates the device.
 *  - Padding mask (TransformerEngine PR #24 "[PyTorch] Build the attention
 *    padding mask without host syncs", Description and Changes): mask =
 *    position >= seqlen, built on the device from cu_seqlens entries 0..B.
 *
 * Tensor layouts (all row-major, contiguous, device memory owned by the
 * caller; the library never allocates, frees or copies caller memory):
 *   q, out  [T_q,  Hq,  D] bfloat16      (row t = token t of the pack)
 *   k, v    [T_kv, Hkv, D] bfloat16
 *   lse     [T_q,  Hq]     float32, natural log of the softmax denominator
 *                          in units of the scaled score
 *   cu_seqlens_q / cu_seqlens_kv  int32[>= B + 1]; sequence b owns rows
 *                          [cu[b], cu[b+1]); entries past B are never read.
 *
 * Errors: host-checkable problems are reported by the return status before
 * anything is enqueued. Problems that are only visible in device data (a
 * length outside [0, s_max], a sequence that would run past the declared
 * row capacity) are never reported through the status, since that would need
 * a host read: the kernels clamp the length so that no access leaves the
 * buffers, compute the clamped rows, and set a bit in the plan's device error
 * word (see vattn_plan_error_word).
 *
 * Streams: every call that touches the device takes a hipStream_t, passed as
 * vattn_stream_t (NULL = the legacy default stream) and enqueues on it only.
 * Threading: a plan owns scratch memory; do not execute one plan on two
 * streams concurrently. Different plans are independent.
 */
#ifndef VATTN_H
#define VATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VATTN_ABI_VERSION 4

typedef void* vattn_stream_t; /* a hipStream_t */

typedef enum {
  VATTN_OK = 0,
  VATTN_ERR_INVALID_ARG = -1,  /* bad size, null or misaligned pointer, B > B_max */
  VATTN_ERR_UNSUPPORTED = -2,  /* e.g. D not in {32, 64, 128, 256} */
  VATTN_ERR_HIP = -3,          /* a HIP runtime call or launch failed */
  VATTN_ERR_OOM = -4,          /* plan scratch could not be allocated */
  VATTN_ERR_TOO_LARGE = -5     /* vattn_execute_noalloc: the plan's scratch exceeds
                                  VATTN_NOALLOC_SCRATCH_BYTES */
} vattn_status;

/* Bits of the device error word (sticky until vattn_plan_clear_error). */
#define VATTN_ERRBIT_Q_LEN   0x1 /* some query length outside [0, s_max_q] was clamped */
#define VATTN_ERRBIT_KV_LEN  0x2 /* some KV length outside [0, s_max_kv] was clamped */
#define VATTN_ERRBIT_ROWS    0x4 /* a sequence ran past q_rows / kv_rows and was cut */
#define VATTN_ERRBIT_INDEX   0x8 /* a gathered K/V row index outside [0, kv_rows) was clamped */

typedef struct vattn_plan_s* vattn_plan_t;

/* Decode compute paths. */
#define VATTN_DECODE_AUTO 0
#define VATTN_DECODE_WAVE 1 /* wavefront dot products + cross-lane reductions (small G) */
#define VATTN_DECODE_MFMA 2 /* G query heads folded into the MFMA dimension */

/*
 * Plan options. Zero means "default" for every field. These serve tests and
 * ablations; nothing is read from the environment on the hot path (the split
 * target that the split-K blog post reads from an environment variable is a
 * plan option here).
 *
 * Decode split rule (split-K blog post, The Thinking Process; AstrAI commit
 * log, split-KV commit): with n_units = B_max * Hkv * head_blocks and
 * n_tiles = ceil(s_max_kv / 64),
 *   nsplit = min(ceil(target_blocks_per_cu * n_cu / n_units), n_tiles,
 *                nsplit_cap, ceil(n_tiles / min_chunk_tiles)),
 * then chunk_tiles = ceil(n_tiles / nsplit), nsplit = ceil(n_tiles /
 * chunk_tiles), and a direct write (no combine) iff nsplit == 1.
 *   - The pages' rule (aim for roughly two workgroups per compute unit, cap
 *     by the tile count and by 32, and write directly once the batch's KV
 *     heads alone fill the device): target_blocks_per_cu = 2,
 *     min_chunk_tiles = 1 (VATTN_PAGES_TARGET, VATTN_PAGES_MIN_CHUNK).
 *   - The default (all fields 0): target_blocks_per_cu =
 *     VATTN_DEFAULT_TARGET * 128 / D (16 at D = 128; 64, 32 and 8 at D = 32,
 *     64 and 256, so that a split workgroup streams about the same bytes at
 *     every head dimension), min_chunk_tiles = 16 (measured faster on this
 *     chip: finer splits even out batches of unequal lengths, and a split
 *     keeps at least 1024 keys).
 */
#define VATTN_DEFAULT_TARGET 16
#define VATTN_DEFAULT_MIN_CHUNK 16
#define VATTN_PAGES_TARGET 2
#define VATTN_PAGES_MIN_CHUNK 1
typedef struct {
  int target_blocks_per_cu; /* 0 = VATTN_DEFAULT_TARGET * 128 / D; the pages' rule: 2 */
  int nsplit_cap;           /* default 32 */
  int force_nsplit;         /* > 0: use this split count (capped by the tile count) */
  int force_decode_path;    /* VATTN_DECODE_* */
  int n_cu_override;        /* > 0: plan as if the device had this many CUs */
  int fuse_combine;         /* where split partials merge: 1 = in the split kernel (the last
                               split workgroup of a unit merges; no second launch);
                               2 = a separate combine kernel; 0 = automatic: in the split
                               kernel when all split workgroups fit on the device at once
                               and the unit count is a multiple of 8, else the combine
                               kernel */
  int decode_waves;         /* 4 or 8 waves per decode workgroup; 0 = automatic */
  int prefill_grid;         /* prefill: 0 = grid sized from B_max and s_max_q whose
                               workgroups exit on dead tiles (default); 1 = device-built
                               schedule of live tiles on a persistent grid */
  int backward;             /* 1: also size the plan for vattn_backward (allocates the
                               row-wise <dO, O> buffer, B_max * s_max_q * Hq floats);
                               G <= 256, and G <= 128 at D = 256 */
  int min_chunk_tiles;      /* fewest 64-key tiles per split at s_max_kv: 0 =
                               VATTN_DEFAULT_MIN_CHUNK (16); 1 = no floor (the pages'
                               rule) */
} vattn_plan_opts;

typedef struct {
  int B_max, s_max_q, s_max_kv, Hq, Hkv, D, causal;
  int is_decode;       /* 1 if s_max_q == 1 */
  int decode_path;     /* VATTN_DECODE_WAVE or VATTN_DECODE_MFMA (decode only) */
  int n_cu;            /* CU count the plan was sized for */
  int block_n;         /* KV keys per tile (split granularity) */
  int n_tiles;         /* ceil(s_max_kv / block_n) */
  int nsplit;          /* KV splits per (sequence, kv head, head block) */
  int chunk_keys;      /* keys per split = chunk_tiles * block_n */
  int direct;          /* 1: one pass writes out/lse, no combine */
  int fused_combine;   /* 1: split workgroups merge in place (no combine launch) */
  int head_blocks;     /* decode: ceil(G / heads per workgroup) */
  int n_units;         /* decode: B_max * Hkv * head_blocks */
  int grid;            /* workgroups of the main kernel */
  int combine_grid;    /* workgroups of the combine kernel (0 if none) */
  int q_tokens_per_tile; /* prefill: query tokens per workgroup (G heads folded) */
  int n_qtiles;        /* prefill: ceil(s_max_q / q_tokens_per_tile) */
  int threads;         /* threads per workgroup of the main kernel */
  int prefill_persistent; /* prefill: 1 = schedule kernel + persistent grid of `grid` */
  int backward;        /* 1 if the plan serves vattn_backward */
  int bwd_q_tokens_per_tile; /* backward dq kernel: query tokens per workgroup
                                (256 / G; 128 / G at D = 256) */
  int bwd_grid_dq;     /* backward: workgroups of the dq kernel */
  int bwd_grid_dkdv;   /* backward: workgroups of the dk/dv kernel (128 keys each; at
                          D = 256 two per key tile, one per 128-column slice) */
  long long scratch_bytes; /* device bytes owned by the plan */
} vattn_plan_info;

/* Human-readable name of a status code (static storage). */
const char* vattn_status_string(vattn_status s);
int vattn_abi_version(void);

/*
 * Create a plan for up to B_max sequences, query lengths <= s_max_q and KV
 * lengths <= s_max_kv. s_max_q == 1 selects decode (split-KV + combine, or a
 * direct pass); otherwise the causal (or full, causal = 0) varlen prefill
 * kernel. Allowed: B_max, s_max_q, s_max_kv >= 1; Hkv >= 1; Hq % Hkv == 0;
 * D in {32, 64, 128, 256}. The plan binds to the device current at this
 * call, allocates its scratch (split partials, counters, error word) there
 * once, and never allocates again. *out receives the handle.
 */
vattn_status vattn_plan(vattn_plan_t* out, int B_max, int s_max_q, int s_max_kv,
                        int Hq, int Hkv, int D, int causal);
vattn_status vattn_plan_ex(vattn_plan_t* out, int B_max, int s_max_q, int s_max_kv,
                           int Hq, int Hkv, int D, int causal,
                           const vattn_plan_opts* opts /* may be NULL */);

/*
 * Host-only: fill *info with the plan that vattn_plan_ex would build, without
 * touching the device when opts->n_cu_override > 0 (otherwise the current
 * device's CU count is queried). Allocates nothing.
 */
vattn_status vattn_plan_describe(int B_max, int s_max_q, int s_max_kv, int Hq,
                                 int Hkv, int D, int causal,
                                 const vattn_plan_opts* opts, vattn_plan_info* info);

/* The chosen plan of an existing handle. */
vattn_status vattn_plan_query(vattn_plan_t p, vattn_plan_info* info);

/*
 * Enqueue one attention pass on `stream` for sequences 0..B-1 (B <= B_max;
 * B = 0 is a no-op). q_rows / kv_rows are the row capacities of q/out/lse and
 * k/v (tokens allocated); no row at or past them is read or written. The call
 * makes no host read of device data, no allocation and no synchronisation: it
 * enqueues one kernel (direct decode, fused split decode, prefill on the
 * s_max grid) or two (split decode + combine; prefill schedule + persistent
 * prefill) and returns. Pointers must be 16-byte aligned (lse and cu:
 * 4-byte). Rows of out/lse that belong to no sequence are not written.
 *
 * Prefill work distribution (cudnn-frontend issue #552, How the other
 * backends avoid this / Proposal to evaluate: the grid is sized at plan time
 * and tiles read lengths on the device): by default the grid covers B_max x
 * ceil(s_max_q / tile) tiles and workgroups on dead tiles exit after reading
 * cu_seqlens; with prefill_grid = 1 a one-workgroup kernel reads
 * cu_seqlens_q, lists the live (sequence, query tile) pairs in the plan's
 * scratch, longest query tiles first, and a persistent grid of one
 * workgroup per CU walks that list.
 */
vattn_status vattn_execute(vattn_plan_t p, int B,
                           const void* q, const void* k, const void* v,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                           void* out, float* lse,
                           int64_t q_rows, int64_t kv_rows,
                           vattn_stream_t stream);

/*
 * Decode over gathered keys (split-K blog post, The Context: Why Split-K
 * Matters and The Message: each query head attends to a selected list of
 * cached tokens, e.g. top-k indices or page-indexed KV): sequence b's query
 * row attends to the K/V rows kv_idx[cu_idx[b] .. cu_idx[b+1]) of k and v
 * ([kv_rows, Hkv, D], packed), in any order, with no causal mask; a row
 * listed twice counts twice. Uses the decode plan's split rule with
 * s_max_kv = the longest list, the same split partials and the LSE combine
 * (the combine kernel also for plans made with fuse_combine = 1). A list
 * length outside [0, s_max_kv] is clamped and flagged as for cu_seqlens_kv
 * (n_idx, the capacity of kv_idx, plays the role of kv_rows); a row index
 * outside [0, kv_rows) is clamped into range and sets VATTN_ERRBIT_INDEX.
 * Decode plans only (VATTN_ERR_UNSUPPORTED otherwise); kv_idx is an int32
 * device array, 4-byte aligned. Enqueue-only, like vattn_execute.
 */
vattn_status vattn_execute_gathered(vattn_plan_t p, int B,
                                    const void* q, const void* k, const void* v,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_idx,
                                    const int32_t* kv_idx, void* out, float* lse,
                                    int64_t q_rows, int64_t kv_rows, int64_t n_idx,
                                    vattn_stream_t stream);

/*
 * vattn_execute on token-row-strided views (cudnn-frontend issue #552,
 * Related / Proposal: binding the caller's ragged layout directly, e.g. q, k
 * and v as slices of one fused QKV buffer). Row t of q starts at element
 * t * q_row_stride of q (likewise k, v and out); within a row the heads are
 * contiguous with stride D. A stride of 0 means packed (H * D). Each stride
 * must be >= H * D of its tensor and a multiple of 8 elements (16 bytes),
 * and for prefill plans the k and v strides below 2^25 elements (the
 * prefill kernel addresses a 64-key tile with 32-bit offsets from its first
 * row); otherwise VATTN_ERR_INVALID_ARG and nothing is enqueued. q_rows / kv_rows
 * count rows: the caller's buffers must hold (rows - 1) * stride + H * D
 * elements. lse stays packed [T_q, Hq]. Same results as vattn_execute on
 * packed copies (bit-identical).
 */
vattn_status vattn_execute_strided(vattn_plan_t p, int B,
                                   const void* q, int64_t q_row_stride,
                                   const void* k, int64_t k_row_stride,
                                   const void* v, int64_t v_row_stride,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                   void* out, int64_t out_row_stride, float* lse,
                                   int64_t q_rows, int64_t kv_rows, vattn_stream_t stream);

/*
 * Backward of the attention (cudnn-frontend issue #552, Related: THD backward
 * engines under the forward's contract — packed or row-strided views, lengths
 * read on the device, no host round trip). Given q, k, v, the forward's out
 * and lse for the same plan, and the output gradient dout ([T_q, Hq, D]
 * bf16), writes the gradients of sum(dout * out):
 *   dq [T_q, Hq, D], dk, dv [T_kv, Hkv, D], bf16 (fp32 accumulation),
 * with dk, dv summed over the G query heads of each KV head. With
 * p_ij = exp(s_ij - lse_i): dv_j = sum_i p_ij dout_i; ds_ij = p_ij
 * (<dout_i, v_j> - <dout_i, out_i>); dq_i = scale sum_j ds_ij k_j;
 * dk_j = scale sum_i ds_ij q_i, over the visible pairs (same causal rule).
 * Rows of dq of every sequence are written (0 for a row without visible
 * keys); rows of dk, dv of every sequence are written (0 for keys no query
 * sees); rows outside all sequences are not touched. Sequences must not share
 * K/V rows. Strides as vattn_execute_strided (0 = packed; >= H * D, a
 * multiple of 8 and, here, below 2^24 elements; q_rs applies to q, out_rs to
 * out, dout_rs to dout, and so on); q_rows bounds q, out, dout, lse and dq,
 * kv_rows bounds k, v, dk and dv.
 * Needs a plan made with opts.backward = 1 (VATTN_ERR_UNSUPPORTED otherwise).
 * Enqueues two kernels (dq, which also stores <dout_i, out_i> in the plan's
 * scratch, then dk/dv) and returns: no allocation, no synchronisation, no
 * host read, so it can be captured. Deterministic: no atomics.
 */
vattn_status vattn_backward(vattn_plan_t p, int B,
                            const void* q, int64_t q_row_stride,
                            const void* k, int64_t k_row_stride,
                            const void* v, int64_t v_row_stride,
                            const void* out, int64_t out_row_stride,
                            const void* dout, int64_t dout_row_stride,
                            const float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                            void* dq, int64_t dq_row_stride,
                            void* dk, int64_t dk_row_stride,
                            void* dv, int64_t dv_row_stride,
                            int64_t q_rows, int64_t kv_rows, vattn_stream_t stream);

/*
 * Prefill comparator that the grid-sizing question asks to be measured
 * (cudnn-frontend issue #552, Proposal to evaluate: exact grid versus
 * oversubscription with early exit). tile_map holds n_tiles int32 entries,
 * each (b << 16) | q_tile listing only live query tiles, computed by the
 * caller (e.g. on the host from the lengths); the kernel runs exactly
 * n_tiles * Hkv workgroups. Same result as vattn_execute on a prefill plan.
 * Entries with b >= B or q_tile out of range are skipped.
 */
vattn_status vattn_execute_exact_grid(vattn_plan_t p, int B,
                                      const void* q, const void* k, const void* v,
                                      const int32_t* cu_seqlens_q,
                                      const int32_t* cu_seqlens_kv,
                                      void* out, float* lse,
                                      int64_t q_rows, int64_t kv_rows,
                                      const int32_t* tile_map, int n_tiles,
                                      vattn_stream_t stream);

/*
 * Padding mask (TransformerEngine PR #24): for b < B and p < max_seqlen,
 * mask[b * max_seqlen + p] = (p >= cu[b+1] - cu[b]) as a 0/1 byte (the
 * layout of a [B, 1, 1, max_seqlen] torch.bool tensor; 1 = padded). The
 * difference is taken in int32 with wraparound. Any int32 values are valid
 * input: a length above max_seqlen gives an all-0 row, a negative one an
 * all-1 row. Entries past cu[B] are never read. B = 0 is a no-op.
 */
vattn_status vattn_padding_mask(const int32_t* cu_seqlens, int B, int max_seqlen,
                                uint8_t* mask, vattn_stream_t stream);

/*
 * Cross-attention padding masks (TransformerEngine PR #24, Equivalence: the
 * query-side and the key-side mask of one batch), built in one launch:
 * mask_q[b * max_seqlen_q + p] = (p >= cu_q[b+1] - cu_q[b]) for p <
 * max_seqlen_q, and mask_kv likewise from cu_kv and max_seqlen_kv. Layout,
 * wraparound, invalid-length and trailing-entry rules as vattn_padding_mask.
 * Either side may have max_seqlen 0 (its pointer may then be NULL). Caller-
 * owned buffers; returns VATTN_ERR_INVALID_ARG for negative sizes or missing
 * pointers, nothing is enqueued then.
 */
vattn_status vattn_cross_padding_mask(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                      int B, int max_seqlen_q, int max_seqlen_kv,
                                      uint8_t* mask_q, uint8_t* mask_kv, vattn_stream_t stream);

/*
 * Device address of the plan's int32 error word (VATTN_ERRBIT_*). The caller
 * reads it after its own synchronisation; the library never does.
 */
const int32_t* vattn_plan_error_word(vattn_plan_t p);
/*
 * Diagnostic host read of the error word: waits for the device to go idle,
 * then copies the word to *value. Synchronising by design; never call it on a
 * hot path or inside graph capture.
 */
vattn_status vattn_plan_read_error(vattn_plan_t p, int32_t* value);
/* Enqueue a reset of the error word to 0 on `stream` (a kernel, no memset). */
vattn_status vattn_plan_clear_error(vattn_plan_t p, vattn_stream_t stream);

/*
 * Measurement hook (profiling, not part of the attention computation). With
 * both handles non-NULL, every later vattn_execute / vattn_execute_exact_grid
 * on this plan launches its main kernel (the split or direct decode kernel,
 * or the prefill kernel) with `start` and `stop` stamped at the start and end
 * of that kernel's dispatch (hipExtLaunchKernelGGL), so that the elapsed time
 * between them is that kernel's duration; a combine kernel that follows is
 * not included. The handles are hipEvent_t values
 * created and owned by the caller, who keeps them alive until that work is
 * done; NULL, NULL turns the hook off. While the hook is set, execute on a
 * capturing stream returns VATTN_ERR_INVALID_ARG (events are not recorded into
 * graphs). Host-only call: no device work, no synchronisation.
 */
vattn_status vattn_plan_set_kernel_events(vattn_plan_t p, void* start, void* stop);

/*
 * For callers that cannot allocate device memory (code under graph capture
 * that must not call hipMalloc, tight serving loops, harnesses that forbid
 * allocation): vattn_plan + vattn_execute in one call that allocates
 * nothing, neither device nor host memory. The plan (B_max, s_max_q, s_max_kv, Hq, Hkv, D,
 * causal; default options) is chosen on the host at each call exactly as
 * vattn_plan would choose it, and its scratch (error word, split partials)
 * lives in a static device array of VATTN_NOALLOC_SCRATCH_BYTES bytes that
 * each GPU the library runs on holds until the process ends. A plan whose
 * scratch would not fit returns VATTN_ERR_TOO_LARGE before anything is
 * enqueued (the split partials take B_max * Hq * nsplit * (4 D + 16) bytes,
 * plus the merge counters: e.g. B_max = 1, Hq = 64, D = 128 at 32 splits
 * needs about 1.1 MB). The arguments B .. kv_rows and the results are as
 * for vattn_execute (packed layouts, same alignment rules, same kernels,
 * bit-identical results). err_word: an int32 in device memory (4-byte
 * aligned) into which the kernels OR the VATTN_ERRBIT_* flags, or NULL to
 * discard them; the caller clears it. All calls on one GPU share that GPU's
 * array: calls that overlap on a GPU (other streams, other host threads)
 * race, so serialise them. The first call on a device looks up the array's
 * device address there (one host-side runtime query, no allocation).
 */
#define VATTN_NOALLOC_SCRATCH_BYTES (8u << 20)
vattn_status vattn_execute_noalloc(int B_max, int s_max_q, int s_max_kv, int Hq, int Hkv, int D,
                                   int causal, int B, const void* q, const void* k,
                                   const void* v, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_kv, void* out, float* lse,
                                   int64_t q_rows, int64_t kv_rows, int32_t* err_word,
                                   vattn_stream_t stream);

/* Free the plan's scratch. Safe on NULL. Work already enqueued must be done.
 * Calls hipFree: not to be called while any stream of the device is being
 * captured in global mode (the capture would be invalidated); the Python
 * binding defers a plan released during a capture of its current stream. */
void vattn_plan_destroy(vattn_plan_t p);

#ifdef __cplusplus
}
#endif

#endif /* VATTN_H */
