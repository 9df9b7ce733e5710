/*
 * libsolattn: block-sparse attention forward (sol-attn, sla and a static local
 * 3-D neighbourhood pattern) for AMD gfx950.
 *
 * The operation (ComfyUI "BlockSparseAttention" node docs, input tables; the
 * minimax-h3-chunk-star7 README, sections "Sol" and "SLA"), per (batch, head):
 *   1. mean-pool Q over block_q tokens and K, V over block_k tokens;
 *   2. score every pooled query block against every pooled key block,
 *      s_ij = q̄_i . k̄_j / sqrt(d);
 *   3. select key blocks per query block: sol-attn keeps s_ij > mean + tau*std
 *      of the row (node docs, sol-attn table, tau row); sla keeps the
 *      ceil(keep_percent*M/100) highest (node docs, sla table, keep_percent
 *      row).  Sink blocks (overlapping [0, sink_range): the packed conditioning
 *      rows, node docs, sink_conditioning row) and the diagonal blocks are kept
 *      on top;
 *   4. add up to extra_tokens individually highest-scoring keys (q̄_i . k_t)
 *      outside the kept blocks (node docs, extra_tokens row);
 *   5. attend exactly over kept-block and extra tokens; for sol-attn every other
 *      key block enters through its centroid (k̄_j, v̄_j) with weight
 *      (tokens of the block not attended exactly) in the same FP32 online
 *      softmax (star7 README, "Sol"); sla drops them (star7 README, "SLA").
 *   Query rows in [dense_row_begin, dense_row_end) attend every key exactly
 *   (node docs, sink_conditioning row: exact_kv_and_rows).
 * Attention is non-causal with scale 1/sqrt(d).
 *
 * All calls are asynchronous on the given HIP stream: a return of SOLATTN_OK
 * means the work was enqueued.  Every argument is validated on the host before
 * anything is launched, so an error return never leaves a partial write.
 */
#ifndef SOLATTN_H
#define SOLATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SOLATTN_OK          0
#define SOLATTN_EINVAL     -1   /* an argument is out of its domain                        */
#define SOLATTN_ENOTSUP    -2   /* valid, but the library does not implement the shape     */
#define SOLATTN_EWORKSPACE -3   /* the caller's workspace is smaller than required        */
#define SOLATTN_EHIP       -4   /* a HIP runtime or launch error (see last_error_detail)   */

/* Element types of q, k, v and out (all four share one type). */
#define SOLATTN_BF16 0
#define SOLATTN_FP32 1
/*
 * bf16 tensors with the fp8-QK flavour of the attention step (the pages' reduced-precision
 * "INT8 QK, FP16 PV" variants, on the FP8 format): the products Q K^T of the exact tokens and of
 * the centroids run on E4M3 operands, Q scaled per query row, K per token and the pooled keys
 * per pooled row by powers of two (the smallest 2^e with max|row| <= 448 * 2^e), rounded to
 * nearest even; the softmax and P V are those of SOLATTN_BF16, and the selection (kept blocks,
 * extra tokens) is unchanged.  Not value-identical to SOLATTN_BF16.  d in {64, 128}.
 */
#define SOLATTN_BF16_FP8QK 2

/* Selection modes. */
#define SOLATTN_MODE_SOL 0
#define SOLATTN_MODE_SLA 1
#define SOLATTN_MODE_LOCAL3D 2

/* Largest extra_tokens value (node docs, extra_tokens row: 0..256). */
#define SOLATTN_MAX_EXTRA 256

/*
 * Optional per-call settings.  Pass NULL for the defaults: bf16, contiguous
 * [B, H, N, d] tensors, no dense rows, the null stream, a library-owned
 * workspace.  Set struct_size = sizeof(solattn_opts) and zero every field you
 * do not use.
 *
 * Workspace.  A caller-owned workspace (opts->workspace) must hold at least
 * solattn_workspace_bytes_ex(...) bytes for the call's mode, dtype, shape,
 * extra_tokens and row window (solattn_workspace_bytes(...) is enough for any
 * dtype), be 256-byte aligned, and not be used by another call that may run at
 * the same time.  The call allocates nothing then.  Without one, the library
 * keeps one grow-only buffer per (device, stream): calls on one stream share it
 * and are ordered by the stream; calls on different streams use different
 * buffers.  Growing a stream's buffer first waits for that stream (so work
 * still queued on the old buffer finishes before it is freed).  The buffers
 * live until solattn_free_default_workspaces() or the end of the process.
 */
typedef struct solattn_opts {
  int struct_size;
  int dtype;                      /* SOLATTN_BF16 or SOLATTN_FP32                          */
  /* Strides in elements of the b, h and n axes; the d axis is contiguous.  A
   * triple of zeros means contiguous [B, H, N, d].  Row starts (every n) must
   * be 16-byte aligned. */
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];
  int dense_row_begin, dense_row_end;   /* query rows attending every key; empty if equal */
  void*  workspace;               /* device buffer owned by the caller, or NULL            */
  size_t workspace_bytes;         /* its size; must be >= solattn_workspace_bytes_ex(...)  */
  void*  stream;                  /* hipStream_t; NULL = null stream                       */
  unsigned flags;                 /* SOLATTN_FLAG_* bits; 0 = defaults                       */
  int64_t* stats;                 /* device int64[SOLATTN_NSTATS] for per-call counters, or NULL */
  /* Query-row window: only rows [q_row_begin, q_row_end) are computed (both multiples of
   * block_q); the other rows of out are left untouched.  Keys are always all N rows.  Both 0
   * means every row.  The workspace then covers the window only (q_rows of the layout
   * calls), which is how a caller splits a long sequence into row chunks that fit in memory.
   * Dense rows are given in whole-sequence coordinates and intersected with the window; the
   * intermediate buffers (qbar, scores, lists, ...) hold the window's query blocks from 0. */
  int q_row_begin, q_row_end;
} solattn_opts;

/*
 * SOLATTN_FLAG_EXACT_EXTRA: the extra-token selection skips its sampled first pass (which
 * seeds each query block's running threshold from a sample of the keys and falls back to the
 * exact pass for the query blocks it leaves short) and runs the exact pass for every query
 * block.  The selected tokens are the same either way; the flag only costs time.  It exists
 * to exercise and check the exact pass on any input.
 */
#define SOLATTN_FLAG_EXACT_EXTRA 1u

/*
 * SOLATTN_FLAG_CHECK_FINITE: also count the NaN and infinite values of q, k, v and out into
 * stats[7] (one extra pass over the four tensors).  Needs opts->stats; without it the call
 * returns SOLATTN_EINVAL.
 */
#define SOLATTN_FLAG_CHECK_FINITE 2u

/*
 * SOLATTN_FLAG_KEEP_SELECTION: also write the kept key blocks as ascending index lists
 * (kept_idx) and every key block's centroid multiplicity (mult), so that a caller can read the
 * whole selection after the call through solattn_selection_view.  Without it a bf16 call writes
 * only what its kernels use: the kept sets as bitmaps, their counts and the extra-token lists.
 * fp32 calls always write both.  The output does not depend on the flag.
 */
#define SOLATTN_FLAG_KEEP_SELECTION 4u

/*
 * Per-call counters (opts->stats != NULL): a device array of SOLATTN_NSTATS int64 values,
 * 8-byte aligned, overwritten asynchronously on the call's stream after the attention (not
 * covered by the per-kernel timing).  Sums over every (batch, head):
 *   [0] kept key blocks of the query blocks that run selection (not dense-row blocks)
 *   [1] query blocks that run selection
 *   [2] exact (query row, key) pairs: kept-block and extra tokens, every key for dense rows
 *   [3] centroid terms (query row, key block): sol-attn only
 *   [4] extra tokens used
 *   [5] key blocks whose score lies within 1e-4 standard deviations of the sol-attn threshold
 *       (recomputed in fp32; a measure of how close the selection is to flipping; 0 for sla,
 *       the local 3-D pattern and tau = -inf)
 *   [6] query blocks whose extra tokens the exact pass selected (see SOLATTN_FLAG_EXACT_EXTRA)
 *   [7] non-finite values among q, k, v and out with SOLATTN_FLAG_CHECK_FINITE, else -1
 * The counters are computed with a fixed reduction order, so they do not vary between runs.
 */
#define SOLATTN_NSTATS 8

/*
 * sol-attn forward.
 *   q, k, v   device pointers, read only, layout given by opts (default [B,H,N,d]).
 *   out       device pointer, same shape and type, fully overwritten; must not
 *             overlap q, k or v.
 *   B, H, N, d  sizes (>= 1).  This build: d in {64, 128}, N % block_q == 0,
 *             N % block_k == 0, and for bf16 at most 4096 key blocks (N <= 262144
 *             at block_k 64); other shapes return SOLATTN_ENOTSUP.
 *   tau       threshold in standard deviations of the row's block scores; any
 *             value but NaN.  -inf keeps every block (dense attention).
 *   block_q   query block size: 64 or 128.   block_k: key block size: 64.
 *   sink_range  0..N; every key block overlapping tokens [0, sink_range) is
 *             attended exactly by every query (0 = none).
 *   extra_tokens  0..256 extra exact keys per query block.
 * Returns a status code.
 */
int sol_attn_fwd(const void* q, const void* k, const void* v, void* out,
                 int B, int H, int N, int d, float tau,
                 int block_q, int block_k, int sink_range, int extra_tokens,
                 const solattn_opts* opts);

/*
 * sla forward: as sol_attn_fwd, but step 3 keeps the ceil(keep_percent*M/100)
 * highest-scoring non-forced key blocks (ties to the lower block index) and
 * skipped blocks contribute nothing.  keep_percent in (0, 100].
 */
int sla_attn_fwd(const void* q, const void* k, const void* v, void* out,
                 int B, int H, int N, int d,
                 int block_q, int block_k, int sink_range, int extra_tokens, float keep_percent,
                 const solattn_opts* opts);

/*
 * Static local 3-D neighbourhood forward (the article on block sparse attention
 * for H3 in ComfyUI, section 1: a fixed pattern that keeps the centre block, its
 * neighbours one frame back and forward and its spatial neighbours one block up,
 * down, left and right, and zeroes every other block).  Step 3 above is replaced
 * by that pattern (no block scores are computed; the workspace's scores are not
 * written) and skipped blocks contribute nothing, as in sla.
 *   frames, height, width  the token grid, >= 1 each, frames*height*width == N
 *             (else SOLATTN_EINVAL).  Token p sits at frame p / (height*width),
 *             row (p % (height*width)) / width, column p % width.
 *   Key block j is kept for query block i when it holds a token of i or a grid
 *   neighbour of one (one step along one axis, no wrap-around).  When a frame is
 *   a whole number of key blocks and a row is a whole number of blocks (or a
 *   block a whole number of rows) this is exactly the centre / +-1 frame / +-1
 *   block row / +-1 block column stencil on the grid of blocks; for other grids
 *   it is the same rule at token level.  Sink blocks, the diagonal, the dense
 *   row range and extra_tokens work as in sol_attn_fwd.
 *   At most 65536 key blocks (SOLATTN_ENOTSUP beyond); the other arguments and
 *   limits are those of sol_attn_fwd.
 */
int local3d_attn_fwd(const void* q, const void* k, const void* v, void* out,
                     int B, int H, int N, int d, int frames, int height, int width,
                     int block_q, int block_k, int sink_range, int extra_tokens,
                     const solattn_opts* opts);

/*
 * Allocation-free sol-attn forward, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.  The same call and
 * result as sol_attn_fwd, but its workspace is a scratch buffer the library holds in device
 * memory: SOLATTN_NOALLOC_SCRATCH_BYTES per GPU, one copy on every GPU the library runs this
 * call on, held until the process ends.  The call allocates nothing (no hipMalloc or hipFree,
 * no HIP events, no library allocation).
 *   opts->workspace must be NULL (SOLATTN_EINVAL otherwise); every other option works as in
 *   sol_attn_fwd, including the query-row window, which bounds the workspace a call needs.
 *   A call whose workspace (solattn_workspace_bytes_ex for its dtype, shape, extra_tokens and
 *   window) exceeds SOLATTN_NOALLOC_SCRATCH_BYTES returns SOLATTN_EWORKSPACE before anything
 *   runs, with the sizes in the error detail.
 *   Every call on one GPU uses that GPU's one buffer, and the buffer keeps the last call's
 *   intermediates (nothing in it needs clearing between calls): calls that may overlap on one
 *   GPU (different streams, or different host threads without ordering) race on it and must
 *   be serialised by the caller.  Calls ordered on one stream are safe.
 * Returns a status code.
 */
#define SOLATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int sol_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out,
                         int B, int H, int N, int d, float tau,
                         int block_q, int block_k, int sink_range, int extra_tokens,
                         const solattn_opts* opts);

/*
 * Host-only argument check: the exact validation sol_attn_fwd / sla_attn_fwd
 * perform, without launching anything.  mode is SOLATTN_MODE_SOL or
 * SOLATTN_MODE_SLA (keep_percent is ignored for sol, tau for sla);
 * SOLATTN_MODE_LOCAL3D returns SOLATTN_EINVAL (use local3d_check_args).
 * Returns a status code.
 */
int solattn_check_args(int mode, const void* q, const void* k, const void* v, void* out,
                       int B, int H, int N, int d, float tau, float keep_percent,
                       int block_q, int block_k, int sink_range, int extra_tokens,
                       const solattn_opts* opts);

/* Host-only argument check of local3d_attn_fwd.  Returns a status code. */
int local3d_check_args(const void* q, const void* k, const void* v, void* out,
                       int B, int H, int N, int d, int frames, int height, int width,
                       int block_q, int block_k, int sink_range, int extra_tokens,
                       const solattn_opts* opts);

/*
 * Workspace layout.  Byte offsets (from the workspace start, each 256-byte aligned) of the
 * intermediate buffers of one call, which stay readable after the call until the workspace is
 * reused.  Mq = query blocks of the computed rows (the window, or N/block_q), M = N/block_k,
 * Mpad = M rounded up to a multiple of 64.  The selection comes first and its offsets depend
 * only on (B, H, Mq, M): they are the same for every dtype, d and extra_tokens.
 *   kept_cnt  int32 [B*H, Mq]         number of kept key blocks (M for dense query blocks)
 *   kept_bm   uint64 [B*H, Mq, Mpad/64] the kept set as a bitmap (bit j%64 of word j/64)
 *   kept_idx  int32 [B*H, Mq, M]      kept key-block indices, ascending, first kept_cnt valid
 *                                     (written with SOLATTN_FLAG_KEEP_SELECTION, or fp32)
 *   mult      uint8 [B*H, Mq, Mpad]   centroid multiplicity of each key block: tokens of the
 *                                     block not attended exactly, 0 for kept blocks (same
 *                                     condition as kept_idx)
 *   extra_cnt int32 [B*H, Mq]         number of extra tokens
 *   extra_idx int32 [B*H, Mq, 256]    extra token indices, ascending, first extra_cnt valid
 *   extra_flag int32 [B*H, Mq]        1 where the extra-token selection's first pass, whose
 *             threshold is seeded from a sample of the keys, kept fewer candidates than the
 *             selection needs, so that the query block was selected again with every
 *             candidate competing (the result is exact either way)
 *   scores    fp32 [B*H, Mq, Mpad]    block scores s_ij (row stride Mpad; columns >= M are
 *                                     padding; not written by local3d_attn_fwd)
 * Then the rest:
 *   qbar      fp32 [B*H, Mq, d]    pooled queries
 *   kbar      fp32 [B*H, M, d]     pooled keys
 *   vbar      fp32 [B*H, M, d]     pooled values
 *   pair_plan int64 [B*H, 8]: for pairing strides s = 1..8, the kept-block union summed over
 *             the pairs of query blocks that one attention workgroup takes together (with
 *             stride s, block t of each run of 2s non-dense query blocks pairs with block t+s);
 *             each head's workgroups use the stride with the least sum.  Scheduling only: no
 *             output depends on it (bf16 tensors with block_q 64 only; offset 0 otherwise)
 *   extra_buf, extra_part: scratch of the extra-token selection (candidate lists per query
 *             block: one per token slice for 16-bit tensors, one per slice and wave for fp32;
 *             and their lengths; only the per-call counters' scratch when extra_tokens is 0);
 *             extra_buf also holds the partial sums of the per-call counters
 *   extra_seed uint32 [B*H, Mq]    scratch of the extra-token selection (16-bit tensors): the
 *             threshold each query block's first pass starts from, seeded from a sample of
 *             the keys, as an order-preserving key of the fp32 score
 *   kbar_bf   bf16 [B*H, Mpad, d], vbar_t bf16 [B*H, Mpad/64, d, 64], v_t bf16
 *             [B*H, M, d, 64]: operand copies for the attention kernel (bf16 only)
 *   k8, kb8   E4M3 tiles [B*H, M] and [B*H, Mpad/64] of 64 * d bytes (64 rows) followed by
 *             the 64 rows' scale codes e + 127 (SOLATTN_BF16_FP8QK only)
 */
typedef struct solattn_ws_layout {
  size_t total;
  size_t kept_cnt, kept_bm, kept_idx, mult, extra_cnt, extra_idx, extra_flag, scores;
  size_t qbar, kbar, vbar;
  size_t extra_buf, extra_part, extra_seed;
  size_t kbar_bf, vbar_t, v_t, k8, kb8, pair_plan;
  int Mq, M, Mpad;
} solattn_ws_layout;

/*
 * Fills *layout for a call of this mode, dtype (SOLATTN_BF16, SOLATTN_FP32 or
 * SOLATTN_BF16_FP8QK), shape and extra_tokens (0..256) over a window of q_rows query rows
 * (q_rows = N: the whole sequence; 1 <= q_rows <= N).  Returns SOLATTN_OK or SOLATTN_EINVAL.
 */
int solattn_workspace_layout(int mode, int dtype, int B, int H, int N, int d, int block_q, int block_k,
                             int extra_tokens, int q_rows, solattn_ws_layout* layout);

/* Total bytes of that layout (0 if the arguments are invalid). */
size_t solattn_workspace_bytes_ex(int mode, int dtype, int B, int H, int N, int d, int block_q,
                                  int block_k, int extra_tokens, int q_rows);

/*
 * Workspace bytes a whole-sequence call of this shape needs with any dtype (the largest of
 * the three layouts); 0 if the arguments are invalid.
 */
size_t solattn_workspace_bytes(int mode, int B, int H, int N, int d, int block_q, int block_k,
                               int extra_tokens);

/*
 * The selection of a call, as device pointers into its workspace (valid once the call has
 * completed on its stream, until the workspace is reused).  Shapes and conditions as in the
 * layout above; kept_idx and mult hold the call's values only if it ran with
 * SOLATTN_FLAG_KEEP_SELECTION (or on fp32 tensors).
 */
typedef struct solattn_selection {
  int Mq, M, Mpad;
  int32_t*  kept_cnt;
  uint64_t* kept_bm;
  int32_t*  kept_idx;
  uint8_t*  mult;
  int32_t*  extra_cnt;
  int32_t*  extra_idx;
  int32_t*  extra_flag;
  float*    scores;
} solattn_selection;

/*
 * Fills *view from opts->workspace (required: a caller-owned workspace) and the query-row window
 * in opts (q_row_begin/q_row_end; both 0 for the whole sequence), for a call of this mode and
 * shape.  Host only: no device access.  Returns SOLATTN_OK or SOLATTN_EINVAL.
 */
int solattn_selection_view(const solattn_opts* opts, int mode, int B, int H, int N, int block_q,
                           int block_k, solattn_selection* view);

/* Frees the library-owned default workspaces (after waiting for the device).  Returns a status. */
int solattn_free_default_workspaces(void);

/* Static text for a status code. */
const char* solattn_status_string(int status);

/* Thread-local detail of the last failing call on this thread, naming the bad argument or the
 * failing HIP call ("" if the last call succeeded). */
const char* solattn_last_error_detail(void);
/* The same text (the name earlier versions of this header used). */
const char* solattn_last_error(void);

/*
 * Scheduling of the bf16 attention kernel with 64-row query blocks (host only, no device
 * call): the query blocks of each workgroup-sized unit of one head, in unit order, for Mq
 * query blocks of which [dense_q0, dense_q1) are dense and pairing stride `stride` (1..8; the
 * kernel takes, per head, the stride with the least sum in the workspace's pair_plan).  The
 * dense blocks' units come first, paired with their neighbours; the other blocks, numbered in
 * order with the dense run cut out, pair block t with block t + stride in each run of
 * 2 * stride of them, and the blocks after the last whole run pair with their neighbours.
 * Fills qa[j], qb[j] (qb[j] = -1: a single block) for j < min(units, cap) and returns the
 * number of units, or SOLATTN_EINVAL.  The pairing decides only which query blocks share a
 * workgroup (and so a walk over the union of their kept blocks); no result depends on it.
 */
int solattn_pair_schedule(int Mq, int dense_q0, int dense_q1, int stride, int* qa, int* qb, int cap);

/*
 * Per-kernel timing.  While enabled, every call records HIP events around each
 * of its kernel launches on the call's stream (local3d_attn_fwd launches no
 * block_score).  solattn_timing_read waits for
 * those events, writes the summed milliseconds and launch counts per kernel
 * (index order: block_pool, block_score, block_select, extra_select,
 * sparse_flash_fwd) into ms[0..n) and launches[0..n), and resets the sums.
 */
#define SOLATTN_NKERNELS 5
int solattn_timing_enable(int enable);
int solattn_timing_read(double* ms, long long* launches, int n);
const char* solattn_kernel_name(int index);

/*
 * Achievable-peak probes (measurement aid; not part of the attention).  Launches one probe on
 * `stream` (hipStream_t, NULL = null stream) and writes the work it does per launch to
 * *work_per_launch; the caller times the launch (e.g. with events) to get the rate:
 *   kind 0: bf16 32x32x16 matrix instructions in a loop, no memory (work: flop)
 *   kind 1: fp32 32x32x2 matrix instructions in a loop (work: flop)
 *   kind 2: copy of the first half of buf to its second half (work: bytes read + written)
 *   kind 3: the kind-0 loop, timed from inside by its first wave: writes two unsigned 64-bit
 *           counts to the start of buf (shader clock ticks, then wall clock ticks, over that
 *           wave's loop) and sets *work_per_launch to the wall clock's rate in Hz, so that
 *           ticks[0] / (ticks[1] / rate) is the shader clock under full matrix load; read the
 *           counts after the stream has finished the launch
 * buf: device memory, 16-byte aligned, at least 2 MiB for kinds 0, 1 and 3 (results that are
 * never stored unless a sum hits one exact value); iters: loop trips for kinds 0, 1 and 3 (>= 1).
 * Returns SOLATTN_OK, SOLATTN_EINVAL or SOLATTN_EHIP.
 */
int solattn_peak_probe(int kind, void* buf, size_t bytes, int iters, void* stream, double* work_per_launch);

#ifdef __cplusplus
}
#endif

#endif /* SOLATTN_H */
