/*
 * flce.h -- C ABI of the MI355X (gfx950) fused linear cross-entropy library.
 *
 * The operation (PR #1554 "skip ignore_index rows in the FLCE GEMMs", Summary;
 * issue #1323 "Reduce FLCE weight-gradient allocation overhead across FP16,
 * BF16, and FP32", Background and motivation):
 *
 *   for the labelled rows i (targets[i] != ignore_index):
 *     z_i      = X[i,:] . W^T                       lm_head logits, never stored for all rows
 *     loss_i   = logsumexp(z_i) - z_i[targets[i]]   cross-entropy
 *     G_i      = s_i * (softmax(z_i) - onehot(targets[i]))
 *     dX[i,:]  = G_i . W                            grad_input
 *     dW      += G_i^T . X[i,:]                     grad_weight
 *   with s_i = g / N (mean), g (sum) or g_i (none); g is the upstream
 *   gradient, N the number of labelled rows.  Ignored rows get a zero dX row
 *   and zero per-token loss and never enter a projection (PR #1554, Details
 *   item 1 and Tests: NaN in ignored rows must not reach the loss or the
 *   gradients).
 *
 * The rows are processed in chunks of chunk_size labelled rows; each chunk
 * runs the logits projection into one reused [chunk_size, V] slab, the
 * softmax-gradient pass in place, the grad_input projection and the
 * grad_weight update written straight into dW (v0.8.3 commit bad6c3ec42,
 * Summary: reusable logits, direct dX, direct dW; issue #1323, Proposed
 * direction: no [V, H] temporary per chunk).  Loss and gradients are all
 * produced by one forward call (PR #1554, Summary).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers to dense row-major arrays,
 *     16-byte aligned, owned by the caller.  The library never allocates
 *     device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All device work is enqueued on it, in order.
 *   - Errors are returned as flce_status_t (0 = OK); nothing throws across
 *     the ABI.  Argument, dtype and workspace errors are found on the host
 *     before any launch and leave every output untouched.
 */
#ifndef FLCE_H
#define FLCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  X, W, dX and the slab use the operand dtype; dW uses the
 * accumulation dtype, which is either the operand dtype or FLCE_F32
 * (issue #1323, Proposed direction: same-dtype direct accumulation, and
 * fp16/bf16 operands with an fp32 destination). */
typedef enum { FLCE_F32 = 0, FLCE_F16 = 1, FLCE_BF16 = 2 } flce_dtype_t;

/* Loss reductions (PR #1554, Tests: mean, sum and none with a per-token
 * upstream gradient). */
typedef enum { FLCE_MEAN = 0, FLCE_SUM = 1, FLCE_NONE = 2 } flce_reduction_t;

typedef enum {
  FLCE_OK = 0,
  FLCE_E_ARG = -1,       /* bad size, pointer, alignment or flag                */
  FLCE_E_DTYPE = -2,     /* unsupported dtype / accumulation-dtype combination  */
  FLCE_E_TARGET = -3,    /* a labelled target lies outside [0, V)               */
  FLCE_E_WORKSPACE = -4, /* workspace smaller than flce_workspace_bytes()       */
  FLCE_E_HIP = -5        /* HIP runtime error; see flce_last_error()            */
} flce_status_t;

/* Geometry and row counts of one flce_fwd_bwd call. */
typedef struct {
  int64_t chunk_size;   /* rows per chunk after flooring / clamping          */
  int64_t chunks_total; /* ceil(BT / chunk_size): chunks with no row skipped */
  int64_t chunks_run;   /* ceil(n_valid / chunk_size): chunks actually run   */
  int64_t n_valid;      /* labelled rows                                      */
  int32_t compacted;    /* 1 when skipping ignored rows removed a chunk       */
  int32_t dx_splits;    /* split factor of the grad_input reduction over V    */
} flce_stats_t;

/*
 * Rows per chunk.
 *   chunk_size > 0 : floored to a power of two, then clamped to BT
 *                    (PR #1439 "expose direct chunk-size control",
 *                    Summary and Testing Done: 100 becomes 64).
 *   chunk_size <= 0: heuristic from the memory constant C = chunk_mem_const
 *                    (>= 1; v0.8.3 commit bad6c3ec42, Summary: public default
 *                    C = 1, per-call override):
 *                    next_pow2(ceil(BT / ceil(V / (C * H)))), clamped to BT.
 *                    This form reproduces every geometry the pages print
 *                    (PR #1439 review thread, C / num_chunks / chunk_size
 *                    table; v0.8.3 commit, H200 memory and latency table).
 * Returns the chunk size (>= 1), or FLCE_E_ARG for BT < 0, H < 1, V < 1,
 * or chunk_size <= 0 with chunk_mem_const < 1.
 */
int64_t flce_chunk_size(int64_t BT, int64_t H, int64_t V, int64_t chunk_size,
                        int32_t chunk_mem_const);

/*
 * MI355X default chunk size.  The pages leave the default geometry open per
 * GPU type (PR #1439 review thread: different defaults for GPUs with different
 * memory, e.g. about 80 GB against about 280 GB; the heuristic's memory
 * constant is only a proxy for the chunk size).  On MI355X (288 GB HBM3E)
 * memory is rarely the bound, so this policy picks the smallest power of two
 * whose per-row cost is within 10 % of the cost at an unbounded chunk, on a
 * model of one chunk of c rows:
 *   GEMM time  = k c' H V / (0.40 x MFMA peak)    k = 6 trained, 4 frozen;
 *                c' = c rounded up to the 256-row tiles of the row-tiled
 *                GEMMs (logits and grad_input; grad_weight tiles over V);
 *                peak 2516.6 TFLOP/s for bf16/fp16, 157.3 for fp32; 0.40 is
 *                the fraction of peak the GEMMs reach on MI355X
 *   HBM time   = (2 V H s + 2 V H a [trained] + 5 c V s) / 5.1 TB/s
 *                (W read by the logits and grad_input GEMMs, the dW
 *                read-modify-write, five passes over the slab; 5.1 TB/s is
 *                the measured device-copy rate)
 *   chunk time = GEMM time + HBM time (the per-chunk weight traffic is not
 *                hidden behind the GEMMs: measured per-step times fit
 *                T(c) = T_inf + (BT / c) x 0.60 ms at BT 8192, H 4096,
 *                V 128256)
 * s / a: operand / accumulation item sizes.  The logits slab is kept within
 * slab_budget_bytes (0: 2 GiB); the result is then floored to a power of two
 * and clamped to BT like an explicit chunk_size.  Returns >= 1, or FLCE_E_ARG.
 */
int64_t flce_chunk_size_mi355x(int64_t BT, int64_t H, int64_t V, flce_dtype_t dtype,
                               flce_dtype_t accum_dtype, int32_t frozen_weight,
                               size_t slab_budget_bytes);

/*
 * Bytes of device workspace flce_fwd_bwd needs for these arguments.  The
 * dominant term is the [chunk_size, V] logits slab in the operand dtype
 * (chunk_size x V x itemsize, PR #1439, Summary), so with an explicit
 * chunk_size it does not grow with BT except for 8 bytes per row of index
 * and per-row loss.  Returns 0 for invalid arguments.
 */
size_t flce_workspace_bytes(int64_t BT, int64_t H, int64_t V, flce_dtype_t dtype,
                            int64_t chunk_size, int32_t chunk_mem_const);

/*
 * Fused linear cross-entropy, forward and backward in one call.
 *
 *   X            [BT, H] dtype        inputs (rows = tokens)
 *   W            [V, H]  dtype        lm_head weight
 *   targets      [BT]    int64        class ids; rows equal to ignore_index are
 *                                     ignored (any int64 value, default -100)
 *   BT, H, V                          BT >= 0, 8 <= H <= 2^20 and H % 8 == 0, V >= 1;
 *                                     with gradients, 256 x round_up(V, 8) x itemsize
 *                                     and (unless frozen) 256 x round_up(chunk, 8) x
 *                                     itemsize must stay under 2 GiB (V <= 4194296 for
 *                                     16-bit operands, 2097144 for fp32).  X may be of
 *                                     any size; beyond 2 GiB - 64 KiB the workspace
 *                                     also holds up to chunk x H x itemsize bytes of
 *                                     gathered rows (at most 2 GiB)
 *   dtype                             FLCE_F32, FLCE_F16 or FLCE_BF16
 *   reduction                         FLCE_MEAN, FLCE_SUM or FLCE_NONE
 *   chunk_size, chunk_mem_const       see flce_chunk_size
 *   accum_dtype                       dtype of dW: FLCE_F32 or == dtype
 *   frozen_weight                     1: no grad_weight work, dW may be NULL
 *                                     (PR #1554, FLCE-alone tables: lm_head frozen)
 *   accumulate_dw                     0: dW is overwritten; 1: dW += this call's gradient
 *   grad_output  float, device        NULL means 1.  mean/sum: [1]; none: [BT].
 *                                     Read only at labelled rows.
 *   loss         float, device        mean/sum: [1]; none: [BT] with ignored rows +0.0
 *                                     (NULL allowed only for none with BT = 0).
 *                                     Mean over zero labelled rows is 0.
 *   dX           [BT, H] dtype        ignored rows +0.0
 *   dW           [V, H] accum_dtype   see accumulate_dw
 *   workspace    device, >= flce_workspace_bytes(...) bytes, 256-byte aligned
 *   stream       hipStream_t as void*
 *   stats        host pointer, may be NULL
 *
 * The call blocks once, on the host, after the row-compaction kernel, to read
 * the labelled-row count and the target range check (PR #1554, Summary: one
 * host sync).  Everything after that is enqueued asynchronously on `stream`;
 * outputs are valid in stream order.  FLCE_E_TARGET is reported at that sync,
 * before any projection runs; outputs are then unspecified.  Outputs must not
 * alias inputs, the workspace or each other: a written buffer whose byte range
 * (as sized above, the workspace by flce_workspace_bytes) overlaps another
 * buffer of the call returns FLCE_E_ARG before any launch.  Calls are
 * reentrant given distinct workspaces.
 */
int flce_fwd_bwd(const void* X, const void* W, const int64_t* targets, int64_t BT, int64_t H,
                 int64_t V, flce_dtype_t dtype, int64_t ignore_index, flce_reduction_t reduction,
                 int64_t chunk_size, int32_t chunk_mem_const, flce_dtype_t accum_dtype,
                 int32_t frozen_weight, int32_t accumulate_dw, const float* grad_output,
                 float* loss, void* dX, void* dW, void* workspace, size_t workspace_bytes,
                 void* stream, flce_stats_t* stats);

/*
 * Optional parts of the method, for flce_fwd_bwd_ex.  A zero-filled struct,
 * or NULL, gives exactly flce_fwd_bwd.
 *
 *   forward_only  1: the call computes the loss and the per-token outputs
 *                 below and nothing else.  No gradient GEMM runs and the
 *                 logits are never stored; dX, dW and grad_bias are not
 *                 touched and may be NULL.  Serves the none reduction, whose
 *                 per-token upstream gradient is only known in backward: the
 *                 forward asks for the loss, and backward calls again with
 *                 grad_output (PR #1554, Tests: the none reduction re-enters
 *                 the chunk loop).
 *   bias          [V] dtype, or NULL: every row's logits become
 *                 z = X W^T + bias (PR #1554, Tests: bias on and off).
 *   grad_bias     [V] accum_dtype, or NULL: the column sums of the logit
 *                 gradient, scaled like dW; overwritten, or added to when
 *                 accumulate_dw = 1.  Computed whenever given and not
 *                 forward_only (frozen_weight does not affect it).
 *   z_loss_scale  lam >= 0: the per-row loss gains lam * lse_i^2, where lse_i
 *                 is the row's log-sum-exp, and the gradient follows it.  The
 *                 pages name a per-token z-loss output without defining it;
 *                 lse^2 with this optional coefficient is the reading taken.
 *   z_loss        NULL, or lse_i^2 per labelled row: none -> [BT] (ignored
 *                 rows 0); mean / sum -> [1], reduced like the loss.
 *   accuracy      NULL, or 1 when the predicted token equals the target, else
 *                 0: none -> [BT] (ignored rows 0); mean / sum -> [1], reduced
 *                 like the loss (the fraction or the count of correct rows).
 *   predicted     NULL, or [BT] int64: the lowest column holding the row's
 *                 largest logit (fp32), -1 at ignored rows (PR #1554, Details
 *                 item 1: the per-token outputs of an ignored row are zero,
 *                 and its predicted token is the sentinel -1).
 * Pointers are device pointers: bias and grad_bias 16-byte aligned,
 * predicted 8-byte, z_loss and accuracy 4-byte.
 */
typedef struct {
  int32_t forward_only;
  const void* bias;
  void* grad_bias;
  float z_loss_scale;
  float* z_loss;
  float* accuracy;
  int64_t* predicted;
} flce_options_t;

/* Workspace for flce_fwd_bwd_ex with these options; with opt NULL it equals
 * flce_workspace_bytes.  A forward_only call needs no logits slab and far
 * less; the per-token outputs and grad_bias add small per-call arrays.
 * 0 when invalid. */
size_t flce_workspace_bytes_ex(int64_t BT, int64_t H, int64_t V, flce_dtype_t dtype,
                               int64_t chunk_size, int32_t chunk_mem_const,
                               const flce_options_t* opt);

/*
 * Where a call leaves its labelled-row index.  The row compaction of
 * flce_fwd_bwd / flce_fwd_bwd_ex (PR #1554, Summary: nonzero() of the
 * not-ignored mask supplies the rows the projections run on) writes the
 * ascending list of labelled row ids as int32 into the workspace, and the
 * chunk loop only reads it.  After a call with these arguments and options
 * returns FLCE_OK, the workspace holds that list at this byte offset,
 * stats.n_valid entries, valid in stream order until the workspace is
 * reused.  The offset is a multiple of 256.  Returns (size_t)-1 for
 * arguments flce_workspace_bytes_ex rejects.
 */
size_t flce_workspace_row_index_offset(int64_t BT, int64_t H, int64_t V, flce_dtype_t dtype,
                                       int64_t chunk_size, int32_t chunk_mem_const,
                                       const flce_options_t* opt);

/*
 * flce_fwd_bwd with the optional parts above; every other argument, the
 * single host sync, the errors and the stream semantics are flce_fwd_bwd's.
 * With forward_only, dX and dW may be NULL.  Invalid options (misaligned
 * pointers, lam < 0 or not finite, forward_only not 0/1) return FLCE_E_ARG
 * before any launch.  The workspace must hold flce_workspace_bytes_ex bytes.
 */
int flce_fwd_bwd_ex(const void* X, const void* W, const int64_t* targets, int64_t BT, int64_t H,
                    int64_t V, flce_dtype_t dtype, int64_t ignore_index,
                    flce_reduction_t reduction, int64_t chunk_size, int32_t chunk_mem_const,
                    flce_dtype_t accum_dtype, int32_t frozen_weight, int32_t accumulate_dw,
                    const float* grad_output, float* loss, void* dX, void* dW, void* workspace,
                    size_t workspace_bytes, void* stream, flce_stats_t* stats,
                    const flce_options_t* opt);

/*
 * flce_fwd_bwd_ex without a workspace argument, for callers that cannot
 * allocate device memory (tight serving loops, harnesses that forbid
 * allocation).  The workspace is a static device array of
 * FLCE_SCRATCH_BYTES inside the library: one per GPU, at its own address,
 * taken when the library's code is loaded on that GPU and held until the
 * process ends.  The call allocates nothing, device or host (the one host
 * sync reads into plain host memory).  It still blocks once at that sync,
 * so it cannot be captured into a HIP graph.
 *
 * Arguments, results, the sync, the errors and the stream semantics are
 * flce_fwd_bwd_ex's.  In addition:
 *   - a call whose flce_workspace_bytes_ex exceeds FLCE_SCRATCH_BYTES
 *     returns FLCE_E_WORKSPACE before any launch (flce_last_error says how
 *     much it needs; a smaller chunk_size needs less);
 *   - the stream must run on the current device (else FLCE_E_ARG): the
 *     current device's array is used;
 *   - every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents (nothing in it needs to start at zero: each call
 *     writes every part before reading it).  Calls that overlap on one GPU,
 *     from several host threads or on several streams without ordering
 *     between them, race on it and must be serialised by the caller.
 */
#define FLCE_SCRATCH_BYTES (256ull << 20)

int flce_fwd_bwd_ex_noalloc(const void* X, const void* W, const int64_t* targets, int64_t BT,
                            int64_t H, int64_t V, flce_dtype_t dtype, int64_t ignore_index,
                            flce_reduction_t reduction, int64_t chunk_size,
                            int32_t chunk_mem_const, flce_dtype_t accum_dtype,
                            int32_t frozen_weight, int32_t accumulate_dw,
                            const float* grad_output, float* loss, void* dX, void* dW,
                            void* stream, flce_stats_t* stats, const flce_options_t* opt);

/*
 * dst[i] = scale * src[i], converted to dst_dtype: the product is rounded to
 * fp32, then to dst_dtype (round to nearest even).  Serves the wrapper's two
 * elementwise steps: the final cast of an fp32 grad_weight to the weight
 * dtype (PR #1554, Tests: chunk storage is released before the final cast)
 * and scaling the stored gradients by the upstream gradient in backward.
 * src [n] src_dtype, dst [n] dst_dtype, device pointers of any alignment
 * (16-byte-aligned ones are moved as 16-byte vectors); scale is a device
 * float (NULL = 1).  src == dst is allowed when the dtypes match; n = 0 does
 * nothing.  Enqueued on `stream`.
 */
int flce_scale_cast(const void* src, flce_dtype_t src_dtype, void* dst, flce_dtype_t dst_dtype,
                    int64_t n, const float* scale, void* stream);

/* Error reporting.  The pages say nothing about how a native library reports
 * failure; these two serve the status codes above, which every entry point
 * returns instead of throwing.
 * flce_status_string: human-readable name of a status code (static storage;
 * "unknown status" for other values). */
const char* flce_status_string(int status);

/* Detail of the last error raised on the calling thread with a message:
 * every FLCE_E_HIP (the failing HIP call and its error string) and the
 * refusals of flce_fwd_bwd_ex_noalloc (thread-local storage, overwritten by
 * the next such error; empty before the first). */
const char* flce_last_error(void);

/* ------------------------------------------------------------------------
 * Measurement.  While a profile is open on the calling thread, every kernel
 * that flce_fwd_bwd enqueues is bracketed by a pair of HIP events on the
 * stream it runs on, and flce_profile_end sums their elapsed times per
 * kernel kind.  This is how per-kernel durations are measured live for the
 * roofline figures (the achieved rate of each kernel against MI355X peak).
 * ---------------------------------------------------------------------- */
typedef enum {
  FLCE_K_MASK_SCAN = 0,   /* ignore mask, prefix sum, labelled-row index, range check */
  FLCE_K_ZERO_ROWS = 1,   /* zero dX / loss at ignored rows                          */
  FLCE_K_LOGITS = 2,      /* logits GEMM into the slab (+ row max / sum-exp)         */
  FLCE_K_SOFTMAX = 3,     /* in-place softmax-gradient pass over the slab            */
  FLCE_K_DX = 4,          /* grad_input GEMM                                          */
  FLCE_K_DX_REDUCE = 5,   /* fixed-order reduction of split grad_input partials      */
  FLCE_K_DW = 6,          /* grad_weight GEMM written into dW                         */
  FLCE_K_FINALIZE = 7,    /* loss reduction                                           */
  FLCE_K_FILL = 8,        /* zero-fill / cast helpers                                 */
  FLCE_K_GATHER = 9,      /* gather of the chunk's labelled X rows (transposed)       */
  FLCE_K_BIAS_GRAD = 10,  /* column sums of the logit gradient into grad_bias         */
  FLCE_K_COUNT = 11
} flce_kernel_kind_t;

typedef struct {
  int64_t launches[FLCE_K_COUNT];
  double total_ms[FLCE_K_COUNT];
} flce_profile_t;

/* Open a profile on the calling thread (clears any previous one). */
int flce_profile_begin(void);

/* The same, bracketing only the kernels whose kind k has bit (1u << k) set
 * in kind_mask: each pair of events adds a few microseconds to the stream,
 * so a timed run brackets only the kernel it measures.  FLCE_E_ARG (and no
 * change) for an empty mask or bits at or above FLCE_K_COUNT. */
int flce_profile_begin_kinds(uint32_t kind_mask);

/* Close it: waits for the recorded events and fills *out.  Returns
 * FLCE_E_ARG if no profile is open. */
int flce_profile_end(flce_profile_t* out);

/* Name of a kernel kind (static storage). */
const char* flce_kernel_name(int kind);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H */
