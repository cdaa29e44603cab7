/*
 * cf.h -- C-ABI of the stitched-subgraph library (libcf.so) for AMD MI355X (gfx950).
 *
 * The library runs a dependency-rich memory-intensive subgraph -- elementwise
 * chains, row reductions feeding broadcasts, an expensive elementwise op
 * feeding a broadcast -- as ONE stitched kernel, and can run such a subgraph
 * as the epilogue of a bf16 MFMA GEMM whose output rows span several tiles.
 *
 * Sources of the method (cited by page title and section):
 *   [ComFuse] "ComFuse: Fusing Complex Memory-Intensive Subgraphs with
 *             Compute-Intensive Kernels For Modern GPU Architectures"
 *   [AStitch] "AStitch: enabling a new multi-dimensional optimization space for
 *             memory-intensive ML training and inference on modern SIMT
 *             architectures" (summary page)
 *   [sass2mlir] "sass2mlir: kernel fusion" (blog page)
 *
 * Conventions for every entry point below
 *   - Tensors are row-major with contiguous rows.  All tensor pointers are
 *     DEVICE pointers owned by the caller; the library never allocates, frees
 *     or synchronizes inside a call.  A call only enqueues work on `stream`
 *     (0 = the null stream) and returns.
 *   - bf16 tensors are passed as arrays of bfloat16 bit patterns (cf_bf16).
 *   - `ws`/`ws_bytes` is a caller-owned DEVICE workspace.  Query its size with
 *     cf_workspace_bytes() (0 means the plan needs none and ws may be NULL).
 *     A fresh workspace must be zero-filled ONCE before its first use (for
 *     example hipMemsetAsync(ws, 0, bytes)); the kernels leave it in a state
 *     that any later call (any shape, any op) accepts, so it never needs
 *     clearing again.  Two calls that may run at the same time must not share
 *     a workspace.  Byte 0..3 of a workspace hold an error word: non-zero
 *     means a cross-workgroup wait gave up (see CF_EOCCUPANCY); the caller may
 *     read and clear it (cf_workspace_error).
 *   - Residency.  Plans whose workgroups wait on each other (rows split over
 *     workgroups, the GEMM epilogues across tiles, the Global scheme of
 *     generated kernels) size their grid to what the device keeps resident
 *     when the call has it to itself, and assume that no other kernel holds
 *     compute units while they run (a kernel on another stream, or another
 *     process's).  If that does not hold, a member that waits for one that
 *     was never scheduled gives up after its spin cap (about a second), sets
 *     the error word, and the call's output is wrong: the call itself still
 *     returns CF_OK, since it only enqueues.  Callers that cannot rule out
 *     concurrent kernels check the word after the stream completes.
 *   - Errors are reported by the return value only.  Argument validation
 *     happens before any HIP call, so an invalid call enqueues nothing.
 *   - Results are bitwise reproducible run to run for a given shape and device:
 *     the row-to-workgroup mapping and every combine order are fixed.
 *   - Thread-safe: the only shared state is a per-device property cache.
 */
#ifndef CF_H
#define CF_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t cf_bf16; /* bfloat16 bit pattern */

typedef enum cf_status {
  CF_OK = 0,
  CF_EINVAL = 1,        /* null pointer, non-positive size, aliasing, bad scalar */
  CF_EUNSUPPORTED = 2,  /* shape outside what the kernels handle (see each call) */
  CF_EALIGN = 3,        /* pointer or row pitch not 16-byte aligned where required */
  CF_EWORKSPACE = 4,    /* ws_bytes smaller than cf_workspace_bytes(), or ws NULL */
  CF_EOCCUPANCY = 5,    /* the workgroups that must wait on each other cannot all be resident */
  CF_EHIP = 6           /* a HIP runtime call failed (the launch, or a device query) */
} cf_status;

/* Read a workspace's error word (bytes 0..3) into *out: 0, or non-zero when a
 * cross-workgroup wait of a call that used `ws` gave up (that call's output is
 * wrong; see "Residency" above).  Enqueues the 4-byte read on `stream` and
 * waits for the stream, so every earlier call on it has completed; with
 * `clear` non-zero the word is then zeroed (by a kernel on `stream`, which the
 * function also waits for).  This call synchronizes: it is not for use under
 * graph capture.  CF_EINVAL for a NULL ws or out, CF_EHIP if a HIP call fails. */
cf_status cf_workspace_error(const void* ws, int clear, uint32_t* out, hipStream_t stream);

/* Operation ids for cf_workspace_bytes / cf_unfused_workspace_bytes. */
enum {
  CF_OP_STITCH_SOFTMAX = 1,       /* d0 = rows, d1 = cols            */
  CF_OP_STITCH_LAYERNORM = 2,     /* d0 = rows, d1 = cols            */
  CF_OP_STITCH_POW_BCAST_ADD = 3, /* d0 = rows, d1 = cols            */
  CF_OP_GEMM_LN = 4,              /* d0 = M, d1 = N, d2 = K          */
  CF_OP_GEMM_SOFTMAX = 5,         /* d0 = M, d1 = N, d2 = D          */
  CF_OP_GEMM_SOFTMAX_GEMM = 6,    /* d0 = M, d1 = N, d2 = D (any Dv <= 128) */
  CF_OP_STITCH_LAYERNORM_AFFINE = 7, /* d0 = rows, d1 = cols         */
  CF_OP_STITCH_RMSNORM = 8,       /* d0 = rows, d1 = cols            */
  CF_OP_GEMM_ACT = 9              /* d0 = M, d1 = N, d2 = K          */
};

/* Unary activations of cf_gemm_act (fp32, applied to u = A.W + bias). */
enum {
  CF_ACT_NONE = 0,      /* y = u                                            */
  CF_ACT_RELU = 1,      /* y = max(u, 0)                                    */
  CF_ACT_GELU_TANH = 2, /* y = 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))) */
  CF_ACT_SILU = 3,      /* y = u / (1 + exp(-u))                            */
  CF_ACT_SQUARE = 4,    /* y = u * u                                        */
  CF_ACT_RSQRT = 5      /* y = 1 / sqrt(u) (inf at 0, NaN below; no eps)   */
};

/* Workspace bytes the fused call needs for this shape on the current device
 * (0 = none).  Returns (size_t)-1 for an unknown op or invalid dims. */
size_t cf_workspace_bytes(int op, int64_t d0, int64_t d1, int64_t d2);

/* Human-readable name of a status code (static storage). */
const char* cf_status_str(cf_status s);

/* Writes a JSON description of the plan chosen by the last cf_* call made on
 * the calling host thread (kernel, grid, block, mapping, split, aggregation)
 * into buf (NUL-terminated, truncated to n).  Returns the untruncated length. */
int cf_last_plan(char* buf, size_t n);

/* ------------------------------------------------------------------------ */
/* Stitched memory-intensive subgraphs (fp32 in, fp32 out, fp32 arithmetic). */
/* Any rows >= 1 and cols >= 1 are accepted (tails are masked).  x and y must */
/* not overlap.  Rows of 4-multiple width with 16-byte aligned x and y use    */
/* 16-byte fragments; other shapes use a 4-byte-fragment variant.            */
/* ------------------------------------------------------------------------ */

/* y = softmax(x) over each row:  m_i = max_j x_ij;  e = exp(x - m_i);
 * s_i = sum_j e_ij;  y = e / s_i.
 * [ComFuse] Stage-Stream Execution Model (fragment compute phase, three-level
 * reduce phase of Fig. 4, stage chaining through the terminal reduction);
 * [AStitch] "What people did before" (a reduction feeding a broadcast).
 * Rows wider than one workgroup holds are split over several workgroups that
 * aggregate through `ws` ([ComFuse] inter-CTA level; [AStitch] task splitting). */
cf_status cf_stitch_softmax(const float* x, float* y, int64_t rows, int64_t cols,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* y = LayerNorm(x) over each row, no affine: mu_i = (sum_j x_ij) / cols;
 * c = x - mu_i;  var_i = (sum_j c_ij^2) / cols;  y = c / sqrt(var_i + eps).
 * eps must be >= 0.  [ComFuse] Stage-Stream Execution Model, bypass path of
 * Fig. 3 (x feeds the mean and, unrecomputed, the x - mean stage);
 * [AStitch] "Adaptive thread mapping" (horizontal packing of short rows). */
cf_status cf_stitch_layernorm(const float* x, float* y, int64_t rows, int64_t cols, float eps,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* Y = x + broadcast_col(v^p)  (Y_ij = x_ij + v_i^p, v has `rows` entries, v_i >= 0),
 * then y = softmax(Y) over each row.  If y_pre is not NULL, Y is also written
 * there.  v^p is computed once per row per workgroup and shared through LDS,
 * never per element.  [AStitch] "What people did before" (power -> broadcast
 * -> add recomputed per consumer when fused through registers only),
 * "Four stitching schemes" (Regional: one-to-many values buffered on chip). */
cf_status cf_stitch_pow_bcast_add(const float* x, const float* v, float p, float* y, float* y_pre,
                                  int64_t rows, int64_t cols, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* y = LayerNorm(x) * gamma + beta over each row (population variance, eps
 * inside the root); gamma, beta fp32 [cols], row-vector broadcasts, not
 * NULL, not overlapping y.  Same planning and rules as cf_stitch_layernorm.
 * [ComFuse] Frontend / Fusion Spec IR (LayerNorm among the stage DAGs the
 * split at reduction nodes covers; 1-D parameters as row-vector broadcasts,
 * the Phi patterns). */
cf_status cf_stitch_layernorm_affine(const float* x, const float* gamma, const float* beta, float* y,
                                     int64_t rows, int64_t cols, float eps, void* ws, size_t ws_bytes,
                                     hipStream_t stream);

/* y = x * rsqrt(mean(x^2) + eps) * gamma over each row (mean over cols);
 * gamma fp32 [cols] or NULL (gain 1); eps >= 0.  One reduction stage whose
 * broadcast result scales the values held from the first stage.  Same
 * planning and rules as cf_stitch_layernorm.  [ComFuse] Stage-Stream
 * Execution Model (bypass path), Frontend / Fusion Spec IR (Phi patterns). */
cf_status cf_stitch_rmsnorm(const float* x, const float* gamma, float* y, int64_t rows, int64_t cols,
                            float eps, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* GEMM with a stitched epilogue across output tiles (bf16 in, fp32          */
/* accumulate, bf16 out by round-to-nearest-even).  Requires N % 8 == 0,      */
/* K % 8 == 0 (D % 8 == 0), 16-byte aligned matrix pointers; M, N, K tails    */
/* against the tile sizes are masked.                                         */
/* ------------------------------------------------------------------------ */

/* Y = LayerNorm(A.W + bias + R) * gamma + beta over each row of length N.
 * A [M x K], W [K x N] (N contiguous), R [M x N] or NULL (no residual),
 * bias/gamma/beta fp32 [N] (row-vector broadcasts), Y [M x N]; eps >= 0.
 * Population variance, eps inside the root, residual before the statistics.
 * [ComFuse] Stage-Stream Execution Model (Fig. 3: x = alpha*Acc + Bias feeds
 * the mean and the x - mean stage; rows spanning several tiles aggregate at
 * the inter-CTA level); [sass2mlir] "Epilogue fusion" (one owner per output). */
cf_status cf_gemm_ln(const cf_bf16* A, const cf_bf16* W, const float* bias, const cf_bf16* R,
                     const float* gamma, const float* beta, float eps, cf_bf16* Y,
                     int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* cf_gemm_ln without a workspace argument, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, kernels and results as cf_gemm_ln; the
 * cross-tile partials and join words live in a 16 MiB static device array of
 * the library (one per GPU, held until the process ends), and nothing is
 * allocated or freed.  Shapes whose workspace (cf_workspace_bytes for
 * CF_OP_GEMM_LN) exceeds 16 MiB return CF_EWORKSPACE before any launch.  Each
 * call first clears the array's error and join words with a small kernel on
 * `stream`.  Every call on one GPU shares the array: calls that overlap on one
 * GPU (other streams, other host threads) race and must not be issued. */
cf_status cf_gemm_ln_noalloc(const cf_bf16* A, const cf_bf16* W, const float* bias, const cf_bf16* R,
                             const float* gamma, const float* beta, float eps, cf_bf16* Y,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* S = softmax(scale * Q.K^T) over each row of length N.
 * Q [M x D], K [N x D] (both D contiguous), S [M x N]; scale finite.
 * Cross-tile max and sum aggregation.  A NaN score makes its whole output
 * row NaN; other rows are unaffected.  [ComFuse] B2BGEMM (eq. 3: S_tile =
 * F(P_tile) formed in the first MatMul's epilogue) and the inter-CTA level. */
cf_status cf_gemm_softmax(const cf_bf16* Q, const cf_bf16* K, float scale, cf_bf16* S,
                          int64_t M, int64_t N, int64_t D, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* O = softmax(scale * Q.K^T) . V: two MatMuls back to back, the row softmax
 * between them, S never written.  Q [M x D], K [N x D] (both D contiguous),
 * V [N x Dv] (Dv contiguous), O [M x Dv]; scale finite; D <= 128,
 * 8 <= Dv <= 128 with Dv % 8 == 0.  The S tile feeds the second MatMul from
 * registers; partial outputs over the contraction dimension N are summed in
 * a fixed order before the commit, so results are deterministic.  A NaN
 * score makes its whole output row NaN; other rows are unaffected.
 * [ComFuse] B2BGEMM (eq. 3: S_tile = F(P_tile); eq. 4: partial products
 * S_tile.W2_tile over the contraction dimension; eq. 5: their sum at the
 * commit; one circular buffer shared by the W1 and W2 tiles), with F the
 * cross-tile softmax of the Stage-Stream Execution Model. */
cf_status cf_gemm_softmax_gemm(const cf_bf16* Q, const cf_bf16* K, const cf_bf16* V, float scale,
                               cf_bf16* O, int64_t M, int64_t N, int64_t D, int64_t Dv,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* Y = act(A.W + bias) per element.  A [M x K], W [K x N] (N contiguous),
 * bias fp32 [N] (row-vector broadcast, 16-byte aligned) or NULL (no bias),
 * act one of CF_ACT_* (anything else: CF_EINVAL), Y [M x N] not overlapping
 * A, W or bias.  The accumulator goes through bias and activation in
 * registers and leaves as bf16; every output element belongs to one tile, so
 * the tiles never wait on each other and the call needs no workspace
 * (cf_workspace_bytes returns 0; ws may be NULL and is not touched).
 * [ComFuse] Frontend / Fusion Spec IR (1-D parameters become row-vector
 * broadcasts, unary functions such as activations, rsqrt and squares become
 * computation nodes) and Stage-Stream Execution Model (Fig. 3: x = alpha*Acc
 * + Bias, here alpha = 1); [sass2mlir] "Epilogue fusion" (consumer math in the
 * producer's registers; one owner per output element). */
cf_status cf_gemm_act(const cf_bf16* A, const cf_bf16* W, const float* bias, int act, cf_bf16* Y,
                      int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Unfused baselines: the same subgraphs as one kernel per operator, with     */
/* fp32 intermediates in the workspace (in HBM) and broadcasts folded into    */
/* the consumer's indexing.  Same arguments and results (up to rounding) as   */
/* the fused calls.  The intermediates sit past the workspace's header and    */
/* join words, so one zero-filled workspace of the larger of the two sizes    */
/* serves both kinds of call.  [AStitch] "What people did before" (kernel     */
/* storm);                                                                    */
/* [sass2mlir] "What graphs deliberately don't do" (round trips remain).      */
/* ------------------------------------------------------------------------ */

size_t cf_unfused_workspace_bytes(int op, int64_t d0, int64_t d1, int64_t d2);

cf_status cf_unfused_stitch_softmax(const float* x, float* y, int64_t rows, int64_t cols,
                                    void* ws, size_t ws_bytes, hipStream_t stream);
cf_status cf_unfused_stitch_layernorm(const float* x, float* y, int64_t rows, int64_t cols,
                                      float eps, void* ws, size_t ws_bytes, hipStream_t stream);
cf_status cf_unfused_stitch_pow_bcast_add(const float* x, const float* v, float p, float* y,
                                          float* y_pre, int64_t rows, int64_t cols, void* ws,
                                          size_t ws_bytes, hipStream_t stream);
cf_status cf_unfused_stitch_layernorm_affine(const float* x, const float* gamma, const float* beta,
                                             float* y, int64_t rows, int64_t cols, float eps, void* ws,
                                             size_t ws_bytes, hipStream_t stream);
cf_status cf_unfused_stitch_rmsnorm(const float* x, const float* gamma, float* y, int64_t rows,
                                    int64_t cols, float eps, void* ws, size_t ws_bytes,
                                    hipStream_t stream);
cf_status cf_unfused_gemm_ln(const cf_bf16* A, const cf_bf16* W, const float* bias,
                             const cf_bf16* R, const float* gamma, const float* beta, float eps,
                             cf_bf16* Y, int64_t M, int64_t N, int64_t K, void* ws,
                             size_t ws_bytes, hipStream_t stream);
cf_status cf_unfused_gemm_softmax(const cf_bf16* Q, const cf_bf16* K, float scale, cf_bf16* S,
                                  int64_t M, int64_t N, int64_t D, void* ws, size_t ws_bytes,
                                  hipStream_t stream);
/* The softmax chain above writes S (bf16, [M x N]) to the workspace; a plain
 * GEMM S.V (fp32 out) and a cast then produce O. */
cf_status cf_unfused_gemm_softmax_gemm(const cf_bf16* Q, const cf_bf16* K, const cf_bf16* V,
                                       float scale, cf_bf16* O, int64_t M, int64_t N, int64_t D,
                                       int64_t Dv, void* ws, size_t ws_bytes, hipStream_t stream);
/* A plain GEMM (fp32 out), the bias add (skipped without bias), the
 * activation (skipped for CF_ACT_NONE) and the cast, one kernel each. */
cf_status cf_unfused_gemm_act(const cf_bf16* A, const cf_bf16* W, const float* bias, int act,
                              cf_bf16* Y, int64_t M, int64_t N, int64_t K, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Graph replay of a captured sequence of calls (used to time the unfused     */
/* chains without per-launch host cost).  [sass2mlir] "Building the DAG"      */
/* (stream capture), "Paying the setup cost once" (instantiate + upload).     */
/* ------------------------------------------------------------------------ */

/* Starts capturing `stream` (global capture mode).  Calls enqueued on the
 * stream until cf_graph_end are recorded, not run. */
cf_status cf_graph_begin(hipStream_t stream);
/* Ends the capture, instantiates the graph and uploads it to `stream`'s device.
 * *exec receives an opaque handle owned by the caller (free with cf_graph_destroy). */
cf_status cf_graph_end(hipStream_t stream, void** exec);
/* Enqueues one replay of the graph on `stream`. */
cf_status cf_graph_launch(void* exec, hipStream_t stream);
cf_status cf_graph_destroy(void* exec);

/* ------------------------------------------------------------------------ */
/* Utilities for measurement (not part of any subgraph).                      */
/* ------------------------------------------------------------------------ */

/* p[i] = value for i < n (writes n*4 bytes; used to evict caches between timed runs). */
cf_status cf_util_fill_f32(float* p, int64_t n, float value, hipStream_t stream);
/* dst[i] = src[i] for i < n (reads and writes n*4 bytes; a copy of known traffic,
 * used to calibrate hardware byte counters).  16-byte aligned pointers. */
cf_status cf_util_copy_f32(const float* src, float* dst, int64_t n, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CF_H */
