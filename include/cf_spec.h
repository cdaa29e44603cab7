/*
 * cf_spec.h -- Fusion Spec IR front end of libcf.so: a captured epilogue or
 * memory-intensive subgraph in, a launchable stitched kernel out.
 *
 * [ComFuse] Frontend / Fusion Spec IR (eq. 9: G_epi --Phi--> S --Psi--> T;
 * eq. 10: S = <N, E, tau, A, C>).  The caller describes the subgraph as a
 * list of raw operator nodes (cf_gnode).  cf_spec_build applies Phi: a
 * top-down traversal from the root (the MatMul, or the 2-D input of a
 * memory-intensive subgraph) that maps
 *   - a binary operator to a broadcast node for each operand that is not a
 *     full tile plus one computation node,
 *   - a constant to a scalar broadcast node,
 *   - a 1-D placeholder to a row-vector broadcast (or, for the per-row
 *     vectors of [AStitch] "What people did before", a column broadcast)
 *     and an entry of the runtime parameter table A,
 *   - a unary function to a computation node,
 *   - a row reduction to a split: the nodes after it form a nested S (C)
 *     whose entry points are a placeholder for the reduction's statistic
 *     and placeholders for the tensors from before the reduction that the
 *     later nodes still read (the passthrough of LayerNorm's x - mean).
 * Psi here does not generate code: it walks S structurally into a canonical
 * form and matches it against the stage DAGs the library's precompiled
 * kernels implement, binding the graph's constants and placeholders to the
 * kernel's arguments.  A graph outside Phi's pattern set, or whose S matches
 * no kernel, is refused with CF_EUNSUPPORTED and nothing else happens (the
 * caller falls back to its own path): a spec that builds computes exactly
 * the graph's semantics.
 *
 * Accepted forms (operand order of ADD and MUL is free; association is not):
 *   softmax        e = exp(x - rowmax(x)); y = e / rowsum(e)
 *   LayerNorm      mu = rowsum(x) / cols; c = x - mu;
 *                  y = c * rsqrt(rowsum(square(c)) / cols + eps)   [* gamma + beta]
 *   RMSNorm        y = x * rsqrt(rowsum(square(x)) / cols + eps)   [* gamma]
 *   pow-softmax    softmax(x + pow(v, p)), v a per-row vector
 *   GEMM+LN        the LayerNorm form on u = (A.W + bias) [+ R], with gamma, beta
 *   GEMM+softmax   the softmax form on A.B^T * scale
 *   GEMM+act       act(A.W [+ bias]), act one of RELU, GELU_TANH, SILU, SQUARE,
 *                  RSQRT, or none (the MatMul, or MatMul + bias, is the output)
 * Constants: the row length in a mean must equal cols; eps >= 0, p, scale
 * are bound as arguments.
 */
#ifndef CF_SPEC_H
#define CF_SPEC_H

#include "cf.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Operator kinds of a captured graph node. */
typedef enum cf_gop {
  CF_G_INPUT = 0,     /* 2-D fp32 input [rows x cols] of a memory-intensive subgraph      */
  CF_G_OPERAND = 1,   /* 2-D bf16 MatMul operand placeholder                             */
  CF_G_MATMUL = 2,    /* in0 . in1 (attr 0: in1 is [K x cols]; attr 1: in1 is [cols x K]) */
  CF_G_ROWVEC = 3,    /* 1-D fp32 placeholder of length cols (row-vector broadcast)      */
  CF_G_COLVEC = 4,    /* 1-D fp32 placeholder of length rows (one value per row)         */
  CF_G_TENSOR = 5,    /* 2-D bf16 placeholder [rows x cols] added elementwise (residual) */
  CF_G_CONST = 6,     /* scalar constant `value`                                         */
  CF_G_ADD = 7,
  CF_G_SUB = 8,
  CF_G_MUL = 9,
  CF_G_DIV = 10,
  CF_G_POW = 11,      /* in0 ^ in1 (in1 a constant): the real power; an integral         */
                      /* exponent takes either sign of in0, x^0 = 1, a negative in0     */
                      /* with a non-integral exponent gives NaN                          */
  CF_G_EXP = 12,
  CF_G_SQUARE = 13,
  CF_G_RSQRT = 14,
  CF_G_RELU = 15,
  CF_G_GELU_TANH = 16,
  CF_G_SILU = 17,
  CF_G_ROWSUM = 18,   /* reduction over the row: one value per row                       */
  CF_G_ROWMAX = 19
} cf_gop;

/* One node of the captured graph.  Inputs refer to earlier nodes (-1 when
 * unused).  Placeholders (INPUT, OPERAND, ROWVEC, COLVEC, TENSOR) name the
 * index of their device pointer in the `args` array of cf_spec_launch. */
typedef struct cf_gnode {
  int32_t op;
  int32_t in0, in1;
  int32_t attr;  /* MATMUL: operand layout (see CF_G_MATMUL) */
  int32_t slot;  /* placeholders: index into args[] */
  double value;  /* CONST */
} cf_gnode;

typedef struct cf_spec cf_spec;

/* Phi then Psi for the graph nodes[0..n) with output node `terminal`, for
 * output rows x cols (and reduction depth k for a MatMul root, else 0).
 * Host-only (no device call).  On success *out receives a spec owned by the
 * caller (free with cf_spec_free).  CF_EINVAL: malformed graph (bad index,
 * cycle, missing input).  CF_EUNSUPPORTED: outside Phi's patterns, or no
 * kernel implements its S. */
cf_status cf_spec_build(const cf_gnode* nodes, int n, int terminal, int64_t rows, int64_t cols, int64_t k,
                        cf_spec** out);

/* JSON description of S (levels, node categories, edges, tau, parameter
 * table A, nesting C) and of Psi's match (kernel, bound constants and
 * arguments), NUL-terminated and truncated to n.  Returns the full length. */
int cf_spec_describe(const cf_spec* s, char* buf, size_t n);

/* Workspace bytes the matched kernel needs (cf_workspace_bytes of its op). */
size_t cf_spec_workspace_bytes(const cf_spec* s);

/* Enqueue the matched kernel: args[slot] are the device pointers of the
 * graph's placeholders, out the terminal's output (fp32 for a
 * memory-intensive subgraph, bf16 for a MatMul root).  Same rules, errors
 * and workspace contract as the entry point it dispatches to. */
cf_status cf_spec_launch(const cf_spec* s, const void* const* args, int nargs, void* out, void* ws,
                         size_t ws_bytes, hipStream_t stream);

void cf_spec_free(cf_spec* s);

/* ------------------------------------------------------------------------ */
/* Automatic stitching of an arbitrary memory-intensive graph.                */
/*                                                                            */
/* [AStitch] "Making it automatic" (dominant ops, index propagation, merging  */
/* of dominants, passive block-locality check), "Four stitching schemes"      */
/* (where each value lives), "Adaptive thread mapping".  For graphs outside   */
/* Psi's kernel set: the scheduler finds the dominants (row reductions,       */
/* expensive ops whose per-row result feeds a broadcast, the output),         */
/* propagates the row-fragment thread mapping from them through the           */
/* one-to-one ops, merges them into one stitched group, decides per edge      */
/* whether the value stays in the thread's registers (Local), crosses waves   */
/* through LDS (Regional) or crosses workgroups through global memory and a   */
/* join (Global), picks the mapping by the row length, and                    */
/* generates one HIP kernel for the group, compiled at build time with        */
/* hiprtc for gfx950.                                                         */
/*                                                                            */
/* Accepted graphs: CF_G_INPUT placeholders (any number, fp32 [rows x cols]), */
/* ROWVEC, COLVEC, CONST, the binary and unary operators, ROWSUM and ROWMAX;  */
/* the terminal is a tile.  Rows of up to 32768 values run one workgroup per  */
/* row at most; wider rows (up to 256 x 8192 values) are cut into slices of   */
/* 8192, one workgroup each, whose members join at every row reduction.       */
/* ------------------------------------------------------------------------ */

typedef struct cf_auto cf_auto;

/* Schedule the graph, generate its kernel and compile it (host only: no
 * device call).  CF_EINVAL: malformed graph; CF_EUNSUPPORTED: outside the
 * accepted graphs; CF_EHIP: the runtime compiler failed. */
cf_status cf_auto_build(const cf_gnode* nodes, int n, int terminal, int64_t rows, int64_t cols,
                        cf_auto** out);

/* JSON: dominants, merged groups, per-edge stitching scheme, thread mapping,
 * parameters, generated source and code sizes.  Returns the full length. */
int cf_auto_describe(const cf_auto* a, char* buf, size_t n);

/* The generated HIP source.  Returns the full length. */
int cf_auto_source(const cf_auto* a, char* buf, size_t n);

/* Workspace bytes the generated kernel needs on the current device: 0 unless
 * rows span workgroups and the graph has a row reduction (members that
 * exchange nothing need none).  Then, in cf.h's fixed workspace layout: the header
 * and join-word region, followed by one 8-byte tagged partial slot per
 * member, row reduction and row of two rounds of co-resident rows.  Every
 * launch clears its slots and joins each row's members once before it reads
 * any slot, so the workspace may serve any op in any order.  Loads the code
 * object on the device.  (size_t)-1 on failure. */
size_t cf_auto_workspace_bytes(cf_auto* a);

/* Enqueue the generated kernel: args[slot] are the placeholders' device
 * pointers, out the fp32 [rows x cols] output (not overlapping any input).
 * Loads the code object on the current device at its first launch there.
 * 16-byte aligned pointers and cols % 4 == 0 select the 16-byte-fragment
 * variant, anything else the 4-byte one.  ws/ws_bytes: the workspace (same
 * contract as cf.h's: zero-filled once, error word at byte 0), needed only
 * when cf_auto_workspace_bytes is non-zero; CF_EOCCUPANCY when not even one
 * row's workgroups can be resident.  The Global scheme's members wait on
 * each other: they assume no other kernel holds compute units meanwhile (see
 * "Residency" in cf.h); a wait that gives up sets the error word and leaves
 * the output wrong, which cf_workspace_error reports after the stream
 * completes.  Free the kernel (cf_auto_free) only after the work it enqueued
 * has completed. */
cf_status cf_auto_launch(cf_auto* a, const void* const* args, int nargs, float* out, void* ws, size_t ws_bytes,
                         hipStream_t stream);

void cf_auto_free(cf_auto* a);

#ifdef __cplusplus
}
#endif

#endif /* CF_SPEC_H */
