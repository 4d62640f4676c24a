/*
 * rmsnorm.h -- C ABI of the MI355X (gfx950) training-RMSNorm library.
 *
 * Operation (FlashInfer training-RMSNorm pages: p1 = "feat(cake_rmsnorm):
 * opt-in non-deterministic weight gradient for the autograd RMSNorm - #8208"
 * with its #8577 commit text, p2 = PR #8899, p3 = "fix(cake_rmsnorm_det):
 * tighten two large-row weight-gradient accuracy edges - #8293"):
 *
 *   forward   rstd = 1/sqrt(mean_j u_j^2 + eps),  y = u * rstd * w
 *             where u = x, or u = h = bf16(x + r) with the fused residual add
 *             (p1 #8577 opening paragraph and "Key": `res` adds the BF16
 *             output h_new).  y and h are BF16, rstd FP32.
 *   backward  xhat = u * rstd,  c = mean_j(xhat_j * w_j * dy_j)
 *             dx = rstd * (w * dy - xhat * c) [+ dres]   (BF16)
 *             dw = sum over all rows of dy * xhat         (FP32)
 *             with deterministic = 1 (fixed-order, bitwise reproducible dw)
 *             or 0 (dw reproducible only within its error budget);
 *             dx is bitwise the same in both modes and from call to call
 *             (p1 #8208 commit message).
 *
 * Tensors.  Every activation tensor (x, r, h, y, dy, dres, dx) is BF16 with
 * the logical shape [T, heads, H] and element strides (stride_t, stride_h, 1);
 * all of them share these strides.  heads = 1 gives plain [T, H] rows
 * (stride_t >= H).  heads > 1 gives per-head views sharing one w[H]
 * (p1 #8577 "Key": [T,24,256] strided and [T,4,256] contiguous), and then the
 * rows are R = T * heads.  rstd is a contiguous FP32 [R] array indexed
 * t * heads + head.  w is [H], BF16 or FP32; dw is a contiguous FP32 [H].
 *
 * Memory and streams.  All pointers are device pointers owned by the caller.
 * The library never allocates, frees or synchronises: a call validates its
 * arguments on the host (before any HIP call), enqueues its kernels on
 * `stream` (a hipStream_t; NULL = the default stream) and returns.
 *
 * Requirements checked on entry (violations return an error, nothing runs):
 *   - H % 8 == 0 and 8 <= H <= RMSN_MAX_H                  else RMSN_ERR_UNSUPPORTED
 *   - T >= 0, heads >= 1, R = T*heads < 2^30, eps finite >= 0
 *   - rows do not overlap: heads == 1: stride_t >= H (or T <= 1);
 *     heads > 1: stride_h >= H and stride_t >= heads*stride_h (or T <= 1)
 *                                                         else RMSN_ERR_INVALID_ARG
 *   - activation pointers and w 16-byte aligned, stride_t and stride_h
 *     multiples of 8 elements; rstd and dw 4-byte aligned;
 *     workspace 256-byte aligned                          else RMSN_ERR_MISALIGNED
 * Aliasing: y may be x, residual_out may be x or residual, dx may be dy or
 * dres (whole tensors with identical strides).  Other overlaps are undefined.
 * Errors in a kernel launch return RMSN_ERR_HIP.  R == 0 is valid: the
 * forward does nothing and the backward writes dw = 0.
 */
#ifndef RMSNORM_MI355X_H
#define RMSNORM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum rmsn_status {
    RMSN_OK = 0,
    RMSN_ERR_INVALID_ARG = 1,
    RMSN_ERR_UNSUPPORTED = 2,
    RMSN_ERR_MISALIGNED = 3,
    RMSN_ERR_WORKSPACE = 4,
    RMSN_ERR_HIP = 5
};

enum rmsn_dtype { RMSN_W_BF16 = 0, RMSN_W_F32 = 1 };

#define RMSN_MAX_H 16384

/*
 * Forward (p1 #8577 opening paragraph: its outputs are y in BF16 and rstd in
 * FP32; p1 #8577 "Key" for `res`, `w32` and the per-head views).
 *   x            [T,heads,H] BF16 input.
 *   residual     [T,heads,H] BF16 r, or NULL.  With r, h = bf16(x + r) (sum in
 *                FP32, one round-to-nearest-even) is written to residual_out
 *                and normalised in place of x.
 *   w            [H] weight, BF16 (w_dtype = RMSN_W_BF16) or FP32 (RMSN_W_F32).
 *   y            [T,heads,H] BF16 output y = bf16(u * rstd * w).
 *   residual_out [T,heads,H] BF16 output h; required iff residual != NULL.
 *   rstd         [R] FP32 output.
 *   eps          added to the mean of squares (the pages measure eps = 1e-6).
 *   deterministic accepted for symmetry with the backward; the forward is
 *                the same program, bit for bit, in both modes (p1 #8577
 *                opening paragraph: both modes share one forward).
 * A row's rstd and y (and h) depend only on that row, w, eps and H: the
 * order of its sum of squares is fixed by H, whatever the row count, the
 * strides or the residual (the grid and the rows per workgroup, which do
 * vary with the row count, never split a row differently).
 */
int rmsnorm_fwd(const void* x, const void* residual, const void* w, int w_dtype,
                void* y, void* residual_out, float* rstd,
                int64_t T, int64_t heads, int64_t H, int64_t stride_t, int64_t stride_h,
                double eps, int deterministic, void* stream);

/*
 * Workspace bytes that rmsnorm_bwd needs for these arguments (p1 #8208 page:
 * the facade exposes backward_workspace_bytes / backward_workspace, which
 * take the backward's arguments and its deterministic flag).
 *   T, heads, H  the backward's shape (as for rmsnorm_bwd).
 *   w_dtype      the weight's dtype (RMSN_W_BF16 or RMSN_W_F32).
 *   residual     the dres pointer the backward will be given, or NULL; only
 *                whether it is NULL matters (it is never dereferenced).
 *   deterministic the backward's flag.
 * The size is that of the route rmsnorm_bwd takes for the same arguments
 * (rmsnorm_bwd_route), and with residual NULL at least that of the route
 * rmsnorm_gated_bwd takes for the same shape, so one size serves both.  A
 * workspace sized for one mode, or for a non-NULL residual, may be too small
 * for the other mode, or for residual NULL: size it with both (the larger)
 * to share it.  A pure
 * function of its arguments; it makes no HIP call.  Always at least the
 * prepared part of rmsnorm_bwd_workspace_init; returns 0 when the shape or
 * w_dtype is invalid or unsupported.
 */
size_t rmsnorm_bwd_workspace_size(int64_t T, int64_t heads, int64_t H, int w_dtype, const void* residual,
                                  int deterministic);

/*
 * Prepare a workspace for first use: zero-fills the part that the
 * non-deterministic backward keeps between calls (arrival tickets and an
 * FP64 [H] accumulator).  Every non-deterministic call leaves that part zero
 * again, so this is needed once per fresh allocation (or after a failed
 * call).  A workspace that is all zero bytes is already prepared.  A
 * deterministic call reads only what it wrote itself earlier in the same
 * call, so it needs no preparation and leaves the tickets and accumulator
 * as it found them.
 */
int rmsnorm_bwd_workspace_init(void* workspace, size_t workspace_bytes, int64_t H, void* stream);

/*
 * Backward (p1 #8577 opening paragraph: its outputs are dx in BF16 and dw in
 * FP32; p1 #8208 commit message for the deterministic flag).
 *   dy        [T,heads,H] BF16 incoming gradient of y.
 *   x         [T,heads,H] BF16 normalised input of the forward (h when the
 *             forward had a residual).
 *   rstd      [R] FP32, as written by rmsnorm_fwd.
 *   w, w_dtype  the forward's weight.
 *   residual  [T,heads,H] BF16 dres, the incoming gradient of h, or NULL; it
 *             is added to dx (dx is then the gradient of both x and r).
 *   dx        [T,heads,H] BF16 output; may be dy (in place).  Then the
 *             column forms run their column tasks, which read dy of every
 *             row, as a launch of their own before the row tasks that
 *             overwrite it: one launch more, the same bits.
 *   dw        [H] FP32 output, overwritten (not accumulated into).
 *   workspace at least rmsnorm_bwd_workspace_size(...) bytes, prepared once
 *             by rmsnorm_bwd_workspace_init; must not be used by two calls
 *             at the same time.
 *   deterministic 1: dw is summed in an order fixed by the shape alone (a
 *             fixed-order pair, or the column form; rmsnorm_bwd_route reports
 *             which), so it is bitwise reproducible for a given shape on any
 *             MI355X, and the workspace may hold anything on entry.
 *             0: the route may also take forms whose order of additions is
 *             not fixed (atomic accumulation) or that keep arrival tickets
 *             in the workspace's prepared part; dw is then reproducible only
 *             within its error budget.  dx is the same in both modes.
 */
int rmsnorm_bwd(const void* dy, const void* x, const float* rstd, const void* w, int w_dtype,
                const void* residual, void* dx, float* dw,
                void* workspace, size_t workspace_bytes,
                int64_t T, int64_t heads, int64_t H, int64_t stride_t, int64_t stride_h,
                int deterministic, void* stream);

/*
 * SiLU-gated forward and backward.  The pages name a SiLU-gated training
 * RMSNorm beside this one, in deterministic and non-deterministic forms
 * (p1 #8208 PR description), without its formula.  Reading taken: the gate
 * scales the normalised, weighted row and does not enter the norm,
 *   y = bf16(u * rstd * w * silu(g)),  silu(g) = g / (1 + exp(-g)),
 * with the gradients of L = sum dy * y:
 *   dg = bf16(dy * (xhat * w) * silu'(g)),
 *   dx, dw = the plain backward's at the gated gradient e = dy * silu(g).
 * No residual.  g and dg are [T,heads,H] BF16 with the activations' strides;
 * dg may be g and dx may be dy.  silu is evaluated in FP32 (sigmoid within
 * ~4 units in the last place while it is a normal number, and rounded once
 * to the subnormal grid below that, down to g ~ -103; g = -inf gives
 * silu = NaN, the formula's IEEE value), so dx, dg and dw carry its error
 * besides their own rounding; all other arithmetic is as in the plain
 * calls.  The workspace is the plain backward's
 * (rmsnorm_bwd_workspace_size with residual NULL) and the same rules apply.
 */
int rmsnorm_gated_fwd(const void* x, const void* gate, const void* w, int w_dtype, void* y, float* rstd,
                      int64_t T, int64_t heads, int64_t H, int64_t stride_t, int64_t stride_h,
                      double eps, int deterministic, void* stream);

int rmsnorm_gated_bwd(const void* dy, const void* x, const void* gate, const float* rstd, const void* w,
                      int w_dtype, void* dx, void* dgate, float* dw, void* workspace, size_t workspace_bytes,
                      int64_t T, int64_t heads, int64_t H, int64_t stride_t, int64_t stride_h,
                      int deterministic, void* stream);

/*
 * Route inspection and override, for the route-table measurement and for
 * tests that cover both sides of a route edge (p3 #8293 commit message: its
 * pairs test exercises each edge from both sides; p1 #8577 "Column-task
 * launch": row-chunk and column-task workgroups in one launch).  A route
 * names how the backward reduces dw over rows:
 *   form   RMSN_FORM_PAIR: each of `chunks` workgroups writes an FP64 column
 *          partial to the workspace and a second kernel sums them in a fixed
 *          order (deterministic; with chunks = 1 the one workgroup writes dw
 *          itself and there is no second kernel).
 *          RMSN_FORM_ATOMIC: the workgroups add their partials to an FP64
 *          accumulator atomically and the last one to finish writes dw (one
 *          launch; order of additions not fixed; non-deterministic only).
 *          RMSN_FORM_COLS: one launch of `chunks` row tasks, which form dx,
 *          beside column tasks, which form dw for slices of 8 * col_vecs
 *          columns straight from x, dy and rstd, each over all rows of its
 *          slice (col_chunks = 1: dw written directly, no workspace beyond
 *          the prepared part) or over one of col_chunks row blocks, whose
 *          FP64 partials a second kernel sums in a fixed order.
 *          Deterministic.
 *          RMSN_FORM_COLS_TICKET: RMSN_FORM_COLS with col_chunks >= 2, where
 *          the column task that finishes a slice last (a per-slice arrival
 *          ticket in the prepared part) sums that slice's partials in the
 *          fixed order: one launch; non-deterministic mode only (it needs
 *          the prepared workspace).
 *   chunks number of row-kernel workgroups (pair, atomic) or row tasks
 *          (column forms), 1 .. 65536; workgroup c takes the row groups c,
 *          c + chunks, c + 2*chunks, ...
 *   col_chunks, col_vecs  column forms only (0 for the others): row blocks
 *          per column slice, 1 .. 4096; 16-byte vectors per slice: 1, 2, 4
 *          or 8.
 *   prefetch  pair and atomic forms: 1 makes each row-kernel workgroup load
 *          its next rows while it reduces the current ones (a second
 *          register tile; pays where a compute unit holds few workgroups);
 *          0 or 1, and 0 for the column forms.  A scheduling choice only: it
 *          changes no bit of dx or dw.  It has no effect with chunks = 1,
 *          on rows wider than 8192 (no registers for a second tile) or on
 *          the gated backward, whose rows up to H 8192 always load ahead.
 * The per-row work, and so dx, does not depend on the route.
 */
enum rmsn_form { RMSN_FORM_PAIR = 0, RMSN_FORM_ATOMIC = 1, RMSN_FORM_COLS = 2, RMSN_FORM_COLS_TICKET = 3 };

typedef struct rmsn_route {
    int32_t form;
    int32_t chunks;
    int32_t col_chunks;
    int32_t col_vecs;
    int32_t prefetch;
} rmsn_route;

/* The route rmsnorm_bwd takes for these arguments.  Returns a status. */
int rmsnorm_bwd_route(int64_t T, int64_t heads, int64_t H, int w_dtype, int has_residual,
                      int deterministic, rmsn_route* out);

/* The route rmsnorm_gated_bwd takes: the plain backward's forms, with the
 * pair's chunk counts measured for the gated rows (which take the next-row
 * tile by width, not by route: prefetch is always 0 here).  Returns a
 * status. */
int rmsnorm_gated_bwd_route(int64_t T, int64_t heads, int64_t H, int w_dtype, int deterministic,
                            rmsn_route* out);

/* Workspace bytes for an explicit route (0 when invalid). */
size_t rmsnorm_bwd_workspace_size_for_route(int64_t T, int64_t heads, int64_t H, rmsn_route route);

/* rmsnorm_bwd with an explicit route.  deterministic = 1 requires the pair
 * or the column form (RMSN_ERR_INVALID_ARG otherwise, and for any
 * malformed route). */
int rmsnorm_bwd_routed(const void* dy, const void* x, const float* rstd, const void* w, int w_dtype,
                       const void* residual, void* dx, float* dw,
                       void* workspace, size_t workspace_bytes,
                       int64_t T, int64_t heads, int64_t H, int64_t stride_t, int64_t stride_h,
                       int deterministic, rmsn_route route, void* stream);

/*
 * rmsnorm_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Arguments and results are those of rmsnorm_bwd,
 * bit for bit (the same route and kernels).  The workspace is the library's
 * own device scratch of RMSN_NOALLOC_SCRATCH_BYTES per GPU, set up on the
 * first call on a device (a symbol lookup, and a clear of its prepared part
 * enqueued on `stream`) and held until the process ends.  Allocates nothing,
 * ever.  Returns RMSN_ERR_WORKSPACE when the workspace of the route it
 * takes (rmsnorm_bwd_workspace_size_for_route of rmsnorm_bwd_route) exceeds
 * the scratch -- every width up to 8192 at every row count fits -- and
 * RMSN_ERR_HIP when the scratch cannot
 * be set up.  Every call on one GPU shares that GPU's scratch: calls that
 * may overlap in time on one GPU (different streams, host threads) race and
 * must be serialised by the caller.
 */
#define RMSN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int rmsnorm_bwd_noalloc(const void* dy, const void* x, const float* rstd, const void* w, int w_dtype,
                        const void* residual, void* dx, float* dw,
                        int64_t T, int64_t heads, int64_t H, int64_t stride_t, int64_t stride_h,
                        int deterministic, void* stream);

/* Human-readable name of a status code (static storage). */
const char* rmsnorm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* RMSNORM_MI355X_H */
