/*
 * oracle.c -- plain FP64 CPU evaluation of training RMSNorm (forward and
 * backward).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this file's library.  It shares no code,
 * header, table or helper with the HIP library and includes nothing from it.
 *
 * What is computed, and where the pages define it
 * -----------------------------------------------
 * Sources: the FlashInfer pull-request pages on the training RMSNorm
 *   p1 = "feat(cake_rmsnorm): opt-in non-deterministic weight gradient for the
 *        autograd RMSNorm - #8208" (with the #8577 commit text on that page),
 *   p2 = PR #8899 (GB300 kb/det windows),
 *   p3 = "fix(cake_rmsnorm_det): tighten two large-row weight-gradient
 *        accuracy edges - #8293".
 *
 *  - Forward returns y (BF16) and rstd (FP32) per row; the backward returns
 *    dx (BF16) and dw (FP32)  [p1 #8577 opening paragraph; p2 description].
 *  - Fused residual: the forward also writes the BF16 sum h = x + r and
 *    normalises it  [p1 #8577 "Key": `res` adds the BF16 output h_new].
 *  - w is BF16 or FP32 ("w32"); eps = 1e-6 in every measurement
 *    [p1 #8577 "Key" and "Baselines and measurement"].
 *  - Per-head views [T,heads,256] share one w[256]; the rows are T*heads and
 *    dw sums over all of them  [p1 #8577 "Key"].
 *  - dw is checked against an FP64 evaluation that uses the kernel's own
 *    FP32 rstd  [p1 #8208 commit message], so the backward takes rstd as an
 *    input.
 *
 * The pages never print the formula.  The plain reading used here (RMS over
 * the H entries, divide by H, eps inside the square root, no bias):
 *    rstd = 1 / sqrt( (1/H) sum_j u_j^2 + eps )
 *    y_j  = u_j * rstd * w_j
 *    with xhat_j = u_j * rho   (rho = the rstd handed to the backward)
 *    c    = (1/H) sum_j xhat_j * w_j * dy_j
 *    dx_j = rho * (w_j * dy_j - xhat_j * c)  [+ dres_j]
 *    dw_j = sum over rows of dy_j * xhat_j
 * These are the derivatives of L = sum_j dy_j * y_j with rstd treated as a
 * function of u; the tests pin them with central finite differences.
 *
 * Everything is evaluated in IEEE double, loops in the plain order.  The only
 * BF16 rounding is a single round-to-nearest-even of the FP64 value
 * (bf16_round below).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------------- */
/* BF16 <-> double                                                          */
/* ---------------------------------------------------------------------- */

/* A BF16 value is the upper 16 bits of an IEEE binary32 value, so the
 * conversion to double is exact. */
double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest BF16 value, ties to even, in one step.
 * BF16 keeps 8 significant bits (1 implicit + 7 stored) and binary32's
 * exponent range.  Normal case: scale |v| into [2^7, 2^8) with frexp/ldexp,
 * round that to an integer with rint (ties-to-even under the default
 * rounding mode), and scale back; the result has at most 8 significant bits
 * and so converts to float exactly.  Below 2^-126 the spacing is fixed at
 * 2^-133 (BF16 subnormals).  Overflow past the largest finite BF16 gives inf. */
uint16_t oracle_bf16_round(double v)
{
    float f;
    uint32_t u;
    if (isnan(v)) return (uint16_t)0x7fc0;
    double a = fabs(v);
    double r;
    if (a == 0.0 || isinf(v)) {
        r = a;
    } else if (a < ldexp(1.0, -126)) {
        r = ldexp(rint(ldexp(a, 133)), -133);
    } else {
        int e;
        double m = frexp(a, &e);          /* a = m * 2^e, m in [0.5, 1)   */
        r = ldexp(rint(ldexp(m, 8)), e - 8);
        /* largest finite BF16 is (2 - 2^-7) * 2^127 */
        if (r > ldexp(2.0 - ldexp(1.0, -7), 127)) r = INFINITY;
    }
    if (signbit(v)) r = -r;
    f = (float)r;                          /* exact: r has <= 8 significant bits */
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

void oracle_bf16_round_array(int64_t n, const double* v, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_round(v[i]);
}

static double weight_at(const void* w, int w_is_f32, int64_t j)
{
    if (w_is_f32) return (double)((const float*)w)[j];
    return oracle_bf16_to_double(((const uint16_t*)w)[j]);
}

/* ---------------------------------------------------------------------- */
/* FP64 core, one row at a time                                            */
/* ---------------------------------------------------------------------- */

/* rstd of one row: 1 / sqrt(mean of squares + eps). */
static double row_rstd(int64_t H, const double* u, double eps)
{
    double ss = 0.0;
    for (int64_t j = 0; j < H; ++j) ss += u[j] * u[j];
    return 1.0 / sqrt(ss / (double)H + eps);
}

/* dx of one row at the given rho (dres may be NULL). */
static void row_dx(int64_t H, const double* u, const double* dy, const double* w,
                   double rho, const double* dres, double* dx)
{
    double c = 0.0;
    for (int64_t j = 0; j < H; ++j) c += (u[j] * rho) * w[j] * dy[j];
    c /= (double)H;
    for (int64_t j = 0; j < H; ++j) {
        double xhat = u[j] * rho;
        dx[j] = rho * (w[j] * dy[j] - xhat * c);
        if (dres) dx[j] += dres[j];
    }
}

/* Forward on FP64 rows: u[R,H] (the normalised input), w[H]. */
void oracle_fwd_f64(int64_t R, int64_t H, const double* u, const double* w,
                    double eps, double* y, double* rstd)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        const double* ur = u + r * H;
        double s = row_rstd(H, ur, eps);
        rstd[r] = s;
        for (int64_t j = 0; j < H; ++j) y[r * H + j] = ur[j] * s * w[j];
    }
}

/* Backward on FP64 rows at the given per-row rho; dres may be NULL.
 * dw[j] = sum over r of dy[r,j] * (u[r,j] * rho[r]), rows summed in order. */
void oracle_bwd_f64(int64_t R, int64_t H, const double* u, const double* dy,
                    const double* w, const double* rho, const double* dres,
                    double* dx, double* dw)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        row_dx(H, u + r * H, dy + r * H, w, rho[r], dres ? dres + r * H : NULL,
               dx + r * H);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < H; ++j) {
        double acc = 0.0;
        for (int64_t r = 0; r < R; ++r) acc += dy[r * H + j] * (u[r * H + j] * rho[r]);
        dw[j] = acc;
    }
}

/* ---------------------------------------------------------------------- */
/* BF16 storage wrappers (rows [R,H] contiguous; views are gathered by the  */
/* caller).  Rows are widened to double one at a time.                    */
/* ---------------------------------------------------------------------- */

/* h = bf16(x + r).  The sum of two BF16 values is exact in double unless
 * their exponents differ by more than 45; then the smaller one is far below
 * half a BF16 unit of the larger and cannot change the rounding. */
void oracle_residual_add(int64_t n, const uint16_t* x, const uint16_t* r, uint16_t* h)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        h[i] = oracle_bf16_round(oracle_bf16_to_double(x[i]) + oracle_bf16_to_double(r[i]));
}

/* Forward from BF16 storage.  With a residual (r != NULL) the stored BF16 sum
 * h is written to h_out and is what gets normalised.  Outputs: y as BF16
 * (one rounding of the FP64 value), rstd in double (the FP64 value). */
int oracle_fwd_bf16(int64_t R, int64_t H, const uint16_t* x, const uint16_t* r,
                    const void* w, int w_is_f32, double eps,
                    uint16_t* y, uint16_t* h_out, double* rstd)
{
    if (R < 0 || H <= 0) return 1;
    if (r && !h_out) return 1;
    double* wd = (double*)malloc((size_t)H * sizeof(double));
    if (!wd) return 2;
    for (int64_t j = 0; j < H; ++j) wd[j] = weight_at(w, w_is_f32, j);
    int failed = 0;
#pragma omp parallel
    {
        double* u = (double*)malloc((size_t)H * sizeof(double));
        if (!u) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t row = 0; row < R; ++row) {
            if (!u) continue;
            const int64_t o = row * H;
            for (int64_t j = 0; j < H; ++j) {
                if (r) {
                    uint16_t hb = oracle_bf16_round(oracle_bf16_to_double(x[o + j]) +
                                                    oracle_bf16_to_double(r[o + j]));
                    h_out[o + j] = hb;
                    u[j] = oracle_bf16_to_double(hb);
                } else {
                    u[j] = oracle_bf16_to_double(x[o + j]);
                }
            }
            double s = row_rstd(H, u, eps);
            rstd[row] = s;
            for (int64_t j = 0; j < H; ++j) y[o + j] = oracle_bf16_round(u[j] * s * wd[j]);
        }
        free(u);
    }
    free(wd);
    return failed ? 2 : 0;
}

/* Backward from BF16 storage at the kernel's FP32 rstd (rho).  u is the
 * normalised input (h when the forward had a residual).  Outputs: dx as BF16
 * (one rounding of the FP64 value; dx64 receives the FP64 value when
 * non-NULL), dw in double.  dres may be NULL. */
int oracle_bwd_bf16(int64_t R, int64_t H, const uint16_t* u16, const uint16_t* dy16,
                    const void* w, int w_is_f32, const float* rho32,
                    const uint16_t* dres16, uint16_t* dx, double* dx64, double* dw)
{
    if (R < 0 || H <= 0) return 1;
    double* wd = (double*)malloc((size_t)H * sizeof(double));
    if (!wd) return 2;
    for (int64_t j = 0; j < H; ++j) wd[j] = weight_at(w, w_is_f32, j);
    int failed = 0;
#pragma omp parallel
    {
        double* buf = (double*)malloc((size_t)H * 4 * sizeof(double));
        if (!buf) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t row = 0; row < R; ++row) {
            if (!buf) continue;
            double *u = buf, *g = buf + H, *dr = buf + 2 * H, *out = buf + 3 * H;
            const int64_t o = row * H;
            for (int64_t j = 0; j < H; ++j) {
                u[j] = oracle_bf16_to_double(u16[o + j]);
                g[j] = oracle_bf16_to_double(dy16[o + j]);
                if (dres16) dr[j] = oracle_bf16_to_double(dres16[o + j]);
            }
            row_dx(H, u, g, wd, (double)rho32[row], dres16 ? dr : NULL, out);
            for (int64_t j = 0; j < H; ++j) {
                dx[o + j] = oracle_bf16_round(out[j]);
                if (dx64) dx64[o + j] = out[j];
            }
        }
        free(buf);
    }
    /* dw: each column summed over the rows in row order. */
#pragma omp parallel for schedule(static)
    for (int64_t j0 = 0; j0 < H; j0 += 64) {
        int64_t j1 = j0 + 64 < H ? j0 + 64 : H;
        double acc[64];
        for (int64_t j = j0; j < j1; ++j) acc[j - j0] = 0.0;
        for (int64_t row = 0; row < R; ++row) {
            const double rho = (double)rho32[row];
            for (int64_t j = j0; j < j1; ++j)
                acc[j - j0] += oracle_bf16_to_double(dy16[row * H + j]) *
                               (oracle_bf16_to_double(u16[row * H + j]) * rho);
        }
        for (int64_t j = j0; j < j1; ++j) dw[j] = acc[j - j0];
    }
    free(wd);
    return failed ? 2 : 0;
}

/* dw alone: dw[j] = sum over rows of dy[r,j] * (u[r,j] * rho[r]), each
 * column summed over the rows in row order -- the same sum as the dw of
 * oracle_bwd_bf16, for full-size checks that do not need dx. */
void oracle_dw_bf16(int64_t R, int64_t H, const uint16_t* u16, const uint16_t* dy16,
                    const float* rho32, double* dw)
{
#pragma omp parallel for schedule(static)
    for (int64_t j0 = 0; j0 < H; j0 += 64) {
        int64_t j1 = j0 + 64 < H ? j0 + 64 : H;
        double acc[64];
        for (int64_t j = j0; j < j1; ++j) acc[j - j0] = 0.0;
        for (int64_t row = 0; row < R; ++row) {
            const double rho = (double)rho32[row];
            for (int64_t j = j0; j < j1; ++j)
                acc[j - j0] += oracle_bf16_to_double(dy16[row * H + j]) *
                               (oracle_bf16_to_double(u16[row * H + j]) * rho);
        }
        for (int64_t j = j0; j < j1; ++j) dw[j] = acc[j - j0];
    }
}

/* ---------------------------------------------------------------------- */
/* SiLU-gated variant                                                      */
/* ---------------------------------------------------------------------- */
/* The pages name a SiLU-gated training RMSNorm next to this one (p1 #8208
 * PR description: the kernel's other variants, deterministic and not) but
 * never state its formula.  Reading taken (the common gated-RMSNorm form,
 * gate applied to the normalised, weighted output; the gate does not enter
 * the norm):
 *    y_j  = u_j * rstd * w_j * silu(g_j),   silu(g) = g * sigmoid(g)
 * and for L = sum_j dy_j * y_j, with a_j = xhat_j * w_j (xhat = u * rho):
 *    dg_j = dy_j * a_j * silu'(g_j),  silu'(g) = s(g) * (1 + g * (1 - s(g))),
 *           s = sigmoid
 *    and dx, dw are the plain backward's at the gated gradient
 *    e_j = dy_j * silu(g_j):
 *    dx_j = rho * (w_j * e_j - xhat_j * c),  c = (1/H) sum_j xhat_j * w_j * e_j
 *    dw_j = sum over rows of e_j * xhat_j
 * The tests pin all three with central finite differences. */

static double sigmoid(double g) { return 1.0 / (1.0 + exp(-g)); }
static double silu(double g) { return g * sigmoid(g); }
static double silu_grad(double g)
{
    const double sg = sigmoid(g);
    return sg * (1.0 + g * (1.0 - sg));
}

/* One row of the gated backward at rho: dx and dg (dw is summed by the
 * callers over rows).  e = dy * silu(g) is the gradient reaching the plain
 * normalised output; e is left in the caller's buffer. */
static void gated_row_bwd(int64_t H, const double* u, const double* g, const double* dy,
                          const double* w, double rho, double* e, double* dx, double* dg)
{
    for (int64_t j = 0; j < H; ++j) {
        e[j] = dy[j] * silu(g[j]);
        dg[j] = dy[j] * ((u[j] * rho) * w[j]) * silu_grad(g[j]);
    }
    row_dx(H, u, e, w, rho, NULL, dx);
}

/* Gated forward on FP64 rows. */
void oracle_gated_fwd_f64(int64_t R, int64_t H, const double* u, const double* g,
                          const double* w, double eps, double* y, double* rstd)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        const double* ur = u + r * H;
        double s = row_rstd(H, ur, eps);
        rstd[r] = s;
        for (int64_t j = 0; j < H; ++j) y[r * H + j] = ur[j] * s * w[j] * silu(g[r * H + j]);
    }
}

/* Gated backward on FP64 rows at the per-row rho. */
void oracle_gated_bwd_f64(int64_t R, int64_t H, const double* u, const double* g,
                          const double* dy, const double* w, const double* rho,
                          double* dx, double* dg, double* dw)
{
    int failed = 0;
#pragma omp parallel
    {
        double* e = (double*)malloc((size_t)H * sizeof(double));
        if (!e) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t r = 0; r < R; ++r) {
            if (!e) continue;
            gated_row_bwd(H, u + r * H, g + r * H, dy + r * H, w, rho[r], e, dx + r * H, dg + r * H);
        }
        free(e);
    }
    (void)failed;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < H; ++j) {
        double acc = 0.0;
        for (int64_t r = 0; r < R; ++r)
            acc += (dy[r * H + j] * silu(g[r * H + j])) * (u[r * H + j] * rho[r]);
        dw[j] = acc;
    }
}

/* Forward from BF16 storage: y (BF16, one rounding) and rstd (FP64). */
int oracle_gated_fwd_bf16(int64_t R, int64_t H, const uint16_t* x, const uint16_t* g,
                          const void* w, int w_is_f32, double eps, uint16_t* y, double* rstd)
{
    if (R < 0 || H <= 0) return 1;
    double* wd = (double*)malloc((size_t)H * sizeof(double));
    if (!wd) return 2;
    for (int64_t j = 0; j < H; ++j) wd[j] = weight_at(w, w_is_f32, j);
    int failed = 0;
#pragma omp parallel
    {
        double* u = (double*)malloc((size_t)H * sizeof(double));
        if (!u) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t row = 0; row < R; ++row) {
            if (!u) continue;
            const int64_t o = row * H;
            for (int64_t j = 0; j < H; ++j) u[j] = oracle_bf16_to_double(x[o + j]);
            double s = row_rstd(H, u, eps);
            rstd[row] = s;
            for (int64_t j = 0; j < H; ++j)
                y[o + j] = oracle_bf16_round(u[j] * s * wd[j] * silu(oracle_bf16_to_double(g[o + j])));
        }
        free(u);
    }
    free(wd);
    return failed ? 2 : 0;
}

/* Backward from BF16 storage at the kernel's FP32 rstd: dx and dg as BF16
 * (one rounding each; the FP64 values go to dx64 / dg64 when non-NULL) and
 * dw in double, each column summed over the rows in row order. */
int oracle_gated_bwd_bf16(int64_t R, int64_t H, const uint16_t* u16, const uint16_t* g16,
                          const uint16_t* dy16, const void* w, int w_is_f32, const float* rho32,
                          uint16_t* dx, uint16_t* dg, double* dx64, double* dg64, double* dw)
{
    if (R < 0 || H <= 0) return 1;
    double* wd = (double*)malloc((size_t)H * sizeof(double));
    if (!wd) return 2;
    for (int64_t j = 0; j < H; ++j) wd[j] = weight_at(w, w_is_f32, j);
    int failed = 0;
#pragma omp parallel
    {
        double* buf = (double*)malloc((size_t)H * 6 * sizeof(double));
        if (!buf) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(static)
        for (int64_t row = 0; row < R; ++row) {
            if (!buf) continue;
            double *u = buf, *gg = buf + H, *d = buf + 2 * H, *e = buf + 3 * H;
            double *ox = buf + 4 * H, *og = buf + 5 * H;
            const int64_t o = row * H;
            for (int64_t j = 0; j < H; ++j) {
                u[j] = oracle_bf16_to_double(u16[o + j]);
                gg[j] = oracle_bf16_to_double(g16[o + j]);
                d[j] = oracle_bf16_to_double(dy16[o + j]);
            }
            gated_row_bwd(H, u, gg, d, wd, (double)rho32[row], e, ox, og);
            for (int64_t j = 0; j < H; ++j) {
                dx[o + j] = oracle_bf16_round(ox[j]);
                dg[o + j] = oracle_bf16_round(og[j]);
                if (dx64) dx64[o + j] = ox[j];
                if (dg64) dg64[o + j] = og[j];
            }
        }
        free(buf);
    }
#pragma omp parallel for schedule(static)
    for (int64_t j0 = 0; j0 < H; j0 += 64) {
        int64_t j1 = j0 + 64 < H ? j0 + 64 : H;
        double acc[64];
        for (int64_t j = j0; j < j1; ++j) acc[j - j0] = 0.0;
        for (int64_t row = 0; row < R; ++row) {
            const double rho = (double)rho32[row];
            for (int64_t j = j0; j < j1; ++j) {
                const double e = oracle_bf16_to_double(dy16[row * H + j]) *
                                 silu(oracle_bf16_to_double(g16[row * H + j]));
                acc[j - j0] += e * (oracle_bf16_to_double(u16[row * H + j]) * rho);
            }
        }
        for (int64_t j = j0; j < j1; ++j) dw[j] = acc[j - j0];
    }
    free(wd);
    return failed ? 2 : 0;
}

int oracle_num_threads(void)
{
    int n = 1;
#ifdef _OPENMP
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
#endif
    return n;
}
