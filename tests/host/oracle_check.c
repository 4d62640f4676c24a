/* Host check of the oracle (oracle/oracle.c) under AddressSanitizer and
 * UBSan: every exported function on small shapes (no rows, one column,
 * ragged widths, both weight dtypes, with and without residual / dres,
 * special values), each buffer allocated to its exact size so that any
 * access past it is caught.  Prints "ok" and exits 0, else exits non-zero.
 * The prototypes repeat those of oracle.c (the oracle has no header: Python
 * loads it through ctypes). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_bf16_to_double(uint16_t b);
uint16_t oracle_bf16_round(double v);
void oracle_bf16_round_array(int64_t n, const double* v, uint16_t* out);
void oracle_fwd_f64(int64_t R, int64_t H, const double* u, const double* w, double eps, double* y, double* rstd);
void oracle_bwd_f64(int64_t R, int64_t H, const double* u, const double* dy, const double* w, const double* rho,
                    const double* dres, double* dx, double* dw);
void oracle_residual_add(int64_t n, const uint16_t* x, const uint16_t* r, uint16_t* h);
int oracle_fwd_bf16(int64_t R, int64_t H, const uint16_t* x, const uint16_t* r, const void* w, int w_is_f32,
                    double eps, uint16_t* y, uint16_t* h_out, double* rstd);
int oracle_bwd_bf16(int64_t R, int64_t H, const uint16_t* u16, const uint16_t* dy16, const void* w, int w_is_f32,
                    const float* rho32, const uint16_t* dres16, uint16_t* dx, double* dx64, double* dw);
void oracle_dw_bf16(int64_t R, int64_t H, const uint16_t* u16, const uint16_t* dy16, const float* rho32, double* dw);
void oracle_gated_fwd_f64(int64_t R, int64_t H, const double* u, const double* g, const double* w, double eps,
                          double* y, double* rstd);
void oracle_gated_bwd_f64(int64_t R, int64_t H, const double* u, const double* g, const double* dy, const double* w,
                          const double* rho, double* dx, double* dg, double* dw);
int oracle_gated_fwd_bf16(int64_t R, int64_t H, const uint16_t* x, const uint16_t* g, const void* w, int w_is_f32,
                          double eps, uint16_t* y, double* rstd);
int oracle_gated_bwd_bf16(int64_t R, int64_t H, const uint16_t* u16, const uint16_t* g16, const uint16_t* dy16,
                          const void* w, int w_is_f32, const float* rho32, uint16_t* dx, uint16_t* dg, double* dx64,
                          double* dg64, double* dw);
int oracle_num_threads(void);

static int fails = 0;
#define CHECK(c, msg)                                                     \
    do {                                                                  \
        if (!(c)) {                                                       \
            printf("%s:%d: %s\n", __FILE__, __LINE__, msg);               \
            ++fails;                                                      \
        }                                                                 \
    } while (0)

/* exact-size allocations (at least one byte, so malloc(0) is never asked) */
static void* xalloc(size_t n) { return malloc(n ? n : 1); }

static uint32_t state = 12345u;
static double rnd(void)
{
    state = state * 1664525u + 1013904223u;
    return ((double)(state >> 8) / 16777216.0) * 4.0 - 2.0;
}

static void check_shape(int64_t R, int64_t H)
{
    const size_t n = (size_t)(R * H);
    uint16_t *x = xalloc(n * 2), *r = xalloc(n * 2), *dy = xalloc(n * 2), *dr = xalloc(n * 2), *g = xalloc(n * 2);
    uint16_t *y = xalloc(n * 2), *h = xalloc(n * 2), *dx = xalloc(n * 2), *dg = xalloc(n * 2);
    uint16_t* wb = xalloc((size_t)H * 2);
    float* wf = xalloc((size_t)H * 4);
    float* rho = xalloc((size_t)R * 4);
    double *rstd = xalloc((size_t)R * 8), *dw = xalloc((size_t)H * 8), *dx64 = xalloc(n * 8), *dg64 = xalloc(n * 8);
    double *u = xalloc(n * 8), *d = xalloc(n * 8), *gd = xalloc(n * 8), *wd = xalloc((size_t)H * 8);
    double *yd = xalloc(n * 8), *dxd = xalloc(n * 8), *dgd = xalloc(n * 8), *rhod = xalloc((size_t)R * 8);
    for (size_t i = 0; i < n; ++i) {
        x[i] = oracle_bf16_round(rnd());
        r[i] = oracle_bf16_round(rnd());
        dy[i] = oracle_bf16_round(rnd());
        dr[i] = oracle_bf16_round(rnd());
        g[i] = oracle_bf16_round(3.0 * rnd());
        u[i] = rnd();
        d[i] = rnd();
        gd[i] = rnd();
    }
    for (int64_t j = 0; j < H; ++j) {
        wf[j] = (float)(1.0 + 0.1 * rnd());
        wb[j] = oracle_bf16_round(wf[j]);
        wd[j] = wf[j];
    }
    for (int w32 = 0; w32 <= 1; ++w32) {
        const void* w = w32 ? (const void*)wf : (const void*)wb;
        CHECK(oracle_fwd_bf16(R, H, x, NULL, w, w32, 1e-6, y, NULL, rstd) == 0, "fwd_bf16");
        CHECK(oracle_fwd_bf16(R, H, x, r, w, w32, 1e-6, y, h, rstd) == 0, "fwd_bf16 residual");
        for (int64_t i = 0; i < R; ++i) rho[i] = (float)rstd[i];
        CHECK(oracle_bwd_bf16(R, H, h, dy, w, w32, rho, NULL, dx, NULL, dw) == 0, "bwd_bf16");
        CHECK(oracle_bwd_bf16(R, H, h, dy, w, w32, rho, dr, dx, dx64, dw) == 0, "bwd_bf16 dres");
        for (int64_t j = 0; j < H; ++j) CHECK(isfinite(dw[j]), "dw finite");
        oracle_dw_bf16(R, H, h, dy, rho, dw);
        CHECK(oracle_gated_fwd_bf16(R, H, x, g, w, w32, 1e-6, y, rstd) == 0, "gated_fwd_bf16");
        for (int64_t i = 0; i < R; ++i) rho[i] = (float)rstd[i];
        CHECK(oracle_gated_bwd_bf16(R, H, x, g, dy, w, w32, rho, dx, dg, NULL, NULL, dw) == 0, "gated_bwd_bf16");
        CHECK(oracle_gated_bwd_bf16(R, H, x, g, dy, w, w32, rho, dx, dg, dx64, dg64, dw) == 0,
              "gated_bwd_bf16 f64 outputs");
    }
    oracle_fwd_f64(R, H, u, wd, 1e-6, yd, rhod);
    oracle_bwd_f64(R, H, u, d, wd, rhod, NULL, dxd, dw);
    oracle_bwd_f64(R, H, u, d, wd, rhod, gd, dxd, dw);
    oracle_gated_fwd_f64(R, H, u, gd, wd, 1e-6, yd, rhod);
    oracle_gated_bwd_f64(R, H, u, gd, d, wd, rhod, dxd, dgd, dw);
    oracle_residual_add((int64_t)n, x, r, h);
    void* bufs[] = {x, r, dy, dr, g, y, h, dx, dg, wb, wf, rho, rstd, dw, dx64, dg64, u, d, gd, wd, yd, dxd, dgd, rhod};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) free(bufs[i]);
}

int main(void)
{
    /* rounding over special values: zeros, subnormals, the largest finite
     * values and their neighbours, infinities, NaN */
    const double specials[] = {0.0, -0.0, 1e-45, -1e-45, 1e-40, 5.877471754111438e-39, 3.3895313892515355e38,
                               3.3961775292304634e38, -3.4e38, INFINITY, -INFINITY, NAN, 1.0, -1.0, 0.1};
    uint16_t out[sizeof specials / sizeof specials[0]];
    oracle_bf16_round_array((int64_t)(sizeof specials / sizeof specials[0]), specials, out);
    for (size_t i = 0; i < sizeof specials / sizeof specials[0]; ++i) (void)oracle_bf16_to_double(out[i]);
    for (uint32_t b = 0; b < 65536; ++b) {
        const double v = oracle_bf16_to_double((uint16_t)b);
        if (!isnan(v)) CHECK(oracle_bf16_round(v) == (uint16_t)b, "BF16 round trip");
    }
    const int64_t shapes[][2] = {{0, 8}, {1, 1}, {1, 8}, {3, 8}, {5, 24}, {7, 1}, {2, 4096}, {33, 520}};
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) check_shape(shapes[i][0], shapes[i][1]);
    CHECK(oracle_fwd_bf16(-1, 8, NULL, NULL, NULL, 0, 1e-6, NULL, NULL, NULL) != 0, "R < 0 refused");
    CHECK(oracle_bwd_bf16(1, 0, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL, NULL) != 0, "H = 0 refused");
    CHECK(oracle_num_threads() >= 1, "threads");
    if (fails) {
        printf("%d failures\n", fails);
        return 1;
    }
    printf("ok\n");
    return 0;
}
