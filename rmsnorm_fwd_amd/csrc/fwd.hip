// fwd.hip -- forward kernel of the training RMSNorm on gfx950.
//
//   rstd = 1/sqrt(mean(u^2) + eps),  y = bf16(u * rstd * w),
//   u = x, or the stored BF16 h = bf16(x + r) with the fused residual add
// (FlashInfer training-RMSNorm pages: p1 #8577 opening paragraph and "Key").
//
// A row group of LPR lanes owns one row; each lane holds V 16-byte vectors of
// it in registers, so x (and r) are read from HBM once and y (and h) written
// once.  The sum of squares: the 8 squares of a vector are exact in FP32 and
// added as a fixed tree, vector sums are added in FP64 and reduced across the
// row group with DPP / ds_swizzle (plus LDS when a row spans several
// wavefronts).  Relative error of the sum stays below 3 * 2^-24, so rstd is
// within 2e-7 of the FP64 value before its final FP32 rounding.  The
// workgroup count is capped and rows are taken grid-stride; results do not
// depend on the grid.  With a SiLU gate (GATE) y is further multiplied by
// silu(g) in FP32.
#include "device_common.h"
#include "kernels.h"

namespace rmsn {

// One iteration's rows of a row group: validity, addresses, x (and r, or
// the gate g) vectors.  RES and GATE never meet.
template <int U, int V, bool RES, bool GATE>
struct FwdTile {
    int row[U];
    bool ok[U];
    int64_t off[U];
    uint4 xv[U][V];
    uint4 rv[(RES || GATE) ? U : 1][(RES || GATE) ? V : 1];
};

template <int U, int V, int SLOTS, bool RES, bool GATE>
__device__ __forceinline__ void fwd_load(FwdTile<U, V, RES, GATE>& t, const FwdParams& p,
                                         const LaneVectors<V>& lv, int base, int slot)
{
#pragma unroll
    for (int u = 0; u < U; ++u) {
        t.row[u] = base + u * SLOTS + slot;
        t.ok[u] = t.row[u] < p.R;
        t.off[u] = row_offset(t.ok[u] ? t.row[u] : p.R - 1, p.rows);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int v = 0; v < V; ++v) {
            t.xv[u][v] = ld16_stream(p.x + t.off[u] + lv.col[v]);
            if constexpr (RES) t.rv[u][v] = ld16_stream(p.r + t.off[u] + lv.col[v]);
            if constexpr (GATE) t.rv[u][v] = ld16_stream(p.g + t.off[u] + lv.col[v]);
        }
}

template <int LPR, int V, int U, bool WF32, bool RES, bool GATE>
__global__ void __launch_bounds__(block_of(LPR)) fwd_kernel(FwdParams p)
{
    constexpr int BLOCK = block_of(LPR);
    constexpr int SLOTS = BLOCK / LPR;
    constexpr int W = LPR > 64 ? LPR / 64 : 1;
    constexpr int RPI = SLOTS * U;
    __shared__ double red[2][RPI][W];

    const int tid = threadIdx.x;
    const int g = tid % LPR;
    const int slot = tid / LPR;
    const LaneVectors<V> lv(g, LPR, p.H >> 3);

    // weights: FP32 in registers, or BF16 kept packed (unpacked per use)
    float wf[WF32 ? V : 1][8];
    uint4 wb[WF32 ? 1 : V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        if constexpr (WF32) {
            const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p.w) + lv.col[v]);
            const float4 a = q[0], b = q[1];
            wf[v][0] = a.x; wf[v][1] = a.y; wf[v][2] = a.z; wf[v][3] = a.w;
            wf[v][4] = b.x; wf[v][5] = b.y; wf[v][6] = b.z; wf[v][7] = b.w;
        } else {
            wb[v] = ld16(static_cast<const uint16_t*>(p.w) + lv.col[v]);
        }
    }

    const int stride = gridDim.x * RPI;
    FwdTile<U, V, RES, GATE> cur;
    int it = 0;
    for (int base = blockIdx.x * RPI; base < p.R; base += stride, ++it) {
        fwd_load<U, V, SLOTS, RES, GATE>(cur, p, lv, base, slot);
        const int* row = cur.row;
        const bool* ok = cur.ok;
        const int64_t* off = cur.off;
        uint4 (&xv)[U][V] = cur.xv;
        if constexpr (RES) {
            // h = bf16(x + r): the FP32 sum of two BF16 values, rounded once
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    float a[8], b[8];
                    unpack8(xv[u][v], a);
                    unpack8(cur.rv[u][v], b);
#pragma unroll
                    for (int e = 0; e < 8; ++e) a[e] += b[e];
                    xv[u][v] = pack8(a);
                    if (ok[u] && lv.ok[v]) st16_stream(p.h + off[u] + lv.col[v], xv[u][v]);
                }
        }
        double ss[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            ss[u] = 0.0;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                float f[8];
                unpack8(xv[u][v], f);
                const float s01 = f[0] * f[0] + f[1] * f[1];
                const float s23 = f[2] * f[2] + f[3] * f[3];
                const float s45 = f[4] * f[4] + f[5] * f[5];
                const float s67 = f[6] * f[6] + f[7] * f[7];
                const float s = (s01 + s23) + (s45 + s67);
                ss[u] += (double)(lv.ok[v] ? s : 0.f);
            }
        }
        // gated rows read one row's wavefront partials at a time (fewer registers;
        // the gated table's row layouts were measured with it)
        row_group_sum<LPR, U, RPI, GATE>(ss, red, it, slot, g);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float rs = rstd_from_ms(ss[u] * p.inv_h + p.eps);
            if (g == 0 && ok[u]) p.rstd[row[u]] = rs;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                float f[8], wv[8];
                unpack8(xv[u][v], f);
                if constexpr (WF32) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) wv[e] = wf[v][e];
                } else {
                    unpack8(wb[v], wv);
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = (f[e] * rs) * wv[e];
                if constexpr (GATE) {
                    // y = (u * rstd * w) * silu(g), all in FP32; sigmoid8
                    // gives sigmoid_f32's bits with fewer instructions
                    float gf[8], sgv[8];
                    unpack8(cur.rv[u][v], gf);
                    sigmoid8(gf, sgv);
#pragma unroll
                    for (int e = 0; e < 8; ++e) f[e] *= gf[e] * sgv[e];
                }
                if (ok[u] && lv.ok[v]) st16_stream(p.y + off[u] + lv.col[v], pack8(f));
            }
        }
    }
}

template <int LPR, int V, int U, bool WF32, bool RES, bool GATE>
static hipError_t fwd_t(const FwdParams& p, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((fwd_kernel<LPR, V, U, WF32, RES, GATE>), dim3(grid), dim3(block_of(LPR)), 0, s, p);
    return hipGetLastError();
}

template <int LPR, int V, int U, bool RES, bool GATE>
static hipError_t fwd_w(bool w_f32, const FwdParams& p, int grid, hipStream_t s)
{
    return w_f32 ? fwd_t<LPR, V, U, true, RES, GATE>(p, grid, s) : fwd_t<LPR, V, U, false, RES, GATE>(p, grid, s);
}

template <int LPR, int V, int U>
static hipError_t fwd_dispatch(bool w_f32, const FwdParams& p, int grid, hipStream_t s)
{
    if (p.r) return fwd_w<LPR, V, U, true, false>(w_f32, p, grid, s);
    return fwd_w<LPR, V, U, false, false>(w_f32, p, grid, s);
}

hipError_t launch_fwd(int table, int layout, bool w_f32, const FwdParams& p, int grid, hipStream_t s)
{
    if ((table == FWD_LONG && (p.r || p.g)) || (table == FWD_RES_LONG && !p.r) || ((table == FWD_GATED) != (p.g != nullptr)))
        return hipErrorInvalidValue;
    if (table == FWD_GATED) {
        switch (layout) {
#define RMSN_FWD_GATED_CASE(id, mh, l, vv, uu, kk) \
    case id: return fwd_w<l, vv, uu, false, true>(w_f32, p, grid, s);
            RMSN_FWD_GATED_LAYOUTS(RMSN_FWD_GATED_CASE)
#undef RMSN_FWD_GATED_CASE
        default: return hipErrorInvalidValue;
        }
    }
    if (table == FWD_LONG) {
        switch (layout) {
#define RMSN_FWD_LONG_CASE(id, mh, l, vv, uu, kk) \
    case id: return fwd_w<l, vv, uu, false, false>(w_f32, p, grid, s);
            RMSN_FWD_LONG_LAYOUTS(RMSN_FWD_LONG_CASE)
#undef RMSN_FWD_LONG_CASE
        default: return hipErrorInvalidValue;
        }
    }
    if (table == FWD_RES_LONG) {
        switch (layout) {
#define RMSN_FWD_RES_CASE(id, mh, l, vv, uu, kk) \
    case id: return fwd_w<l, vv, uu, true, false>(w_f32, p, grid, s);
            RMSN_FWD_RES_LONG_LAYOUTS(RMSN_FWD_RES_CASE)
#undef RMSN_FWD_RES_CASE
        default: return hipErrorInvalidValue;
        }
    }
    switch (layout) {
#define RMSN_FWD_CASE(id, mh, l, vv, uu, kk) \
    case id: return fwd_dispatch<l, vv, uu>(w_f32, p, grid, s);
        RMSN_FWD_LAYOUTS(RMSN_FWD_CASE)
#undef RMSN_FWD_CASE
    default: return hipErrorInvalidValue;
    }
}

}  // namespace rmsn
