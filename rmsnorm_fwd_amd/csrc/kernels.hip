// kernels.hip -- gfx950 (CDNA4) kernels of the training RMSNorm.
//
// The operation (FlashInfer training-RMSNorm pages, p1 #8577 opening
// paragraph and "Key"; p2 description):
//   forward   rstd = 1/sqrt(mean(u^2) + eps), y = bf16(u * rstd * w),
//             u = x or the stored BF16 h = bf16(x + r)
//   backward  dx = bf16(rstd * (w*dy - xhat * mean(xhat*w*dy)) [+ dres]),
//             dw = sum over rows of dy * xhat, xhat = u * rstd
//
// Every kernel here streams rows from HBM once; there is no matrix product,
// so the design goal is bytes in flight, not matrix-core throughput:
//   * 16-byte loads and stores, consecutive lanes on consecutive vectors;
//   * one wavefront (or a few, through LDS) per row, reduced with DPP row
//     operations and ds_swizzle, never with a workgroup-wide tree;
//   * exact products in FP32 (BF16*BF16 has 16 significant bits) widened to
//     FP64 for every sum: the row's sum of squares, the row dot
//     S = sum(x*w*dy) and the dw column sums.  FP64 runs at the FP32 rate on
//     this chip, and it makes y, dx and dw rounding-exact up to the final
//     BF16/FP32 rounding (dx is formed in FP64 and rounded once to FP32,
//     then to BF16);
//   * dw: each chunk of rows keeps FP64 column partials in registers; a
//     workgroup with several row groups combines them in LDS in slot order;
//     the chunk partial then goes either to a workspace row (pair form, summed
//     by dw_reduce_kernel in a fixed order: deterministic) or into an FP64
//     accumulator by atomic add, with the last-arriving workgroup writing dw
//     and clearing the accumulator (atomic form: one launch).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "layouts.h"

namespace rmsn {

#define RMSN_CHECK_LAYOUT(id, mh, l, vv, uu) static_assert((mh) == (l) * (vv) * 8, "layout width");
RMSN_FWD_LAYOUTS(RMSN_CHECK_LAYOUT)
RMSN_BWD_LAYOUTS(RMSN_CHECK_LAYOUT)
#undef RMSN_CHECK_LAYOUT

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- BF16 ----

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two floats -> two BF16 (round to nearest even; v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ void unpack8(const uint4& v, float f[8])
{
    f[0] = bf_lo(v.x); f[1] = bf_hi(v.x);
    f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
    f[4] = bf_lo(v.z); f[5] = bf_hi(v.z);
    f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
}

__device__ __forceinline__ uint4 pack8(const float f[8])
{
    uint4 v;
    v.x = pack_bf16x2(f[0], f[1]);
    v.y = pack_bf16x2(f[2], f[3]);
    v.z = pack_bf16x2(f[4], f[5]);
    v.w = pack_bf16x2(f[6], f[7]);
    return v;
}

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(uint16_t* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// ------------------------------------------------- cross-lane FP64 sums ----

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}

// Lane i <-> lane i ^ 16 inside each 32-lane half (ds_swizzle bit mode:
// and_mask 0x1F, or_mask 0, xor_mask 0x10).
__device__ __forceinline__ double swizzle_xor16_f64(double v)
{
    const int lo = __builtin_amdgcn_ds_swizzle(__double2loint(v), 0x401F);
    const int hi = __builtin_amdgcn_ds_swizzle(__double2hiint(v), 0x401F);
    return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double readlane_f64(double v, int lane)
{
    const int lo = __builtin_amdgcn_readlane(__double2loint(v), lane);
    const int hi = __builtin_amdgcn_readlane(__double2hiint(v), lane);
    return __hiloint2double(hi, lo);
}

// Sum over aligned groups of L lanes (L = 8, 16, 32 or 64).  Each step adds
// the value of a partner lane chosen symmetrically (xor 1, xor 2, mirror in
// 8, mirror in 16, xor 16, halves), so every lane of a group ends with the
// bitwise same result, and the order depends only on L.
template <int L>
__device__ __forceinline__ double group_sum_f64(double v)
{
    static_assert(L == 8 || L == 16 || L == 32 || L == 64, "group size");
    v += dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f64<0x141>(v);  // row_half_mirror
    if (L >= 16) v += dpp_f64<0x140>(v);  // row_mirror
    if (L >= 32) v += swizzle_xor16_f64(v);
    if (L >= 64) v = readlane_f64(v, 0) + readlane_f64(v, 32);
    return v;
}

__device__ __forceinline__ int64_t row_offset(int row, int heads, int64_t st, int64_t sh)
{
    if (heads == 1) return (int64_t)row * st;
    const int t = row / heads;
    const int hd = row - t * heads;
    return (int64_t)t * st + (int64_t)hd * sh;
}

// 1/sqrt(m) in FP64: hardware estimate refined by two Newton steps, then
// rounded to FP32 (the error before the final rounding is far below 2^-40).
__device__ __forceinline__ float rstd_from_ms(double m)
{
    double y = __builtin_amdgcn_rsq(m);
    if (__builtin_isinf(y)) return (float)y;  // m == 0 (eps == 0 and a zero row)
    const double hm = 0.5 * m;
    y = y * (1.5 - hm * y * y);
    y = y * (1.5 - hm * y * y);
    return (float)y;
}

// Reduce U per-row values across the LPR lanes of each row group.  For
// LPR > 64 the wavefronts of a row meet in LDS (double-buffered by iteration
// parity, one barrier per iteration); the sum over wavefronts runs in
// wavefront order.
template <int LPR, int U, int RPI>
__device__ __forceinline__ void row_group_sum(double (&s)[U], double (*red)[RPI][LPR > 64 ? LPR / 64 : 1],
                                              int it, int slot, int g)
{
    constexpr int W = LPR > 64 ? LPR / 64 : 1;
    constexpr int SLOTS = RPI / U;
#pragma unroll
    for (int u = 0; u < U; ++u) s[u] = group_sum_f64<(LPR < 64 ? LPR : 64)>(s[u]);
    if constexpr (W > 1) {
        const int wave = g >> 6;
        if ((g & 63) == 0) {
#pragma unroll
            for (int u = 0; u < U; ++u) red[it & 1][u * SLOTS + slot][wave] = s[u];
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            double t = red[it & 1][u * SLOTS + slot][0];
#pragma unroll
            for (int k = 1; k < W; ++k) t += red[it & 1][u * SLOTS + slot][k];
            s[u] = t;
        }
    }
}

template <int V, bool WF32>
__device__ __forceinline__ void load_weights(const void* w, int g, int lpr, int nv, float (&wf)[V][8])
{
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int k = g + lpr * v;
        if (k < nv) {
            if constexpr (WF32) {
                const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(w) + 8 * k);
                const float4 a = p[0], b = p[1];
                wf[v][0] = a.x; wf[v][1] = a.y; wf[v][2] = a.z; wf[v][3] = a.w;
                wf[v][4] = b.x; wf[v][5] = b.y; wf[v][6] = b.z; wf[v][7] = b.w;
            } else {
                unpack8(ld16(static_cast<const uint16_t*>(w) + 8 * k), wf[v]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) wf[v][e] = 0.f;
        }
    }
}

// ============================================================ forward ====

template <int LPR, int V, int U, bool WF32>
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
    const int nv = p.H >> 3;

    float wf[V][8];
    load_weights<V, WF32>(p.w, g, LPR, nv, wf);

    int it = 0;
    for (int base = blockIdx.x * RPI; base < p.R; base += gridDim.x * RPI, ++it) {
        int row[U];
        int64_t off[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            row[u] = base + u * SLOTS + slot;
            ok[u] = row[u] < p.R;
            off[u] = ok[u] ? row_offset(row[u], p.heads, p.stride_t, p.stride_h) : 0;
        }
        uint4 xv[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int k = g + LPR * v;
                xv[u][v] = (ok[u] && k < nv) ? ld16(p.x + off[u] + 8 * k) : make_uint4(0, 0, 0, 0);
            }
        if (p.r) {
            // h = bf16(x + r): the FP32 sum of two BF16 values, rounded once
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    const int k = g + LPR * v;
                    if (ok[u] && k < nv) {
                        const uint4 rv = ld16(p.r + off[u] + 8 * k);
                        float a[8], b[8];
                        unpack8(xv[u][v], a);
                        unpack8(rv, b);
#pragma unroll
                        for (int e = 0; e < 8; ++e) a[e] += b[e];
                        xv[u][v] = pack8(a);
                        st16(p.h + off[u] + 8 * k, xv[u][v]);
                    }
                }
        }
        // sum of squares: the 8 squares of a vector are exact in FP32 and
        // summed as a fixed tree; vector sums are accumulated in FP64.
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
                ss[u] += (double)((s01 + s23) + (s45 + s67));
            }
        }
        row_group_sum<LPR, U, RPI>(ss, red, it, slot, g);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float rs = rstd_from_ms(ss[u] * p.inv_h + p.eps);
            if (g == 0 && ok[u]) p.rstd[row[u]] = rs;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int k = g + LPR * v;
                if (ok[u] && k < nv) {
                    float f[8];
                    unpack8(xv[u][v], f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) f[e] = (f[e] * rs) * wf[v][e];
                    st16(p.y + off[u] + 8 * k, pack8(f));
                }
            }
        }
    }
}

// =========================================================== backward ====

template <int LPR, int V, int U, bool WF32>
__global__ void __launch_bounds__(block_of(LPR)) bwd_kernel(BwdParams p)
{
    constexpr int BLOCK = block_of(LPR);
    constexpr int SLOTS = BLOCK / LPR;
    constexpr int W = LPR > 64 ? LPR / 64 : 1;
    constexpr int RPI = SLOTS * U;
    __shared__ double red[2][RPI][W];
    __shared__ int last_block;
    extern __shared__ double slot_part[];  // [SLOTS][H] when SLOTS > 1

    const int tid = threadIdx.x;
    const int g = tid % LPR;
    const int slot = tid / LPR;
    const int H = p.H;
    const int nv = H >> 3;
    const int chunk = blockIdx.x;
    const int row0 = chunk * p.rows_per_chunk;
    const int row1 = min(row0 + p.rows_per_chunk, p.R);

    float wf[V][8];
    load_weights<V, WF32>(p.w, g, LPR, nv, wf);

    double acc[V][8];
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[v][e] = 0.0;

    int it = 0;
    for (int base = row0; base < row1; base += RPI, ++it) {
        int row[U];
        int64_t off[U];
        bool ok[U];
        double rho[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            row[u] = base + u * SLOTS + slot;
            ok[u] = row[u] < row1;
            off[u] = ok[u] ? row_offset(row[u], p.heads, p.stride_t, p.stride_h) : 0;
            rho[u] = ok[u] ? (double)p.rstd[row[u]] : 0.0;
        }
        uint4 xv[U][V], dv[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int k = g + LPR * v;
                const bool in = ok[u] && k < nv;
                xv[u][v] = in ? ld16(p.x + off[u] + 8 * k) : make_uint4(0, 0, 0, 0);
                dv[u][v] = in ? ld16(p.dy + off[u] + 8 * k) : make_uint4(0, 0, 0, 0);
            }
        // Row dot S = sum x*w*dy and the dw column sums, both from the exact
        // FP32 product x*dy (16 significant bits) widened to FP64; its
        // products with w (<= 24 bits) and with rstd (24 bits) are exact in
        // FP64, so only the additions round.
        double S[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            S[u] = 0.0;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                float xf[8], df[8];
                unpack8(xv[u][v], xf);
                unpack8(dv[u][v], df);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const double pd = (double)(xf[e] * df[e]);
                    S[u] = __builtin_fma(pd, (double)wf[v][e], S[u]);
                    acc[v][e] = __builtin_fma(pd, rho[u], acc[v][e]);
                }
            }
        }
        row_group_sum<LPR, U, RPI>(S, red, it, slot, g);
        // dx = rstd*(w*dy) - x*(rstd^3 * S / H), in FP64, rounded once to
        // FP32 and then to BF16.
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const double Lr = rho[u] * rho[u] * rho[u] * S[u] * p.inv_h;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int k = g + LPR * v;
                if (ok[u] && k < nv) {
                    float xf[8], df[8], out[8], rf[8];
                    unpack8(xv[u][v], xf);
                    unpack8(dv[u][v], df);
                    if (p.dres) unpack8(ld16(p.dres + off[u] + 8 * k), rf);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        double gw;
                        if constexpr (WF32) gw = (double)wf[v][e] * (double)df[e];
                        else gw = (double)(wf[v][e] * df[e]);  // exact: 8 x 8 bits
                        double d = __builtin_fma(gw, rho[u], -((double)xf[e] * Lr));
                        if (p.dres) d += (double)rf[e];
                        out[e] = (float)d;
                    }
                    st16(p.dx + off[u] + 8 * k, pack8(out));
                }
            }
        }
    }

    // ---- chunk partial of dw ------------------------------------------
    if constexpr (SLOTS > 1) {
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int k = g + LPR * v;
            if (k < nv) {
#pragma unroll
                for (int e = 0; e < 8; ++e) slot_part[slot * H + 8 * k + e] = acc[v][e];
            }
        }
        __syncthreads();
        for (int col = tid; col < H; col += BLOCK) {
            double s = slot_part[col];
#pragma unroll
            for (int sl = 1; sl < SLOTS; ++sl) s += slot_part[sl * H + col];
            if (p.atomic_form) unsafeAtomicAdd(p.acc + col, s);
            else p.part[(int64_t)chunk * H + col] = s;
        }
    } else {
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int k = g + LPR * v;
            if (k < nv) {
                if (p.atomic_form) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) unsafeAtomicAdd(p.acc + 8 * k + e, acc[v][e]);
                } else {
                    double2* dst = reinterpret_cast<double2*>(p.part + (int64_t)chunk * H + 8 * k);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[e] = make_double2(acc[v][2 * e], acc[v][2 * e + 1]);
                }
            }
        }
    }

    if (p.atomic_form) {
        // Last-arriver: every workgroup publishes its atomics (agent-scope
        // fence) before taking a ticket; the one that draws the last ticket
        // reads and clears the accumulator and writes dw.  No workgroup ever
        // waits for another.
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const unsigned t = __hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            last_block = (t == (unsigned)(gridDim.x - 1));
        }
        __syncthreads();
        if (last_block) {
            __threadfence();
            for (int col = tid; col < H; col += BLOCK) {
                unsigned long long* a = reinterpret_cast<unsigned long long*>(p.acc + col);
                const unsigned long long bits =
                    __hip_atomic_exchange(a, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                p.dw[col] = (float)__longlong_as_double((long long)bits);
            }
            if (tid == 0) __hip_atomic_store(p.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ------------------------------------------------ fixed-order dw reduce ----
// dw[col] = sum over chunks of part[chunk][col].  A workgroup takes 16
// columns; its 16 lane groups q sum chunks q, q+16, q+32, ... in order and
// the 16 group sums are added in q order.  The order depends only on the
// chunk count.
constexpr int kReduceCols = 16;
constexpr int kReduceGroups = 16;

__global__ void __launch_bounds__(kReduceCols * kReduceGroups)
dw_reduce_kernel(const double* __restrict__ part, int chunks, int H, float* __restrict__ dw)
{
    constexpr int DEPTH = 16;  // loads in flight per lane
    __shared__ double sums[kReduceGroups][kReduceCols];
    const int c = threadIdx.x % kReduceCols;
    const int q = threadIdx.x / kReduceCols;
    const int col = blockIdx.x * kReduceCols + c;
    double s = 0.0;
    if (col < H) {
        for (int k = q; k < chunks; k += DEPTH * kReduceGroups) {
            double a[DEPTH];
#pragma unroll
            for (int i = 0; i < DEPTH; ++i) {
                const int kk = k + i * kReduceGroups;
                a[i] = kk < chunks ? part[(int64_t)kk * H + col] : 0.0;
            }
#pragma unroll
            for (int i = 0; i < DEPTH; ++i) s += a[i];
        }
    }
    sums[q][c] = s;
    __syncthreads();
    if (q == 0 && col < H) {
        double t = sums[0][c];
#pragma unroll
        for (int j = 1; j < kReduceGroups; ++j) t += sums[j][c];
        dw[col] = (float)t;
    }
}

__global__ void fill_zero_kernel(uint32_t* p, int64_t words)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// ----------------------------------------------------------- launchers ----

template <int LPR, int V, int U, bool WF32>
static hipError_t fwd_t(const FwdParams& p, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((fwd_kernel<LPR, V, U, WF32>), dim3(grid), dim3(block_of(LPR)), 0, s, p);
    return hipGetLastError();
}

template <int LPR, int V, int U, bool WF32>
static hipError_t bwd_t(const BwdParams& p, hipStream_t s)
{
    constexpr int SLOTS = slots_of(LPR);
    const size_t lds = SLOTS > 1 ? (size_t)SLOTS * p.H * sizeof(double) : 0;
    hipLaunchKernelGGL((bwd_kernel<LPR, V, U, WF32>), dim3(p.chunks), dim3(block_of(LPR)), lds, s, p);
    return hipGetLastError();
}

hipError_t launch_fwd(int layout, bool w_f32, const FwdParams& p, int grid, hipStream_t s)
{
    switch (layout) {
#define RMSN_FWD_CASE(id, mh, l, vv, uu) \
    case id: return w_f32 ? fwd_t<l, vv, uu, true>(p, grid, s) : fwd_t<l, vv, uu, false>(p, grid, s);
        RMSN_FWD_LAYOUTS(RMSN_FWD_CASE)
#undef RMSN_FWD_CASE
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bwd(int layout, bool w_f32, const BwdParams& p, hipStream_t s)
{
    switch (layout) {
#define RMSN_BWD_CASE(id, mh, l, vv, uu) \
    case id: return w_f32 ? bwd_t<l, vv, uu, true>(p, s) : bwd_t<l, vv, uu, false>(p, s);
        RMSN_BWD_LAYOUTS(RMSN_BWD_CASE)
#undef RMSN_BWD_CASE
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dw_reduce(const double* part, int chunks, int H, float* dw, hipStream_t s)
{
    const int grid = (H + kReduceCols - 1) / kReduceCols;
    hipLaunchKernelGGL(dw_reduce_kernel, dim3(grid), dim3(kReduceCols * kReduceGroups), 0, s, part, chunks, H, dw);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void* ptr, int64_t bytes, hipStream_t s)
{
    const int64_t words = bytes / 4;
    if (words <= 0) return hipSuccess;
    int64_t blocks = (words + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((int)blocks), dim3(256), 0, s, static_cast<uint32_t*>(ptr), words);
    return hipGetLastError();
}

}  // namespace rmsn
