// device_common.h -- device helpers shared by the forward and backward
// kernels: BF16 packing, cross-lane FP64 sums (DPP / ds_swizzle), row
// addressing and the per-row LDS meeting point of multi-wavefront rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "layouts.h"

namespace rmsn {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two floats -> two BF16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Same, for values just rounded from FP64.  The empty asm keeps the compiler
// from fusing the FP64->FP32->BF16 pair into one correctly rounded FP64->BF16
// conversion, which it emulates with eight extra instructions per value; the
// two-step rounding is within one BF16 unit of the exact result, which is
// the accuracy the backward guarantees.
__device__ __forceinline__ uint32_t pack_bf16x2_from_f64(double lo, double hi)
{
    float a = (float)lo, b = (float)hi;
    __asm__("" : "+v"(a), "+v"(b));
    return pack_bf16x2(a, b);
}

// SiLU gate in FP32: sigmoid(g) = 1 / (1 + exp(-g)), silu = g * sigmoid,
// silu' = sigmoid * (1 + g * (1 - sigmoid)).  exp(-g) = 2^t with
// t = -g * log2(e) carried as a rounded product p plus its error (an FMA
// gives the product's rounding error exactly; log2(e)'s own tail is added),
// so the hardware 2^p (v_exp_f32, 1 unit) is corrected by 2^lo ~ 1 + lo ln 2.
// For p > 64 (g < -44.4) numerator and denominator are scaled by 2^-64:
// sigmoid = 2^-64 / (2^-64 + 2^(p-64)), the final 2^-64 applied by ldexp,
// which rounds once into the subnormal range.  So 2^p never overflows and
// sigmoid(g) follows e^g down to FP32's smallest subnormal (g near -103)
// instead of stopping at 2^-126.  g is first clamped to [-128, 128]: beyond
// that sigmoid is 1, or rounds to 0 either way.  The reciprocal is v_rcp_f32
// (1 unit).  Relative error: ~4 units in the last place while sigmoid is a
// normal FP32 number; below 2^-126 (g < -87.3) the result is the correctly
// scaled value rounded once to the subnormal grid (absolute error <= 2^-149
// plus the same ~4 units relative).  Infinite g gives sigmoid 1 or 0, so
// silu(-inf) = -inf * 0 is NaN, as the formula g * sigmoid(g) reads in IEEE
// arithmetic.
__device__ __forceinline__ float sigmoid_f32(float g)
{
    constexpr float kL2eHi = 1.44269502162933349609375f;   // log2(e) rounded to float
    constexpr float kL2eLo = 1.925963033500011e-08f;        // log2(e) - kL2eHi
    constexpr float kLn2 = 0.693147180559945309f;
    const float gc = __builtin_amdgcn_fmed3f(g, -128.0f, 128.0f);
    const float p = -gc * kL2eHi;
    const float lo = __builtin_fmaf(-gc, kL2eLo, __builtin_fmaf(-gc, kL2eHi, -p));
    const bool big = p > 64.0f;
    const float e0 = __builtin_amdgcn_exp2f(p - (big ? 64.0f : 0.0f));
    const float e = __builtin_fmaf(e0, lo * kLn2, e0);
    const float r = __builtin_amdgcn_rcpf((big ? 0x1p-64f : 1.0f) + e);
    return __builtin_amdgcn_ldexpf(r, big ? -64 : 0);
}

// sigmoid_f32 of 8 values, bit for bit.  For p <= 64 (g >= -44.4) the
// scaling above is the identity (2^(p - 0), ldexp by 0), so the 8 values
// are evaluated without it, 6 instructions fewer each; a lane that holds a
// value with p > 64 evaluates its 8 values again with sigmoid_f32 (a branch
// taken only when some lane of the wavefront has such a gate).
__device__ __forceinline__ void sigmoid8(const float (&g)[8], float (&s)[8])
{
    constexpr float kL2eHi = 1.44269502162933349609375f;
    constexpr float kL2eLo = 1.925963033500011e-08f;
    constexpr float kLn2 = 0.693147180559945309f;
    bool far = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float gc = __builtin_amdgcn_fmed3f(g[e], -128.0f, 128.0f);
        const float p = -gc * kL2eHi;
        const float lo = __builtin_fmaf(-gc, kL2eLo, __builtin_fmaf(-gc, kL2eHi, -p));
        far |= p > 64.0f;
        const float e0 = __builtin_amdgcn_exp2f(p);
        s[e] = __builtin_amdgcn_rcpf(1.0f + __builtin_fmaf(e0, lo * kLn2, e0));
    }
    if (far) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] = sigmoid_f32(g[e]);
    }
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

// Streaming accesses of the activations: each element is read or written
// exactly once per launch.
#ifndef RMSN_NT_LOAD
#define RMSN_NT_LOAD 1
#endif
#ifndef RMSN_NT_STORE
#define RMSN_NT_STORE 1
#endif
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const uint16_t* p)
{
#if RMSN_NT_LOAD
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
#else
    return ld16(p);
#endif
}
__device__ __forceinline__ void st16_stream(uint16_t* p, const uint4& v)
{
#if RMSN_NT_STORE
    const u32x4_t t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t*>(p));
#else
    st16(p, v);
#endif
}

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
// 8, mirror in 16, xor 16, the two halves), so every lane of a group ends
// with the bitwise same result and the order depends only on L.
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

__device__ __forceinline__ int64_t row_offset(int row, const RowMap& m)
{
    if (m.heads == 1) return (int64_t)row * m.stride_t;
    const uint32_t n = (uint32_t)row;
    const uint32_t hi = __umulhi(n, m.magic);
    const uint32_t t = (hi + ((n - hi) >> 1)) >> (m.shift - 1);
    const uint32_t hd = n - t * m.heads;
    return (int64_t)t * m.stride_t + (int64_t)hd * m.stride_h;
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
// parity, one barrier per iteration); the wavefront partials are added in
// wavefront order.  With ONE_ROW_AT_A_TIME the partials of one row are read
// and added before the next row's are read (an empty asm with a memory
// clobber keeps the compiler from hoisting the reads), so at most one row's
// partials occupy registers; otherwise all of them may be in flight at once.
// The sums are the same either way.
template <int LPR, int U, int RPI, bool ONE_ROW_AT_A_TIME = false>
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
            if constexpr (ONE_ROW_AT_A_TIME) __asm__ volatile("" : "+v"(t)::"memory");
            s[u] = t;
        }
    }
}

// Vector indices a lane owns.  Lanes past the row's last vector read the last
// vector again (always in bounds) and are masked where it matters, so loads
// need no per-element predication.
template <int V>
struct LaneVectors {
    int col[V];   // first element of the (clamped) vector
    bool ok[V];   // the vector belongs to this lane
    __device__ __forceinline__ LaneVectors(int g, int lpr, int nv)
    {
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int k = g + lpr * v;
            ok[v] = k < nv;
            col[v] = 8 * (ok[v] ? k : nv - 1);
        }
    }
};

}  // namespace rmsn
