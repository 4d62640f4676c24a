// kernels.h -- internal interface between the C-ABI layer (api.cpp) and the
// HIP kernels (kernels.hip).  Not installed; the public ABI is
// include/rmsnorm.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace rmsn {

struct FwdParams {
    const uint16_t* x;    // [T,heads,H] BF16
    const uint16_t* r;    // residual or nullptr
    const void* w;        // [H] BF16 or FP32
    uint16_t* y;          // [T,heads,H] BF16
    uint16_t* h;          // residual output (when r != nullptr)
    float* rstd;          // [R]
    int64_t stride_t, stride_h;
    int R, heads, H;
    double eps, inv_h;
};

struct BwdParams {
    const uint16_t* dy;
    const uint16_t* x;    // normalised input (h with a residual)
    const float* rstd;
    const void* w;
    const uint16_t* dres; // or nullptr
    uint16_t* dx;
    float* dw;
    double* part;         // [P,H] FP64 chunk partials (pair form)
    double* acc;          // [H] FP64 accumulator (atomic form), zero on entry and exit
    unsigned* ticket;     // arrival counter (atomic form), zero on entry and exit
    int64_t stride_t, stride_h;
    int R, heads, H;
    int chunks;           // workgroups; workgroup c takes row groups c, c + chunks, ...
    int form;             // FORM_PAIR or FORM_ATOMIC (route.h)
    int direct_dw;        // pair form with one chunk: write dw, skip the reduce
    double inv_h;
};

// Launchers; return the launch's hipError_t.
hipError_t launch_fwd(int layout, bool w_f32, const FwdParams& p, int grid, hipStream_t s);
hipError_t launch_bwd(int layout, bool w_f32, const BwdParams& p, hipStream_t s);
hipError_t launch_dw_reduce(const double* part, int chunks, int H, float* dw, hipStream_t s);
hipError_t launch_fill_zero(void* ptr, int64_t bytes, hipStream_t s);

}  // namespace rmsn
