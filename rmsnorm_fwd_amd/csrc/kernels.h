// kernels.h -- internal interface between the C-ABI layer (api.cpp) and the
// HIP kernels (fwd.hip, bwd.hip).  Not installed; the public ABI is
// include/rmsnorm.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace rmsn {

// Where row r = t * heads + head of a [T, heads, H] tensor starts:
// t * stride_t + head * stride_h elements.  t = r / heads is taken by the
// multiply-shift method for invariant divisors (Granlund and Montgomery,
// "Division by invariant integers using multiplication", 1994), valid for
// every 32-bit r: with l = ceil(log2(heads)) and
// magic = floor(2^32 (2^l - heads) / heads) + 1,
// t = (hi + ((r - hi) >> 1)) >> (l - 1), hi = the high 32 bits of r * magic.
struct RowMap {
    int64_t stride_t, stride_h;
    uint32_t heads, magic, shift;
};

inline RowMap make_row_map(int64_t heads, int64_t stride_t, int64_t stride_h)
{
    RowMap m{stride_t, stride_h, (uint32_t)heads, 0u, 0u};
    if (heads > 1) {
        uint32_t l = 0;
        while ((1ull << l) < (uint64_t)heads) ++l;
        m.magic = (uint32_t)(((1ull << 32) * ((1ull << l) - (uint64_t)heads)) / (uint64_t)heads + 1);
        m.shift = l;
    }
    return m;
}

struct FwdParams {
    const uint16_t* x;    // [T,heads,H] BF16
    const uint16_t* r;    // residual or nullptr
    const void* w;        // [H] BF16 or FP32
    uint16_t* y;          // [T,heads,H] BF16
    uint16_t* h;          // residual output (when r != nullptr)
    const uint16_t* g;    // SiLU gate [T,heads,H] or nullptr (never with r)
    float* rstd;          // [R]
    RowMap rows;
    int R, H;
    double eps, inv_h;
};

struct BwdParams {
    const uint16_t* dy;
    const uint16_t* x;    // normalised input (h with a residual)
    const float* rstd;
    const void* w;
    const uint16_t* dres; // or nullptr
    const uint16_t* g;    // SiLU gate or nullptr (never with dres)
    uint16_t* dg;         // gate gradient (when g != nullptr)
    uint16_t* dx;
    float* dw;
    double* part;         // [P,H] FP64 partials (pair form: P = chunks; column forms: P = col_chunks)
    double* acc;          // [H] FP64 accumulator (atomic form), zero on entry and exit
    unsigned* ticket;     // arrival counter (atomic form), zero on entry and exit
    unsigned* slice_ticket;  // [slices] arrival counters (column ticket form), zero on entry and exit
    RowMap rows;
    int R, H;
    int chunks;           // row workgroups; workgroup c takes row groups c, c + chunks, ...
    int form;             // FORM_* (route.h)
    int direct_dw;        // pair form with one chunk: write dw, skip the reduce
    int col_chunks;       // column forms: row blocks per column slice
    int col_vecs;         // column forms: 16-byte vectors per column slice (1, 2, 4 or 8)
    int slices;           // column forms: column slices, ceil(H / (8 col_vecs))
    int col_tasks;        // column forms: column tasks at the start of this launch's grid (0: row tasks only)
    int prefetch;         // row kernel over several chunks, plain rows: 1 = next-row register tile
    int one_row;          // per-head view with gaps between rows: one row per row group (H 129-256)
    double inv_h;
};

// Launchers; return the launch's hipError_t.
// launch_fwd: `layout` indexes the forward table `table` (FWD_PLAIN, FWD_LONG
// or FWD_RES_LONG of layouts.h; FWD_LONG only without residual and gate,
// FWD_RES_LONG only with a residual).
hipError_t launch_fwd(int table, int layout, bool w_f32, const FwdParams& p, int grid, hipStream_t s);
hipError_t launch_bwd(int layout, bool w_f32, const BwdParams& p, hipStream_t s);
// launch_bwd_cols: a launch of the column forms' kernel: p.col_tasks column
// tasks, then (with rows) p.chunks row tasks.
hipError_t launch_bwd_cols(int layout, bool w_f32, const BwdParams& p, bool rows, hipStream_t s);
hipError_t launch_dw_reduce(const double* part, int chunks, int H, float* dw, hipStream_t s);
hipError_t launch_fill_zero(void* ptr, int64_t bytes, hipStream_t s);

// The library's own device scratch for callers that cannot allocate: a
// file-scope device array of kScratchBytes per GPU.  scratch_region returns
// its device address on the current device (looked up once per device, when
// its prepared part is also cleared on `s`); hipSuccess or the lookup's error.
constexpr size_t kScratchBytes = size_t(32) << 20;
hipError_t scratch_region(void** out, hipStream_t s);

}  // namespace rmsn
