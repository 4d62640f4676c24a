// api.cpp -- the C ABI declared in include/rmsnorm.h: argument validation
// (host only, before any HIP call), routing, and kernel launches on the
// caller's stream.  No allocation, no synchronisation.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdint>

#include "../../include/rmsnorm.h"
#include "kernels.h"
#include "layouts.h"
#include "route.h"

using namespace rmsn;

namespace {

// R = T * heads must stay below 2^30 (row indices are 32-bit in the kernels,
// with room for a whole grid's step beyond the last row).
constexpr int64_t kMaxRows = int64_t(1) << 30;

bool rows_ok(int64_t T, int64_t heads) { return T >= 0 && heads >= 1 && T <= (kMaxRows - 1) / heads; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Shape {
    int64_t T, heads, H, st, sh, R;
};

// Shape checks shared by every entry point.
int check_shape(int64_t T, int64_t heads, int64_t H, int64_t st, int64_t sh, Shape* out)
{
    if (T < 0 || heads < 1 || H < 1) return RMSN_ERR_INVALID_ARG;
    if (H % 8 != 0 || H > RMSN_MAX_H) return RMSN_ERR_UNSUPPORTED;
    if (!rows_ok(T, heads)) return RMSN_ERR_INVALID_ARG;
    const int64_t R = T * heads;
    if (st < 0 || sh < 0) return RMSN_ERR_INVALID_ARG;
    if (heads == 1) {
        if (T > 1 && st < H) return RMSN_ERR_INVALID_ARG;
    } else {
        if (sh < H) return RMSN_ERR_INVALID_ARG;
        if (T > 1 && st < heads * sh) return RMSN_ERR_INVALID_ARG;
    }
    if (st % 8 != 0 || (heads > 1 && sh % 8 != 0)) return RMSN_ERR_MISALIGNED;
    *out = Shape{T, heads, H, st, sh, R};
    return RMSN_OK;
}

std::atomic<int> g_cu_count[64];

int cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        g_cu_count[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

int status_of(hipError_t e) { return e == hipSuccess ? RMSN_OK : RMSN_ERR_HIP; }

BwdRoute internal(const rmsn_route& r) { return BwdRoute{r.form, r.chunks, r.col_chunks, r.col_vecs, r.prefetch}; }

int bwd_impl(const void* dy, const void* x, const float* rstd, const void* w, int w_dtype,
             const void* dres, void* dx, float* dw, void* workspace,
             const Shape& s, const BwdRoute& r, hipStream_t stream,
             const void* gate = nullptr, void* dgate = nullptr)
{
    if (s.R == 0) return status_of(launch_fill_zero(dw, s.H * 4, stream));

    const int layout = pick_layout(kBwdLayouts, kNumBwdLayouts, s.H);
    BwdParams p{};
    p.dy = static_cast<const uint16_t*>(dy);
    p.x = static_cast<const uint16_t*>(x);
    p.rstd = rstd;
    p.w = w;
    p.dres = static_cast<const uint16_t*>(dres);
    p.g = static_cast<const uint16_t*>(gate);
    p.dg = static_cast<uint16_t*>(dgate);
    p.dx = static_cast<uint16_t*>(dx);
    p.dw = dw;
    char* ws = static_cast<char*>(workspace);
    p.ticket = reinterpret_cast<unsigned*>(ws);
    p.acc = reinterpret_cast<double*>(ws + ws_acc_offset());
    p.slice_ticket = reinterpret_cast<unsigned*>(ws + ws_slice_ticket_offset(s.H));
    p.part = reinterpret_cast<double*>(ws + ws_part_offset(s.H));
    p.rows = make_row_map(s.heads, s.st, s.sh);
    p.R = (int)s.R;
    p.H = (int)s.H;
    p.chunks = r.chunks;
    p.form = r.form;
    p.direct_dw = r.form == FORM_PAIR && r.chunks == 1;
    p.prefetch = r.prefetch;
    p.one_row = s.heads > 1 && (s.sh != s.H || s.st != s.heads * s.H);
    p.inv_h = 1.0 / (double)s.H;
    const bool w32 = w_dtype == RMSN_W_F32;
    if (r.form == FORM_COLS || r.form == FORM_COLS_TICKET) {
        p.col_chunks = r.col_chunks;
        p.col_vecs = r.col_vecs;
        p.slices = (int)col_slices(s.H, r.col_vecs);
        p.col_tasks = p.slices * r.col_chunks;
        // In place (dx over dy, or dg over the gate) the column tasks, which
        // read dy and the gate of every row, run first as a launch of their
        // own and the row tasks after them: the same kernels and order of
        // sums, so the same bits.
        const bool in_place = dx == dy || (gate && dgate == gate);
        hipError_t e = launch_bwd_cols(layout, w32, p, !in_place, stream);
        if (e != hipSuccess) return RMSN_ERR_HIP;
        if (r.form == FORM_COLS && r.col_chunks > 1) e = launch_dw_reduce(p.part, r.col_chunks, p.H, dw, stream);
        if (e != hipSuccess) return RMSN_ERR_HIP;
        if (in_place) {
            p.col_tasks = 0;
            e = launch_bwd_cols(layout, w32, p, true, stream);
        }
        return status_of(e);
    }
    hipError_t e = launch_bwd(layout, w32, p, stream);
    if (e != hipSuccess) return RMSN_ERR_HIP;
    if (r.form == FORM_PAIR && !p.direct_dw) e = launch_dw_reduce(p.part, p.chunks, p.H, dw, stream);
    return status_of(e);
}

int check_bwd_args(const void* dy, const void* x, const float* rstd, const void* w, int w_dtype,
                   const void* dres, const void* dx, const float* dw, const void* workspace,
                   const Shape& s)
{
    if (w_dtype != RMSN_W_BF16 && w_dtype != RMSN_W_F32) return RMSN_ERR_INVALID_ARG;
    if (!dw) return RMSN_ERR_INVALID_ARG;
    if (!aligned(dw, 4)) return RMSN_ERR_MISALIGNED;
    if (s.R == 0) return RMSN_OK;
    if (!dy || !x || !rstd || !w || !dx || !workspace) return RMSN_ERR_INVALID_ARG;
    if (!aligned(dy, 16) || !aligned(x, 16) || !aligned(w, 16) || !aligned(dx, 16) ||
        (dres && !aligned(dres, 16)) || !aligned(rstd, 4) || !aligned(workspace, 256))
        return RMSN_ERR_MISALIGNED;
    return RMSN_OK;
}

// Forward with an optional residual (r, h) or an optional SiLU gate.
int fwd_impl(const void* x, const void* residual, const void* gate, const void* w, int w_dtype,
             void* y, void* residual_out, float* rstd,
             int64_t T, int64_t heads, int64_t H, int64_t stride_t, int64_t stride_h,
             double eps, void* stream)
{
    Shape s;
    int st = check_shape(T, heads, H, stride_t, stride_h, &s);
    if (st != RMSN_OK) return st;
    if (w_dtype != RMSN_W_BF16 && w_dtype != RMSN_W_F32) return RMSN_ERR_INVALID_ARG;
    if (!(std::isfinite(eps) && eps >= 0.0)) return RMSN_ERR_INVALID_ARG;
    if (s.R == 0) return RMSN_OK;
    if (!x || !w || !y || !rstd) return RMSN_ERR_INVALID_ARG;
    if ((residual != nullptr) != (residual_out != nullptr)) return RMSN_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16) || !aligned(rstd, 4) ||
        (residual && (!aligned(residual, 16) || !aligned(residual_out, 16))) || (gate && !aligned(gate, 16)))
        return RMSN_ERR_MISALIGNED;

    const int kind = fwd_table_kind(s.R, residual != nullptr, gate != nullptr);
    const Layout* table = fwd_table(kind);
    const int layout = pick_layout(table, kNumFwdLayouts, s.H);
    const Layout& L = table[layout];
    const int64_t rpi = (int64_t)slots_of(L.lpr) * L.u;
    const int64_t iters = (s.R + rpi - 1) / rpi;
    const int64_t cap = (int64_t)cu_count() * L.k;
    const int grid = (int)(iters < cap ? iters : cap);

    FwdParams p{};
    p.x = static_cast<const uint16_t*>(x);
    p.r = static_cast<const uint16_t*>(residual);
    p.w = w;
    p.y = static_cast<uint16_t*>(y);
    p.h = static_cast<uint16_t*>(residual_out);
    p.g = static_cast<const uint16_t*>(gate);
    p.rstd = rstd;
    p.rows = make_row_map(s.heads, s.st, s.sh);
    p.R = (int)s.R;
    p.H = (int)s.H;
    p.eps = eps;
    p.inv_h = 1.0 / (double)s.H;
    return status_of(launch_fwd(kind, layout, w_dtype == RMSN_W_F32, p, grid, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int rmsnorm_fwd(const void* x, const void* residual, const void* w, int w_dtype,
                void* y, void* residual_out, float* rstd,
                int64_t T, int64_t heads, int64_t H, int64_t stride_t, int64_t stride_h,
                double eps, int deterministic, void* stream)
{
    (void)deterministic;  // the forward is one program for both modes
    return fwd_impl(x, residual, nullptr, w, w_dtype, y, residual_out, rstd, T, heads, H, stride_t,
                    stride_h, eps, stream);
}

int rmsnorm_gated_fwd(const void* x, const void* gate, const void* w, int w_dtype, void* y, float* rstd,
                      int64_t T, int64_t heads, int64_t H, int64_t stride_t, int64_t stride_h,
                      double eps, int deterministic, void* stream)
{
    (void)deterministic;
    Shape s;
    const int st = check_shape(T, heads, H, stride_t, stride_h, &s);
    if (st != RMSN_OK) return st;
    if (s.R > 0 && !gate) return RMSN_ERR_INVALID_ARG;
    return fwd_impl(x, nullptr, gate, w, w_dtype, y, nullptr, rstd, T, heads, H, stride_t, stride_h, eps,
                    stream);
}

size_t rmsnorm_bwd_workspace_size(int64_t T, int64_t heads, int64_t H, int w_dtype, const void* residual,
                                  int deterministic)
{
    if (w_dtype != RMSN_W_BF16 && w_dtype != RMSN_W_F32) return 0;
    if (!rows_ok(T, heads) || H < 1 || H % 8 != 0 || H > RMSN_MAX_H) return 0;
    const int64_t R = T * heads;
    return bwd_workspace_bytes(R, H, w_dtype == RMSN_W_F32, residual != nullptr, deterministic != 0);
}

size_t rmsnorm_bwd_workspace_size_for_route(int64_t T, int64_t heads, int64_t H, rmsn_route route)
{
    if (!rows_ok(T, heads) || H < 1 || H % 8 != 0 || H > RMSN_MAX_H) return 0;
    const BwdRoute r = internal(route);
    if (!route_valid(r, false)) return 0;
    return ws_bytes_for(T * heads, H, r);
}

int rmsnorm_bwd_workspace_init(void* workspace, size_t workspace_bytes, int64_t H, void* stream)
{
    if (!workspace || H < 1 || H % 8 != 0 || H > RMSN_MAX_H) return RMSN_ERR_INVALID_ARG;
    if (!aligned(workspace, 256)) return RMSN_ERR_MISALIGNED;
    const size_t need = ws_part_offset(H);
    if (workspace_bytes < need) return RMSN_ERR_WORKSPACE;
    return status_of(launch_fill_zero(workspace, (int64_t)need, static_cast<hipStream_t>(stream)));
}

static int route_query(int64_t T, int64_t heads, int64_t H, int w_dtype, int has_residual, int deterministic,
                       bool gated, rmsn_route* out)
{
    if (!out) return RMSN_ERR_INVALID_ARG;
    if (w_dtype != RMSN_W_BF16 && w_dtype != RMSN_W_F32) return RMSN_ERR_INVALID_ARG;
    if (!rows_ok(T, heads) || H < 1) return RMSN_ERR_INVALID_ARG;
    if (H % 8 != 0 || H > RMSN_MAX_H) return RMSN_ERR_UNSUPPORTED;
    const bool w32 = w_dtype == RMSN_W_F32;
    const BwdRoute r = gated ? gated_bwd_route(T * heads, H, w32, deterministic != 0)
                             : default_bwd_route(T * heads, H, w32, has_residual != 0, deterministic != 0);
    out->form = r.form;
    out->chunks = r.chunks;
    out->col_chunks = r.col_chunks;
    out->col_vecs = r.col_vecs;
    out->prefetch = r.prefetch;
    return RMSN_OK;
}

int rmsnorm_bwd_route(int64_t T, int64_t heads, int64_t H, int w_dtype, int has_residual,
                      int deterministic, rmsn_route* out)
{
    return route_query(T, heads, H, w_dtype, has_residual, deterministic, false, out);
}

int rmsnorm_gated_bwd_route(int64_t T, int64_t heads, int64_t H, int w_dtype, int deterministic,
                            rmsn_route* out)
{
    return route_query(T, heads, H, w_dtype, 0, deterministic, true, out);
}

int rmsnorm_bwd_routed(const void* dy, const void* x, const float* rstd, const void* w, int w_dtype,
                       const void* residual, void* dx, float* dw,
                       void* workspace, size_t workspace_bytes,
                       int64_t T, int64_t heads, int64_t H, int64_t stride_t, int64_t stride_h,
                       int deterministic, rmsn_route route, void* stream)
{
    Shape s;
    int st = check_shape(T, heads, H, stride_t, stride_h, &s);
    if (st != RMSN_OK) return st;
    st = check_bwd_args(dy, x, rstd, w, w_dtype, residual, dx, dw, workspace, s);
    if (st != RMSN_OK) return st;
    const BwdRoute r = internal(route);
    if (!route_valid(r, deterministic != 0)) return RMSN_ERR_INVALID_ARG;
    if (s.R > 0 && workspace_bytes < ws_bytes_for(s.R, s.H, r)) return RMSN_ERR_WORKSPACE;
    return bwd_impl(dy, x, rstd, w, w_dtype, residual, dx, dw, workspace, s, r, static_cast<hipStream_t>(stream));
}

int rmsnorm_bwd(const void* dy, const void* x, const float* rstd, const void* w, int w_dtype,
                const void* residual, void* dx, float* dw,
                void* workspace, size_t workspace_bytes,
                int64_t T, int64_t heads, int64_t H, int64_t stride_t, int64_t stride_h,
                int deterministic, void* stream)
{
    Shape s;
    int st = check_shape(T, heads, H, stride_t, stride_h, &s);
    if (st != RMSN_OK) return st;
    st = check_bwd_args(dy, x, rstd, w, w_dtype, residual, dx, dw, workspace, s);
    if (st != RMSN_OK) return st;
    const BwdRoute r = default_bwd_route(s.R, s.H, w_dtype == RMSN_W_F32, residual != nullptr, deterministic != 0);
    if (s.R > 0 && workspace_bytes < ws_bytes_for(s.R, s.H, r)) return RMSN_ERR_WORKSPACE;
    return bwd_impl(dy, x, rstd, w, w_dtype, residual, dx, dw, workspace, s, r, static_cast<hipStream_t>(stream));
}

int rmsnorm_bwd_noalloc(const void* dy, const void* x, const float* rstd, const void* w, int w_dtype,
                        const void* residual, void* dx, float* dw,
                        int64_t T, int64_t heads, int64_t H, int64_t stride_t, int64_t stride_h,
                        int deterministic, void* stream)
{
    Shape s;
    int st = check_shape(T, heads, H, stride_t, stride_h, &s);
    if (st != RMSN_OK) return st;
    // the scratch stands in for the workspace: validate everything else first
    alignas(256) static char stand_in;
    st = check_bwd_args(dy, x, rstd, w, w_dtype, residual, dx, dw, &stand_in, s);
    if (st != RMSN_OK) return st;
    const BwdRoute r = default_bwd_route(s.R, s.H, w_dtype == RMSN_W_F32, residual != nullptr, deterministic != 0);
    if (s.R > 0 && ws_bytes_for(s.R, s.H, r) > kScratchBytes) return RMSN_ERR_WORKSPACE;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    void* scratch = nullptr;
    if (s.R > 0 && scratch_region(&scratch, hs) != hipSuccess) return RMSN_ERR_HIP;
    return bwd_impl(dy, x, rstd, w, w_dtype, residual, dx, dw, scratch, s, r, hs);
}

int rmsnorm_gated_bwd(const void* dy, const void* x, const void* gate, const float* rstd, const void* w,
                      int w_dtype, void* dx, void* dgate, float* dw, void* workspace, size_t workspace_bytes,
                      int64_t T, int64_t heads, int64_t H, int64_t stride_t, int64_t stride_h,
                      int deterministic, void* stream)
{
    Shape s;
    int st = check_shape(T, heads, H, stride_t, stride_h, &s);
    if (st != RMSN_OK) return st;
    st = check_bwd_args(dy, x, rstd, w, w_dtype, nullptr, dx, dw, workspace, s);
    if (st != RMSN_OK) return st;
    if (s.R > 0 && (!gate || !dgate)) return RMSN_ERR_INVALID_ARG;
    if (s.R > 0 && (!aligned(gate, 16) || !aligned(dgate, 16))) return RMSN_ERR_MISALIGNED;
    const BwdRoute r = gated_bwd_route(s.R, s.H, w_dtype == RMSN_W_F32, deterministic != 0);
    if (s.R > 0 && workspace_bytes < ws_bytes_for(s.R, s.H, r)) return RMSN_ERR_WORKSPACE;
    return bwd_impl(dy, x, rstd, w, w_dtype, nullptr, dx, dw, workspace, s, r, static_cast<hipStream_t>(stream),
                    gate, dgate);
}

const char* rmsnorm_status_string(int status)
{
    switch (status) {
    case RMSN_OK: return "ok";
    case RMSN_ERR_INVALID_ARG: return "invalid argument";
    case RMSN_ERR_UNSUPPORTED: return "unsupported shape (H must be a multiple of 8 and at most RMSN_MAX_H)";
    case RMSN_ERR_MISALIGNED: return "misaligned pointer or stride";
    case RMSN_ERR_WORKSPACE: return "workspace missing or too small";
    case RMSN_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
    }
}

}  // extern "C"
