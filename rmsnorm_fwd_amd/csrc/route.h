// route.h -- per-shape choices of the library: which layout a width uses,
// how the backward cuts rows into chunks, which dw form it takes, and the
// workspace that follows from them.  Pure host functions (no HIP calls), so
// the CPU tests can check them.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace rmsn {

// pair: FP64 partials + fixed-order reduce kernel (with one chunk the row
// kernel writes dw itself); atomic: FP64 atomic adds, last workgroup writes dw.
enum { FORM_PAIR = 0, FORM_ATOMIC = 1 };

struct BwdRoute {
    int form;    // FORM_PAIR or FORM_ATOMIC
    int chunks;  // workgroups of the row kernel (= FP64 partial rows of the pair form)
};

// Workspace layout: [0, 256) header (arrival ticket at offset 0),
// [256, 256 + pad256(8H)) FP64 accumulator for the atomic form,
// then chunks * H FP64 partials for the pair form.
constexpr size_t kWsHeader = 256;
inline size_t pad256(size_t b) { return (b + 255) & ~(size_t)255; }
inline size_t ws_acc_offset() { return kWsHeader; }
inline size_t ws_part_offset(int64_t H) { return kWsHeader + pad256((size_t)H * 8); }
size_t ws_bytes_for(int64_t R, int64_t H, const BwdRoute& r);

// The measured route table (route.cpp).
BwdRoute default_bwd_route(int64_t R, int64_t H, bool w_f32, bool residual, bool deterministic);

// Rows one iteration covers when a single workgroup does every row (chunks
// = 1, dw written directly) for this width.
int bwd_direct_rows_per_iter(int64_t H);

// Largest chunk count a route may ask for.
constexpr int64_t kMaxChunks = 1 << 16;

}  // namespace rmsn
