// route.h -- per-shape choices of the library: which layout a width uses,
// how the backward cuts rows into chunks, which dw form it takes, and the
// workspace that follows from them.  Pure host functions (no HIP calls), so
// the CPU tests can check them.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace rmsn {

// How the backward forms dw (the column sum over all rows):
//   FORM_PAIR    row kernel writes one FP64 partial row per chunk of rows, a
//                second kernel sums them in a fixed order (with one chunk the
//                row kernel writes dw itself and there is no second kernel);
//   FORM_ATOMIC  row kernel adds its chunk partials into an FP64 accumulator
//                atomically, the last workgroup to finish writes dw;
//   FORM_COLS    one launch of two kinds of workgroups: row tasks form dx
//                only; column tasks form dw for a slice of columns straight
//                from u, dy and rstd, in a fixed order.  With col_chunks > 1
//                each slice's rows are cut into col_chunks blocks whose FP64
//                partials the fixed-order reduce kernel sums (a second
//                launch, but over col_chunks rows instead of one per chunk);
//   FORM_COLS_TICKET  FORM_COLS with col_chunks > 1, where the column task
//                that finishes a slice last (a per-slice arrival ticket) sums
//                that slice's partials in the fixed order: one launch.
enum { FORM_PAIR = 0, FORM_ATOMIC = 1, FORM_COLS = 2, FORM_COLS_TICKET = 3 };

struct BwdRoute {
    int form;        // FORM_*
    int chunks;      // workgroups that walk the rows (row kernel, or row tasks of the column forms)
    int col_chunks;  // column forms: row blocks per column slice (1: one pass over all rows)
    int col_vecs;    // column forms: 16-byte vectors (8 columns each) per column slice: 1, 2, 4 or 8
    int prefetch;    // pair and atomic forms: 1 = the row kernel loads a workgroup's next rows while
                     // it reduces the current ones (plain rows; no effect on any result bit)
};

// Workspace layout (bytes, every part 256-aligned):
//   [0, 256)                  header: the arrival ticket of the atomic form at offset 0
//   [256, +pad256(8H))        FP64 [H] accumulator of the atomic form
//   [.., +pad256(4*ceil(H/8))) per-slice arrival tickets of FORM_COLS_TICKET
//   [ws_part_offset(H), ...)  FP64 partials: chunks x H (pair), col_chunks x H (column forms)
// Everything before ws_part_offset is the "prepared" part: zero before the
// first non-deterministic call and left zero by every call.
constexpr size_t kWsHeader = 256;
inline size_t pad256(size_t b) { return (b + 255) & ~(size_t)255; }
inline size_t ws_acc_offset() { return kWsHeader; }
inline size_t ws_slice_ticket_offset(int64_t H) { return kWsHeader + pad256((size_t)H * 8); }
inline size_t ws_part_offset(int64_t H)
{
    return ws_slice_ticket_offset(H) + pad256((size_t)((H + 7) / 8) * sizeof(unsigned));
}
size_t ws_bytes_for(int64_t R, int64_t H, const BwdRoute& r);

// Column slices of a column form: ceil(H / (8 * col_vecs)).
inline int64_t col_slices(int64_t H, int col_vecs) { return (H + 8 * col_vecs - 1) / (8 * col_vecs); }

// The measured route table (route.cpp): the plain backward's (residual:
// rows with dres) and the SiLU-gated backward's.
BwdRoute default_bwd_route(int64_t R, int64_t H, bool w_f32, bool residual, bool deterministic);
BwdRoute gated_bwd_route(int64_t R, int64_t H, bool w_f32, bool deterministic);

// The pair's chunking and next-row tile alone.
BwdRoute pair_route(int64_t R, int64_t H, bool residual, bool gated);

// Workspace bytes the size query reports: the plain route's, and without
// dres at least the gated route's too (one size serves both backwards).
size_t bwd_workspace_bytes(int64_t R, int64_t H, bool w_f32, bool residual, bool deterministic);

// Largest chunk count a route may ask for, and largest row-block count per
// column slice.
constexpr int64_t kMaxChunks = 1 << 16;
constexpr int64_t kMaxColChunks = 1 << 12;

// Whether a route is well formed for this mode (host validation of the route
// override): the atomic and ticket forms only without determinism.
bool route_valid(const BwdRoute& r, bool deterministic);

}  // namespace rmsn
