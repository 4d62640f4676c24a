// route.cpp -- backward route table.
//
// The pages route by token-count windows per (architecture, width, weight
// dtype, residual, mode) and keep the deterministic "pair" (main kernel +
// fixed-order dw reduce) next to single-kernel forms (p1 #8577 "Two GB300
// windows"; p2 windows list).  Their windows were measured on other hardware;
// this table is MI355X's own.
#include "route.h"

#include "layouts.h"

namespace rmsn {

int bwd_rows_per_iter(int64_t H)
{
    const int id = pick_layout(kBwdLayouts, kNumBwdLayouts, H);
    if (id < 0) return 0;
    const Layout& L = kBwdLayouts[id];
    return slots_of(L.lpr) * L.u;
}

size_t ws_bytes_for(int64_t R, int64_t H, const BwdRoute& r)
{
    size_t b = ws_part_offset(H);
    if (r.form == FORM_PAIR) b += (size_t)chunks_of(R, r.rows_per_chunk) * (size_t)H * 8;
    return b;
}

BwdRoute default_bwd_route(int64_t R, int64_t H, bool w_f32, bool residual, bool deterministic)
{
    (void)w_f32;
    (void)residual;
    const int rpi = bwd_rows_per_iter(H);
    BwdRoute r;
    r.form = deterministic ? FORM_PAIR : FORM_ATOMIC;
    // Aim for about 1024 workgroups (4 per compute unit) once there are
    // enough rows; a chunk is a whole number of iterations.
    const int64_t target = 1024;
    int64_t per = (R + target - 1) / target;
    per = ((per + rpi - 1) / rpi) * rpi;
    if (per < rpi) per = rpi;
    r.rows_per_chunk = (int)per;
    return r;
}

}  // namespace rmsn
