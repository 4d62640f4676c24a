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
    (void)R;
    if (r.form == FORM_PAIR) b += (size_t)r.chunks * (size_t)H * 8;
    return b;
}

BwdRoute default_bwd_route(int64_t R, int64_t H, bool w_f32, bool residual, bool deterministic)
{
    (void)w_f32;
    (void)residual;
    (void)deterministic;
    const int64_t rpi = bwd_rows_per_iter(H);
    const int64_t groups = (R + rpi - 1) / rpi;
    BwdRoute r;
    // Measured on MI355X (T 65536, H 1536 to 6144, both weight dtypes):
    // 512 workgroups -- two per compute unit -- beat 256, 768, 1024 and more
    // by 4-20 %, and the fixed-order pair beats the atomic form by 25-50 %,
    // so both modes take the pair at these sizes.
    r.form = FORM_PAIR;
    r.chunks = (int)(groups < 512 ? (groups > 0 ? groups : 1) : 512);
    return r;
}

}  // namespace rmsn
