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

int bwd_direct_rows_per_iter(int64_t H)
{
    const int id = pick_layout(kBwdLayouts, kNumBwdLayouts, H);
    if (id < 0) return 0;
    const Layout& L = kBwdLayouts[id];
    return slots_of(L.lpr) * direct_max_u(L.lpr, L.v, L.u);
}

size_t ws_bytes_for(int64_t R, int64_t H, const BwdRoute& r)
{
    size_t b = ws_part_offset(H);
    (void)R;
    if (r.form == FORM_PAIR && r.chunks > 1) b += (size_t)r.chunks * (size_t)H * 8;
    return b;
}

BwdRoute default_bwd_route(int64_t R, int64_t H, bool w_f32, bool residual, bool deterministic)
{
    (void)w_f32;
    (void)residual;
    (void)deterministic;
    const int id = pick_layout(kBwdLayouts, kNumBwdLayouts, H);
    const Layout& L = kBwdLayouts[id < 0 ? 0 : id];
    const int64_t rpi = (int64_t)slots_of(L.lpr) * L.u;
    const int64_t groups = (R + rpi - 1) / rpi;
    BwdRoute r;
    // Measured on MI355X with cold caches, T*H from 2^23 to 2^30 elements,
    // both weight dtypes: the layout's chunk count (512 -- two workgroups per
    // compute unit -- for H <= 6144, 256 above) beats the other counts by
    // 4-20 %, and the fixed-order pair beats the atomic form at every shape
    // (FP64 atomics from hundreds of workgroups to the same H addresses
    // serialise), so both modes take the pair.
    r.form = FORM_PAIR;
    // Below that size each workgroup should still get about four rows: the
    // chunk partials (chunks * H * 8 bytes, written and read back) would
    // otherwise cost more than the rows themselves.  Measured at H 1536 to
    // 6144, T 256 to 2048: 4 rows per workgroup, but never fewer than 128
    // workgroups, is best or within 1.4 us of the best count, and 1.5-3 us
    // faster than one row group per workgroup at T 256 to 1024.
    const int64_t per = (4 + rpi - 1) / rpi;  // row groups per workgroup
    int64_t c = (groups + per - 1) / per;
    if (c < 128) c = groups < 128 ? groups : 128;
    if (c > L.k) c = L.k;
    r.chunks = (int)(c > 0 ? c : 1);
    // When one iteration of a single workgroup covers every row (it may take
    // more rows per iteration than the multi-workgroup layout, see
    // direct_max_u), that workgroup writes dw itself and the reduce launch
    // goes: measured at T 1-128, H 256-6144, 0.5-2 us faster than the pair
    // with one row group per workgroup; one more iteration already costs
    // 1.3-4 us (cold loads in series), more than the reduce launch.
    if (groups <= 2 || R <= (int64_t)bwd_direct_rows_per_iter(H)) r.chunks = 1;
    return r;
}

}  // namespace rmsn
