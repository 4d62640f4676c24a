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

size_t ws_bytes_for(int64_t R, int64_t H, const BwdRoute& r)
{
    size_t b = ws_part_offset(H);
    (void)R;
    if (r.form == FORM_PAIR && r.chunks > 1) b += (size_t)r.chunks * (size_t)H * 8;
    if ((r.form == FORM_COLS || r.form == FORM_COLS_TICKET) && r.col_chunks > 1)
        b += (size_t)r.col_chunks * (size_t)H * 8;
    return b;
}

bool route_valid(const BwdRoute& r, bool deterministic)
{
    if (r.chunks < 1 || r.chunks > kMaxChunks) return false;
    if (r.prefetch != 0 && r.prefetch != 1) return false;
    switch (r.form) {
    case FORM_PAIR:
        return r.col_chunks == 0 && r.col_vecs == 0;
    case FORM_ATOMIC:
        return !deterministic && r.col_chunks == 0 && r.col_vecs == 0;
    case FORM_COLS:
    case FORM_COLS_TICKET: {
        if (r.prefetch != 0) return false;
        if (r.form == FORM_COLS_TICKET && (deterministic || r.col_chunks < 2)) return false;
        const int v = r.col_vecs;
        return r.col_chunks >= 1 && r.col_chunks <= kMaxColChunks && (v == 1 || v == 2 || v == 4 || v == 8);
    }
    default:
        return false;
    }
}

// Column forms (measured on MI355X, cold caches, BF16 w, H 256-8192, R 16 to
// 16384; per-head views [T,4,256] too).  The one-pass form -- dw written by
// column tasks that each read all rows of an 8 * col_vecs-column slice, one
// launch, no workspace -- beats the pair at every width up to R = 384 (H <=
// 3072), 512 (H <= 6144) and 1024 (wider rows): H 4096, R 16: 6.2 against
// 10.7 us; R 256: 8.2 against 12.2 us; H 6144, R 512: 13.0 against 18.8 us
// (HIP events around a one-element fill read 6.0 us on the same machine).
// Its slice width: about one batch of four rows per column-task lane at
// R <= 128 (8 vectors); above that wider rows, having more slices, keep
// wider slices (fewer, longer column tasks):
static int cols1_vecs(int64_t R, int64_t H)
{
    if (R <= 128 || H > 6144) return 8;
    if (R <= 256) return 4;
    if (R <= 512) return H <= 4096 ? 2 : 4;
    return H <= 1024 ? 1 : 2;
}

static int64_t cols1_max_rows(int64_t H) { return H <= 3072 ? 384 : (H <= 6144 ? 512 : 1024); }

// Beyond that the two-launch column form -- 8-vector slices cut into
// col_chunks row blocks whose partials the reduce kernel sums, about 192
// column tasks in all (col_chunks ~ 12288 / H) -- beats the pair up to about
// R * H = 3.2 M elements at H <= 2048 (H 1536, R 2048: 13.5 against 16.2 us),
// 4.8 M at H 3072 and 6.4 M up to H 6144 (H 4096, R 1536: 20.8 against 21.8
// us; H 6144, R 1024: 21.2 against 22.8 us); past those the pair, whose rows
// are read once, wins (H 4096, R 4096: 32.3 against 41.5 us).
static int64_t cols_max_elems(int64_t H)
{
    if (H <= 2048) return 3200000;
    if (H <= 3072) return 4800000;
    if (H <= 6144) return 6400000;
    return 8400000;
}

// The next-row tile of the row kernel (BwdRoute::prefetch), by width: the
// largest row count that takes it on plain rows, the row count from which
// it takes 512 workgroups instead of 256, and the same two for rows with
// dres.  Measured on MI355X with cold caches (BF16 w; T 2048-131072,
// chunk counts 128-512 with and without the tile): on plain rows the tile
// wins 7-16 % at a few thousand rows, where each compute unit holds one or
// two workgroups and no other wavefront covers the load latency (T 4096,
// H 1536: 18.6 -> 16.6 us; T 2048, H 5120: 28.0 -> 23.5 us; T 4096,
// H 4096: 32.6 -> 28.3 us), 3-5 % up to 16384 rows, and at H 1024, 1536
// and 8192 at every row count measured (T 65536, H 8192: 586 -> 559 us);
// elsewhere beyond 16384-65536 rows it only adds registers and loses 1-6 %
// (T 65536, H 4096: 268 -> 272 us; T 65536, H 2048: 139 -> 146 us).  256
// workgroups (two or more iterations each, which the tile overlaps) beat
// 384 and 512 except at H 1024 from 16384 rows.  With dres, three loads
// per element, the tile (without the deferred rstd, see bwd.hip) wins at
// every row count measured from H 1024 to 6144 (T 131072, H 6144: 1176 ->
// 1048 us; T 65536, H 4096: 373 -> 351 us).  It spills at H 16384.  With
// dres a route never takes more workgroups than without at the same row
// count, so a workspace sized for plain rows also serves rows with dres.
struct TileWindow {
    int64_t max_h;       // serves H <= max_h (the smallest such entry)
    int64_t rows;        // plain rows: the tile up to this many rows
    int64_t wide_rows;   // ... with 512 workgroups from this many rows (else 256)
    int64_t dres_rows;   // rows with dres: the tile up to this many rows
    int64_t dres_wide;   // ... with 512 workgroups from this many rows
};
constexpr int64_t kAllRows = int64_t(1) << 40;
static constexpr TileWindow kTileWindows[] = {
    {128, 0, 0, 0, 0},                                // not measured beyond 1-3 %
    {256, 65536, kAllRows, 65536, kAllRows},          // T 32768: 19.2 -> 18.4 us
    {512, 32768, kAllRows, 32768, kAllRows},          // T 65536: 2.8 % slower
    {1024, kAllRows, 16384, kAllRows, 16384},         // T 65536: 78.2 -> 75.5 us
    {1536, kAllRows, kAllRows, kAllRows, kAllRows},   // T 65536: 108.7 -> 104.8 us
    {2048, 16384, kAllRows, kAllRows, kAllRows},      // T 65536: 5 % slower
    {3072, 32768, kAllRows, kAllRows, kAllRows},      // T 65536: 1.3 % slower
    {4096, 16384, kAllRows, kAllRows, kAllRows},      // T 32768: 0.9 % slower
    {5120, 16384, kAllRows, kAllRows, kAllRows},      // T 32768 even
    {6144, 16384, kAllRows, kAllRows, kAllRows},      // T 32768: 1.4 % slower
    {8192, kAllRows, kAllRows, 0, 0},                 // dres: even
    {16384, 0, 0, 0, 0},
};

static const TileWindow& tile_window(int64_t H)
{
    int i = 0;
    while (kTileWindows[i].max_h < H && kTileWindows[i].max_h < 16384) ++i;
    return kTileWindows[i];
}

// The fixed-order pair's chunking for R rows of width H.
BwdRoute pair_route(int64_t R, int64_t H, bool residual, bool gated)
{
    const int id = pick_layout(kBwdLayouts, kNumBwdLayouts, H);
    const Layout& L = kBwdLayouts[id < 0 ? 0 : id];
    const int64_t rpi = (int64_t)slots_of(L.lpr) * L.u;
    const int64_t groups = (R + rpi - 1) / rpi;
    const TileWindow& tw = tile_window(H);
    if (!gated && R <= (residual ? tw.dres_rows : tw.rows)) {
        // with the tile, 256 workgroups (two or more iterations each, which
        // the tile overlaps) beat 384 and 512 by 3-15 % at a few thousand
        // rows, 512 where one row group is little work (H 1024) or many
        // rows fall to each (H 3072 from 8192 rows)
        const int64_t c = R >= (residual ? tw.dres_wide : tw.wide_rows) ? 512 : 256;
        return BwdRoute{FORM_PAIR, (int)(c < groups ? c : groups), 0, 0, 1};
    }
    // Measured on MI355X with cold caches, T*H from 2^23 to 2^30 elements,
    // both weight dtypes: the layout's chunk count (512 -- two workgroups per
    // compute unit -- for H <= 6144, 256 above) beats the other counts by
    // 4-20 %, and the fixed-order pair beats the atomic form at every shape
    // (FP64 atomics from hundreds of workgroups to the same H addresses
    // serialise).
    // Below that size each workgroup should still get about four rows: the
    // chunk partials (chunks * H * 8 bytes, written and read back) would
    // otherwise cost more than the rows themselves.  Measured at H 1536 to
    // 6144, T 256 to 2048: 4 rows per workgroup, but never fewer than 128
    // workgroups, is best or within 1.4 us of the best count.
    // Halving the partials' bytes with FP32 partials was slower at every
    // size, measured twice (with the next-row tile: 18.1 -> 21.8 us at
    // T 4096, H 1536, 26.3 with 32-column reduce workgroups; 265 -> 269 us
    // at T 65536, H 4096).
    const int64_t per = (4 + rpi - 1) / rpi;  // row groups per workgroup
    int64_t c = (groups + per - 1) / per;
    if (c < 128) c = groups < 128 ? groups : 128;
    if (gated && H > 1024 && H <= 8192) {
        // The gated rows (which always load their next rows ahead) fill a
        // compute unit with one or two workgroups, so their counts are
        // multiples of the 256 compute units (384 left units idle: T 4096,
        // H 3072: 44.7 against 36.1 us at 256): 512 at H 1536 (T 4096:
        // 27.4 -> 24.8 us at 512; T 131072: 409 against 522 us at 256),
        // 256 at every row count from H 1537 to 6144 (T 131072, H 6144:
        // 1472 against 1549 us at 512; H 4096, whose rows then run at two
        // wavefronts per SIMD: 921 against 1206 us), and 256 up to 65536
        // rows and 512 above for the wider rows (T 16384, H 8192: 277 ->
        // 235 us at 256; T 131072: 512 by 1.8 %).
        const int64_t g = H <= 1536 ? 512 : (H <= 6144 || R <= 65536) ? 256 : 512;
        c = g < groups ? g : groups;
    } else {
        // narrower and wider gated rows: as measured before the tile
        if (gated && R * H <= 12000000 && c > 384) c = 384;
        if (c > L.k) c = L.k;
    }
    return BwdRoute{FORM_PAIR, (int)(c > 0 ? c : 1), 0, 0, 0};
}

static BwdRoute route_of(int64_t R, int64_t H, bool residual, bool gated)
{
    const int id = pick_layout(kBwdLayouts, kNumBwdLayouts, H);
    const Layout& L = kBwdLayouts[id < 0 ? 0 : id];
    // column forms: row tasks take one row per row group, so a row group is
    // slots_of(lpr) rows there
    const int64_t cgroups = (R + slots_of(L.lpr) - 1) / slots_of(L.lpr);
    if (R <= cols1_max_rows(H)) {
        const int64_t c = cgroups < 1 ? 1 : cgroups;
        return BwdRoute{FORM_COLS, (int)c, 1, cols1_vecs(R, H), 0};
    }
    if (R * H <= cols_max_elems(H)) {
        const int64_t c = cgroups < 512 ? cgroups : 512;
        int64_t cc = (12288 + H / 2) / H;
        if (cc < 2) cc = 2;
        return BwdRoute{FORM_COLS, (int)c, (int)cc, 8, 0};
    }
    return pair_route(R, H, residual, gated);
}

BwdRoute default_bwd_route(int64_t R, int64_t H, bool w_f32, bool residual, bool deterministic)
{
    (void)w_f32;
    (void)deterministic;  // every routed form is deterministic: both modes take the same route
    return route_of(R, H, residual, false);
}

BwdRoute gated_bwd_route(int64_t R, int64_t H, bool w_f32, bool deterministic)
{
    (void)w_f32;
    (void)deterministic;
    return route_of(R, H, false, true);
}

size_t bwd_workspace_bytes(int64_t R, int64_t H, bool w_f32, bool residual, bool deterministic)
{
    const size_t a = ws_bytes_for(R, H, default_bwd_route(R, H, w_f32, residual, deterministic));
    if (residual) return a;
    const size_t b = ws_bytes_for(R, H, gated_bwd_route(R, H, w_f32, deterministic));
    return a > b ? a : b;
}

}  // namespace rmsn
