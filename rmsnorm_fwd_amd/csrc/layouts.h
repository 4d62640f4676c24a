// layouts.h -- how a row of H BF16 values is spread over the lanes of a
// workgroup, for the forward and the backward kernels.  Internal to the
// library (host and device code both read these tables).
//
// A row is read as H/8 vectors of 16 bytes (8 BF16 values).  A "row group"
// of LPR lanes covers one row: lane g owns vectors g, g + LPR, ...,
// g + (V-1)*LPR, so each load instruction of a wavefront touches consecutive
// 16-byte vectors.  LPR <= 64 keeps a row inside one wavefront (reduced with
// DPP and ds_swizzle only); LPR > 64 spans LPR/64 wavefronts that combine
// their partial sums through LDS.  A workgroup has BLOCK = max(256, LPR)
// lanes, i.e. SLOTS = BLOCK/LPR row groups, and each row group takes U rows
// per iteration, so one iteration covers RPI = SLOTS*U rows.  LPR and V are
// a function of H alone (the forward's U and grid cap also follow the row
// count and the residual, through the tables below, which all agree on LPR
// and V), which keeps the order of every row reduction -- and so y, rstd
// and dx -- independent of T, of the route and of the mode.
#pragma once

namespace rmsn {

struct Layout {
    int max_h;  // the layout serves H <= max_h (H % 8 == 0)
    int lpr;    // lanes per row
    int v;      // 16-byte vectors per lane per row
    int u;      // rows per row group per iteration
    int k;      // forward: workgroups per compute unit (grid cap);
                // backward: workgroups ("chunks") of the row kernel
};

// X(id, max_h, lpr, v, u, k); max_h == lpr * v * 8.  Every entry was picked
// by timing the candidates on MI355X with cold caches (T*H between 2^25 and
// 2^30 elements); the smallest max_h >= H serves H.  At H 2048, 4096 and
// 5120 the forward's grid cap is 64 workgroups per compute unit (one or two
// iterations each): against 32, 1-3 % faster from T 32768 up (T 131072,
// H 4096: 358 -> 348 us; gated T 65536, H 4096: 269 -> 262 us; T 65536,
// H 2048: 91.3 -> 89.5 us) and equal below.  At H 6144 a larger cap pays
// only in long runs (48: T 131072 548 -> 540 us), and was 2 % slower at
// T 16384, so only the long-run table takes it; at H 1536 and 3072 it made
// no difference.  At H 16384 both long-run tables take 32 instead of 8
// (T 65536: 767 -> 731 us with FP32 w, 752 -> 739 us, residual 1641 -> 1605
// us); at T 4096 it was mixed, so the plain table keeps 8.  A tuning build may
// supply its own candidate tables (all four, and the two row thresholds) through
// RMSN_LAYOUTS_OVERRIDE.
#ifdef RMSN_LAYOUTS_OVERRIDE
#include RMSN_LAYOUTS_OVERRIDE
#else
#define RMSN_FWD_LAYOUTS(X)    \
    X(0, 64, 8, 1, 4, 64)      \
    X(1, 128, 16, 1, 4, 64)    \
    X(2, 256, 8, 4, 1, 64)     \
    X(3, 512, 32, 2, 2, 64)    \
    X(4, 1024, 32, 4, 1, 64)   \
    X(5, 1536, 32, 6, 1, 16)   \
    X(6, 2048, 256, 1, 4, 64)  \
    X(7, 3072, 64, 6, 1, 32)   \
    X(8, 4096, 512, 1, 2, 64)  \
    X(9, 5120, 320, 2, 2, 64)  \
    X(10, 6144, 768, 1, 2, 24) \
    X(11, 8192, 512, 2, 2, 32) \
    X(12, 16384, 512, 4, 1, 8)

// Plain forwards over at least kFwdLongRows rows.  Same lanes and vectors
// per row as the plain table (so the same row sums); at H 4096 and 5120 three
// rows per row group and iteration instead of two: T 65536, H 4096: 180 ->
// 175 us; T 131072, H 4096: 364 -> 358 us; T 65536, H 5120: 228 -> 224 us.
// Below that the extra rows cost more than they bring (T 16384, H 4096:
// 47.4 -> 48.6 us; T 32768, H 5120: 110.9 -> 113.6 us), and at H 6144 and the
// narrower widths they were slower at every row count measured.
constexpr long long kFwdLongRows = 65536;
#define RMSN_FWD_LONG_LAYOUTS(X) \
    X(0, 64, 8, 1, 4, 64)        \
    X(1, 128, 16, 1, 4, 64)      \
    X(2, 256, 8, 4, 1, 64)       \
    X(3, 512, 32, 2, 2, 64)      \
    X(4, 1024, 32, 4, 1, 64)     \
    X(5, 1536, 32, 6, 1, 16)     \
    X(6, 2048, 256, 1, 4, 64)    \
    X(7, 3072, 64, 6, 1, 32)     \
    X(8, 4096, 512, 1, 3, 64)    \
    X(9, 5120, 320, 2, 3, 64)    \
    X(10, 6144, 768, 1, 2, 48)   \
    X(11, 8192, 512, 2, 2, 32)   \
    X(12, 16384, 512, 4, 1, 32)

// The forward with a fused residual add streams four tensors (x, r in; h, y
// out) instead of two.  Over at least kFwdResLongRows rows it keeps the plain
// forward's lanes and vectors per row for every width -- so its row sums,
// rstd and y are the plain forward's bits for the same input h -- and at
// H 5120 and 6144 takes four rows per row group and iteration, twice the
// loads in flight: T 131072, H 6144: 1183 -> 1104 us; T 65536, H 6144:
// 572 -> 543 us; T 32768, H 6144: 279 -> 271 us; T 65536, H 5120: 497 ->
// 475 us (the grid cap made no difference between 8 and 32 workgroups per
// compute unit).  Below that it takes the plain table: at T 16384 four rows
// were already 1 % slower, at T 4096 6 %, and at T 1 the 768-lane
// workgroup's three unused rows cost 1.2 us.  At H 4096 four rows were
// slower at T 65536 (372 -> 386 us), so the plain layout stays there and
// below.
constexpr long long kFwdResLongRows = 32768;
#define RMSN_FWD_RES_LONG_LAYOUTS(X) \
    X(0, 64, 8, 1, 4, 64)       \
    X(1, 128, 16, 1, 4, 64)     \
    X(2, 256, 8, 4, 1, 64)      \
    X(3, 512, 32, 2, 2, 64)     \
    X(4, 1024, 32, 4, 1, 64)    \
    X(5, 1536, 32, 6, 1, 16)    \
    X(6, 2048, 256, 1, 4, 32)   \
    X(7, 3072, 64, 6, 1, 32)    \
    X(8, 4096, 512, 1, 2, 32)   \
    X(9, 5120, 320, 2, 4, 16)   \
    X(10, 6144, 768, 1, 4, 16)  \
    X(11, 8192, 512, 2, 2, 32)  \
    X(12, 16384, 512, 4, 1, 32)

// The SiLU-gated forward is an operation of its own (its rstd need not equal
// the plain forward's bits), with its own table, measured on MI355X with the
// eight-gate sigmoid (cold, T 4096-131072, BF16 and FP32 w): one row per row
// group of two to four vectors per lane from H 1024 to 5120 (T 65536, H 2048:
// 146 -> 130 us; H 4096: 279 -> 257 us, 128 x 4 beating 256 x 2 from 65536
// rows; H 5120: 389 -> 362 us), 256 lanes x 3 vectors at H 6144 (T 65536:
// 421-425 against 473-478 us for 768 x 1; 384 x 2: 444 us), and the plain
// table's layouts at H 3072 and 8192 (the alternatives measured there were
// not faster at every row count); 64 workgroups per compute unit at every
// width up to 8192 (against 32 at H 3072-8192: T 65536, H 6144 423 -> 400
// us, H 3072 200 -> 193 us; 16 was slower), 32 at H 16384 (against 8, with
// the eight-gate sigmoid: T 4096 78 -> 73 us, T 65536 1128 -> 1096 us).
#define RMSN_FWD_GATED_LAYOUTS(X) \
    X(0, 64, 8, 1, 4, 64)         \
    X(1, 128, 16, 1, 4, 64)       \
    X(2, 256, 8, 4, 1, 64)        \
    X(3, 512, 32, 2, 2, 64)       \
    X(4, 1024, 64, 2, 1, 64)      \
    X(5, 1536, 64, 3, 1, 64)      \
    X(6, 2048, 128, 2, 1, 64)     \
    X(7, 3072, 64, 6, 1, 64)      \
    X(8, 4096, 128, 4, 1, 64)     \
    X(9, 5120, 320, 2, 1, 64)     \
    X(10, 6144, 256, 3, 1, 64)    \
    X(11, 8192, 512, 2, 2, 64)    \
    X(12, 16384, 512, 4, 1, 32)

#define RMSN_BWD_LAYOUTS(X)       \
    X(0, 64, 8, 1, 2, 512)        \
    X(1, 128, 16, 1, 2, 512)      \
    X(2, 256, 16, 2, 2, 512)      \
    X(3, 512, 32, 2, 2, 512)      \
    X(4, 1024, 64, 2, 1, 512)     \
    X(5, 1536, 64, 3, 1, 512)     \
    X(6, 2048, 128, 2, 2, 512)    \
    X(7, 3072, 128, 3, 1, 512)    \
    X(8, 4096, 256, 2, 2, 512)    \
    X(9, 6144, 256, 3, 1, 512)    \
    X(10, 8192, 1024, 1, 1, 256)  \
    X(11, 16384, 512, 4, 1, 256)
#endif

#define RMSN_CHECK_LAYOUT(id, mh, l, vv, uu, kk) static_assert((mh) == (l) * (vv) * 8, "layout width");
RMSN_FWD_LAYOUTS(RMSN_CHECK_LAYOUT)
RMSN_FWD_LONG_LAYOUTS(RMSN_CHECK_LAYOUT)
RMSN_FWD_RES_LONG_LAYOUTS(RMSN_CHECK_LAYOUT)
RMSN_FWD_GATED_LAYOUTS(RMSN_CHECK_LAYOUT)
RMSN_BWD_LAYOUTS(RMSN_CHECK_LAYOUT)
#undef RMSN_CHECK_LAYOUT

// The backward adds its row groups' FP64 column sums through LDS, one row
// of H doubles per wavefront (per row group when a row group spans
// wavefronts): at most (256 / min(LPR, 64)) * H * 8 bytes when LPR < 256,
// which must stay within kMaxSlotLds.
constexpr long kMaxSlotLds = 64 * 1024;
#define RMSN_CHECK_LDS(id, mh, l, vv, uu, kk)                                                        \
    static_assert((l) >= 256 || (long)(256 / ((l) < 64 ? 64 : (l))) * (mh) * 8 <= kMaxSlotLds, \
                  "backward layout needs too much LDS");
RMSN_BWD_LAYOUTS(RMSN_CHECK_LDS)
#undef RMSN_CHECK_LDS

#define RMSN_LAYOUT_ENTRY(id, mh, l, vv, uu, kk) Layout{mh, l, vv, uu, kk},
static constexpr Layout kFwdLayouts[] = {RMSN_FWD_LAYOUTS(RMSN_LAYOUT_ENTRY)};
static constexpr Layout kFwdLongLayouts[] = {RMSN_FWD_LONG_LAYOUTS(RMSN_LAYOUT_ENTRY)};
static constexpr Layout kFwdResLongLayouts[] = {RMSN_FWD_RES_LONG_LAYOUTS(RMSN_LAYOUT_ENTRY)};
static constexpr Layout kFwdGatedLayouts[] = {RMSN_FWD_GATED_LAYOUTS(RMSN_LAYOUT_ENTRY)};
static constexpr Layout kBwdLayouts[] = {RMSN_BWD_LAYOUTS(RMSN_LAYOUT_ENTRY)};
#undef RMSN_LAYOUT_ENTRY

static constexpr int kNumFwdLayouts = sizeof(kFwdLayouts) / sizeof(kFwdLayouts[0]);
static_assert(sizeof(kFwdResLongLayouts) == sizeof(kFwdLayouts), "one residual layout per forward layout");
static_assert(sizeof(kFwdLongLayouts) == sizeof(kFwdLayouts), "one long-run layout per forward layout");
static_assert(sizeof(kFwdGatedLayouts) == sizeof(kFwdLayouts), "one gated layout per forward layout");

// Same widths, lanes and vectors per row in every forward table.
constexpr bool fwd_tables_agree(const Layout* t, int i = 0)
{
    return i == kNumFwdLayouts || (t[i].max_h == kFwdLayouts[i].max_h && t[i].lpr == kFwdLayouts[i].lpr &&
                                   t[i].v == kFwdLayouts[i].v && fwd_tables_agree(t, i + 1));
}
static_assert(fwd_tables_agree(kFwdResLongLayouts), "the residual forward keeps the plain forward's row layout");
static_assert(fwd_tables_agree(kFwdLongLayouts), "long runs keep the plain forward's row layout");

// Which forward table serves a call: the gated table for gated forwards;
// the long-run tables for plain forwards over at least kFwdLongRows rows and
// residual forwards over at least kFwdResLongRows rows; else the plain
// table, which serves the plain and residual kernels alike.
enum { FWD_PLAIN = 0, FWD_LONG = 1, FWD_RES_LONG = 2, FWD_GATED = 3 };
inline int fwd_table_kind(long long R, bool residual, bool gated)
{
    if (gated) return FWD_GATED;
    if (residual) return R >= kFwdResLongRows ? FWD_RES_LONG : FWD_PLAIN;
    return R >= kFwdLongRows ? FWD_LONG : FWD_PLAIN;
}
inline const Layout* fwd_table(int kind)
{
    return kind == FWD_GATED ? kFwdGatedLayouts
                             : (kind == FWD_RES_LONG ? kFwdResLongLayouts : (kind == FWD_LONG ? kFwdLongLayouts : kFwdLayouts));
}
static constexpr int kNumBwdLayouts = sizeof(kBwdLayouts) / sizeof(kBwdLayouts[0]);

// Workgroup size: the largest multiple of LPR not above 256, or LPR itself
// when a row spans more than 256 lanes.
constexpr int block_of(int lpr) { return lpr >= 256 ? lpr : lpr * (256 / lpr); }
constexpr int slots_of(int lpr) { return block_of(lpr) / lpr; }

// The backward's single-workgroup path (small T: one workgroup takes every
// row and writes dw itself) runs with the fewest rows per row group and
// iteration (U = 1, 2 or 4) that covers all rows in one iteration: measured
// at T 1-16, each extra iteration costs 1.3-2.5 us of cold loads in series,
// while a larger U costs 0.4-1.5 us even when its rows are not needed.
// Lanes and vectors per row stay the layout's, so every per-row sum -- and
// dx -- is the one of the multi-workgroup path.  Largest U: 4 for rows of up
// to 2 vectors per lane, 2 for 3; rows spanning more than 256 lanes keep
// the layout's U (their workgroups are too large for more registers).
#ifdef RMSN_DIRECT_U_AS_LAYOUT  // tuning builds: only the table's U
constexpr int direct_max_u(int, int, int u) { return u; }
#else
constexpr int direct_max_u(int lpr, int v, int u) { return lpr > 256 ? u : (v <= 2 ? 4 : (v == 3 ? 2 : u)); }
#endif

// Smallest layout that covers H (tables are sorted by max_h); -1 if none.
inline int pick_layout(const Layout* t, int n, long long H)
{
    for (int i = 0; i < n; ++i)
        if (H <= t[i].max_h) return i;
    return -1;
}

}  // namespace rmsn
