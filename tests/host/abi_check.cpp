// Host check of the C-ABI layer (api.cpp, route.cpp), built for the host with
// AddressSanitizer and UBSan.  The kernel launchers are replaced by stubs that
// record what they would launch, and the two HIP queries api.cpp makes are
// stubbed too, so no GPU and no HIP runtime is involved.  Pointers are
// addresses in a host array that the ABI layer never dereferences.
//
// Checked:
//   * every error path returns its status before any launch;
//   * for a sweep of shapes, the backward's workspace accesses (ticket,
//     FP64 accumulator, chunk partials) stay inside rmsnorm_bwd_workspace_size,
//     one byte less is refused, and the launch parameters are in range;
//   * the same for explicit column-form routes (slice tickets inside the
//     prepared part, row-block partials inside the workspace, the reduce
//     launched exactly for the deterministic multi-block form);
//   * rmsnorm_bwd_noalloc runs the route rmsnorm_bwd takes on the scratch,
//     refuses routes whose workspace exceeds it, and rejects bad arguments
//     before touching it;
//   * the forward grid is within [1, compute units * layout cap] and every
//     launch gets the row count and width it was given.
// Prints "ok" and exits 0, or prints the first failures and exits 1.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/rmsnorm.h"
#include "kernels.h"
#include "layouts.h"
#include "route.h"

namespace rmsn {

struct Calls {
    int fwd = 0, bwd = 0, cols = 0, cols_rows = 0, cols_col_tasks = 0, reduce = 0, fill = 0, scratch = 0;
    FwdParams fp{};
    BwdParams bp{};
    int grid = 0, layout = -1, fwd_table = -1, reduce_chunks = 0, reduce_h = 0;
    int64_t fill_bytes = 0;
    const void* fill_ptr = nullptr;
};
static Calls g;

hipError_t launch_fwd(int table, int layout, bool, const FwdParams& p, int grid, hipStream_t)
{
    ++g.fwd;
    g.fwd_table = table;
    g.fp = p;
    g.grid = grid;
    g.layout = layout;
    return hipSuccess;
}
hipError_t launch_bwd(int layout, bool, const BwdParams& p, hipStream_t)
{
    ++g.bwd;
    g.bp = p;
    g.layout = layout;
    return hipSuccess;
}
hipError_t launch_bwd_cols(int layout, bool, const BwdParams& p, bool rows, hipStream_t)
{
    ++g.cols;
    g.cols_rows += rows ? 1 : 0;
    g.cols_col_tasks += p.col_tasks;
    g.bp = p;
    g.layout = layout;
    return hipSuccess;
}
alignas(256) static char fake_scratch[64];
hipError_t scratch_region(void** out, hipStream_t)
{
    ++g.scratch;
    *out = fake_scratch;
    return hipSuccess;
}
hipError_t launch_dw_reduce(const double*, int chunks, int H, float*, hipStream_t)
{
    ++g.reduce;
    g.reduce_chunks = chunks;
    g.reduce_h = H;
    return hipSuccess;
}
hipError_t launch_fill_zero(void* ptr, int64_t bytes, hipStream_t)
{
    ++g.fill;
    g.fill_ptr = ptr;
    g.fill_bytes = bytes;
    return hipSuccess;
}

}  // namespace rmsn

// the two device queries api.cpp makes (compute-unit count for the forward grid)
extern "C" hipError_t hipGetDevice(int* d)
{
    *d = 0;
    return hipSuccess;
}
extern "C" hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int)
{
    *v = 256;
    return hipSuccess;
}

using namespace rmsn;

static long fails = 0;
#define CHECK(c, ...)                                   \
    do {                                                \
        if (!(c)) {                                     \
            if (fails < 20) {                           \
                std::printf("%s:%d: ", __FILE__, __LINE__); \
                std::printf(__VA_ARGS__);               \
                std::printf("\n");                      \
            }                                           \
            ++fails;                                    \
        }                                               \
    } while (0)

alignas(256) static char mem[16][1024];
static void* P(int i) { return mem[i]; }

static void reset() { g = Calls{}; }

static int bwd(int64_t T, int64_t heads, int64_t H, size_t ws_bytes, int det, const void* dres = nullptr,
               int64_t st = -1, int64_t sh = -1)
{
    if (sh < 0) sh = H;
    if (st < 0) st = heads * sh;
    return rmsnorm_bwd(P(0), P(1), (const float*)P(2), P(3), RMSN_W_F32, dres, P(4), (float*)P(5), P(6), ws_bytes,
                       T, heads, H, st, sh, det, nullptr);
}

static void check_error_paths()
{
    const int64_t H = 512;
    float* rstd = (float*)P(2);
    // forward
    reset();
    CHECK(rmsnorm_fwd(P(0), nullptr, P(1), RMSN_W_BF16, P(2), nullptr, rstd, 4, 1, 7, 7, 7, 1e-6, 1, nullptr) ==
              RMSN_ERR_UNSUPPORTED, "H = 7");
    CHECK(rmsnorm_fwd(P(0), nullptr, P(1), RMSN_W_BF16, P(2), nullptr, rstd, 4, 1, RMSN_MAX_H + 8, RMSN_MAX_H + 8,
                      RMSN_MAX_H + 8, 1e-6, 1, nullptr) == RMSN_ERR_UNSUPPORTED, "H too large");
    CHECK(rmsnorm_fwd(P(0), nullptr, P(1), RMSN_W_BF16, P(2), nullptr, rstd, -1, 1, H, H, H, 1e-6, 1, nullptr) ==
              RMSN_ERR_INVALID_ARG, "T < 0");
    CHECK(rmsnorm_fwd(P(0), nullptr, P(1), RMSN_W_BF16, P(2), nullptr, rstd, 4, 0, H, H, H, 1e-6, 1, nullptr) ==
              RMSN_ERR_INVALID_ARG, "heads = 0");
    CHECK(rmsnorm_fwd(P(0), nullptr, P(1), RMSN_W_BF16, P(2), nullptr, rstd, 4, 1, H, H - 8, H, 1e-6, 1, nullptr) ==
              RMSN_ERR_INVALID_ARG, "overlapping rows");
    CHECK(rmsnorm_fwd(P(0), nullptr, P(1), RMSN_W_BF16, P(2), nullptr, rstd, 4, 2, H, 2 * H - 8, H, 1e-6, 1,
                      nullptr) == RMSN_ERR_INVALID_ARG, "overlapping tokens");
    CHECK(rmsnorm_fwd(P(0), nullptr, P(1), RMSN_W_BF16, P(2), nullptr, rstd, 4, 1, H, H + 4, H, 1e-6, 1, nullptr) ==
              RMSN_ERR_MISALIGNED, "stride not a multiple of 8");
    CHECK(rmsnorm_fwd((char*)P(0) + 2, nullptr, P(1), RMSN_W_BF16, P(2), nullptr, rstd, 4, 1, H, H, H, 1e-6, 1,
                      nullptr) == RMSN_ERR_MISALIGNED, "misaligned x");
    CHECK(rmsnorm_fwd(P(0), nullptr, P(1), RMSN_W_BF16, P(2), nullptr, rstd, 4, 1, H, H, H, NAN, 1, nullptr) ==
              RMSN_ERR_INVALID_ARG, "eps NaN");
    CHECK(rmsnorm_fwd(P(0), nullptr, P(1), RMSN_W_BF16, P(2), nullptr, rstd, 4, 1, H, H, H, -1.0, 1, nullptr) ==
              RMSN_ERR_INVALID_ARG, "eps < 0");
    CHECK(rmsnorm_fwd(P(0), nullptr, P(1), 2, P(2), nullptr, rstd, 4, 1, H, H, H, 1e-6, 1, nullptr) ==
              RMSN_ERR_INVALID_ARG, "w dtype");
    CHECK(rmsnorm_fwd(P(0), P(3), P(1), RMSN_W_BF16, P(2), nullptr, rstd, 4, 1, H, H, H, 1e-6, 1, nullptr) ==
              RMSN_ERR_INVALID_ARG, "residual without residual_out");
    CHECK(rmsnorm_fwd(nullptr, nullptr, P(1), RMSN_W_BF16, P(2), nullptr, rstd, 4, 1, H, H, H, 1e-6, 1, nullptr) ==
              RMSN_ERR_INVALID_ARG, "x null");
    CHECK(rmsnorm_fwd(P(0), nullptr, P(1), RMSN_W_BF16, P(2), nullptr, rstd, INT64_MAX, 1, H, H, H, 1e-6, 1,
                      nullptr) == RMSN_ERR_INVALID_ARG, "T huge");
    CHECK(rmsnorm_fwd(P(0), nullptr, P(1), RMSN_W_BF16, P(2), nullptr, rstd, INT64_MAX / 2, 4, H, 4 * H, H, 1e-6, 1,
                      nullptr) == RMSN_ERR_INVALID_ARG, "T * heads overflows");
    CHECK(rmsnorm_fwd(P(0), nullptr, P(1), RMSN_W_BF16, P(2), nullptr, rstd, int64_t(1) << 30, 1, H, H, H, 1e-6, 1,
                      nullptr) == RMSN_ERR_INVALID_ARG, "R = 2^30");
    CHECK(rmsnorm_gated_fwd(P(0), nullptr, P(1), RMSN_W_BF16, P(2), rstd, 4, 1, H, H, H, 1e-6, 1, nullptr) ==
              RMSN_ERR_INVALID_ARG, "gate null");
    CHECK(rmsnorm_gated_fwd(P(0), (char*)P(3) + 8, P(1), RMSN_W_BF16, P(2), rstd, 4, 1, H, H, H, 1e-6, 1,
                            nullptr) == RMSN_ERR_MISALIGNED, "gate misaligned");
    CHECK(g.fwd == 0, "a rejected forward launched");

    // backward
    const size_t ws = rmsnorm_bwd_workspace_size(64, 1, H, RMSN_W_F32, nullptr, 1);
    rmsn_route rt64{};
    CHECK(rmsnorm_bwd_route(64, 1, H, RMSN_W_F32, 0, 1, &rt64) == RMSN_OK, "route query");
    reset();
    CHECK(bwd(64, 1, H, rmsnorm_bwd_workspace_size_for_route(64, 1, H, rt64) - 1, 1) == RMSN_ERR_WORKSPACE,
          "workspace one byte short");
    CHECK(rmsnorm_bwd(P(0), P(1), (const float*)P(2), P(3), RMSN_W_F32, nullptr, P(4), (float*)P(5),
                      (char*)P(6) + 128, ws, 64, 1, H, H, H, 1, nullptr) == RMSN_ERR_MISALIGNED,
          "workspace misaligned");
    CHECK(rmsnorm_bwd(P(0), P(1), (const float*)P(2), P(3), RMSN_W_F32, nullptr, P(4), nullptr, P(6), ws, 64, 1, H,
                      H, H, 1, nullptr) == RMSN_ERR_INVALID_ARG, "dw null");
    CHECK(rmsnorm_bwd(P(0), P(1), (const float*)((char*)P(2) + 2), P(3), RMSN_W_F32, nullptr, P(4), (float*)P(5),
                      P(6), ws, 64, 1, H, H, H, 1, nullptr) == RMSN_ERR_MISALIGNED, "rstd misaligned");
    CHECK(rmsnorm_bwd(P(0), P(1), (const float*)P(2), P(3), RMSN_W_F32, (char*)P(7) + 8, P(4), (float*)P(5), P(6),
                      ws, 64, 1, H, H, H, 1, nullptr) == RMSN_ERR_MISALIGNED, "dres misaligned");
    const rmsn_route atomic{RMSN_FORM_ATOMIC, 8, 0, 0}, zero{RMSN_FORM_PAIR, 0, 0, 0},
        many{RMSN_FORM_PAIR, 65537, 0, 0}, bad_form{7, 8, 0, 0}, pair_cols{RMSN_FORM_PAIR, 8, 1, 8},
        cols_zero{RMSN_FORM_COLS, 8, 0, 8}, cols_many{RMSN_FORM_COLS, 8, 4097, 8}, cols_v3{RMSN_FORM_COLS, 8, 1, 3},
        cols_v16{RMSN_FORM_COLS, 8, 1, 16}, ticket_one{RMSN_FORM_COLS_TICKET, 8, 1, 8},
        ticket{RMSN_FORM_COLS_TICKET, 8, 4, 8};
    for (const rmsn_route& r : {zero, many, bad_form, pair_cols, cols_zero, cols_many, cols_v3, cols_v16, ticket_one})
        CHECK(rmsnorm_bwd_routed(P(0), P(1), (const float*)P(2), P(3), RMSN_W_F32, nullptr, P(4), (float*)P(5), P(6),
                                 ws, 64, 1, H, H, H, 0, r, nullptr) == RMSN_ERR_INVALID_ARG,
              "route (%d, %d, %d, %d)", r.form, r.chunks, r.col_chunks, r.col_vecs);
    for (const rmsn_route& r : {atomic, ticket})
        CHECK(rmsnorm_bwd_routed(P(0), P(1), (const float*)P(2), P(3), RMSN_W_F32, nullptr, P(4), (float*)P(5), P(6),
                                 ws, 64, 1, H, H, H, 1, r, nullptr) == RMSN_ERR_INVALID_ARG,
              "deterministic route of form %d", r.form);
    CHECK(rmsnorm_gated_bwd(P(0), P(1), nullptr, (const float*)P(2), P(3), RMSN_W_F32, P(4), P(7), (float*)P(5),
                            P(6), ws, 64, 1, H, H, H, 1, nullptr) == RMSN_ERR_INVALID_ARG, "gate null");
    CHECK(rmsnorm_gated_bwd(P(0), P(1), P(8), (const float*)P(2), P(3), RMSN_W_F32, P(4), (char*)P(7) + 4,
                            (float*)P(5), P(6), ws, 64, 1, H, H, H, 1, nullptr) == RMSN_ERR_MISALIGNED,
          "dgate misaligned");
    CHECK(rmsnorm_bwd_workspace_init(P(6), ws, 12, nullptr) == RMSN_ERR_INVALID_ARG, "init H = 12");
    CHECK(rmsnorm_bwd_workspace_init(P(6), 100, H, nullptr) == RMSN_ERR_WORKSPACE, "init too small");
    // the allocation-free backward: argument errors before the scratch is looked up
    CHECK(rmsnorm_bwd_noalloc(P(0), P(1), (const float*)P(2), P(3), RMSN_W_F32, nullptr, P(4), nullptr, 64, 1, H, H,
                              H, 1, nullptr) == RMSN_ERR_INVALID_ARG, "noalloc dw null");
    CHECK(rmsnorm_bwd_noalloc(P(0), P(1), (const float*)P(2), P(3), 3, nullptr, P(4), (float*)P(5), 64, 1, H, H, H,
                              1, nullptr) == RMSN_ERR_INVALID_ARG, "noalloc w dtype");
    CHECK(rmsnorm_bwd_noalloc((char*)P(0) + 2, P(1), (const float*)P(2), P(3), RMSN_W_F32, nullptr, P(4),
                              (float*)P(5), 64, 1, H, H, H, 1, nullptr) == RMSN_ERR_MISALIGNED, "noalloc dy misaligned");
    CHECK(rmsnorm_bwd_noalloc(P(0), P(1), (const float*)P(2), P(3), RMSN_W_F32, nullptr, P(4), (float*)P(5), 65536,
                              1, 16384, 16384, 16384, 1, nullptr) == RMSN_ERR_WORKSPACE,
          "noalloc route beyond the scratch");
    CHECK(g.bwd == 0 && g.cols == 0 && g.reduce == 0 && g.fill == 0 && g.scratch == 0,
          "a rejected backward launched or touched the scratch");
    CHECK(rmsnorm_bwd_workspace_size(4, 1, 12, RMSN_W_BF16, nullptr, 1) == 0 &&
              rmsnorm_bwd_workspace_size(-1, 1, H, RMSN_W_BF16, nullptr, 1) == 0 &&
              rmsnorm_bwd_workspace_size(int64_t(1) << 30, 1, H, RMSN_W_BF16, nullptr, 1) == 0 &&
              rmsnorm_bwd_workspace_size(4, 1, H, 2, nullptr, 1) == 0,
          "workspace size of an invalid shape or dtype is not 0");

    // R = 0: the backward zero-fills dw and launches nothing else
    reset();
    CHECK(bwd(0, 1, H, 0, 1) == RMSN_OK && g.fill == 1 && g.fill_bytes == H * 4 && g.bwd == 0,
          "R = 0 backward");
    reset();
    CHECK(rmsnorm_fwd(P(0), nullptr, P(1), RMSN_W_BF16, P(2), nullptr, rstd, 0, 1, H, H, H, 1e-6, 1, nullptr) ==
              RMSN_OK && g.fwd == 0, "R = 0 forward");

    for (int s = -1; s <= 6; ++s) CHECK(rmsnorm_status_string(s) != nullptr, "status string %d", s);
}

// Where the workspace accesses of the launch just recorded fall, for a
// workspace of ws bytes at `base`: every one inside it.
static void check_ws_accesses(const char* base, size_t ws, int64_t H, int form, const char* what)
{
    const BwdParams& p = g.bp;
    CHECK((const char*)p.ticket == base && (const char*)p.acc >= base + sizeof(unsigned),
          "%s: ticket/accumulator placement", what);
    CHECK((size_t)((const char*)p.acc - base) + (size_t)H * 8 <= (size_t)((const char*)p.slice_ticket - base),
          "%s: accumulator runs into the slice tickets", what);
    CHECK((size_t)((const char*)p.acc - base) % 8 == 0 && (size_t)((const char*)p.part - base) % 16 == 0 &&
              (size_t)((const char*)p.slice_ticket - base) % 4 == 0,
          "%s: workspace alignment", what);
    CHECK((size_t)((const char*)p.part - base) <= ws, "%s: partials start past the workspace", what);
    if (form == FORM_PAIR && p.chunks > 1)
        CHECK((size_t)((const char*)p.part - base) + (size_t)p.chunks * H * 8 <= ws,
              "%s: pair partials past the workspace (chunks %d)", what, p.chunks);
    if (form == FORM_COLS || form == FORM_COLS_TICKET) {
        CHECK(p.slices == (int)col_slices(H, p.col_vecs) && (int64_t)p.slices * p.col_vecs * 8 >= H &&
                  (int64_t)(p.slices - 1) * p.col_vecs * 8 < H,
              "%s: slices %d for H %lld", what, p.slices, (long long)H);
        CHECK((size_t)((const char*)p.slice_ticket - base) + (size_t)p.slices * sizeof(unsigned) <=
                  (size_t)((const char*)p.part - base),
              "%s: slice tickets run into the partials", what);
        if (p.col_chunks > 1)
            CHECK((size_t)((const char*)p.part - base) + (size_t)p.col_chunks * H * 8 <= ws,
                  "%s: row-block partials past the workspace (col_chunks %d)", what, p.col_chunks);
    }
}

// One backward call at (T, heads, H) in both modes, both weight dtypes,
// with and without dres: bounds of every workspace access, launch
// parameters, and the one-byte-short refusal.
static void check_backward_shape(int64_t T, int64_t heads, int64_t H)
{
    const int64_t R = T * heads;
    for (int det = 0; det <= 1; ++det)
        for (int wd = 0; wd <= 1; ++wd)
            for (int res = 0; res <= 1; ++res) {
                const void* dres = res ? P(7) : nullptr;
                const size_t ws = rmsnorm_bwd_workspace_size(T, heads, H, wd, dres, det);
                CHECK(ws > 0, "workspace size 0 for T=%lld heads=%lld H=%lld", (long long)T, (long long)heads,
                      (long long)H);
                rmsn_route rt{};
                CHECK(rmsnorm_bwd_route(T, heads, H, wd, res, det, &rt) == RMSN_OK, "route query");
                const size_t own = rmsnorm_bwd_workspace_size_for_route(T, heads, H, rt);
                CHECK(ws >= own && (res == 0 || ws == own), "size of the route");
                CHECK(!det || rt.form == RMSN_FORM_PAIR || rt.form == RMSN_FORM_COLS, "deterministic route form");
                reset();
                const int64_t sh = H, st = heads * sh;
                const int st_ = rmsnorm_bwd(P(0), P(1), (const float*)P(2), P(3), wd, dres, P(4), (float*)P(5), P(6),
                                            ws, T, heads, H, st, sh, det, nullptr);
                CHECK(st_ == RMSN_OK, "status %d for T=%lld heads=%lld H=%lld", st_, (long long)T, (long long)heads,
                      (long long)H);
                if (st_ != RMSN_OK || R == 0) continue;
                const BwdParams& p = g.bp;
                CHECK(g.bwd + g.cols == 1 && p.R == R && p.H == H, "launch R/H");
                CHECK(g.cols == 0 || (g.cols_rows == 1 && p.col_tasks == p.slices * p.col_chunks),
                      "one column-form launch holds the column and the row tasks");
                CHECK(p.chunks >= 1 && p.chunks <= kMaxChunks, "chunks %d", p.chunks);
                CHECK(p.form == rt.form && p.chunks == rt.chunks && p.prefetch == rt.prefetch,
                      "launch follows the route");
                CHECK(rt.prefetch == 0 || rt.prefetch == 1, "prefetch flag");
                check_ws_accesses((const char*)P(6), ws, H, p.form, "rmsnorm_bwd");
                if (p.form == FORM_PAIR && p.chunks > 1)
                    CHECK(!p.direct_dw && g.reduce == 1 && g.reduce_chunks == p.chunks && g.reduce_h == H,
                          "pair launches its reduce");
                if (p.form == FORM_PAIR && p.chunks == 1) CHECK(p.direct_dw && g.reduce == 0, "one chunk writes dw");
                reset();
                const size_t need = rmsnorm_bwd_workspace_size_for_route(T, heads, H, rt);
                CHECK(rmsnorm_bwd(P(0), P(1), (const float*)P(2), P(3), wd, dres, P(4), (float*)P(5), P(6), need - 1,
                                  T, heads, H, st, sh, det, nullptr) == RMSN_ERR_WORKSPACE &&
                          g.bwd + g.cols == 0,
                      "a workspace one byte short of the route's is refused");
                // in place (dx = dy): the same route; a column form runs its
                // column tasks alone, then its row tasks alone
                reset();
                CHECK(rmsnorm_bwd(P(0), P(1), (const float*)P(2), P(3), wd, dres, P(0), (float*)P(5), P(6), ws, T,
                                  heads, H, st, sh, det, nullptr) == RMSN_OK && g.bp.form == rt.form,
                      "an in-place backward");
                if (rt.form == RMSN_FORM_COLS)
                    CHECK(g.cols == 2 && g.cols_rows == 1 && g.bp.col_tasks == 0 &&
                              g.cols_col_tasks == (int)col_slices(H, rt.col_vecs) * rt.col_chunks,
                          "in place, the column tasks run before the row tasks, in launches of their own");
                else
                    CHECK(g.bwd == 1 && g.cols == 0, "in place, the row kernel");
                check_ws_accesses((const char*)P(6), ws, H, rt.form, "in place");
                // the allocation-free entry point takes the same route on the scratch
                reset();
                const int sn = rmsnorm_bwd_noalloc(P(0), P(1), (const float*)P(2), P(3), wd, dres, P(4), (float*)P(5),
                                                   T, heads, H, st, sh, det, nullptr);
                if (own <= kScratchBytes) {
                    CHECK(sn == RMSN_OK && g.scratch == 1 && g.bwd + g.cols == 1 && g.bp.form == rt.form &&
                              g.bp.chunks == rt.chunks && (const char*)g.bp.ticket == fake_scratch,
                          "noalloc runs the route on the scratch (status %d)", sn);
                } else {
                    CHECK(sn == RMSN_ERR_WORKSPACE && g.bwd + g.cols == 0 && g.scratch == 0,
                          "noalloc refuses a route beyond the scratch");
                }
                // the size query without dres also serves the gated backward
                if (res == 0) {
                    reset();
                    const int sg = rmsnorm_gated_bwd(P(0), P(1), P(8), (const float*)P(2), P(3), wd, P(4), P(7),
                                                     (float*)P(5), P(6), ws, T, heads, H, st, sh, det, nullptr);
                    rmsn_route gr{};
                    CHECK(rmsnorm_gated_bwd_route(T, heads, H, wd, det, &gr) == RMSN_OK && gr.prefetch == 0 &&
                              rmsnorm_bwd_workspace_size_for_route(T, heads, H, gr) <= ws,
                          "gated route query");
                    CHECK(sg == RMSN_OK && g.bwd + g.cols >= 1 && g.bp.prefetch == 0 && g.bp.form == gr.form &&
                              g.bp.chunks == gr.chunks,
                          "gated backward on the size query's workspace follows its route (status %d)", sg);
                    check_ws_accesses((const char*)P(6), ws, H, g.bp.form, "gated");
                }
            }
}

// Explicit column-form routes: launch parameters and workspace bounds.
static void check_column_routes(int64_t T, int64_t H)
{
    for (int form : {RMSN_FORM_COLS, RMSN_FORM_COLS_TICKET})
        for (int vecs : {1, 2, 4, 8})
            for (int cc : {1, 2, 3, 16, 4096}) {
                if (form == RMSN_FORM_COLS_TICKET && cc < 2) continue;
                const rmsn_route r{form, 37, cc, vecs};
                const size_t ws = rmsnorm_bwd_workspace_size_for_route(T, 1, H, r);
                CHECK(ws >= ws_part_offset(H), "column route workspace");
                reset();
                const int det = form == RMSN_FORM_COLS;
                const int st = rmsnorm_bwd_routed(P(0), P(1), (const float*)P(2), P(3), RMSN_W_BF16, nullptr, P(4),
                                                  (float*)P(5), P(6), ws, T, 1, H, H, H, det, r, nullptr);
                CHECK(st == RMSN_OK, "column route status %d", st);
                if (st != RMSN_OK || T == 0) continue;
                CHECK(g.cols == 1 && g.bwd == 0 && g.bp.col_chunks == cc && g.bp.col_vecs == vecs && g.bp.chunks == 37,
                      "column launch parameters");
                CHECK(g.reduce == (form == RMSN_FORM_COLS && cc > 1 ? 1 : 0) && (g.reduce == 0 || g.reduce_chunks == cc),
                      "reduce launch of the column form");
                check_ws_accesses((const char*)P(6), ws, H, form, "column route");
                reset();
                CHECK(rmsnorm_bwd_routed(P(0), P(1), (const float*)P(2), P(3), RMSN_W_BF16, nullptr, P(4),
                                         (float*)P(5), P(6), ws - 1, T, 1, H, H, H, det, r, nullptr) ==
                          RMSN_ERR_WORKSPACE,
                      "column route one byte short");
            }
}

static void check_forward_shape(int64_t T, int64_t heads, int64_t H, bool residual)
{
    reset();
    const int st = rmsnorm_fwd(P(0), residual ? P(4) : nullptr, P(1), RMSN_W_BF16, P(2), residual ? P(5) : nullptr,
                               (float*)P(3), T, heads, H, heads * H, H, 1e-6, 1, nullptr);
    CHECK(st == RMSN_OK, "forward status %d", st);
    if (T * heads == 0) return;
    const int64_t R = T * heads;
    const int kind = residual ? (R >= kFwdResLongRows ? FWD_RES_LONG : FWD_PLAIN)
                              : (R >= kFwdLongRows ? FWD_LONG : FWD_PLAIN);
    CHECK(g.fwd_table == kind, "forward table %d for R=%lld", g.fwd_table, (long long)(T * heads));
    const Layout* table = fwd_table(kind);
    const Layout& L = table[g.layout];
    CHECK(H <= L.max_h && (g.layout == 0 || H > table[g.layout - 1].max_h), "forward layout for H=%lld",
          (long long)H);
    CHECK(g.grid >= 1 && g.grid <= 256 * L.k, "forward grid %d", g.grid);
    CHECK(g.fp.R == T * heads && g.fp.H == H, "forward R/H");
    CHECK((g.fp.r != nullptr) == residual && (g.fp.h != nullptr) == residual, "forward residual pointers");
}

// The gated forward always takes its own table, whatever the row count.
static void check_gated_forward_table()
{
    const int64_t Ts[] = {1, 32768, 65535, 65536, 131072};
    for (int64_t T : Ts) {
        reset();
        const int st = rmsnorm_gated_fwd(P(0), P(4), P(1), RMSN_W_BF16, P(2), (float*)P(3), T, 1, 4096, 4096, 4096,
                                         1e-6, 1, nullptr);
        CHECK(st == RMSN_OK && g.fwd == 1 && g.fwd_table == FWD_GATED && g.fp.g != nullptr,
              "gated forward table for T=%lld", (long long)T);
    }
}

// Explicit row-kernel routes with and without the next-row tile: the flag
// reaches the launch; a column form refuses it.
static void check_prefetch_routes()
{
    const int64_t T = 4099, H = 1536;
    for (int form : {RMSN_FORM_PAIR, RMSN_FORM_ATOMIC})
        for (int pf : {0, 1}) {
            const rmsn_route r{form, 256, 0, 0, pf};
            const size_t ws = rmsnorm_bwd_workspace_size_for_route(T, 1, H, r);
            reset();
            const int st = rmsnorm_bwd_routed(P(0), P(1), (const float*)P(2), P(3), RMSN_W_BF16, nullptr, P(4),
                                              (float*)P(5), P(6), ws, T, 1, H, H, H, form == RMSN_FORM_PAIR, r, nullptr);
            CHECK(st == RMSN_OK && g.bwd == 1 && g.bp.prefetch == pf && g.bp.chunks == 256, "prefetch route launch");
        }
    const rmsn_route bad{RMSN_FORM_COLS, 8, 2, 8, 1};
    CHECK(rmsnorm_bwd_workspace_size_for_route(T, 1, H, bad) == 0, "column form with prefetch has no size");
    CHECK(rmsnorm_bwd_routed(P(0), P(1), (const float*)P(2), P(3), RMSN_W_BF16, nullptr, P(4), (float*)P(5), P(6),
                             size_t(1) << 30, T, 1, H, H, H, 1, bad, nullptr) == RMSN_ERR_INVALID_ARG,
          "column form refuses prefetch");
}

int main()
{
    check_error_paths();
    check_prefetch_routes();
    check_gated_forward_table();
    const int64_t Ts[] = {1, 2, 3, 4, 5, 7, 16, 63, 64, 65, 255, 256, 257, 1000, 1024, 4096, 4099,
                          16384, 32767, 32768, 65535, 65536, 131072, 1 << 20, (int64_t(1) << 30) - 1};
    for (int64_t H : {int64_t(8), int64_t(64), int64_t(72), int64_t(1536), int64_t(6144), int64_t(16384)})
        for (int64_t T : {int64_t(1), int64_t(5), int64_t(4099)}) check_column_routes(T, H);
    for (int64_t H = 8; H <= RMSN_MAX_H; H += (H < 1024 ? 8 : (H < 8192 ? 72 : 520))) {
        for (int64_t T : Ts) {
            check_backward_shape(T, 1, H);
            check_forward_shape(T, 1, H, false);
            check_forward_shape(T, 1, H, true);
        }
    }
    for (int64_t H : {int64_t(8), int64_t(256), int64_t(1536), int64_t(4096), int64_t(6144), int64_t(16384)})
        for (int64_t heads : {int64_t(2), int64_t(3), int64_t(24), int64_t(1000)})
            for (int64_t T : {int64_t(1), int64_t(5), int64_t(4097), int64_t(32768), ((int64_t(1) << 30) - 1) / 1000}) {
                if (T * heads >= (int64_t(1) << 30)) continue;
                check_backward_shape(T, heads, H);
                check_forward_shape(T, heads, H, false);
                check_forward_shape(T, heads, H, true);
            }
    if (fails) {
        std::printf("%ld failures\n", fails);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
