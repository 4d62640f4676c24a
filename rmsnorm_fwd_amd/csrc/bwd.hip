// bwd.hip -- backward kernels of the training RMSNorm on gfx950.
//
//   xhat = u * rstd,  c = mean(xhat * w * dy)
//   dx   = bf16(rstd * (w * dy - xhat * c) [+ dres])
//   dw   = sum over rows of dy * xhat
// (FlashInfer training-RMSNorm pages: p1 #8577 opening paragraph; the dw
// reference is an FP64 evaluation that takes the kernel's FP32 rstd, p1
// #8208 commit message.)
//
// Row kernel.  Workgroup c of `chunks` takes every chunks-th group of rows
// (its "chunk"); a row group of LPR lanes owns a row, each lane V 16-byte
// vectors of it.  Per element:
// p = x*dy is exact in FP32 (two 8-bit significands) and is widened to FP64;
// p*w (<= 24 + 16 bits) and p*rstd (24 + 16 bits) are exact in FP64, so the
// row dot S = sum(x*w*dy) and the dw column sums round only in their FP64
// additions.  dx = rstd*(w*dy) - x*(rstd^3 S / H) is formed in FP64 and
// rounded to FP32, then BF16 (within one BF16 unit of the exact value).  The
// row dot's order depends only on H, so dx is the same in both modes and for
// every chunking.  The weights live in registers as FP64 (0 for vectors a
// lane does not own); rows wider than 8192 keep them as loaded and widen
// each where it is used.
//
// Loads.  A workgroup loads an iteration's rows (x or h, dy, rstd, and dres
// or the gate) before it uses any of them.  With the next-row tile (a route
// choice for plain rows, always for gated rows up to H 8192) it loads the
// next iteration's rows while it works on the current ones; the order of
// its waits on the memory counter, which also counts stores, is chosen per
// kernel (BwdTile): the tile needs them to leave the next rows' loads in
// flight, full-occupancy rows are faster when each wait drains the
// wavefront's earlier stores first.  None of this changes a result bit.
//
// dw.  Each lane keeps FP64 column sums over the chunk's rows in registers;
// row groups of one workgroup are added by lane exchanges inside a
// wavefront, then across wavefronts through LDS, in a fixed order.  With a
// single chunk that sum is dw and is written directly; otherwise the chunk
// sum goes
//   pair form:   to row `chunk` of a workspace [chunks, H] (FP64), summed by
//                dw_reduce_kernel in a fixed order -- deterministic;
//   atomic form: into an FP64 [H] accumulator by atomic add; the workgroup
//                that draws the last arrival ticket writes dw and zeroes the
//                accumulator and ticket -- one launch, no waiting.
//
// Column forms (bwd_cols_kernel).  dw needs no row dot: dw_j = sum over rows
// of dy_j * u_j * rstd, all three inputs of the backward.  So one launch runs
// two kinds of workgroup side by side: row tasks form dx (the row kernel's
// per-row work, without column sums) and column tasks form dw for a slice of
// 8 * col_vecs columns, reading that slice of every row (or of a block of
// rows) again.  No workgroup waits for another and no partial leaves the
// chip when one column task covers all rows of its slice; with col_chunks
// row blocks per slice the blocks' FP64 partials are summed in a fixed
// order, by the reduce kernel or by the slice's last-arriving column task.
//
// SiLU gate (GATE).  With a gate g the gradient reaching the normalised row
// is e = dy * silu(g).  silu is an FP32 evaluation (relative error up to
// ~2^-22), so the gated arithmetic does not keep the plain path's exact
// products: x*dy*silu(g) is rounded once in FP32 before it joins the FP64
// row and column sums, and dx = rstd*(w*e) - x*L and dg = dy * (xhat * w) *
// silu'(g) are formed in FP32; every one of these roundings stays inside the
// bound silu's error sets (the tolerance the tests derive).
#include <atomic>
#include <mutex>
#include <type_traits>

#include "../../include/rmsnorm.h"
#include "device_common.h"
#include "kernels.h"
#include "route.h"

namespace rmsn {

// ------------------------------------------------ fixed-order dw reduce ----
// dw[col] = sum over chunks of part[chunk][col], in one fixed order: lane
// group q (of 16) sums chunks q, q+16, q+32, ... in that order, 16 loads in
// flight (missing chunks add +0.0), and the 16 group sums are added in q
// order.  The order depends only on the chunk count.
constexpr int kReduceCols = 16;
constexpr int kReduceGroups = 16;

__device__ __forceinline__ double chunk_group_sum(const double* part, int chunks, int H, int col, int q)
{
    constexpr int DEPTH = 16;
    double s = 0.0;
    for (int k = q; k < chunks; k += DEPTH * kReduceGroups) {
        double a[DEPTH];
#pragma unroll
        for (int i = 0; i < DEPTH; ++i) {
            const int kk = k + i * kReduceGroups;
            a[i] = kk < chunks ? part[(int64_t)kk * H + col] : 0.0;
        }
#pragma unroll
        for (int i = 0; i < DEPTH; ++i) s += a[i];
    }
    return s;
}

// One iteration's rows of a row group: addresses, rstd and the x / dy (and
// dres, or the gate g) vectors, all loaded before any of them is used.
// DRES and GATE never meet.
//
// rstd, three ways (one memory counter covers loads and stores, and a wait
// on it drains everything issued before):
//   DEFER    loaded unconditionally (rr is in range) and widened and masked
//            only where it is used, so nothing in the load waits and the
//            rows' other loads go out behind it at once;
//   PER_ROW  masked and widened as each row's value arrives, a wait per row,
//            each of which also drains the wavefront's earlier stores;
//   else     all U rows' values loaded, one wait, then widened and masked.
// The waits that drain the stores before a row's loads go out are faster
// where rows stream at full occupancy (each wavefront's reads and writes
// stay in separate phases: T 131072, H 6144: 738 against 865 us deferred),
// one wait for all rows is 1-2 % faster than one per row at most widths,
// and DEFER is faster where few wavefronts share a compute unit and the
// next-row tile is in use (T 4096, H 1536: 18.0 -> 16.8 us; gated T 16384,
// H 3072: 169 -> 110 us).
template <int U, int V, bool DRES, bool GATE, bool DEFER>
struct BwdTile {
    bool ok[U];
    int64_t off[U];
    typename std::conditional<DEFER, float, double>::type rho[U];
    uint4 xv[U][V], dv[U][V];
    uint4 rv[(DRES || GATE) ? U : 1][(DRES || GATE) ? V : 1];
};

template <int U, int V, int SLOTS, bool DRES, bool GATE, bool DEFER, bool PER_ROW>
__device__ __forceinline__ void bwd_load(BwdTile<U, V, DRES, GATE, DEFER>& t, const BwdParams& p,
                                         const LaneVectors<V>& lv, int base, int slot, int row1)
{
    float rf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int row = base + u * SLOTS + slot;
        t.ok[u] = row < row1;
        const int rr = t.ok[u] ? row : row1 - 1;  // rows past the end re-read the last row
        t.off[u] = row_offset(rr, p.rows);
        if constexpr (DEFER) t.rho[u] = p.rstd[rr];
        else if constexpr (PER_ROW) t.rho[u] = t.ok[u] ? (double)p.rstd[rr] : 0.0;  // ... and add nothing to dw
        else rf[u] = p.rstd[rr];
    }
    if constexpr (!DEFER && !PER_ROW) {
        // one wait for all U rows' rstd (not one per row), which also drains
        // the wavefront's earlier stores before the rows' loads go out
        __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
        for (int u = 0; u < U; ++u) t.rho[u] = t.ok[u] ? (double)rf[u] : 0.0;  // ... rows past the end add nothing
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int v = 0; v < V; ++v) {
            t.xv[u][v] = ld16_stream(p.x + t.off[u] + lv.col[v]);
            t.dv[u][v] = ld16_stream(p.dy + t.off[u] + lv.col[v]);
            if constexpr (DRES) t.rv[u][v] = ld16_stream(p.dres + t.off[u] + lv.col[v]);
            if constexpr (GATE) t.rv[u][v] = ld16_stream(p.g + t.off[u] + lv.col[v]);
        }
}

// The row work of workgroup `chunk` of `nchunks`: row groups chunk,
// chunk + nchunks, ... (interleaved, so that at any moment all workgroups
// stream neighbouring rows, which keeps the HBM pages they touch together --
// measured 1.1-1.25x over contiguous chunks of rows on MI355X).  Writes dx
// (and dg) for those rows; with DW it also adds each row's dy * xhat into
// the lane's column sums acc (which it first sets to zero).
template <int LPR, int V, int U, bool WF32, bool DRES, bool GATE, bool DW, bool PFP = false>
__device__ __forceinline__ void bwd_rows(const BwdParams& p, int chunk, int nchunks, double (&acc)[V][8])
{
    constexpr int BLOCK = block_of(LPR);
    constexpr int SLOTS = BLOCK / LPR;
    constexpr int W = LPR > 64 ? LPR / 64 : 1;
    constexpr int RPI = SLOTS * U;
    __shared__ double red[2][RPI][W];

    const int tid = threadIdx.x;
    const int g = tid % LPR;
    const int slot = tid / LPR;
    const LaneVectors<V> lv(g, LPR, p.H >> 3);
    const int first = chunk * RPI;
    const int step = nchunks * RPI;
    const int row1 = p.R;

    // weights as loaded (FP32: two float4 per vector; BF16: one uint4 in wa)
    float4 wa[V], wb[WF32 ? V : 1];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        if constexpr (WF32) {
            const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p.w) + lv.col[v]);
            wa[v] = q[0];
            wb[v] = q[1];
        } else {
            const uint4 r = ld16(static_cast<const uint16_t*>(p.w) + lv.col[v]);
            wa[v] = *reinterpret_cast<const float4*>(&r);
        }
    }
    if constexpr (DW) {
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[v][e] = 0.0;
    }

    // With PF the workgroup loads its next rows while the current ones are
    // reduced (a second register tile), the first rows before the weights
    // are widened.  Gated rows always do, up to H 8192: their arithmetic per
    // element is long and one or two workgroups fill a compute unit, so no
    // other wavefront covers the load latency (gated T 65536, H 4096: 509 ->
    // 467 us with the tile, although its two-vector rows drop to one
    // wavefront per SIMD; wider gated rows would spill).  Plain rows do when
    // the route asks (PFP): where each compute unit holds few workgroups, as
    // at a few thousand rows.  Results do not depend on it.
    constexpr bool PF = GATE ? LPR * V * 8 <= 8192 : PFP;
    // see BwdTile: with the tile, no dres (the column forms' plain row
    // tasks, one or a few iterations each beside the column tasks, measured
    // 1-2 % slower deferred: T 449, H 6144: 12.15 -> 12.43 us)
    constexpr bool DEFER = PF && !DRES;
    // Without DEFER the row kernel waits once for an iteration's rstd
    // values; the workgroup-wide rows of two per iteration (H 4096) and the
    // column forms' row tasks keep one wait per row (1 % faster there: T
    // 65536, H 4096: 266.4 against 267.8 us; T 449, H 6144: 12.3 against
    // 12.5 us), where the other row kernels gain 1-2 % from one wait.
    constexpr bool PER_ROW = !DEFER && ((U > 1 && SLOTS == 1) || !DW);
    using Tile = BwdTile<U, V, DRES, GATE, DEFER>;
    Tile cur;
    BwdTile<PF ? U : 1, PF ? V : 1, DRES, GATE, DEFER> nxt;
    if constexpr (PF) {
        if (first < row1) bwd_load<U, V, SLOTS, DRES, GATE, DEFER, PER_ROW>(cur, p, lv, first, slot, row1);
    }
    // The weights in FP64 registers, 0 for vectors a lane does not own; rows
    // wider than 8192 (four or more vectors per lane) keep them as loaded
    // and widen each one where it is used, since FP64 copies would not fit
    // the registers a lane has beside its column sums.
    constexpr bool WRAW = LPR * V * 8 > 8192;
    double w64[WRAW ? 1 : V][8];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        if constexpr (WRAW) {
            if (!lv.ok[v]) wa[v] = wb[WF32 ? v : 0] = make_float4(0.f, 0.f, 0.f, 0.f);
        } else {
            float wv[8];
            if constexpr (WF32) {
                wv[0] = wa[v].x; wv[1] = wa[v].y; wv[2] = wa[v].z; wv[3] = wa[v].w;
                wv[4] = wb[v].x; wv[5] = wb[v].y; wv[6] = wb[v].z; wv[7] = wb[v].w;
            } else {
                unpack8(*reinterpret_cast<const uint4*>(&wa[v]), wv);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) w64[v][e] = lv.ok[v] ? (double)wv[e] : 0.0;
        }
    }
    // weight e of vector v, as FP32 (exact for BF16 and FP32 weights)
    auto wf32 = [&](int v, int e) -> float {
        if constexpr (!WRAW) {
            return (float)w64[v][e];
        } else if constexpr (WF32) {
            const float4& q = e < 4 ? wa[v] : wb[v];
            const int k = e & 3;
            return k == 0 ? q.x : k == 1 ? q.y : k == 2 ? q.z : q.w;
        } else {
            const float4& q = wa[v];
            const int k = e >> 1;
            const unsigned word = __float_as_uint(k == 0 ? q.x : k == 1 ? q.y : k == 2 ? q.z : q.w);
            return __uint_as_float((e & 1) ? (word & 0xffff0000u) : (word << 16));
        }
    };
    auto wf64 = [&](int v, int e) -> double {
        if constexpr (WRAW) return (double)wf32(v, e);
        else return w64[v][e];
    };
    // The work on one iteration's rows, already loaded into t.
    auto work = [&](Tile& t, int it) {
        const bool* ok = t.ok;
        const int64_t* off = t.off;
        // rstd in FP64; rows past the end add nothing to dw
        double rho_d[DEFER ? U : 1];
        const double* rho;
        if constexpr (DEFER) {
#pragma unroll
            for (int u = 0; u < U; ++u) rho_d[u] = ok[u] ? (double)t.rho[u] : 0.0;
            rho = rho_d;
        } else {
            rho = t.rho;
        }
        uint4 (&xv)[U][V] = t.xv;
        uint4 (&dv)[U][V] = t.dv;
        double S[U];
        // Gated rows take sigmoid(g) eight values at a time (sigmoid8) in
        // the first pass and keep it for the second, up to H 4096 and in
        // the one-vector rows of 768 lanes (H 5120, 6144).  The two-vector
        // rows of 512 lanes and more (H 8192, 16384) have no registers for
        // it (they spill) and evaluate sigmoid per element in both passes;
        // both forms give the same bits.
        constexpr bool KEEP_SG = GATE && (LPR * V * 8 <= 4096 || LPR == 768);
        float sgk[KEEP_SG ? U : 1][KEEP_SG ? V : 1][8];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            S[u] = 0.0;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                float xf[8], df[8];
                unpack8(xv[u][v], xf);
                unpack8(dv[u][v], df);
                float sg[8];  // silu(g) with a gate, else unused
                if constexpr (GATE) {
                    float gf[8];
                    unpack8(t.rv[u][v], gf);
                    if constexpr (KEEP_SG) {
                        sigmoid8(gf, sgk[u][v]);
#pragma unroll
                        for (int e = 0; e < 8; ++e) sg[e] = gf[e] * sgk[u][v][e];
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) sg[e] = gf[e] * sigmoid_f32(gf[e]);
                    }
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    // x * dy is exact in FP32.  With a gate, x * dy * silu(g) is
                    // rounded once in FP32 (2^-24 relative, far inside silu's
                    // own error bound) before it joins the FP64 sums.
                    double pd = GATE ? (double)((xf[e] * df[e]) * sg[e]) : (double)(xf[e] * df[e]);
                    if constexpr (DW) acc[v][e] = __builtin_fma(pd, rho[u], acc[v][e]);
                    S[u] = __builtin_fma(pd, wf64(v, e), S[u]);
                }
            }
        }
        row_group_sum<LPR, U, RPI, true>(S, red, it, slot, g);
        if constexpr (WRAW || (GATE && LPR >= 1024)) {
            // Wide rows: unpack the tile again in the second pass rather
            // than hold the first pass's FP32 values across the row
            // reduction (an empty asm hides that they are unchanged; it
            // emits no instruction).
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    asm volatile("" : "+v"(xv[u][v].x), "+v"(xv[u][v].y), "+v"(xv[u][v].z), "+v"(xv[u][v].w));
                    asm volatile("" : "+v"(dv[u][v].x), "+v"(dv[u][v].y), "+v"(dv[u][v].z), "+v"(dv[u][v].w));
                    if constexpr (DRES || GATE)
                        asm volatile("" : "+v"(t.rv[u][v].x), "+v"(t.rv[u][v].y), "+v"(t.rv[u][v].z),
                                     "+v"(t.rv[u][v].w));
                }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const double L = rho[u] * rho[u] * rho[u] * S[u] * p.inv_h;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                float xf[8], df[8], rf[8];
                unpack8(xv[u][v], xf);
                unpack8(dv[u][v], df);
                if constexpr (DRES || GATE) unpack8(t.rv[u][v], rf);
                uint4 o;
                if constexpr (GATE) {
                    // The gated gradient e = dy * silu(g) carries silu's FP32
                    // error (2^-20 relative at most), so dx is formed in FP32:
                    // its roundings (~3 * 2^-24 of |w e rstd| + |x L|) stay
                    // inside the bound that error already sets.  dg = dy *
                    // (xhat * w) * silu'(g), FP32 as well.
                    const float rf32 = (float)rho[u];  // exact: rstd is an FP32 input
                    const float lf = (float)L;
                    float d[8], q[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float wf = wf32(v, e);
                        const float sgm = KEEP_SG ? sgk[u][v][e] : sigmoid_f32(rf[e]);
                        // silu' = sigmoid * (1 + g (1 - sigmoid)) = sigmoid + silu (1 - sigmoid)
                        const float sl = rf[e] * sgm;  // silu(g), as in the first pass
                        const float dsilu = __builtin_fmaf(sl, 1.0f - sgm, sgm);
                        const float ef = df[e] * sl;
                        q[e] = (df[e] * ((xf[e] * rf32) * wf)) * dsilu;
                        d[e] = __builtin_fmaf(wf * ef, rf32, -(xf[e] * lf));
                    }
                    if (ok[u] && lv.ok[v]) st16_stream(p.dg + off[u] + lv.col[v], pack8(q));
                    o = pack8(d);
                } else {
                    double d[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const double gw = wf64(v, e) * (double)df[e];  // exact
                        d[e] = __builtin_fma(gw, rho[u], -((double)xf[e] * L));
                        if constexpr (DRES) d[e] += (double)rf[e];
                    }
                    o.x = pack_bf16x2_from_f64(d[0], d[1]);
                    o.y = pack_bf16x2_from_f64(d[2], d[3]);
                    o.z = pack_bf16x2_from_f64(d[4], d[5]);
                    o.w = pack_bf16x2_from_f64(d[6], d[7]);
                }
                if (ok[u] && lv.ok[v]) st16_stream(p.dx + off[u] + lv.col[v], o);
            }
        }
    };
    if constexpr (PF && DEFER) {
        // The loop runs while a next iteration exists and loads it
        // unconditionally, the last iteration after it: every path into the
        // work then has the same loads in flight, so the wait before the
        // work leaves the next rows' loads outstanding (with a conditional
        // load the paths' waits merge into one that drains them all).
        if (first < row1) {
            int it = 0;
            int base = first;
            for (; base + step < row1; base += step, ++it) {
                bwd_load<U, V, SLOTS, DRES, GATE, DEFER, PER_ROW>(nxt, p, lv, base + step, slot, row1);
                work(cur, it);
                cur = nxt;
            }
            work(cur, it);
        }
    } else {
        int it = 0;
        for (int base = first; base < row1; base += step, ++it) {
            if constexpr (PF) {
                if (base + step < row1) bwd_load<U, V, SLOTS, DRES, GATE, DEFER, PER_ROW>(nxt, p, lv, base + step, slot, row1);
            } else {
                bwd_load<U, V, SLOTS, DRES, GATE, DEFER, PER_ROW>(cur, p, lv, base, slot, row1);
            }
            work(cur, it);
            if constexpr (PF) {
                if (base + step < row1) cur = nxt;
            }
        }
    }
}

template <int LPR, int V, int U, bool WF32, bool DRES, bool GATE, bool PFP>
__global__ void __launch_bounds__(block_of(LPR)) bwd_kernel(BwdParams p)
{
    constexpr int BLOCK = block_of(LPR);
    constexpr int SLOTS = BLOCK / LPR;
    __shared__ int last_block;
    extern __shared__ double slot_part[];  // [wavefronts][H] when SLOTS > 1

    const int chunk = blockIdx.x;
    double acc[V][8];
    bwd_rows<LPR, V, U, WF32, DRES, GATE, true, PFP>(p, chunk, p.chunks, acc);

    const int tid = threadIdx.x;
    const int g = tid % LPR;
    const int slot = tid / LPR;
    const int H = p.H;
    const LaneVectors<V> lv(g, LPR, H >> 3);

    // ---- chunk sum of dw ----------------------------------------------
    if constexpr (SLOTS > 1) {
        // Row groups of this workgroup hold column sums for the same
        // columns.  Those sharing a wavefront are added with a butterfly of
        // lane exchanges (every lane ends with the wavefront's sum); each
        // wavefront's first row group then stores that sum in its own LDS
        // row, and the rows are added in wavefront order.  Fixed order
        // throughout; LDS use is (BLOCK/max(LPR,64)) * H doubles.
        constexpr int SPW = LPR < 64 ? 64 / LPR : 1;  // row groups per wavefront
        constexpr int GROUPS = SLOTS / SPW;
        if constexpr (SPW > 1) {
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
                for (int v = 0; v < V; ++v)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[v][e] += __shfl_xor(acc[v][e], off);
        }
        if (slot % SPW == 0) {
            double* row = slot_part + (slot / SPW) * H;
#pragma unroll
            for (int v = 0; v < V; ++v)
                if (lv.ok[v]) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) row[lv.col[v] + e] = acc[v][e];
                }
        }
        __syncthreads();
        for (int col = tid; col < H; col += BLOCK) {
            double s = slot_part[col];
#pragma unroll
            for (int gi = 1; gi < GROUPS; ++gi) s += slot_part[gi * H + col];
            if (p.form == FORM_ATOMIC) unsafeAtomicAdd(p.acc + col, s);
            else if (p.direct_dw) p.dw[col] = (float)s;
            else p.part[(int64_t)chunk * H + col] = s;
        }
    } else {
#pragma unroll
        for (int v = 0; v < V; ++v)
            if (lv.ok[v]) {
                if (p.form == FORM_ATOMIC) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) unsafeAtomicAdd(p.acc + lv.col[v] + e, acc[v][e]);
                } else if (p.direct_dw) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) p.dw[lv.col[v] + e] = (float)acc[v][e];
                } else {
                    double2* dst = reinterpret_cast<double2*>(p.part + (int64_t)chunk * H + lv.col[v]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[e] = make_double2(acc[v][2 * e], acc[v][2 * e + 1]);
                }
            }
    }

    if (p.form == FORM_ATOMIC) {
        // Every workgroup publishes its atomics (agent-scope fence) before it
        // takes a ticket; the one that draws the last ticket reads and clears
        // the accumulator and writes dw.  No workgroup ever waits for another.
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const unsigned t = __hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            last_block = (t == (unsigned)(gridDim.x - 1));
        }
        __syncthreads();
        if (last_block) {
            __threadfence();
            for (int col = tid; col < H; col += BLOCK) {
                unsigned long long* a = reinterpret_cast<unsigned long long*>(p.acc + col);
                const unsigned long long bits =
                    __hip_atomic_exchange(a, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                p.dw[col] = (float)__longlong_as_double((long long)bits);
            }
            if (tid == 0) __hip_atomic_store(p.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ----------------------------------------------------- column forms ----
// Column task `task` of a column-form launch: slice s = task % slices covers
// the columns [8 col_vecs s, 8 col_vecs (s + 1)) (the last slice may end
// early), row block k = task / slices the rows [k rpc, (k + 1) rpc) with
// rpc = ceil(R / col_chunks).  Lane l reads vector l % col_vecs of the slice
// in rows q, q + NQ, ... of the block (q = l / col_vecs, NQ = BLOCK /
// col_vecs), four rows in flight, and adds dy * u * rstd (dy * silu(g) * u *
// rstd with a gate) in FP64 from exact products, as the row kernel does.
// Lanes of one vector are then added by a butterfly of lane exchanges inside
// each wavefront and the wavefronts' sums through LDS in wavefront order: a
// fixed order that depends only on R, H, col_chunks, col_vecs and BLOCK.
template <int BLOCK, bool GATE>
__device__ __forceinline__ void dw_column_task(const BwdParams& p, int task)
{
    constexpr int W = BLOCK / 64;
    constexpr int B = 4;  // rows per lane in flight
    __shared__ double cs[W][64];
    __shared__ int last_task;

    const int tid = threadIdx.x;
    const int VC = p.col_vecs;
    const int lg = __builtin_ctz((unsigned)VC);
    const int v = tid & (VC - 1);
    const int q = tid >> lg;
    const int NQ = BLOCK >> lg;
    const int s = task % p.slices;
    const int k = task / p.slices;
    const int nv = p.H >> 3;
    const int vec = s * VC + v;
    const int col = 8 * (vec < nv ? vec : nv - 1);  // lanes past the row's end re-read its last vector
    const int rpc = (p.R + p.col_chunks - 1) / p.col_chunks;
    const int r0 = k * rpc;
    const int r1 = r0 + rpc < p.R ? r0 + rpc : p.R;

    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    for (int base = r0 + q; base < r1; base += B * NQ) {
        bool ok[B];
        float rho[B];
        uint4 xv[B], dv[B], gv[GATE ? B : 1];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int r = base + b * NQ;
            ok[b] = r < r1;
            const int rr = ok[b] ? r : base;
            const int64_t off = row_offset(rr, p.rows) + col;
            rho[b] = p.rstd[rr];
            xv[b] = ld16(p.x + off);
            dv[b] = ld16(p.dy + off);
            if constexpr (GATE) gv[b] = ld16(p.g + off);
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            float xf[8], df[8];
            unpack8(xv[b], xf);
            unpack8(dv[b], df);
            float gf[8];
            if constexpr (GATE) unpack8(gv[b], gf);
            const double rh = (double)rho[b];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // the row kernel's product: with a gate, x * dy * silu(g)
                // rounded once in FP32
                const double pd =
                    GATE ? (double)((xf[e] * df[e]) * (gf[e] * sigmoid_f32(gf[e]))) : (double)(xf[e] * df[e]);
                const double a = __builtin_fma(pd, rh, acc[e]);
                acc[e] = ok[b] ? a : acc[e];
            }
        }
    }
    for (int off = VC; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off);
    const int wave = tid >> 6;
    if ((tid & 63) < VC) {
#pragma unroll
        for (int e = 0; e < 8; ++e) cs[wave][8 * v + e] = acc[e];
    }
    __syncthreads();
    const int c = tid;                  // column within the slice (threads 0 .. 8 VC - 1)
    const int cc = 8 * s * VC + c;      // column of H
    const bool mine = c < 8 * VC && cc < p.H;
    double t = 0.0;
    if (mine) {
        t = cs[0][c];
#pragma unroll
        for (int w = 1; w < W; ++w) t += cs[w][c];
    }
    if (p.col_chunks == 1) {
        if (mine) p.dw[cc] = (float)t;
        return;
    }
    if (mine) p.part[(int64_t)k * p.H + cc] = t;
    if (p.form != FORM_COLS_TICKET) return;
    // Ticket form: publish the block's partial (agent-scope fence), then take
    // the slice's arrival ticket; the task that draws the last one sums the
    // slice's col_chunks partials in block order, writes dw and clears the
    // ticket.  No task waits for another.
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const unsigned n = __hip_atomic_fetch_add(p.slice_ticket + s, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        last_task = n == (unsigned)(p.col_chunks - 1);
    }
    __syncthreads();
    if (!last_task) return;
    __threadfence();
    if (mine) {
        double a = 0.0;
        for (int kk = 0; kk < p.col_chunks; ++kk) a += p.part[(int64_t)kk * p.H + cc];
        p.dw[cc] = (float)a;
    }
    if (tid == 0) __hip_atomic_store(p.slice_ticket + s, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Column-form launch: workgroups [0, col_tasks) are column tasks (col_tasks
// = slices * col_chunks, or 0 for a launch of row tasks alone), the rest
// (p.chunks of them) row tasks that form dx with one row per row group and
// iteration.  A row's arithmetic is the row kernel's (same lanes and vectors
// per row), so dx is bitwise the same in every form.  In place (dx = dy, or
// dg = g) the caller runs the column tasks and the row tasks as two launches
// in that order: column tasks read dy (and g) of rows whose row tasks are
// other workgroups.
template <int LPR, int V, bool WF32, bool DRES, bool GATE>
__global__ void __launch_bounds__(block_of(LPR)) bwd_cols_kernel(BwdParams p)
{
    const int ncol = p.col_tasks;
    if ((int)blockIdx.x < ncol) {
        dw_column_task<block_of(LPR), GATE>(p, blockIdx.x);
        return;
    }
    double none[V][8];
    bwd_rows<LPR, V, 1, WF32, DRES, GATE, false>(p, blockIdx.x - ncol, p.chunks, none);
}

__global__ void __launch_bounds__(kReduceCols * kReduceGroups)
dw_reduce_kernel(const double* __restrict__ part, int chunks, int H, float* __restrict__ dw)
{
    __shared__ double sums[kReduceGroups][kReduceCols];
    const int c = threadIdx.x % kReduceCols;
    const int q = threadIdx.x / kReduceCols;
    const int col = blockIdx.x * kReduceCols + c;
    sums[q][c] = col < H ? chunk_group_sum(part, chunks, H, col, q) : 0.0;
    __syncthreads();
    if (q == 0 && col < H) {
        double t = sums[0][c];
#pragma unroll
        for (int j = 1; j < kReduceGroups; ++j) t += sums[j][c];
        dw[col] = (float)t;
    }
}

__global__ void fill_zero_kernel(uint32_t* p, int64_t words)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// ----------------------------------------------------------- launchers ----

template <int LPR, int V, int U, bool WF32, bool DRES, bool GATE, bool PFP>
static hipError_t bwd_t(const BwdParams& p, hipStream_t s)
{
    constexpr int SLOTS = slots_of(LPR);
    constexpr int ROWS = LPR < 64 ? block_of(LPR) / 64 : SLOTS;
    const size_t lds = SLOTS > 1 ? (size_t)ROWS * p.H * sizeof(double) : 0;
    if (lds > (size_t)kMaxSlotLds) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_kernel<LPR, V, U, WF32, DRES, GATE, PFP>), dim3(p.chunks), dim3(block_of(LPR)), lds, s, p);
    return hipGetLastError();
}

template <int LPR, int V, int U, bool DRES, bool GATE, bool PFP = false>
static hipError_t bwd_w(bool w_f32, const BwdParams& p, hipStream_t s)
{
    return w_f32 ? bwd_t<LPR, V, U, true, DRES, GATE, PFP>(p, s) : bwd_t<LPR, V, U, false, DRES, GATE, PFP>(p, s);
}

// Gated rows hold one more input per element and sigmoid(g) between the two
// passes: with more than one row per row group they outgrow the 256
// registers a lane has at two wavefronts per SIMD, so they take one.
template <int LPR, int V, int U>
constexpr int gated_u() { return LPR <= 256 ? 1 : U; }

#ifndef RMSN_GATED_WIDE_V3
#define RMSN_GATED_WIDE_V3 1
#endif
// Gated rows of three vectors per lane spill even at one row per row group;
// they run as rows of three times the lanes and one vector each instead
// (the gated variant's row order is then its own, fixed per H), which also
// gives them the double-buffered loads of one-vector gated rows.  Rows of
// two vectors stay as they are: as rows of twice the lanes they ran 1.2-1.4x
// slower, and the second tile does not fit their registers.
// Gated rows of 1024 lanes x 1 vector (H 8192) have the 128 registers of
// four wavefronts per SIMD and spill; they run as 512 lanes x 2 vectors.
template <int LPR, int V>
constexpr bool gated_halve_lanes() { return LPR == 1024 && V == 1; }

template <int LPR, int V, int U>
static hipError_t bwd_gated(bool w_f32, const BwdParams& p, hipStream_t s)
{
    if constexpr (RMSN_GATED_WIDE_V3 && V == 3 && LPR <= 256) return bwd_w<3 * LPR, 1, 1, false, true>(w_f32, p, s);
    else if constexpr (gated_halve_lanes<LPR, V>()) return bwd_w<LPR / 2, 2 * V, 1, false, true>(w_f32, p, s);
    else return bwd_w<LPR, V, gated_u<LPR, V, U>(), false, true>(w_f32, p, s);
}

// Plain rows over several chunks, with or without the next-row tile (rows
// wider than 8192 have no registers for a second tile and ignore it).
template <int LPR, int V, int U>
static hipError_t bwd_plain(bool w_f32, const BwdParams& p, hipStream_t s)
{
    if constexpr (LPR * V * 8 > 8192) {
        if (p.dres) return bwd_w<LPR, V, U, true, false>(w_f32, p, s);
        return bwd_w<LPR, V, U, false, false>(w_f32, p, s);
    } else {
        if (p.dres)
            return p.prefetch ? bwd_w<LPR, V, U, true, false, true>(w_f32, p, s)
                              : bwd_w<LPR, V, U, true, false>(w_f32, p, s);
        return p.prefetch ? bwd_w<LPR, V, U, false, false, true>(w_f32, p, s)
                          : bwd_w<LPR, V, U, false, false>(w_f32, p, s);
    }
}

// Per-head views with gaps between rows (a [T, heads, 256] slice of a wider
// row) take one row per row group at H 129-256 instead of two: on the
// [32768, 24, 256] view with token stride 8192, 220.7 -> 213.5 us, while
// contiguous rows of the same width lose 1-3 % with one.  Each row is
// reduced as before, so dx keeps its bits; the deterministic dw follows the
// row groups' fixed order, as at every other layout.
template <int LPR, int V, int U>
static hipError_t bwd_dispatch(bool w_f32, const BwdParams& p, hipStream_t s)
{
    if (p.g) return bwd_gated<LPR, V, U>(w_f32, p, s);
    if constexpr (LPR == 16 && V == 2 && U == 2) {
        if (p.one_row) return bwd_plain<LPR, V, 1>(w_f32, p, s);
    }
    return bwd_plain<LPR, V, U>(w_f32, p, s);
}

// Single-workgroup path: the smallest U in {1, 2, 4} (up to direct_max_u)
// whose one iteration covers every row; gated rows keep gated_u.
template <int LPR, int V, int U, bool DRES, bool GATE>
static hipError_t bwd_direct_t(bool w_f32, const BwdParams& p, hipStream_t s)
{
    constexpr int UM = direct_max_u(LPR, V, U);
    constexpr int UMAX = GATE ? gated_u<LPR, V, U>() : UM;
    constexpr int SL = slots_of(LPR);
    if constexpr (UMAX >= 2) {
        if (p.R <= SL) return bwd_w<LPR, V, 1, DRES, GATE>(w_f32, p, s);
        if constexpr (UMAX >= 4)
            if (p.R > 2 * SL) return bwd_w<LPR, V, 4, DRES, GATE>(w_f32, p, s);
        return bwd_w<LPR, V, 2, DRES, GATE>(w_f32, p, s);
    } else {
        return bwd_w<LPR, V, UMAX, DRES, GATE>(w_f32, p, s);
    }
}

template <int LPR, int V, int U>
static hipError_t bwd_direct(bool w_f32, const BwdParams& p, hipStream_t s)
{
    if (p.dres) return bwd_direct_t<LPR, V, U, true, false>(w_f32, p, s);
    if (p.g) return bwd_gated<LPR, V, U>(w_f32, p, s);
    return bwd_direct_t<LPR, V, U, false, false>(w_f32, p, s);
}

hipError_t launch_bwd(int layout, bool w_f32, const BwdParams& p, hipStream_t s)
{
    switch (layout) {
#define RMSN_BWD_CASE(id, mh, l, vv, uu, kk)                                                 \
    case id:                                                                                 \
        return p.direct_dw ? bwd_direct<l, vv, uu>(w_f32, p, s) : bwd_dispatch<l, vv, uu>(w_f32, p, s);
        RMSN_BWD_LAYOUTS(RMSN_BWD_CASE)
#undef RMSN_BWD_CASE
    default: return hipErrorInvalidValue;
    }
}

template <int LPR, int V, bool WF32, bool DRES, bool GATE>
static hipError_t bwd_cols_t(const BwdParams& p, bool rows, hipStream_t s)
{
    const int grid = p.col_tasks + (rows ? p.chunks : 0);
    if (grid < 1) return hipSuccess;
    hipLaunchKernelGGL((bwd_cols_kernel<LPR, V, WF32, DRES, GATE>), dim3(grid), dim3(block_of(LPR)), 0, s, p);
    return hipGetLastError();
}

template <int LPR, int V, bool DRES, bool GATE>
static hipError_t bwd_cols_w(bool w_f32, const BwdParams& p, bool rows, hipStream_t s)
{
    return w_f32 ? bwd_cols_t<LPR, V, true, DRES, GATE>(p, rows, s) : bwd_cols_t<LPR, V, false, DRES, GATE>(p, rows, s);
}

// Gated rows of three vectors per lane run as rows of three times the lanes,
// as in the row kernel (same row order).
template <int LPR, int V>
static hipError_t bwd_cols_dispatch(bool w_f32, const BwdParams& p, bool rows, hipStream_t s)
{
    if (p.dres) return bwd_cols_w<LPR, V, true, false>(w_f32, p, rows, s);
    if (p.g) {
        if constexpr (RMSN_GATED_WIDE_V3 && V == 3 && LPR <= 256)
            return bwd_cols_w<3 * LPR, 1, false, true>(w_f32, p, rows, s);
        else if constexpr (gated_halve_lanes<LPR, V>()) return bwd_cols_w<LPR / 2, 2 * V, false, true>(w_f32, p, rows, s);
        else return bwd_cols_w<LPR, V, false, true>(w_f32, p, rows, s);
    }
    return bwd_cols_w<LPR, V, false, false>(w_f32, p, rows, s);
}

hipError_t launch_bwd_cols(int layout, bool w_f32, const BwdParams& p, bool rows, hipStream_t s)
{
    switch (layout) {
#define RMSN_BWD_COLS_CASE(id, mh, l, vv, uu, kk) \
    case id: return bwd_cols_dispatch<l, vv>(w_f32, p, rows, s);
        RMSN_BWD_LAYOUTS(RMSN_BWD_COLS_CASE)
#undef RMSN_BWD_COLS_CASE
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dw_reduce(const double* part, int chunks, int H, float* dw, hipStream_t s)
{
    const int grid = (H + kReduceCols - 1) / kReduceCols;
    hipLaunchKernelGGL(dw_reduce_kernel, dim3(grid), dim3(kReduceCols * kReduceGroups), 0, s, part, chunks, H, dw);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void* ptr, int64_t bytes, hipStream_t s)
{
    const int64_t words = bytes / 4;
    if (words <= 0) return hipSuccess;
    int64_t blocks = (words + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((int)blocks), dim3(256), 0, s, static_cast<uint32_t*>(ptr), words);
    return hipGetLastError();
}

// ------------------------------------------------ library-owned scratch ----
// For callers that cannot allocate (rmsnorm_bwd_noalloc): a file-scope device
// array, one per GPU the library runs on, held until the process ends.  Host
// code never uses the array's name as an address (on the host it names a
// stand-in, not device memory): the device address is looked up with
// hipGetSymbolAddress once per device, with that device current, and kept.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t scratch_region(void** out, hipStream_t s)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (!ptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ptr = g_scratch[dev].load(std::memory_order_acquire);
        if (!ptr) {
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!ptr) return hipErrorInvalidSymbol;
            // the prepared part (tickets and accumulator) must start at zero;
            // every call leaves it zero again
            e = launch_fill_zero(ptr, (int64_t)ws_part_offset(RMSN_MAX_H), s);
            if (e != hipSuccess) return e;
            g_scratch[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return hipSuccess;
}

}  // namespace rmsn
