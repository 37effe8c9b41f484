// adaln_kernels.hip -- gfx950 kernels of libadaln: LayerNorm / RMSNorm fused with
// the adaLN modulate epilogue, optionally preceded by the residual-gate prologue or
// (LayerNorm) followed by a static FP8 quantisation of the output.
//
// One row is owned by one wave (H < 2048) or by one workgroup of two waves
// (H < 4096) or four waves.  The row is read from HBM once with 16-byte loads and
// kept in registers; the statistic is reduced in the fixed order of the numerics contract
// (include/adaln.h), which depends on H only, so the bits of a row never depend on
// the batch it is launched in or on the grid.  Sources, by page title and section:
//  - kernels guide, "selection matrix / Norm + scale/shift": column ownership
//    (v fastest, then b), squares rounded on their own, ordered add chain,
//    adjacent-pair butterfly, one final rounding of the RMS output, the three
//    roundings of the modulate chain, the residual variant's two roundings;
//  - ERNIE PR report, kernel snippet: one program per row, 64-bit row offsets,
//    per-batch vector base b*stride, the gated variant storing the residual;
//  - FLUX PR report, motivation: LayerNorm by per-element Welford updates and a
//    count-weighted combine; test snippet `_eager` for the modulate chain.
// Built with -ffp-contract=off; fp32 sqrt and divide are the correctly rounded
// expansions (__builtin_sqrtf and '/'; HIP's __fsqrt_rn is the approximate one),
// or for the LayerNorm rstd the exact shortcut of row_rstd (the same bits).
//
// Execution: a persistent grid of row groups (a wave, or a workgroup of W waves),
// at most as many as can be resident at once.  A group owns either a contiguous
// range of rows or every G-th row (interleaved; then the groups together stream a
// contiguous band of the tensor at any moment; with several batch entries each
// entry can get its own share of the groups, so that no group changes entry).  The
// LayerNorm ops are interleaved; the RMS ops take contiguous ranges.  Launches of at
// least 2^25 elements (all ops but LN+FP8) take a one-shot grid instead: every group
// takes one ring's worth of consecutive rows and the hardware dispatches the groups
// as slots free up, which keeps the rows in flight a compact band of the tensor.  A
// group keeps the per-column constants of its current batch entry in registers
// (bf16(1 + scale), shift, weight, gate: computed once per batch entry, not once per
// row) and keeps its next rows' loads in flight (non-temporal 16-byte loads) while it
// reduces the current one, so HBM traffic never waits on the reduction.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "adaln_device.hpp"
#include "adaln_fold.hpp"
#include "adaln_internal.hpp"

// Launch tuning (never changes the numerics): for contiguous row ranges, groups per
// resident group slot for one-, two- and four-wave rows.  Measured on MI355X: the
// narrower rows need more, shorter groups to keep every SIMD busy.
#ifndef ADALN_GROUP_OVERSUBSCRIBE_W1
#define ADALN_GROUP_OVERSUBSCRIBE_W1 3
#endif
#ifndef ADALN_GROUP_OVERSUBSCRIBE_W2
#define ADALN_GROUP_OVERSUBSCRIBE_W2 2
#endif
#ifndef ADALN_GROUP_OVERSUBSCRIBE_W4
#define ADALN_GROUP_OVERSUBSCRIBE_W4 1
#endif
// Row assignment per op (never changes the numerics): interleaved (group g takes
// rows g, g + G, ...) or contiguous ranges.  Measured on MI355X: the LayerNorm ops
// gain from the interleaved assignment (more groups, shorter chains), the RMS ops
// stream slightly faster over contiguous ranges (below ADALN_ONESHOT_MIN_ELEMS).
#ifndef ADALN_INTERLEAVE_LN
#define ADALN_INTERLEAVE_LN 1  // LayerNorm and LayerNorm + FP8
#endif
#ifndef ADALN_INTERLEAVE_RMS
#define ADALN_INTERLEAVE_RMS 0
#endif
#ifndef ADALN_INTERLEAVE_RG
#define ADALN_INTERLEAVE_RG 0
#endif
#ifndef ADALN_INTERLEAVE_RGLN
#define ADALN_INTERLEAVE_RGLN 1
#endif
// Interleaved ops switch to a one-slot ring when each resident group would get at
// least this many rows (measured on MI355X: more resident groups then beat a deeper
// ring; with fewer rows per group the deeper ring is faster).
#ifndef ADALN_SHALLOW_ROWS_PER_GROUP
#define ADALN_SHALLOW_ROWS_PER_GROUP 3
#endif
// The RMS op (no gate) with four-wave rows takes the one-slot ring when every
// resident one-slot group gets at most this many rows (measured on MI355X at H
// 4096: +3% at 1024 rows, +11% at 2048, +39% at 256 against the three-row ring,
// which fills fewer groups; from a few thousand rows on the three-row ring is
// faster, and with the gate the one-slot ring was slower).
#ifndef ADALN_CONTIG_SHALLOW_MAX_ROWS_PER_GROUP
#define ADALN_CONTIG_SHALLOW_MAX_ROWS_PER_GROUP 2
#endif
// From this many elements (rows * H) per launch on, every op but LN+FP8 takes the
// one-shot grid: one pass of the default ring per group, consecutive rows, as many
// groups as that takes (measured on MI355X against the persistent grid: +0.7% to
// +16% at 2^25 elements and above, for one-, two- and four-wave rows of every such
// op; mixed or slower below; LN+FP8, bound by its arithmetic, 4-5% slower).
#ifndef ADALN_ONESHOT_MIN_ELEMS
#define ADALN_ONESHOT_MIN_ELEMS (int64_t(1) << 25)
#endif

namespace adaln {
namespace {

constexpr bool interleaved(int op) {
    return ((op == OP_LN || op == OP_LNQ) && ADALN_INTERLEAVE_LN) ||
           (op == OP_RMS && ADALN_INTERLEAVE_RMS) || (op == OP_RG && ADALN_INTERLEAVE_RG) ||
           (op == OP_RGLN && ADALN_INTERLEAVE_RGLN);
}

// ---------------------------------------------------------------------------
// the fused row kernel
// ---------------------------------------------------------------------------
// Rows in flight per group (prefetch depth + 1), by lane footprint: enough bytes
// outstanding per CU to cover HBM latency without costing occupancy.
#ifndef ADALN_SLOTS_SMALL
#define ADALN_SLOTS_SMALL 3  // <= 16 bf16 of x per lane
#endif
#ifndef ADALN_SLOTS_MID
#define ADALN_SLOTS_MID 3    // <= 32 per lane
#endif
#ifndef ADALN_SLOTS_LARGE
#define ADALN_SLOTS_LARGE 2  // more
#endif
// Per-column constants as fp32 (no unpacking per row) when they fit in at most
// ADALN_KF_MAX registers per lane, else as packed bf16 pairs.
#ifndef ADALN_KF_MAX
#define ADALN_KF_MAX 96
#endif
constexpr bool consts_as_f32(int W, int C, int op, bool weight) {
    const int nvec = 2 + (weight ? 1 : 0) + (op_gated(op) ? 1 : 0);
    return W > 1 || 8 * C * nvec <= ADALN_KF_MAX;
}
#ifndef ADALN_SLOTS_W2
#define ADALN_SLOTS_W2 2     // two-wave rows without the gate (2048 <= H < 4096)
#endif
constexpr int ring_slots(int W, int C, bool gated) {
    if (W == 2 && !gated) return ADALN_SLOTS_W2;
    const int per_lane = C * 8 * (gated ? 2 : 1);
    return per_lane <= 16 ? ADALN_SLOTS_SMALL : per_lane <= 32 ? ADALN_SLOTS_MID
                                                               : ADALN_SLOTS_LARGE;
}

// OP: Op; W: waves per row; C: chunks per lane; TAIL: the last chunk is partial;
// WEIGHT: RMS weight present; IL: interleaved rows (per-row descriptors); RING: the
// ring depth when not 0 (one or two slots), else ring_slots.  A workgroup is four independent one-wave groups (W == 1) or one
// group of W waves.
//
// Per-lane constants of the current batch entry are kept as fp32 (no unpacking
// per row) or, for wide rows on one wave, as packed bf16 pairs (every constant is
// a bf16 value); see consts_as_f32.
template <int OP, int W, int C, bool TAIL, bool WEIGHT, bool IL, int RING>
__global__ __launch_bounds__(256) void fused_norm_modulate(Params p) {
    constexpr int P = 64 * W;
    constexpr bool KF = consts_as_f32(W, C, OP, WEIGHT);
    constexpr int NK = KF ? 8 * C : 4 * C;           // constants per vector per lane
    constexpr bool GATED = op_gated(OP);
    constexpr bool FP8 = op_fp8(OP);
    constexpr bool LNSTAT = op_layernorm(OP);
    constexpr int HFULL = C * 8 * P;                 // H when no chunk is partial

    const int lane = threadIdx.x & 63;
    // readfirstlane: the wave index is uniform, and the compiler must know it so
    // that a group's row range and buffer descriptors live in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t group = (W == 1) ? (int64_t)blockIdx.x * 4 + wave : (int64_t)blockIdx.x;
    // a whole wave (W == 1) or workgroup (W > 1) leaves, before any barrier
    if (group >= p.groups) return;
    // Group g owns the rows r_begin, r_begin + step, ... below r_end: a contiguous
    // range (step 1) or every gpb-th row of its block (the interleaved assignment).
    const int64_t blk = p.gpb == p.groups ? 0 : (int64_t)((uint32_t)group / (uint32_t)p.gpb);
    const int64_t blk_begin = blk * p.blk_rows;
    const int64_t r_begin = blk_begin + (group - blk * p.gpb) * p.group_stride;
    int64_t r_end = r_begin + p.span < p.rows ? r_begin + p.span : p.rows;
    if (r_end > blk_begin + p.blk_rows) r_end = blk_begin + p.blk_rows;
    if (r_begin >= r_end) return;
    const int64_t step = IL ? p.step : 1;
    const int t = (W == 1) ? lane : wave * 64 + lane;  // lane index within the row
    const int64_t H = TAIL ? p.H : HFULL;
    constexpr bool POW2H = !TAIL && (HFULL & (HFULL - 1)) == 0;
    const float rH = 1.0f / (float)H;  // a constant unless the row is ragged

    __shared__ float xwave[2][4][3];  // cross-wave partials, double-buffered by row parity

    int col[C];
    bool ok[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        col[c] = c * 8 * P + 8 * t;
        ok[c] = !TAIL || c < C - 1 || col[c] < H;
    }

    // ---- per-column constants of batch entry b --------------------------------
    float ka[KF ? NK : 1], kh[KF ? NK : 1], kw[KF ? NK : 1], kg[KF ? NK : 1];
    u32 pa[KF ? 1 : NK], ph[KF ? 1 : NK], pw[KF ? 1 : NK], pg[KF ? 1 : NK];
    auto load_consts = [&](int64_t b) {
        const uint16_t* sc_row = p.scale + b * p.scale_bs;
        const uint16_t* sh_row = p.shift + b * p.shift_bs;
        const uint16_t* g_row = GATED ? p.gate + b * p.gate_bs : nullptr;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            uint4 sc = make_uint4(0u, 0u, 0u, 0u), sh = sc, wv = sc, gv = sc;
            if (ok[c]) {
                sc = ld16(sc_row + col[c]);
                sh = ld16(sh_row + col[c]);
                if (WEIGHT) wv = ld16(p.weight + col[c]);
                if (GATED) gv = ld16(g_row + col[c]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32 s = word(sc, j);
                const u32 a = pack_bf16(1.0f + bf_lo(s), 1.0f + bf_hi(s));  // bf16(1 + scale)
                const u32 w = word(wv, j);
                const float w0 = bf_lo(w) + 0.0f, w1 = bf_hi(w) + 0.0f;    // (w + 0.0): -0 -> +0
                if (KF) {
                    const int e = c * 8 + 2 * j;
                    ka[e] = round_bf16(1.0f + bf_lo(s));  // the same values as a, unpacked
                    ka[e + 1] = round_bf16(1.0f + bf_hi(s));
                    kh[e] = bf_lo(word(sh, j));
                    kh[e + 1] = bf_hi(word(sh, j));
                    kw[e] = w0;
                    kw[e + 1] = w1;
                    kg[e] = bf_lo(word(gv, j));
                    kg[e + 1] = bf_hi(word(gv, j));
                } else {
                    const int e = c * 4 + j;
                    pa[e] = a;
                    ph[e] = word(sh, j);
                    pw[e] = pack_bf16(w0, w1);  // exact: w + 0 is a bf16 value
                    pg[e] = word(gv, j);
                }
            }
        }
    };
    auto K_a = [&](int c, int v) {
        return KF ? ka[c * 8 + v] : ((v & 1) ? bf_hi(pa[c * 4 + (v >> 1)]) : bf_lo(pa[c * 4 + (v >> 1)]));
    };
    auto K_h = [&](int c, int v) {
        return KF ? kh[c * 8 + v] : ((v & 1) ? bf_hi(ph[c * 4 + (v >> 1)]) : bf_lo(ph[c * 4 + (v >> 1)]));
    };
    auto K_w = [&](int c, int v) {
        return KF ? kw[c * 8 + v] : ((v & 1) ? bf_hi(pw[c * 4 + (v >> 1)]) : bf_lo(pw[c * 4 + (v >> 1)]));
    };
    auto K_g = [&](int c, int v) {
        return KF ? kg[c * 8 + v] : ((v & 1) ? bf_hi(pg[c * 4 + (v >> 1)]) : bf_lo(pg[c * 4 + (v >> 1)]));
    };

    // ---- addressing through buffer descriptors ---------------------------------
    // Interleaved rows (IL): one descriptor per row spanning exactly its 2H bytes,
    // an empty one for a row past the end, and a lane offset that is the same for
    // every row.  Contiguous rows: one descriptor per tensor over the group's range
    // and a per-row offset; a row past the range lands beyond it.  Either way lanes
    // past a ragged row end get an out-of-range offset, and an access out of range
    // reads zero or is dropped.
    // ES: bytes per element of a tensor (2 for bf16, 1 for the FP8 output)
    auto range_rsrc = [&](const void* base, int ES) {
        return make_rsrc(IL ? base : static_cast<const char*>(base) + r_begin * H * ES,
                         IL ? 0 : (r_end - r_begin) * H * ES);
    };
    auto rsrc_of = [&](const void* base, const rsrc_t& range, int64_t row, int ES) {
        if (!IL) return range;
        return row < r_end ? make_rsrc(static_cast<const char*>(base) + row * H * ES, H * ES)
                           : make_rsrc(base, 0);
    };
    auto off_of = [&](int64_t row, int c, int ES) {
        if (IL) return ok[c] ? ES * col[c] : kOutOfRange;
        const int64_t rr = row < r_end ? row : r_end;  // keeps the offset arithmetic in range
        return ok[c] ? (int)((rr - r_begin) * H * ES) + ES * col[c] : kOutOfRange;
    };
    constexpr int OES = FP8 ? 1 : 2;  // output bytes per element
    const rsrc_t gx = range_rsrc(p.x, 2);
    const rsrc_t gy = FP8 ? range_rsrc(p.q, 1) : range_rsrc(p.y, 2);
    const rsrc_t gres = GATED ? range_rsrc(p.res, 2) : gx;
    const rsrc_t gr = GATED ? range_rsrc(p.r, 2) : gy;
    auto load_row = [&](int64_t row, uint4 (&xv)[C], uint4 (&rv)[C]) {
        const rsrc_t rx = rsrc_of(p.x, gx, row, 2);
        const rsrc_t rres = GATED ? rsrc_of(p.res, gres, row, 2) : rx;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int off = off_of(row, c, 2);
            xv[c] = ld16_stream(rx, off);
            if (GATED) rv[c] = ld16_stream(rres, off);
        }
    };
    const rsrc_t r_none = make_rsrc(p.x, 0);  // an empty range: every store dropped
    // LNQ: the reciprocal of the static quantisation scale, correctly rounded
    const float inv_qscale = FP8 ? 1.0f / *p.qscale : 0.0f;

    auto store_out = [&](const rsrc_t& r, int off, const u32 (&w)[4]) {
        if (FP8) st8_stream(r, off, w[0], w[1]);
        else st16_stream(r, off, make_uint4(w[0], w[1], w[2], w[3]));
    };

    // LN+FP8: whether every modulation constant of this lane is finite; with finite
    // row statistics too, no output can be NaN and the clamp can be one median.  The
    // answer is wave-uniform (true only if it holds in every lane of the wave).  The
    // NaN-propagating maximum of the magnitudes is finite exactly when every value
    // is: a NaN stays NaN, an infinity stays infinite.
    auto consts_finite = [&]() {
        float m = 0.0f;
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int v = 0; v < 8; ++v)
                m = __builtin_elementwise_maximum(
                    __builtin_elementwise_maximum(m, __builtin_fabsf(K_a(c, v))),
                    __builtin_fabsf(K_h(c, v)));
        return __builtin_amdgcn_ballot_w64(!__builtin_isfinite(m)) == 0;
    };
    // blocks of one batch entry each: the block is the batch entry
    int64_t b = p.blk_rows == p.T ? blk : r_begin / p.T;
    int64_t t_in = r_begin - b * p.T;
    load_consts(b);
    // and a finite, non-zero 1/scale (0 * inf and inf * 0 are the other NaN sources)
    const bool inv_ok = FP8 && __builtin_isfinite(inv_qscale) && inv_qscale != 0.0f;
    bool fast_q = inv_ok && consts_finite();

    // A ring of S row slots: slot k holds the group's row row0 + k*G; after a row is
    // finished its slot is refilled with the group's row S ahead, so S rows' loads
    // stay in flight.
    constexpr int S = RING ? RING : ring_slots(W, C, GATED);
    uint4 xs[S][C], rs[S][C];
    // Prologue in the steady state's order: before slot k's loads, stand-ins for
    // slot k-1's stores (out of range: dropped), so that at the loop head the
    // outstanding operations after slot 0's loads are the same on the first pass
    // as on every later one.
#pragma unroll
    for (int k = 0; k < S; ++k) {
        if (k > 0) {
#pragma unroll
            for (int i = 0; i < (GATED ? 2 * C : C); ++i)  // distinct, so none is merged
                st16_stream(r_none, kOutOfRange - 16 * i, make_uint4(0u, 0u, 0u, 0u));
        }
        load_row(r_begin + k * step, xs[k], rs[k]);
    }

    // One exit test per pass over the S slots, at the loop head: the only way back
    // to the head runs through all S slots, so the compiler knows exactly which
    // loads and stores are still outstanding at each slot and waits only for that
    // slot's own data.  In the last pass a slot past the group's last row holds
    // zeros (its loads were out of range) and its stores are dropped.
    int seq = 0;  // index of the current row among the group's rows
    for (int64_t row0 = r_begin; row0 < r_end; row0 += S * step) {
#pragma unroll
    for (int k = 0; k < S; ++k) {
        const int64_t row = row0 + k * step;
        uint4 (&xa)[C] = xs[k];
        uint4 (&ra)[C] = rs[k];
        const int par = seq & 1;  // alternates over the group's consecutive rows
        const rsrc_t ry = FP8 ? rsrc_of(p.q, gy, row, 1) : rsrc_of(p.y, gy, row, 2);
        const rsrc_t rr_out = GATED ? rsrc_of(p.r, gr, row, 2) : ry;

        // Residual gate (gated ops): r = bf16(res + bf16(gate * x)), stored; r is the
        // norm input.  The norm input is widened to binary32 once and kept for the
        // statistic and the normalisation.
        float xf[C][8];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            u32 rr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                u32 xw = word(xa[c], j);
                if (GATED) {
                    const u32 rw = word(ra[c], j);
                    const float g0 = round_bf16(K_g(c, 2 * j) * bf_lo(xw));
                    const float g1 = round_bf16(K_g(c, 2 * j + 1) * bf_hi(xw));
                    const float s0 = bf_lo(rw) + g0;
                    const float s1 = bf_hi(rw) + g1;
                    xw = pack_bf16(s0, s1);
                    rr[j] = xw;
                }
                xf[c][2 * j] = bf_lo(xw);
                xf[c][2 * j + 1] = bf_hi(xw);
            }
            if (GATED) st16_stream(rr_out, off_of(row, c, 2), make_uint4(rr[0], rr[1], rr[2], rr[3]));
        }

        // Interleaved rows: the statistic and the normalisation run only for a real
        // row (a uniform branch with no HBM access inside) and the y stores follow
        // it, issued either way, so every pass issues the same memory operations in
        // the same order.  Contiguous rows (only the last group can have an idle
        // slot): no branch, and each chunk's store leaves as soon as it is ready.
        u32 yw_out[C][4];
        if (IL) {
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int j = 0; j < 4; ++j) yw_out[c][j] = 0u;
        }
        if (!IL || row < r_end) {

        // Statistic: ordered per-lane chain, butterfly, cross-wave pairs, finalize.
        float mean = 0.0f, rstd, m2_row = 0.0f;
        if (LNSTAT) {
            float wm = 0.0f, w2 = 0.0f;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                if (!ok[c]) continue;
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    const float x = xf[c][v];
                    const float rho = 1.0f / (float)(c * 8 + v + 1);  // RN(1/n), folded
                    const float d = x - wm;
                    const float step = d * rho;
                    wm = wm + step;
                    const float e = x - wm;
                    const float q = d * e;
                    w2 = w2 + q;
                }
            }
            if (!TAIL) {
                constexpr int N = 8 * C;
                wave_welford_equal<N>(wm, w2);
                if (W > 1) {
                    if (lane == 0) {
                        xwave[par][wave][0] = wm;
                        xwave[par][wave][1] = w2;
                    }
                    __syncthreads();
                    if (W == 2) {
                        combine_equal<64 * N>(xwave[par][0][0], xwave[par][1][0],
                                              xwave[par][0][1] + xwave[par][1][1], wm, w2);
                    } else {
                        float ma, qa, mb, qb;
                        combine_equal<64 * N>(xwave[par][0][0], xwave[par][1][0],
                                              xwave[par][0][1] + xwave[par][1][1], ma, qa);
                        combine_equal<64 * N>(xwave[par][2][0], xwave[par][3][0],
                                              xwave[par][2][1] + xwave[par][3][1], mb, qb);
                        combine_equal<128 * N>(ma, mb, qa + qb, wm, w2);
                    }
                }
            } else {
                Welford w{ok[C - 1] ? 8.0f * C : 8.0f * (C - 1), wm, w2};
                w = wave_welford(w, lane);
                if (W > 1) {
                    if (lane == 0) {
                        xwave[par][wave][0] = w.n;
                        xwave[par][wave][1] = w.mean;
                        xwave[par][wave][2] = w.m2;
                    }
                    __syncthreads();
                    Welford q[W];
#pragma unroll
                    for (int i = 0; i < W; ++i)
                        q[i] = Welford{xwave[par][i][0], xwave[par][i][1], xwave[par][i][2]};
                    if (W == 2)
                        w = combine(q[0], q[W - 1]);
                    else
                        w = combine(combine(q[0], q[1 % W]), combine(q[2 % W], q[3 % W]));
                }
                wm = w.mean;
                w2 = w.m2;
            }
            mean = wm;
            m2_row = w2;
            rstd = row_rstd<POW2H>(w2, (float)H, rH, p.eps);
        } else {
            float s = 0.0f;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                if (!ok[c]) continue;
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    const float q = xf[c][v] * xf[c][v];
                    s = s + q;
                }
            }
            s = wave_sum(s);
            if (W > 1) {
                if (lane == 0) xwave[par][wave][0] = s;
                __syncthreads();
                if (W == 2) {
                    s = xwave[par][0][0] + xwave[par][1][0];
                } else {
                    const float a = xwave[par][0][0] + xwave[par][1][0];
                    const float bb = xwave[par][2][0] + xwave[par][3][0];
                    s = a + bb;
                }
            }
            // (the general steps here: the shortcut's uniform test costs the RMS ops
            // more latency than its instructions save)
            rstd = finalize(s / (float)H, p.eps);
        }

        // LN+FP8: the row statistics are the same in every lane; the one-median clamp
        // is exact when no output of the row can be NaN (see consts_finite)
        const bool fast_row =
            FP8 && fast_q &&
            __builtin_amdgcn_ballot_w64(!(__builtin_isfinite(mean) && __builtin_isfinite(m2_row) &&
                                          __builtin_isfinite(rstd))) == 0;
        // Normalise from registers, modulate.
#pragma unroll
        for (int c = 0; c < C; ++c) {
            u32 (&out)[4] = yw_out[c];
            float qv[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float n0, n1;
                if (LNSTAT) {
                    const float d0 = xf[c][2 * j] - mean;
                    const float d1 = xf[c][2 * j + 1] - mean;
                    n0 = d0 * rstd;
                    n1 = d1 * rstd;
                } else {
                    n0 = xf[c][2 * j] * rstd;
                    n1 = xf[c][2 * j + 1] * rstd;
                    if (WEIGHT) {
                        n0 = n0 * K_w(c, 2 * j);
                        n1 = n1 * K_w(c, 2 * j + 1);
                    }
                }
                const float y0 = round_bf16(n0), y1 = round_bf16(n1);               // yn
                const float p0 = round_bf16(y0 * K_a(c, 2 * j));                   // bf16(yn*a)
                const float p1 = round_bf16(y1 * K_a(c, 2 * j + 1));
                if (!FP8) {
                    out[j] = pack_bf16(p0 + K_h(c, 2 * j), p1 + K_h(c, 2 * j + 1));  // bf16(p+shift)
                } else {
                    // y = bf16(p + shift) as binary32, times 1/scale
                    qv[2 * j] = round_bf16(p0 + K_h(c, 2 * j)) * inv_qscale;
                    qv[2 * j + 1] = round_bf16(p1 + K_h(c, 2 * j + 1)) * inv_qscale;
                }
            }
            if (FP8) {
                if (fast_row) {
                    out[0] = quant4_no_nan(qv[0], qv[1], qv[2], qv[3]);
                    out[1] = quant4_no_nan(qv[4], qv[5], qv[6], qv[7]);
                } else {
                    out[0] = quant4(qv[0], qv[1], qv[2], qv[3]);
                    out[1] = quant4(qv[4], qv[5], qv[6], qv[7]);
                }
            }
            if (!IL) store_out(ry, off_of(row, c, OES), out);
        }
        }  // row < r_end

        // non-temporal stores of y (16 bytes) or q (8 bytes) per chunk (interleaved rows)
        if (IL) {
#pragma unroll
            for (int c = 0; c < C; ++c) store_out(ry, off_of(row, c, OES), yw_out[c]);
        }

        // refill this slot S rows ahead; switch batch entry if the next row needs it
        load_row(row + S * step, xa, ra);
        ++seq;
        const int64_t next = row + step;
        if (next < r_end) {  // uniform over the group
            t_in += step;
            if (t_in >= p.T) {
                if (IL) {
                    b = next / p.T;
                    t_in = next - b * p.T;
                } else {  // consecutive rows: the next batch entry
                    ++b;
                    t_in = 0;
                }
                load_consts(b);
                if (FP8) fast_q = inv_ok && consts_finite();
            }
        }
    }
    }
    // Never true (rows > 0): gives the ring registers a use after the loop, so the
    // compiler cannot sink a refill load below the exit test into the next pass.
    // Even if executed, the stores land out of range and are dropped.
    if (p.rows < 0) {
#pragma unroll
        for (int k = 0; k < S; ++k)
#pragma unroll
            for (int c = 0; c < C; ++c) {
                st16_stream(r_none, kOutOfRange, xs[k][c]);
                if (GATED) st16_stream(r_none, kOutOfRange, rs[k][c]);
            }
    }
}

__global__ __launch_bounds__(256) void diag_round(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
    {
        // both conversion slots of v_cvt_pk_bf16_f32 are used by the kernels; a
        // disagreement between them is reported as the quiet NaN 0x7FC1
        const u32 lo = pack_bf16(in[i], 0.0f) & 0xFFFFu;
        const u32 hi = __float_as_uint(round_bf16(in[i])) >> 16;
        out[i] = (uint16_t)(lo == hi ? lo : 0x7FC1u);
    }
}

__global__ __launch_bounds__(256) void diag_finalize(const float* in, float* out, int64_t n,
                                                     float H, float eps) {
    const float rH = 1.0f / H;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        out[i] = row_rstd<false>(in[i], H, rH, eps);
}

// The fused LNQ kernel's quantisation step on binary32 inputs: out = E4M3 of
// clamp(in * RN(1/qscale)), four values per thread.
__global__ __launch_bounds__(256) void diag_quant(const float4* __restrict__ in,
                                                  u32* __restrict__ out, int64_t n4,
                                                  const float* qscale) {
    const float inv = 1.0f / *qscale;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * blockDim.x) {
        const float4 v = in[i];
        out[i] = quant4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
    }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
using KernelFn = void (*)(Params);

template <int OP, int W, int C, bool TAIL, int RING>
KernelFn pick_weight(bool weight) {
    constexpr bool IL = interleaved(OP);
    if constexpr (op_layernorm(OP)) {
        return fused_norm_modulate<OP, W, C, TAIL, false, IL, RING>;  // no weight
    } else {
        return weight ? fused_norm_modulate<OP, W, C, TAIL, true, IL, RING>
                      : fused_norm_modulate<OP, W, C, TAIL, false, IL, RING>;
    }
}

// ring 1 (the one-slot ring) is instantiated for the interleaved ops and for the
// ungated contiguous ops' four-wave rows, ring 2 for the latter only; ring 0 is the
// default depth
template <int OP, int W, int C>
KernelFn pick_tail(bool tail, bool weight, int ring) {
    constexpr bool contig4 = !interleaved(OP) && W == 4 && !op_gated(OP);
    if constexpr (interleaved(OP) || contig4) {
        if (ring == 1)
            return tail ? pick_weight<OP, W, C, true, 1>(weight)
                        : pick_weight<OP, W, C, false, 1>(weight);
    }
    if constexpr (contig4) {
        if (ring == 2)
            return tail ? pick_weight<OP, W, C, true, 2>(weight)
                        : pick_weight<OP, W, C, false, 2>(weight);
    }
    if (ring != 0) return nullptr;
    return tail ? pick_weight<OP, W, C, true, 0>(weight)
                : pick_weight<OP, W, C, false, 0>(weight);
}

template <int OP>
KernelFn pick(const Layout& L, bool weight, int ring) {
    // H < 2048: one wave, C = 1..4; 2048 <= H < 4096: two waves, C = 2..4;
    // H >= 4096: four waves, C = 2..4.
    if (L.waves == 1) {
        switch (L.chunks) {
            case 1: return pick_tail<OP, 1, 1>(L.ragged, weight, ring);
            case 2: return pick_tail<OP, 1, 2>(L.ragged, weight, ring);
            case 3: return pick_tail<OP, 1, 3>(L.ragged, weight, ring);
            case 4: return pick_tail<OP, 1, 4>(L.ragged, weight, ring);
        }
    } else if (L.waves == 2) {
        switch (L.chunks) {
            case 2: return pick_tail<OP, 2, 2>(L.ragged, weight, ring);
            case 3: return pick_tail<OP, 2, 3>(L.ragged, weight, ring);
            case 4: return pick_tail<OP, 2, 4>(L.ragged, weight, ring);
        }
    } else {
        switch (L.chunks) {
            case 2: return pick_tail<OP, 4, 2>(L.ragged, weight, ring);
            case 3: return pick_tail<OP, 4, 3>(L.ragged, weight, ring);
            case 4: return pick_tail<OP, 4, 4>(L.ragged, weight, ring);
        }
    }
    return nullptr;
}

}  // namespace

// Resident workgroups per CU for a kernel on the current device (cached).
struct OccEntry {
    const void* fn;
    int device;
    int blocks_per_cu;
    int cus;
};

bool occupancy(const void* fn, int block, int* blocks_per_cu, int* cus) {
    static std::mutex mu;
    static OccEntry cache[256];
    static int n_cache = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n_cache; ++i)
        if (cache[i].fn == fn && cache[i].device == dev) {
            *blocks_per_cu = cache[i].blocks_per_cu;
            *cus = cache[i].cus;
            return true;
        }
    int nb = 0, ncu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, block, 0) != hipSuccess)
        return false;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return false;
    if (nb < 1) nb = 1;
    if (n_cache < 256) cache[n_cache++] = OccEntry{fn, dev, nb, ncu};
    *blocks_per_cu = nb;
    *cus = ncu;
    return true;
}

Layout layout_of(int64_t H) {
    Layout L;
    L.waves = H < 2048 ? 1 : H < 4096 ? 2 : 4;
    L.lanes = 64 * L.waves;
    L.chunks = (int)((H + 8 * L.lanes - 1) / (8 * L.lanes));
    L.ragged = (H % (8 * L.lanes)) != 0;
    return L;
}

Plan plan_launch(Op op, int64_t rows, int64_t H, int64_t T, int64_t resident,
                 int64_t resident_shallow, int64_t resident_two, int64_t cus) {
    const Layout L = layout_of(H);
    Plan pl{};
    pl.block_threads = L.waves == 1 ? 256 : 64 * L.waves;
    // a grid holds fewer than 2^32 work-items
    const int64_t max_groups =
        int64_t(0xFFFFFFFF) / pl.block_threads * (L.waves == 1 ? 4 : 1);
    // the most rows of a contiguous group with s ring slots: its descriptors address
    // them with 32-bit byte offsets, and the last pass reaches s rows past its range,
    // so (rows + s) rows stay below 2^31 bytes
    auto max_rows = [&](int s) { return ((int64_t(0x7FFFFFFF) - 64) / (2 * H) - s) / s * s; };
    // Large launches: the one-shot grid.  Group g takes the consecutive rows
    // g*per .. g*per + per - 1, per = S (one pass of the default ring), unless the
    // grid would then pass 2^32 work-items, when per grows by whole passes.  The
    // interleaved ops' kernels address any row, so they take the same ranges.
    if (op != OP_LNQ && rows >= (ADALN_ONESHOT_MIN_ELEMS + H - 1) / H) {
        const int S = ring_slots(L.waves, L.chunks, op_gated(op));
        const int64_t passes = ((rows + S - 1) / S + max_groups - 1) / max_groups;
        int64_t per = passes * S;
        // (only past 2^55 bytes of rows could a group need more than 32-bit offsets;
        // the grid is then too large and the launch is refused)
        if (!interleaved(op) && per > max_rows(S)) per = max_rows(S);
        pl.shallow = false;
        pl.slots = S;
        pl.ring = 0;
        pl.groups = (rows + per - 1) / per;
        pl.gpb = pl.groups;
        pl.blk_rows = rows;
        pl.group_stride = per;
        pl.step = 1;
        pl.span = per;
        pl.blocks = L.waves == 1 ? (pl.groups + 3) / 4 : pl.groups;
        return pl;
    }
    // Interleaved ops with many rows per group: the one-slot ring (more resident
    // groups, the latency covered by the other groups) streams faster; with few
    // rows per group the deeper ring does.  Contiguous four-wave RMS rows: the other
    // way round, the one-slot ring only for launches of one or two rows per group
    // (with the gate it measured slower; tuning; the bits never depend on it).
    pl.shallow = resident_shallow > 0 &&
                 (interleaved(op) ? rows >= ADALN_SHALLOW_ROWS_PER_GROUP * resident
                                  : L.waves == 4 && !op_gated(op) &&
                                        rows <= ADALN_CONTIG_SHALLOW_MAX_ROWS_PER_GROUP *
                                                    resident_shallow);
    if (pl.shallow) resident = resident_shallow;
    const int S = pl.shallow ? 1 : ring_slots(L.waves, L.chunks, op_gated(op));
    pl.slots = S;
    pl.ring = pl.shallow ? 1 : 0;
    if (interleaved(op)) {
        // one group per resident group slot (at most one per row); a group's ring
        // slots past its last row skip their arithmetic.  With several batch entries
        // and enough groups, each entry gets its own share of the groups, so that a
        // group never changes entry (its per-column constants are loaded once), as
        // long as the split leaves at most 1/16 of the slots idle.
        int64_t G = rows < resident ? rows : resident;
        if (G > max_groups) G = max_groups;
        const int64_t B = rows / T;
        const int64_t per_entry = B > 1 ? (G / B < T ? G / B : T) : 0;
        if (per_entry > 0 && 16 * (G - per_entry * B) <= G) {
            pl.groups = per_entry * B;
            pl.gpb = per_entry;
            pl.blk_rows = T;
            pl.span = T;
        } else {
            pl.groups = G;
            pl.gpb = G;
            pl.blk_rows = rows;
            pl.span = rows;
        }
        pl.group_stride = 1;
        pl.step = pl.gpb;
    } else {
        // `per` contiguous rows per group, a multiple of S so that only the last
        // group can end with idle ring slots; the group's descriptors address its
        // rows with 32-bit byte offsets and the last pass reaches S rows past its
        // range, so (per + S) rows stay below 2^31 bytes
        const int over = L.waves == 1   ? ADALN_GROUP_OVERSUBSCRIBE_W1
                         : L.waves == 2 ? ADALN_GROUP_OVERSUBSCRIBE_W2
                                        : ADALN_GROUP_OVERSUBSCRIBE_W4;
        auto per_of = [&](int64_t res, int s) {
            int64_t slots = res * over;
            if (slots > max_groups) slots = max_groups;
            const int64_t groups0 = rows < slots ? rows : slots;
            int64_t q = (rows + groups0 - 1) / groups0;
            q = (q + s - 1) / s * s;
            return q < max_rows(s) ? q : max_rows(s);
        };
        int64_t per = per_of(resident, S);
        // Ungated four-wave rows: the two-row ring instead of the deeper one when it
        // leaves the most loaded CU fewer rows (its groups spread over the CUs more
        // evenly), weighing a two-row ring's row 3.5% dearer (measured at 65536 rows).
        if (!pl.shallow && L.waves == 4 && !op_gated(op) &&
            resident_two > 0 && cus > 0 && S > 2) {
            const int64_t per2 = per_of(resident_two, 2);
            const int64_t g2 = (rows + per2 - 1) / per2, g = (rows + per - 1) / per;
            const int64_t load2 = (g2 + cus - 1) / cus * per2, load = (g + cus - 1) / cus * per;
            if (load2 * 1035 < load * 1000) {
                per = per2;
                pl.slots = 2;
                pl.ring = 2;
            }
        }
        pl.groups = (rows + per - 1) / per;
        pl.gpb = pl.groups;
        pl.blk_rows = rows;
        pl.group_stride = per;
        pl.step = 1;
        pl.span = per;
    }
    pl.blocks = L.waves == 1 ? (pl.groups + 3) / 4 : pl.groups;
    return pl;
}

Plan decide(Op op, int64_t rows, int64_t H, int64_t T, const int64_t resident[3], int64_t cus) {
    return plan_launch(op, rows, H, T, resident[0], resident[1], resident[2], cus);
}

namespace {

KernelFn pick_op(Op op, const Layout& L, bool weight, int ring) {
    return op == OP_LN     ? pick<OP_LN>(L, false, ring)
           : op == OP_RMS  ? pick<OP_RMS>(L, weight, ring)
           : op == OP_RG   ? pick<OP_RG>(L, weight, ring)
           : op == OP_RGLN ? pick<OP_RGLN>(L, false, ring)
           : op == OP_LNQ  ? pick<OP_LNQ>(L, false, ring)
                           : nullptr;
}

}  // namespace

bool device_plan(Op op, int64_t rows, int64_t H, int64_t T, bool weight, Plan* pl,
                 int64_t resident[3], int64_t* cus_out) {
    const Layout L = layout_of(H);
    KernelFn deep = pick_op(op, L, weight, 0);
    if (!deep) return false;
    // one-wave rows: four independent waves per workgroup; else one row group per
    // workgroup of W waves
    const int block = L.waves == 1 ? 256 : 64 * L.waves;
    const int groups_per_block = L.waves == 1 ? 4 : 1;
    int blocks_per_cu = 0, cus = 0;
    if (!occupancy(reinterpret_cast<const void*>(deep), block, &blocks_per_cu, &cus)) {
        (void)hipGetLastError();
        return false;
    }
    resident[0] = (int64_t)cus * blocks_per_cu * groups_per_block;
    // the optional kernels (one-slot ring, two-row ring): one whose query fails is not
    // used, and its error is cleared so that the launch reports only its own
    for (int ring = 1; ring <= 2; ++ring) {
        resident[ring] = 0;
        KernelFn fn = pick_op(op, L, weight, ring);
        int bpc = 0, c2 = 0;
        if (!fn) continue;
        if (occupancy(reinterpret_cast<const void*>(fn), block, &bpc, &c2))
            resident[ring] = (int64_t)c2 * bpc * groups_per_block;
        else
            (void)hipGetLastError();
    }
    *cus_out = cus;
    *pl = decide(op, rows, H, T, resident, cus);
    return true;
}

hipError_t launch(Op op, const Params& p_in, hipStream_t stream) {
    const bool weight = p_in.weight != nullptr;
    Plan pl;
    int64_t resident[3], cus = 0;
    if (!device_plan(op, p_in.rows, p_in.H, p_in.T, weight, &pl, resident, &cus))
        return hipErrorInvalidDeviceFunction;
    if (pl.blocks * pl.block_threads > int64_t(0xFFFFFFFF)) return hipErrorInvalidValue;
    KernelFn fn = pick_op(op, layout_of(p_in.H), weight, pl.ring);
    if (!fn) return hipErrorInvalidValue;
    Params p = p_in;
    p.groups = pl.groups;
    p.gpb = pl.gpb;
    p.blk_rows = pl.blk_rows;
    p.group_stride = pl.group_stride;
    p.step = pl.step;
    p.span = pl.span;
    hipLaunchKernelGGL(fn, dim3((unsigned)pl.blocks), dim3(pl.block_threads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_diag_round(const float* in, uint16_t* out, int64_t n, hipStream_t stream) {
    const int64_t blocks = n / 256 + 1 < 65536 ? n / 256 + 1 : 65536;
    hipLaunchKernelGGL(diag_round, dim3((unsigned)blocks), dim3(256), 0, stream, in, out, n);
    return hipGetLastError();
}

hipError_t launch_diag_finalize(const float* in, float* out, int64_t n, int64_t H, float eps,
                                hipStream_t stream) {
    const int64_t blocks = n / 256 + 1 < 65536 ? n / 256 + 1 : 65536;
    hipLaunchKernelGGL(diag_finalize, dim3((unsigned)blocks), dim3(256), 0, stream, in, out, n,
                       (float)H, eps);
    return hipGetLastError();
}

hipError_t launch_diag_quant(const float* in, uint8_t* out, int64_t n, const float* qscale,
                             hipStream_t stream) {
    const int64_t n4 = n / 4;
    const int64_t blocks = n4 / 256 + 1 < 65536 ? n4 / 256 + 1 : 65536;
    hipLaunchKernelGGL(diag_quant, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const float4*>(in), reinterpret_cast<u32*>(out), n4,
                       qscale);
    return hipGetLastError();
}

}  // namespace adaln
