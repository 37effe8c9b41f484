// adaln_fold.hpp -- the fixed-order reductions shared by the fused kernels of
// libadaln (gfx950): the Chan pairwise combine of Welford partials and the butterfly
// over a wave's 64 lanes (distances 1..32), for sums of squares and for Welford
// partials, in the order of the numerics contract (include/adaln.h): at distance k
// lane t combines (partial of lane t & ~k, partial of lane t | k) in that order.
// Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include "adaln_device.hpp"

namespace adaln {
namespace {

// ---------------------------------------------------------------------------
// statistics
// ---------------------------------------------------------------------------
struct Welford {
    float n, mean, m2;
};

// Chan pairwise combine of (lo, hi) in that order; an empty side yields the other.
// n = na + nb, delta = mean_b - mean_a, wb = RN(nb/n), mean = mean_a + delta*wb,
// M2 = (M2a + M2b) + (delta*delta)*(na*wb).
__device__ __forceinline__ Welford combine(const Welford& lo, const Welford& hi) {
    const float n = lo.n + hi.n;
    const float delta = hi.mean - lo.mean;
    const float wb = hi.n / n;
    const float step = delta * wb;
    const float mean = lo.mean + step;
    const float msum = lo.m2 + hi.m2;
    const float dd = delta * delta;
    const float nw = lo.n * wb;
    const float corr = dd * nw;
    const float m2 = msum + corr;
    Welford o{n, mean, m2};
    if (hi.n == 0.0f) o = lo;
    if (lo.n == 0.0f) o = hi;
    return o;
}

// The same combine when both sides hold NA > 0 elements (every level of a row
// whose H fills all chunks): wb = RN(NA/2NA) = 1/2 and na*wb = NA/2 exactly, so
// the two constants below give the bits of the general formula.  m2 enters as
// the sum M2a + M2b, which fp32 addition makes independent of operand order.
template <int NA>
__device__ __forceinline__ void combine_equal(float lo_mean, float hi_mean, float m2_sum,
                                              float& mean, float& m2) {
    const float delta = hi_mean - lo_mean;
    const float step = delta * 0.5f;
    mean = lo_mean + step;
    const float dd = delta * delta;
    const float corr = dd * (0.5f * (float)NA);
    m2 = m2_sum + corr;
}

// One in-row butterfly level at distance K (1, 2, 4 or 8) for Welford partials
// with runtime counts (ragged rows).
template <int K, int CTRL>
__device__ __forceinline__ Welford welford_level(const Welford& me, int lane) {
    Welford other{dpp<CTRL>(me.n), dpp<CTRL>(me.mean), dpp<CTRL>(me.m2)};
    const bool upper = (lane & K) != 0;
    Welford lo{upper ? other.n : me.n, upper ? other.mean : me.mean, upper ? other.m2 : me.m2};
    Welford hi{upper ? me.n : other.n, upper ? me.mean : other.mean, upper ? me.m2 : other.m2};
    return combine(lo, hi);
}

// The same level when both partners hold NA elements: the partners are read in
// their fixed order directly (lo from lane t & ~K, hi from lane t | K).
template <int K, int CTRL, int NA>
__device__ __forceinline__ void welford_level_equal(float& mean, float& m2) {
    const float lo = partner_lo<K>(mean);
    const float hi = partner_hi<K>(mean);
    combine_equal<NA>(lo, hi, m2 + dpp<CTRL>(m2), mean, m2);
}

__device__ __forceinline__ Welford readlane(const Welford& w, int lane) {
    return Welford{readlane(w.n, lane), readlane(w.mean, lane), readlane(w.m2, lane)};
}

// Butterfly over the 64 lanes of a wave (distances 1..32).  Distances 16 and 32
// combine the four uniform rows of 16 lanes: ((r0 (+) r1) (+) (r2 (+) r3)), every
// lane ending with the wave's value.
__device__ __forceinline__ float wave_sum(float s) {
    s = s + dpp<DPP_XOR1>(s);
    s = s + dpp<DPP_XOR2>(s);
    s = s + dpp<DPP_HALF_MIRROR>(s);
    s = s + dpp<DPP_MIRROR>(s);
    float lo, hi;
    pair16(s, lo, hi);
    s = lo + hi;
    pair32(s, lo, hi);
    return lo + hi;
}

__device__ __forceinline__ Welford wave_welford(Welford w, int lane) {
    w = welford_level<1, DPP_XOR1>(w, lane);
    w = welford_level<2, DPP_XOR2>(w, lane);
    w = welford_level<4, DPP_HALF_MIRROR>(w, lane);
    w = welford_level<8, DPP_MIRROR>(w, lane);
    const Welford a = combine(readlane(w, 0), readlane(w, 16));
    const Welford b = combine(readlane(w, 32), readlane(w, 48));
    return combine(a, b);
}

// Wave butterfly when every lane holds N elements.
template <int N>
__device__ __forceinline__ void wave_welford_equal(float& mean, float& m2) {
    welford_level_equal<1, DPP_XOR1, N>(mean, m2);
    welford_level_equal<2, DPP_XOR2, 2 * N>(mean, m2);
    welford_level_equal<4, DPP_HALF_MIRROR, 4 * N>(mean, m2);
    welford_level_equal<8, DPP_MIRROR, 8 * N>(mean, m2);
    float mlo, mhi, qlo, qhi;
    pair16(mean, mlo, mhi);
    pair16(m2, qlo, qhi);
    combine_equal<16 * N>(mlo, mhi, qlo + qhi, mean, m2);
    pair32(mean, mlo, mhi);
    pair32(m2, qlo, qhi);
    combine_equal<32 * N>(mlo, mhi, qlo + qhi, mean, m2);
}


}  // namespace
}  // namespace adaln
