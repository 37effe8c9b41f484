// adaln_kernels.hip -- gfx950 kernels of libadaln: LayerNorm / RMSNorm fused with
// the adaLN modulate epilogue, optionally preceded by the residual-gate prologue.
//
// One row is owned by one wave (H < 4096) or by one workgroup of 4 waves
// (H >= 4096).  The row is read from HBM once with 16-byte loads and kept in
// registers; the statistic is reduced in the fixed order of the numerics contract
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
// expansions (__builtin_sqrtf and '/'; HIP's __fsqrt_rn is the approximate one).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "adaln_internal.hpp"

namespace adaln {
namespace {

using u32 = uint32_t;

// ---------------------------------------------------------------------------
// bf16 <-> binary32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf_lo(u32 p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf_hi(u32 p) { return __uint_as_float(p & 0xFFFF0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round two binary32 values to bf16, nearest-even (v_cvt_pk_bf16_f32), lo in bits 0..15.
__device__ __forceinline__ u32 pack_bf16(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(u32, r);
}

__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st16(uint16_t* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ __forceinline__ u32 word(const uint4& v, int j) {
    return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------------------
// cross-lane moves for the butterfly
// ---------------------------------------------------------------------------
// DPP controls: quad_perm [1,0,3,2] reads lane t^1; quad_perm [2,3,0,1] reads
// t^2; row_half_mirror reads 7-i within 8 lanes and row_mirror 15-i within 16.
// After the earlier levels all lanes of a group hold equal bits, so the mirrors
// deliver the partner group's value exactly as t^4 and t^8 would.
constexpr int DPP_XOR1 = 0xB1;
constexpr int DPP_XOR2 = 0x4E;
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float readlane(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// ---------------------------------------------------------------------------
// statistics
// ---------------------------------------------------------------------------
struct Welford {
    float n, mean, m2;
};

// Chan pairwise combine of (lo, hi) in that order; an empty side yields the other.
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

// One in-row butterfly level at distance K (1, 2, 4 or 8) for Welford partials.
template <int K, int CTRL>
__device__ __forceinline__ Welford welford_level(const Welford& me, int lane) {
    Welford other{dpp<CTRL>(me.n), dpp<CTRL>(me.mean), dpp<CTRL>(me.m2)};
    const bool upper = (lane & K) != 0;
    Welford lo{upper ? other.n : me.n, upper ? other.mean : me.mean, upper ? other.m2 : me.m2};
    Welford hi{upper ? me.n : other.n, upper ? me.mean : other.mean, upper ? me.m2 : other.m2};
    return combine(lo, hi);
}

__device__ __forceinline__ Welford readlane(const Welford& w, int lane) {
    return Welford{readlane(w.n, lane), readlane(w.mean, lane), readlane(w.m2, lane)};
}

// Butterfly over the 64 lanes of a wave (distances 1..32).  Distances 16 and 32
// combine the four uniform rows of 16 lanes: ((r0 (+) r1) (+) (r2 (+) r3)).
__device__ __forceinline__ float wave_sum(float s) {
    s = s + dpp<DPP_XOR1>(s);
    s = s + dpp<DPP_XOR2>(s);
    s = s + dpp<DPP_HALF_MIRROR>(s);
    s = s + dpp<DPP_MIRROR>(s);
    const float r0 = readlane(s, 0), r1 = readlane(s, 16);
    const float r2 = readlane(s, 32), r3 = readlane(s, 48);
    const float a = r0 + r1;
    const float b = r2 + r3;
    return a + b;
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

// rstd = RN(1 / RN(sqrt(RN(stat + eps)))), correctly rounded steps.
__device__ __forceinline__ float finalize(float stat, float eps) {
    const float v = stat + eps;
    const float root = __builtin_sqrtf(v);
    return 1.0f / root;
}

// ---------------------------------------------------------------------------
// the fused row kernel
// ---------------------------------------------------------------------------
// OP: Op; W: waves per row; C: chunks per lane; TAIL: the last chunk is partial;
// WEIGHT: RMS weight present.  256 threads per workgroup.
template <int OP, int W, int C, bool TAIL, bool WEIGHT>
__global__ __launch_bounds__(256) void fused_norm_modulate(Params p) {
    constexpr int P = 64 * W;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t group = (W == 1) ? (int64_t)blockIdx.x * 4 + wave : (int64_t)blockIdx.x;
    if (W == 1 && group >= p.groups) return;  // whole wave leaves (no barriers when W == 1)
    const int64_t row_begin = group * p.rows / p.groups;
    const int64_t row_end = (group + 1) * p.rows / p.groups;
    const int t = (W == 1) ? lane : wave * 64 + lane;  // lane index within the row
    const int64_t H = p.H;
    const float Hf = (float)H;

    __shared__ float xwave[2][4][3];  // cross-wave partials, double-buffered by row parity

    for (int64_t row = row_begin; row < row_end; ++row) {
        const int64_t b = row / p.T;
        const int64_t base = row * H;

        // A1 (+A2): load the row once; the gated variant forms r and stores it.
        uint4 xb[C];
        bool ok[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int col = c * 8 * P + 8 * t;
            ok[c] = !TAIL || c < C - 1 || col < H;
            xb[c] = make_uint4(0u, 0u, 0u, 0u);
            if (ok[c]) {
                uint4 v = ld16(p.x + base + col);
                if (OP == OP_RG) {
                    const uint4 rs = ld16(p.res + base + col);
                    const uint4 g = ld16(p.gate + b * p.gate_bs + col);
                    u32 rr[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const u32 gw = word(g, j), xw = word(v, j), rw = word(rs, j);
                        const float g0 = bf_lo(gw) * bf_lo(xw);
                        const float g1 = bf_hi(gw) * bf_hi(xw);
                        const u32 gx = pack_bf16(g0, g1);
                        const float r0 = bf_lo(rw) + bf_lo(gx);
                        const float r1 = bf_hi(rw) + bf_hi(gx);
                        rr[j] = pack_bf16(r0, r1);
                    }
                    v = make_uint4(rr[0], rr[1], rr[2], rr[3]);
                    st16(p.r + base + col, v);
                }
                xb[c] = v;
            }
        }

        // A3: per-lane ordered statistic, b-major then v-minor.
        float mean = 0.0f, rstd;
        if (OP == OP_LN) {
            Welford w{0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int c = 0; c < C; ++c) {
                if (!ok[c]) continue;
#pragma unroll
                for (int v = 0; v < 8; ++v) {
                    const u32 wd = word(xb[c], v >> 1);
                    const float x = (v & 1) ? bf_hi(wd) : bf_lo(wd);
                    const float rho = 1.0f / (float)(c * 8 + v + 1);  // RN(1/n), folded
                    const float d = x - w.mean;
                    const float step = d * rho;
                    w.mean = w.mean + step;
                    const float e = x - w.mean;
                    const float q = d * e;
                    w.m2 = w.m2 + q;
                }
            }
            w.n = TAIL ? (ok[C - 1] ? 8.0f * C : 8.0f * (C - 1)) : 8.0f * C;
            // A4: wave butterfly; A5: cross-wave pairs through LDS.
            w = wave_welford(w, lane);
            if (W > 1) {
                const int par = (int)((row - row_begin) & 1);
                if (lane == 0) {
                    xwave[par][wave][0] = w.n;
                    xwave[par][wave][1] = w.mean;
                    xwave[par][wave][2] = w.m2;
                }
                __syncthreads();
                Welford q[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    q[i] = Welford{xwave[par][i][0], xwave[par][i][1], xwave[par][i][2]};
                w = combine(combine(q[0], q[1]), combine(q[2], q[3]));
            }
            // A6
            mean = w.mean;
            rstd = finalize(w.m2 / Hf, p.eps);
        } else {
            float s = 0.0f;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                if (!ok[c]) continue;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32 wd = word(xb[c], j);
                    const float x0 = bf_lo(wd), x1 = bf_hi(wd);
                    const float q0 = x0 * x0;
                    s = s + q0;
                    const float q1 = x1 * x1;
                    s = s + q1;
                }
            }
            s = wave_sum(s);
            if (W > 1) {
                const int par = (int)((row - row_begin) & 1);
                if (lane == 0) xwave[par][wave][0] = s;
                __syncthreads();
                const float a = xwave[par][0][0] + xwave[par][1][0];
                const float bb = xwave[par][2][0] + xwave[par][3][0];
                s = a + bb;
            }
            rstd = finalize(s / Hf, p.eps);
        }

        // A7 + A8: normalise from registers, modulate, 16-byte stores.
        const uint16_t* sc_row = p.scale + b * p.scale_bs;
        const uint16_t* sh_row = p.shift + b * p.shift_bs;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if (!ok[c]) continue;
            const int col = c * 8 * P + 8 * t;
            const uint4 sc = ld16(sc_row + col);
            const uint4 sh = ld16(sh_row + col);
            uint4 wv = make_uint4(0u, 0u, 0u, 0u);
            if (WEIGHT) wv = ld16(p.weight + col);
            u32 out[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32 xw = word(xb[c], j);
                float n0, n1;
                if (OP == OP_LN) {
                    const float d0 = bf_lo(xw) - mean;
                    const float d1 = bf_hi(xw) - mean;
                    n0 = d0 * rstd;
                    n1 = d1 * rstd;
                } else {
                    n0 = bf_lo(xw) * rstd;
                    n1 = bf_hi(xw) * rstd;
                    if (WEIGHT) {
                        const u32 ww = word(wv, j);
                        const float w0 = bf_lo(ww) + 0.0f;  // (w + 0.0): -0 -> +0
                        const float w1 = bf_hi(ww) + 0.0f;
                        n0 = n0 * w0;
                        n1 = n1 * w1;
                    }
                }
                const u32 yn = pack_bf16(n0, n1);
                const u32 scw = word(sc, j);
                const u32 a = pack_bf16(1.0f + bf_lo(scw), 1.0f + bf_hi(scw));
                const u32 pr = pack_bf16(bf_lo(yn) * bf_lo(a), bf_hi(yn) * bf_hi(a));
                const u32 shw = word(sh, j);
                out[j] = pack_bf16(bf_lo(pr) + bf_lo(shw), bf_hi(pr) + bf_hi(shw));
            }
            st16(p.y + base + col, make_uint4(out[0], out[1], out[2], out[3]));
        }
    }
}

__global__ __launch_bounds__(256) void diag_round(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        out[i] = (uint16_t)(pack_bf16(in[i], 0.0f) & 0xFFFFu);
}

__global__ __launch_bounds__(256) void diag_finalize(const float* in, float* out, int64_t n,
                                                     float eps) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        out[i] = finalize(in[i], eps);
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
using KernelFn = void (*)(Params);

template <int OP, int W, int C, bool TAIL>
KernelFn pick_weight(bool weight) {
    if (OP == OP_LN) return fused_norm_modulate<OP, W, C, TAIL, false>;
    return weight ? fused_norm_modulate<OP, W, C, TAIL, true>
                  : fused_norm_modulate<OP, W, C, TAIL, false>;
}

template <int OP, int W, int C>
KernelFn pick_tail(bool tail, bool weight) {
    return tail ? pick_weight<OP, W, C, true>(weight) : pick_weight<OP, W, C, false>(weight);
}

template <int OP>
KernelFn pick(const Layout& L, bool weight) {
    if (L.waves == 1) {
        switch (L.chunks) {
            case 1: return pick_tail<OP, 1, 1>(L.ragged, weight);
            case 2: return pick_tail<OP, 1, 2>(L.ragged, weight);
            case 3: return pick_tail<OP, 1, 3>(L.ragged, weight);
            case 4: return pick_tail<OP, 1, 4>(L.ragged, weight);
            case 5: return pick_tail<OP, 1, 5>(L.ragged, weight);
            case 6: return pick_tail<OP, 1, 6>(L.ragged, weight);
            case 7: return pick_tail<OP, 1, 7>(L.ragged, weight);
            case 8: return pick_tail<OP, 1, 8>(L.ragged, weight);
        }
    } else {
        switch (L.chunks) {
            case 2: return pick_tail<OP, 4, 2>(L.ragged, weight);
            case 3: return pick_tail<OP, 4, 3>(L.ragged, weight);
            case 4: return pick_tail<OP, 4, 4>(L.ragged, weight);
        }
    }
    return nullptr;
}

}  // namespace

Layout layout_of(int64_t H) {
    Layout L;
    L.waves = H < 4096 ? 1 : 4;
    L.lanes = 64 * L.waves;
    L.chunks = (int)((H + 8 * L.lanes - 1) / (8 * L.lanes));
    L.ragged = (H % (8 * L.lanes)) != 0;
    return L;
}

hipError_t launch(Op op, const Params& p_in, hipStream_t stream) {
    const Layout L = layout_of(p_in.H);
    const bool weight = p_in.weight != nullptr;
    KernelFn fn = op == OP_LN ? pick<OP_LN>(L, false)
                : op == OP_RMS ? pick<OP_RMS>(L, weight)
                               : pick<OP_RG>(L, weight);
    if (!fn) return hipErrorInvalidValue;
    Params p = p_in;
    // One row per group; very large inputs give each group a contiguous range.
    const int64_t max_groups = int64_t(1) << 30;
    p.groups = p.rows < max_groups ? p.rows : max_groups;
    const int64_t blocks = L.waves == 1 ? (p.groups + 3) / 4 : p.groups;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_diag_round(const float* in, uint16_t* out, int64_t n, hipStream_t stream) {
    const int64_t blocks = n / 256 + 1 < 65536 ? n / 256 + 1 : 65536;
    hipLaunchKernelGGL(diag_round, dim3((unsigned)blocks), dim3(256), 0, stream, in, out, n);
    return hipGetLastError();
}

hipError_t launch_diag_finalize(const float* in, float* out, int64_t n, float eps,
                                hipStream_t stream) {
    const int64_t blocks = n / 256 + 1 < 65536 ? n / 256 + 1 : 65536;
    hipLaunchKernelGGL(diag_finalize, dim3((unsigned)blocks), dim3(256), 0, stream, in, out, n,
                       eps);
    return hipGetLastError();
}

}  // namespace adaln
