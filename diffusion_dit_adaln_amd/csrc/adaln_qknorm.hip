// adaln_qknorm.hip -- gfx950 kernel of libadaln: per-head RMSNorm of Q and K fused
// with the interleaved rotary embedding (kernels guide, RoPE / QK-norm: the QK-norm
// chain folded into the rotary embedding; Qwen PR report, implementation item 3:
// one kernel does the Q/K RMS reduction and the RoPE from an fp32 cos/sin cache,
// head_dim 128, Q/K read through the packed QKV projection's strided views).
//
// The statistic follows the library's fixed order for H = 128: 16 lanes of the
// 64-lane layout own 8 columns each (lane t: columns 8t .. 8t+7), square them in
// order, and fold the 16 partials by the butterfly at distances 1, 2, 4, 8 (lanes
// past column 128 hold +0 and add nothing).  Here a head is owned by 8 lanes and
// lane l plays the layout's lanes l and l + 8: it keeps their two partials apart,
// folds both at distances 1, 2, 4 across the 8 lanes, and adds them in-lane for
// distance 8, which is the same sum of the same operands.  Then
// yn = bf16(x * rstd * (w + 0)) with one rounding, and each pair (yn[2i], yn[2i+1])
// is rotated by the token's (cos_i, sin_i) in binary32 with every product and sum
// rounded, then rounded once to bf16.
//
// Work: a task is eight consecutive heads of Q or of K of one token, one head per
// 8-lane group of a wave.  The number of waves is a multiple of the tasks per
// token and wave w takes the tasks w, w + waves, ..., so a wave always meets the
// same side and heads (its weights stay in registers) and steps a fixed number of
// tokens.  The next task's loads are issued when the current one's stores leave;
// a task past the last token gets empty descriptors (its loads read zero, its
// stores are dropped), so every pass issues the same memory operations.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "adaln_device.hpp"
#include "adaln_internal.hpp"

namespace adaln {
namespace {

#ifndef ADALN_QK_SLOTS
#define ADALN_QK_SLOTS 1  // tasks in flight per wave (launch tuning; never the bits)
#endif
constexpr int kQKSlots = ADALN_QK_SLOTS;

// A 16-byte load that stays in the caches: every task of a token reads the token's
// cos/sin row, so it is read from HBM about once and then hit in L2 (measured: 3.5%
// faster than streaming it like the activations).
__device__ __forceinline__ uint4 ld16_cached(rsrc_t r, int off) {
    const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(t.x, t.y, t.z, t.w);
}

__global__ __launch_bounds__(256) void qk_rmsnorm_rope(QKParams p) {
    constexpr int D = 128;
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 3;  // head within the task
    const int l = lane & 7;     // columns 8l .. 8l+7 (chunk A) and 64+8l .. 64+8l+7 (B)
    const int64_t wave = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (wave >= p.waves) return;

    // the wave's side and heads (uniform)
    const int64_t j = wave % p.tasks_per_token;
    const bool is_q = j < p.q_tasks;
    const int64_t head0 = 8 * (is_q ? j : j - p.q_tasks);
    const int64_t heads = is_q ? p.heads_q : p.heads_k;
    const uint16_t* in = is_q ? p.q : p.k;
    const int64_t in_tstride = is_q ? p.q_tstride : p.k_tstride;
    uint16_t* out = is_q ? p.q_out : p.k_out;
    const uint16_t* wp = is_q ? p.q_weight : p.k_weight;
    const int64_t tok_step = p.waves / p.tasks_per_token;

    // (w + 0.0) of the lane's 16 columns
    float w[16];
    {
        uint4 a = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u), b = a;  // 1.0
        if (wp) {
            a = ld16(wp + 8 * l);
            b = ld16(wp + 64 + 8 * l);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[2 * i] = bf_lo(word(a, i)) + 0.0f;
            w[2 * i + 1] = bf_hi(word(a, i)) + 0.0f;
            w[8 + 2 * i] = bf_lo(word(b, i)) + 0.0f;
            w[8 + 2 * i + 1] = bf_hi(word(b, i)) + 0.0f;
        }
    }

    // the lane's byte offset in a token's row of heads (chunk B 128 bytes further);
    // heads past the count land past the descriptor's range
    const int off = (int)((head0 + grp) * D * 2) + 16 * l;
    const int in_bytes = (int)(heads * D * 2);
    auto in_rsrc = [&](int64_t t) {
        return t < p.tokens ? make_rsrc(in + t * in_tstride, in_bytes) : make_rsrc(in, 0);
    };
    auto out_rsrc = [&](int64_t t) {
        return t < p.tokens ? make_rsrc(out + t * heads * D, in_bytes) : make_rsrc(out, 0);
    };
    auto cs_rsrc = [&](int64_t t) {
        return t < p.tokens ? make_rsrc(p.cos_sin + t * D, D * 4) : make_rsrc(p.cos_sin, 0);
    };

    struct Slot {
        uint4 xa, xb, ca, cb, sa, sb;
    };
    auto load_task = [&](int64_t t, Slot& sl) {
        const rsrc_t ri = in_rsrc(t);
        sl.xa = ld16_stream(ri, off);
        sl.xb = ld16_stream(ri, off + 128);
        const rsrc_t rc = cs_rsrc(t);
        sl.ca = ld16_cached(rc, 16 * l);        // cos of pairs 4l .. 4l+3
        sl.cb = ld16_cached(rc, 128 + 16 * l);  // cos of pairs 32+4l .. 32+4l+3
        sl.sa = ld16_cached(rc, 256 + 16 * l);  // sin, likewise
        sl.sb = ld16_cached(rc, 384 + 16 * l);
    };

    const rsrc_t r_none = make_rsrc(p.q_out, 0);
    constexpr int S = kQKSlots;
    Slot ring[S];
    const int64_t tok0 = wave / p.tasks_per_token;
#pragma unroll
    for (int k = 0; k < S; ++k) {
        if (k > 0) {  // stand-ins for the previous slot's stores (dropped)
            st16_stream(r_none, kOutOfRange, make_uint4(0u, 0u, 0u, 0u));
            st16_stream(r_none, kOutOfRange - 16, make_uint4(0u, 0u, 0u, 0u));
        }
        load_task(tok0 + k * tok_step, ring[k]);
    }

    // rotate one 8-column chunk: x (bf16 pairs), its 4 cos and 4 sin, weights w8
    auto chunk = [&](const uint4& xv, const uint4& cv, const uint4& sv, const float* w8,
                     float rstd) {
        const float c4[4] = {__uint_as_float(cv.x), __uint_as_float(cv.y),
                             __uint_as_float(cv.z), __uint_as_float(cv.w)};
        const float s4[4] = {__uint_as_float(sv.x), __uint_as_float(sv.y),
                             __uint_as_float(sv.z), __uint_as_float(sv.w)};
        u32 o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float n0 = bf_lo(word(xv, i)) * rstd, n1 = bf_hi(word(xv, i)) * rstd;
            const float a = round_bf16(n0 * w8[2 * i]), b = round_bf16(n1 * w8[2 * i + 1]);
            const float ac = a * c4[i], bs = b * s4[i], bc = b * c4[i], as = a * s4[i];
            const float o1 = ac - bs;
            const float o2 = bc + as;
            o[i] = pack_bf16(o1, o2);
        }
        return make_uint4(o[0], o[1], o[2], o[3]);
    };

    for (int64_t t0 = tok0; t0 < p.tokens; t0 += S * tok_step) {
#pragma unroll
        for (int k = 0; k < S; ++k) {
            const int64_t t = t0 + k * tok_step;
            Slot& sl = ring[k];
            // the arithmetic only for a real task (uniform branch, no memory operation
            // inside); the stores below are issued either way
            uint4 oa = make_uint4(0u, 0u, 0u, 0u), ob = oa;
            if (t < p.tokens) {
                // ordered squares of the two chunks, each chunk's partial folded at
                // distances 1, 2, 4 over the head's 8 lanes, then the two added
                float sa = 0.0f, sb = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float a0 = bf_lo(word(sl.xa, i)), a1 = bf_hi(word(sl.xa, i));
                    const float q0 = a0 * a0;
                    sa = sa + q0;
                    const float q1 = a1 * a1;
                    sa = sa + q1;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float b0 = bf_lo(word(sl.xb, i)), b1 = bf_hi(word(sl.xb, i));
                    const float q0 = b0 * b0;
                    sb = sb + q0;
                    const float q1 = b1 * b1;
                    sb = sb + q1;
                }
                sa = sa + dpp<DPP_XOR1>(sa);
                sb = sb + dpp<DPP_XOR1>(sb);
                sa = sa + dpp<DPP_XOR2>(sa);
                sb = sb + dpp<DPP_XOR2>(sb);
                sa = sa + dpp<DPP_HALF_MIRROR>(sa);
                sb = sb + dpp<DPP_HALF_MIRROR>(sb);
                const float sum = sa + sb;
                const float rstd = finalize(sum / (float)D, p.eps);
                oa = chunk(sl.xa, sl.ca, sl.sa, w, rstd);
                ob = chunk(sl.xb, sl.cb, sl.sb, w + 8, rstd);
            }
            const rsrc_t ro = out_rsrc(t);
            st16_stream(ro, off, oa);
            st16_stream(ro, off + 128, ob);
            load_task(t + S * tok_step, sl);
        }
    }
    // never true (tokens > 0): keeps the ring's last loads inside the loop
    if (p.tokens < 0) {
#pragma unroll
        for (int k = 0; k < S; ++k) {
            st16_stream(r_none, kOutOfRange, ring[k].xa);
            st16_stream(r_none, kOutOfRange, ring[k].xb);
            st16_stream(r_none, kOutOfRange, ring[k].ca);
            st16_stream(r_none, kOutOfRange, ring[k].cb);
            st16_stream(r_none, kOutOfRange, ring[k].sa);
            st16_stream(r_none, kOutOfRange, ring[k].sb);
        }
    }
}

}  // namespace

hipError_t launch_qk(const QKParams& p_in, hipStream_t stream) {
    QKParams p = p_in;
    p.q_tasks = (p.heads_q + 7) / 8;
    p.tasks_per_token = p.q_tasks + (p.heads_k + 7) / 8;
    const int64_t tasks = p.tokens * p.tasks_per_token;
    int blocks_per_cu = 0, cus = 0;
    if (!occupancy(reinterpret_cast<const void*>(qk_rmsnorm_rope), 256, &blocks_per_cu, &cus)) {
        (void)hipGetLastError();  // the query's error is reported as this status only
        return hipErrorInvalidDeviceFunction;
    }
    // as many waves as fit at once (at most one per task), a multiple of the tasks
    // per token; at least one wave per task of a token
    const int64_t slots = (int64_t)blocks_per_cu * cus * 4;
    const int64_t fit = tasks < slots ? tasks : slots;
    p.waves = fit / p.tasks_per_token * p.tasks_per_token;
    if (p.waves < p.tasks_per_token) p.waves = p.tasks_per_token;
    const int64_t blocks = (p.waves + 3) / 4;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(qk_rmsnorm_rope, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace adaln
