// adaln_qknorm.hip -- gfx950 kernel of libadaln: per-head RMSNorm of Q and K fused
// with the interleaved rotary embedding (kernels guide, RoPE / QK-norm: the QK-norm
// chain folded into the rotary embedding; Qwen PR report, implementation item 3:
// one kernel does the Q/K RMS reduction and the RoPE from an fp32 cos/sin cache,
// head_dim 128, Q/K read through the packed QKV projection's strided views).
//
// A head vector (128 bf16, 256 bytes) is owned by 16 lanes, 8 columns each, so a
// wave processes four heads at a time.  The statistic follows the library's fixed
// order for H = 128: each lane squares its 8 columns in order, the 16 partials are
// folded by the butterfly at distances 1, 2, 4, 8 (the lanes past column 128 of the
// 64-lane layout hold +0 and add nothing).  Then yn = bf16(x * rstd * (w + 0)) with
// one rounding, and each pair (yn[2i], yn[2i+1]) is rotated by the token's
// (cos_i, sin_i) in binary32 with every product and sum rounded, then rounded once
// to bf16.
//
// Work: a task is four consecutive heads of Q or of K of one token.  Waves walk
// the tasks interleaved (wave w takes tasks w, w + G, ...) with the next task's
// loads issued before the current one's arithmetic ends (a ring of S slots); the
// loads and stores of a pass are unconditional (descriptor ranges drop what lies
// past the end, and a slot without a task skips its arithmetic), so each slot
// waits only for its own data.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "adaln_device.hpp"
#include "adaln_internal.hpp"

namespace adaln {
namespace {

// Tasks in flight per wave (launch tuning; never changes the bits).  Measured on
// MI355X: one task per wave, with seven waves per SIMD covering the latency, beats
// deeper rings (1: 4.72 TB/s, 2: 4.57, 3: 4.55, 4: 4.40 on [4608, 24+24, 128]).
#ifndef ADALN_QK_SLOTS
#define ADALN_QK_SLOTS 1
#endif
constexpr int kQKSlots = ADALN_QK_SLOTS;
#ifndef ADALN_QK_OVERSUB
#define ADALN_QK_OVERSUB 1  // waves per resident wave slot
#endif

__global__ __launch_bounds__(256) void qk_rmsnorm_rope(QKParams p) {
    constexpr int D = 128;
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4;  // head within the task
    const int l = lane & 15;    // lane within the head: columns 8l .. 8l+7
    const int64_t wave = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (wave >= p.waves) return;
    const int64_t G = p.waves;

    // weights of Q and K for this lane's 8 columns, (w + 0.0) applied
    float wq[8], wk[8];
    {
        uint4 a = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u), b = a;  // 1.0
        if (p.q_weight) a = ld16(p.q_weight + 8 * l);
        if (p.k_weight) b = ld16(p.k_weight + 8 * l);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            wq[2 * j] = bf_lo(word(a, j)) + 0.0f;
            wq[2 * j + 1] = bf_hi(word(a, j)) + 0.0f;
            wk[2 * j] = bf_lo(word(b, j)) + 0.0f;
            wk[2 * j + 1] = bf_hi(word(b, j)) + 0.0f;
        }
    }

    // task id = token * tasks_per_token + j; tasks j < q_tasks are Q heads 4j..4j+3,
    // the rest K heads.  A slot tracks (token, j) of its task; stepping S*G tasks
    // ahead adds the host's quotient and remainder of S*G by tasks_per_token, so
    // the loop divides nothing.  All uniform over the wave.
    struct Task {
        int64_t token;
        bool is_q;
        int64_t head0;
    };
    auto task_at = [&](int64_t tok, int64_t j) {
        const bool q = j < p.q_tasks;
        return Task{tok, q, 4 * (q ? j : j - p.q_tasks)};
    };
    // descriptors: the task's input heads, its output heads, the token's cache row;
    // a task past the end gets empty ones (its token and head then do not matter)
    auto in_rsrc = [&](int64_t id, const Task& t) {
        if (id >= p.tasks) return make_rsrc(p.q, 0);
        const uint16_t* base = t.is_q ? p.q + t.token * p.q_tstride : p.k + t.token * p.k_tstride;
        return make_rsrc(base, (t.is_q ? p.heads_q : p.heads_k) * D * 2);
    };
    auto out_rsrc = [&](int64_t id, const Task& t) {
        if (id >= p.tasks) return make_rsrc(p.q_out, 0);
        const int64_t h = t.is_q ? p.heads_q : p.heads_k;
        uint16_t* base = (t.is_q ? p.q_out : p.k_out) + t.token * h * D;
        return make_rsrc(base, h * D * 2);
    };
    auto cs_rsrc = [&](int64_t id, const Task& t) {
        if (id >= p.tasks) return make_rsrc(p.cos_sin, 0);
        return make_rsrc(p.cos_sin + t.token * D, D * 4);
    };
    // the lane's offset inside its head's row (heads past the count land out of range)
    auto head_off = [&](const Task& t) { return (int)((t.head0 + grp) * D * 2) + 16 * l; };

    struct Slot {
        uint4 x, c, s;
    };
    auto load_task = [&](int64_t id, const Task& t, Slot& sl) {
        sl.x = ld16_stream(in_rsrc(id, t), head_off(t));
        const rsrc_t rc = cs_rsrc(id, t);
        sl.c = ld16_stream(rc, 16 * l);           // cos[4l .. 4l+3]
        sl.s = ld16_stream(rc, D * 2 + 16 * l);   // sin[4l .. 4l+3]
    };

    const rsrc_t r_none = make_rsrc(p.q_out, 0);
    constexpr int S = kQKSlots;
    Slot ring[S];
    int64_t tok[S], jj[S];
#pragma unroll
    for (int k = 0; k < S; ++k) {
        const int64_t id = wave + k * G;
        tok[k] = id / p.tasks_per_token;
        jj[k] = id - tok[k] * p.tasks_per_token;
        if (k > 0) st16_stream(r_none, kOutOfRange, make_uint4(0u, 0u, 0u, 0u));
        load_task(id, task_at(tok[k], jj[k]), ring[k]);
    }

    for (int64_t id0 = wave; id0 < p.tasks; id0 += S * G) {
#pragma unroll
        for (int k = 0; k < S; ++k) {
            const int64_t id = id0 + k * G;
            Slot& sl = ring[k];
            const Task t = task_at(tok[k], jj[k]);

            // the arithmetic only for a real task (uniform branch, no memory operation
            // inside); the store below is issued either way
            u32 out[4] = {0u, 0u, 0u, 0u};
            if (id < p.tasks) {
            float x[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[2 * j] = bf_lo(word(sl.x, j));
                x[2 * j + 1] = bf_hi(word(sl.x, j));
            }
            // ordered per-lane sum of squares, butterfly over the head's 16 lanes
            float sum = 0.0f;
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                const float q = x[v] * x[v];
                sum = sum + q;
            }
            sum = sum + dpp<DPP_XOR1>(sum);
            sum = sum + dpp<DPP_XOR2>(sum);
            sum = sum + dpp<DPP_HALF_MIRROR>(sum);
            sum = sum + dpp<DPP_MIRROR>(sum);
            const float rstd = finalize(sum / (float)D, p.eps);

            const float c4[4] = {__uint_as_float(sl.c.x), __uint_as_float(sl.c.y),
                                 __uint_as_float(sl.c.z), __uint_as_float(sl.c.w)};
            const float s4[4] = {__uint_as_float(sl.s.x), __uint_as_float(sl.s.y),
                                 __uint_as_float(sl.s.z), __uint_as_float(sl.s.w)};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float w0 = t.is_q ? wq[2 * j] : wk[2 * j];
                const float w1 = t.is_q ? wq[2 * j + 1] : wk[2 * j + 1];
                const float n0 = x[2 * j] * rstd, n1 = x[2 * j + 1] * rstd;
                const float a = round_bf16(n0 * w0), b = round_bf16(n1 * w1);  // yn pair
                const float ac = a * c4[j], bs = b * s4[j], bc = b * c4[j], as = a * s4[j];
                const float o1 = ac - bs;
                const float o2 = bc + as;
                out[j] = pack_bf16(o1, o2);
            }
            }  // id < tasks
            st16_stream(out_rsrc(id, t), head_off(t), make_uint4(out[0], out[1], out[2], out[3]));

            // the slot's task S*G ahead
            tok[k] += p.sg_div;
            jj[k] += p.sg_mod;
            if (jj[k] >= p.tasks_per_token) {
                jj[k] -= p.tasks_per_token;
                tok[k] += 1;
            }
            load_task(id + S * G, task_at(tok[k], jj[k]), sl);
        }
    }
    // never true (tasks > 0): keeps the ring's last loads inside the loop
    if (p.tasks < 0) {
#pragma unroll
        for (int k = 0; k < S; ++k) {
            st16_stream(r_none, kOutOfRange, ring[k].x);
            st16_stream(r_none, kOutOfRange, ring[k].c);
            st16_stream(r_none, kOutOfRange, ring[k].s);
        }
    }
}

}  // namespace

hipError_t launch_qk(const QKParams& p_in, hipStream_t stream) {
    QKParams p = p_in;
    p.q_tasks = (p.heads_q + 3) / 4;
    p.tasks_per_token = p.q_tasks + (p.heads_k + 3) / 4;
    p.tasks = p.tokens * p.tasks_per_token;
    // resident waves, one per task at most
    int blocks_per_cu = 0, cus = 0;
    if (!occupancy(reinterpret_cast<const void*>(qk_rmsnorm_rope), 256, &blocks_per_cu, &cus))
        return hipErrorInvalidDeviceFunction;
    const int64_t slots = (int64_t)blocks_per_cu * cus * 4 * ADALN_QK_OVERSUB;
    p.waves = p.tasks < slots ? p.tasks : slots;
    const int64_t sg = (int64_t)kQKSlots * p.waves;
    p.sg_div = sg / p.tasks_per_token;
    p.sg_mod = sg % p.tasks_per_token;
    const int64_t blocks = (p.waves + 3) / 4;
    hipLaunchKernelGGL(qk_rmsnorm_rope, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace adaln
