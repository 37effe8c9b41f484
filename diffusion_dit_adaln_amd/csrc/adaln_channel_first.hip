// adaln_channel_first.hip -- gfx950 kernel of libadaln: residual gating on the
// channel-first layout (kernels guide, norm variants / residual gating: the
// transposed dense path reads `update` in its logical row-major order through
// on-chip tiles while the residual reads and the output writes stay coalesced on
// their [B, hidden, tokens] layout, with no .contiguous() copy).
//
//   out[b][h][t] = bf16(res[b][h][t] + bf16(gate[b][h] * update[b][t][h]))
//
// A workgroup of 256 threads owns a 64 (hidden) x 64 (tokens) tile of one batch
// entry.  Phase 1 reads the tile of `update` with 16-byte loads along hidden,
// forms g = bf16(gate * update) and writes it to LDS as rows of tokens (16-byte
// writes).  Phase 2 reads res along tokens (16-byte loads, eight lanes cover one
// 128-byte hidden row), picks g for its (hidden, 8 tokens) from LDS and stores the
// sum along tokens (with T % 8 != 0 the token rows are not 16-byte aligned and
// phase 2 moves single elements instead).  The LDS tile is unpadded; a 16-byte column chunk is stored at
// chunk (hidden/8) XOR (token/8 mod 8), so the phase-2 reads of one instruction
// (8 hidden rows x 8 token groups) fall in 32 distinct banks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "adaln_device.hpp"
#include "adaln_internal.hpp"

namespace adaln {
namespace {

constexpr int kTile = 64;

// RAGGED: T % 8 != 0, so a token row of res/out is not 16-byte aligned; phase 2
// then moves one element per access (lane tc of a hidden row takes the tokens
// 8j + tc, so each access of the 8 lanes covers 8 consecutive tokens).
template <bool RAGGED>
__global__ __launch_bounds__(256) void residual_gate_cf(CFParams p) {
    const int tid = threadIdx.x;
    const int64_t tiles_h = (p.H + kTile - 1) / kTile;
    const int64_t tiles_t = (p.T + kTile - 1) / kTile;
    const int64_t tile = blockIdx.x;
    const int64_t b = tile / (tiles_h * tiles_t);
    const int64_t rem = tile - b * tiles_h * tiles_t;
    const int64_t h0 = (rem / tiles_t) * kTile;
    const int64_t t0 = (rem % tiles_t) * kTile;

    __shared__ uint4 g_lds[kTile][kTile / 8];  // [token][hidden chunk ^ swizzle], 8 bf16 each

    // phase 1: update rows (tokens), 8 lanes x 16 bytes per 64-hidden row
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int tl = (tid >> 3) + 32 * it;  // local token
        const int hc = tid & 7;               // hidden chunk of 8
        const int64_t t = t0 + tl, h = h0 + 8 * hc;
        uint4 g = make_uint4(0u, 0u, 0u, 0u);
        if (t < p.T && h < p.H) {
            const uint4 u = ld16_nt(p.update + (b * p.T + t) * p.H + h);
            const uint4 gv = ld16(p.gate + b * p.gate_bs + h);
            u32 w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float g0 = bf_lo(word(gv, j)) * bf_lo(word(u, j));
                const float g1 = bf_hi(word(gv, j)) * bf_hi(word(u, j));
                w[j] = pack_bf16(g0, g1);  // bf16(gate * update)
            }
            g = make_uint4(w[0], w[1], w[2], w[3]);
        }
        g_lds[tl][hc ^ ((tl >> 3) & 7)] = g;
    }
    __syncthreads();

    // phase 2: residual rows (hidden), 8 lanes x 16 bytes per 64-token row
    const uint16_t* g16 = reinterpret_cast<const uint16_t*>(&g_lds[0][0]);
    if (RAGGED) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int hl = (tid >> 3) + 32 * it;  // local hidden
            const int tc = tid & 7;
            const int64_t h = h0 + hl;
            if (h >= p.H) continue;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int tl = 8 * j + tc;  // local token
                const int64_t t = t0 + tl;
                if (t >= p.T) continue;
                const int64_t off = (b * p.H + h) * p.T + t;
                const float r = __uint_as_float((u32)__builtin_nontemporal_load(p.res + off) << 16);
                // g of token tl at hidden hl: row tl, chunk (hl/8) ^ (tl/8 mod 8), slot hl%8
                const int col = (((hl >> 3) ^ j) << 3) | (hl & 7);
                const float g = __uint_as_float((u32)g16[tl * kTile + col] << 16);
                const float s = r + g;
                __builtin_nontemporal_store((uint16_t)(pack_bf16(s, 0.0f) & 0xFFFFu), p.out + off);
            }
        }
        return;
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int hl = (tid >> 3) + 32 * it;  // local hidden
        const int tc = tid & 7;               // token group of 8
        const int64_t h = h0 + hl, t = t0 + 8 * tc;
        if (h >= p.H || t >= p.T) continue;
        const int64_t off = (b * p.H + h) * p.T + t;
        const uint4 r = ld16_nt(p.res + off);
        // g of tokens 8tc .. 8tc+7 at hidden hl: row 8tc+k, chunk (hl/8) ^ tc, slot hl%8
        const int col = (((hl >> 3) ^ tc) << 3) | (hl & 7);
        u32 o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float ga = __uint_as_float((u32)g16[(8 * tc + 2 * j) * kTile + col] << 16);
            const float gb = __uint_as_float((u32)g16[(8 * tc + 2 * j + 1) * kTile + col] << 16);
            const float s0 = bf_lo(word(r, j)) + ga;
            const float s1 = bf_hi(word(r, j)) + gb;
            o[j] = pack_bf16(s0, s1);  // bf16(res + g)
        }
        st16_nt(p.out + off, make_uint4(o[0], o[1], o[2], o[3]));
    }
}

}  // namespace

hipError_t launch_cf(const CFParams& p, hipStream_t stream) {
    const int64_t tiles = p.B * ((p.H + kTile - 1) / kTile) * ((p.T + kTile - 1) / kTile);
    // a grid holds fewer than 2^32 work-items
    if (tiles > int64_t(0xFFFFFFFF) / 256) return hipErrorInvalidValue;
    if (p.T % 8 == 0)
        hipLaunchKernelGGL(residual_gate_cf<false>, dim3((unsigned)tiles), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(residual_gate_cf<true>, dim3((unsigned)tiles), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace adaln
