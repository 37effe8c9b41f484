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
// sum along tokens (when T % 8 != 0 the token rows are not 16-byte aligned, and
// phase 2 moves 4, 2 or 1 tokens per access, whichever keeps accesses aligned).  The LDS tile is unpadded; a 16-byte column chunk is stored at
// chunk (hidden/8) XOR (token/8 mod 8), so the phase-2 reads of one instruction
// (8 hidden rows x 8 token groups) fall in 32 distinct banks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "adaln_device.hpp"
#include "adaln_internal.hpp"

namespace adaln {
namespace {

constexpr int kTile = 64;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// VEC: tokens per phase-2 access, the largest of 8, 4, 2, 1 that divides T, so that
// every access of a token row of res/out is naturally aligned (a row starts at
// element (b*H + h)*T).  Lane tc of a hidden row takes the token groups 8j + tc
// (j < 8/VEC) of VEC tokens each, so the 8 lanes of a row cover 8*VEC consecutive
// tokens per access.
template <int VEC>
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

    // phase 2: residual rows (hidden) along tokens
    const uint16_t* g16 = reinterpret_cast<const uint16_t*>(&g_lds[0][0]);
    constexpr int NW = VEC >= 2 ? VEC / 2 : 1;  // 32-bit words per access
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int hl = (tid >> 3) + 32 * it;  // local hidden
        const int tc = tid & 7;
        const int64_t h = h0 + hl;
        if (h >= p.H) continue;
#pragma unroll
        for (int j = 0; j < 8 / VEC; ++j) {
            const int tl = VEC * (8 * j + tc);  // first local token of the group
            const int64_t t = t0 + tl;
            if (t >= p.T) continue;  // VEC divides T: the group is all in or all out
            const int64_t off = (b * p.H + h) * p.T + t;
            u32 rw[NW];
            if constexpr (VEC == 8) {
                const uint4 v = ld16_nt(p.res + off);
                rw[0] = v.x; rw[1] = v.y; rw[2] = v.z; rw[3] = v.w;
            } else if constexpr (VEC == 4) {
                const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p.res + off));
                rw[0] = v.x; rw[1] = v.y;
            } else if constexpr (VEC == 2) {
                rw[0] = __builtin_nontemporal_load(reinterpret_cast<const u32*>(p.res + off));
            } else {
                rw[0] = __builtin_nontemporal_load(p.res + off);
            }
            // g of token tl + k at hidden hl: row tl + k, chunk (hl/8) ^ (tl/8 mod 8),
            // slot hl % 8 (the VEC tokens share tl/8)
            const int col = (((hl >> 3) ^ ((tl >> 3) & 7)) << 3) | (hl & 7);
            u32 o[NW];
#pragma unroll
            for (int k = 0; k < NW; ++k) {
                const float ga = __uint_as_float((u32)g16[(tl + 2 * k) * kTile + col] << 16);
                const float s0 = bf_lo(rw[k]) + ga;  // bf16(res + g)
                if constexpr (VEC >= 2) {
                    const float gb = __uint_as_float((u32)g16[(tl + 2 * k + 1) * kTile + col] << 16);
                    const float s1 = bf_hi(rw[k]) + gb;
                    o[k] = pack_bf16(s0, s1);
                } else {
                    o[k] = pack_bf16(s0, 0.0f) & 0xFFFFu;
                }
            }
            if constexpr (VEC == 8) {
                st16_nt(p.out + off, make_uint4(o[0], o[1], o[2], o[3]));
            } else if constexpr (VEC == 4) {
                const u32x2 v = {o[0], o[1]};
                __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p.out + off));
            } else if constexpr (VEC == 2) {
                __builtin_nontemporal_store(o[0], reinterpret_cast<u32*>(p.out + off));
            } else {
                __builtin_nontemporal_store((uint16_t)o[0], p.out + off);
            }
        }
    }
}

}  // namespace

hipError_t launch_cf(const CFParams& p, hipStream_t stream) {
    const int64_t tiles = p.B * ((p.H + kTile - 1) / kTile) * ((p.T + kTile - 1) / kTile);
    // a grid holds fewer than 2^32 work-items
    if (tiles > int64_t(0xFFFFFFFF) / 256) return hipErrorInvalidValue;
    const dim3 grid((unsigned)tiles), block(256);
    if (p.T % 8 == 0)
        hipLaunchKernelGGL(residual_gate_cf<8>, grid, block, 0, stream, p);
    else if (p.T % 4 == 0)
        hipLaunchKernelGGL(residual_gate_cf<4>, grid, block, 0, stream, p);
    else if (p.T % 2 == 0)
        hipLaunchKernelGGL(residual_gate_cf<2>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(residual_gate_cf<1>, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace adaln
