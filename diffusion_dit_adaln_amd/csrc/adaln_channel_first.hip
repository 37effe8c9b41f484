// adaln_channel_first.hip -- gfx950 kernels of libadaln: residual gating on the
// channel-first layout (kernels guide, norm variants / residual gating: the
// transposed dense path reads `update` in its logical row-major order through
// on-chip tiles while the residual reads and the output writes stay coalesced on
// their [B, hidden, tokens] layout, with no .contiguous() copy).
//
//   out[b][h][t] = bf16(res[b][h][t] + bf16(gate[b][h] * update[b][t][h]))
//
// A workgroup of 256 threads owns 64 hidden rows of one batch entry and a span of
// tokens.  Phase 1 reads `update` for the span with 16-byte loads along hidden,
// forms g = bf16(gate * update) and writes it to LDS as rows of tokens.  Phase 2
// reads res along tokens with 16-byte loads (eight lanes per hidden row), adds the
// gated values picked from LDS and stores the sums along tokens.
//
// When T % 8 == 0 every residual row starts on a 16-byte boundary and a tile is
// 64 hidden x 64 tokens.  Otherwise row (b, h) starts mis = ((b*H + h)*T) mod 8
// elements past a boundary; phase 2 then walks each row's own aligned 16-byte
// blocks (the tile's eight blocks of row h span the tokens 64j - mis .. 64j - mis
// + 63), so every access is a full aligned 16-byte one except the block that holds
// a row's first or last token together with a neighbouring row's tokens, which is
// accessed element by element.  Phase 1 provides the gated values of the 72 tokens
// 64j - 8 .. 64j + 63 that cover every mis.
//
// The LDS tile is unpadded; the 16-byte chunk of hidden/8 at token row r is stored
// at chunk (hidden/8) XOR (r/8 mod 8), spreading a phase-2 instruction's reads over
// the banks.  Tiles are numbered so that consecutive ones (neighbouring token spans
// of the same hidden rows, which share update rows and cache lines of res and out)
// run on the same XCD: workgroup i goes to XCD i mod 8, so it takes tile
// (i mod 8) * (tiles / 8) + i / 8.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "adaln_device.hpp"
#include "adaln_internal.hpp"

namespace adaln {
namespace {

constexpr int kTile = 64;  // hidden rows per tile
static_assert(kCfTokens % 64 == 0 && kCfTokens >= 64 && kCfTokens <= 256, "tokens per tile");

// The tile of workgroup `bid` under the XCD-aware numbering, or -1 when the grid's
// round-up to a multiple of eight leaves it without one.
__device__ __forceinline__ int64_t tile_of(int64_t bid, int64_t tiles) {
    const int64_t per_xcd = (tiles + 7) / 8;
    const int64_t t = (bid & 7) * per_xcd + (bid >> 3);
    return t < tiles ? t : -1;
}

__device__ __forceinline__ float lds_g(const uint16_t* g16, int row, int hl) {
    const int col = (((hl >> 3) ^ ((row >> 3) & 7)) << 3) | (hl & 7);
    return __uint_as_float((u32)g16[row * kTile + col] << 16);
}

// T % 8 == 0: tiles of 64 hidden x TT tokens, every row 16-byte aligned.
template <int TT>
__global__ __launch_bounds__(256) void residual_gate_cf_aligned(CFParams p, int64_t tiles) {
    const int64_t tile = tile_of(blockIdx.x, tiles);
    if (tile < 0) return;
    const int tid = threadIdx.x;
    const int64_t tiles_h = (p.H + kTile - 1) / kTile;
    const int64_t tiles_t = (p.T + TT - 1) / TT;
    const int64_t b = tile / (tiles_h * tiles_t);
    const int64_t rem = tile - b * tiles_h * tiles_t;
    const int64_t h0 = (rem / tiles_t) * kTile;
    const int64_t t0 = (rem % tiles_t) * TT;

    __shared__ uint4 g_lds[TT][kTile / 8];  // [token][hidden chunk ^ swizzle], 8 bf16 each

    // phase 1: update rows (tokens), 8 lanes x 16 bytes per 64-hidden row
#pragma unroll
    for (int it = 0; it < TT / 32; ++it) {
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

    // phase 2: residual rows (hidden) along tokens; lane tc of a hidden row takes the
    // blocks 8j + tc of 8 tokens, so the 8 lanes cover 64 consecutive tokens per access
    const uint16_t* g16 = reinterpret_cast<const uint16_t*>(&g_lds[0][0]);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int hl = (tid >> 3) + 32 * it;  // local hidden
        const int64_t h = h0 + hl;
        if (h >= p.H) continue;
#pragma unroll
        for (int j = 0; j < TT / 64; ++j) {
            const int tl = 8 * (8 * j + (tid & 7));  // first local token of the lane's block
            const int64_t t = t0 + tl;
            if (t >= p.T) continue;  // T % 8 == 0: a block is all in or all out
            const int64_t off = (b * p.H + h) * p.T + t;
            const uint4 v = ld16_nt(p.res + off);
            u32 o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float s0 = bf_lo(word(v, k)) + lds_g(g16, tl + 2 * k, hl);  // bf16(res + g)
                const float s1 = bf_hi(word(v, k)) + lds_g(g16, tl + 2 * k + 1, hl);
                o[k] = pack_bf16(s0, s1);
            }
            st16_nt(p.out + off, make_uint4(o[0], o[1], o[2], o[3]));
        }
    }
}

// T % 8 != 0: each hidden row walks its own aligned 16-byte blocks; tile j covers the
// row's blocks whose first token lies in TT*j - mis .. TT*j - mis + TT - 1.
template <int TT>
__global__ __launch_bounds__(256) void residual_gate_cf_ragged(CFParams p, int64_t tiles) {
    constexpr int kSpan = TT + 8;  // gated tokens held per tile: TT*j - 8 .. TT*j + TT - 1
    const int64_t tile = tile_of(blockIdx.x, tiles);
    if (tile < 0) return;
    const int tid = threadIdx.x;
    const int64_t tiles_h = (p.H + kTile - 1) / kTile;
    const int64_t tiles_t = (p.T + 7 + TT - 1) / TT;
    const int64_t b = tile / (tiles_h * tiles_t);
    const int64_t rem = tile - b * tiles_h * tiles_t;
    const int64_t h0 = (rem / tiles_t) * kTile;
    const int64_t jt = (rem % tiles_t) * TT;  // TT*j
    const int64_t g0 = jt - 8;                // token of LDS row 0

    __shared__ uint4 g_lds[kSpan][kTile / 8];

    // phase 1: gated values of tokens g0 .. g0 + kSpan - 1 (those inside [0, T))
#pragma unroll
    for (int it = 0; it < (kSpan * 8 + 255) / 256; ++it) {
        const int item = tid + 256 * it;
        if (item >= kSpan * 8) break;
        const int tl = item >> 3;
        const int hc = item & 7;
        const int64_t t = g0 + tl, h = h0 + 8 * hc;
        if (t >= 0 && t < p.T && h < p.H) {
            const uint4 u = ld16_nt(p.update + (b * p.T + t) * p.H + h);
            const uint4 gv = ld16(p.gate + b * p.gate_bs + h);
            u32 w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float ga = bf_lo(word(gv, j)) * bf_lo(word(u, j));
                const float gb = bf_hi(word(gv, j)) * bf_hi(word(u, j));
                w[j] = pack_bf16(ga, gb);  // bf16(gate * update)
            }
            g_lds[tl][hc ^ ((tl >> 3) & 7)] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
    __syncthreads();

    // phase 2: lane tc of hidden row h takes the row's aligned blocks 8m + tc of the tile
    const uint16_t* g16 = reinterpret_cast<const uint16_t*>(&g_lds[0][0]);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int hl = (tid >> 3) + 32 * it;
        const int64_t h = h0 + hl;
        if (h >= p.H) continue;
        const int64_t row = (b * p.H + h) * p.T;   // flat index of token 0 of the row
        const int mis = (int)(row & 7);
#pragma unroll
        for (int m = 0; m < TT / 64; ++m) {
            const int tc = 8 * m + (tid & 7);
            const int64_t tb = jt + 8 * tc - mis;  // token of the block's first element
            if (tb >= p.T) continue;               // the block lies past the row
            const int rb = (int)(tb - g0);         // its LDS row: 1 .. TT
            if (tb >= 0 && tb + 8 <= p.T) {
                const int64_t off = row + tb;      // a multiple of 8: 16-byte aligned
                const uint4 v = ld16_nt(p.res + off);
                u32 o[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float s0 = bf_lo(word(v, k)) + lds_g(g16, rb + 2 * k, hl);
                    const float s1 = bf_hi(word(v, k)) + lds_g(g16, rb + 2 * k + 1, hl);
                    o[k] = pack_bf16(s0, s1);
                }
                st16_nt(p.out + off, make_uint4(o[0], o[1], o[2], o[3]));
            } else {
                // the block shared with the previous or next row: only this row's tokens
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int64_t t = tb + e;
                    if (t < 0 || t >= p.T) continue;
                    const float r =
                        __uint_as_float((u32)__builtin_nontemporal_load(p.res + row + t) << 16);
                    const float sum = r + lds_g(g16, rb + e, hl);
                    __builtin_nontemporal_store((uint16_t)(pack_bf16(sum, 0.0f) & 0xFFFFu),
                                                p.out + row + t);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_cf(const CFParams& p, hipStream_t stream) {
    const int64_t tiles = cf_tiles(p.B, p.H, p.T);
    const int64_t grid = cf_grid(tiles);
    // a grid holds fewer than 2^32 work-items
    if (grid > int64_t(0xFFFFFFFF) / 256) return hipErrorInvalidValue;
    if (p.T % 8 == 0)
        hipLaunchKernelGGL(residual_gate_cf_aligned<kCfTokens>, dim3((unsigned)grid), dim3(256),
                           0, stream, p, tiles);
    else
        hipLaunchKernelGGL(residual_gate_cf_ragged<kCfTokens>, dim3((unsigned)grid), dim3(256),
                           0, stream, p, tiles);
    return hipGetLastError();
}

}  // namespace adaln
