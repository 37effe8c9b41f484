// adaln_channel_first.hip -- gfx950 kernel of libadaln: residual gating on the
// channel-first layout (kernels guide, norm variants / residual gating: the
// transposed dense path reads `update` in its logical row-major order through
// on-chip tiles while the residual reads and the output writes stay coalesced on
// their [B, hidden, tokens] layout, with no .contiguous() copy).
//
//   out[b][h][t] = bf16(res[b][h][t] + bf16(gate[b][h] * update[b][t][h]))
//
// A workgroup of 256 threads owns 64 hidden rows of one batch entry and a span of
// kCfTokens tokens of each of them.  Each lane owns whole 16-byte blocks of residual
// rows: lane 8i + k of the workgroup takes block k (and k + 8, ... for wider tiles)
// of hidden rows i and i + 32, so the eight lanes of a row cover 128 consecutive
// bytes per access.  A row's blocks start on a kCfAlign-element boundary of the flat
// tensor: row (b, h) starts mis = ((b*H + h)*T) mod kCfAlign elements past one, and
// in tile j it takes the blocks whose first token lies in
// kCfTokens*j - mis .. kCfTokens*j - mis + kCfTokens - 1, so the eight lanes of a row
// cover whole 128-byte lines.  Every residual load is a whole aligned 16-byte access
// (a block that also holds a neighbouring row's tokens, when T % 8 != 0, is loaded
// whole and only this row's halfwords are used; only a block reaching past the end of
// the tensor is gathered element by element), and so is every output store except
// those of the blocks shared with a neighbouring row, which are stored element by
// element.
//
// Order of work: the lane first issues its loads of `update` (two tokens x 8 hidden
// values per item, 16-byte loads along hidden; cached when the rows are not all
// aligned, since a tile then reads kCfAlign update rows that the tile before it
// also read, non-temporal otherwise), then its residual blocks, so both
// streams are in flight together; it forms g = bf16(gate * update) as soon as the
// update values arrive and writes them to LDS as rows of hidden, two tokens per
// 32-bit word; after one barrier it adds, to each residual block, the eight gated
// values of the same row and tokens read from LDS, and stores the sums.  The LDS
// rows hold the tile's tokens from kCfTokens*j - kCfAlign on (just kCfTokens*j on
// when every row is aligned), unshifted, so a block's eight values are consecutive
// halfwords read from one address with immediate offsets whatever its row's mis.
// The row stride is 4 bytes past a multiple of 32, which puts the eight hidden rows
// of a phase-1 write instruction on distinct banks.
//
// Tiles are numbered so that consecutive ones (neighbouring token spans of the same
// hidden rows, which share update rows and cache lines of res and out) run on the
// same XCD: workgroup i goes to XCD i mod 8, so it takes tile
// (i mod 8) * ceil(tiles / 8) + i / 8.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "adaln_device.hpp"
#include "adaln_internal.hpp"

namespace adaln {
namespace {

constexpr int kTile = 64;  // hidden rows per tile
static_assert(kCfTokens == 64 || kCfTokens == 128, "tokens per tile");
static_assert(kCfAlign == 8 || kCfAlign == 64, "block alignment");

// LDS row stride in bytes for n tokens: 4 past a multiple of 32.
constexpr int lds_stride(int n) { return (n * 2) % 32 == 0 ? n * 2 + 4 : n * 2 + 20; }

__device__ __forceinline__ float bf_at(const uint16_t* p, int i) {
    return __uint_as_float((u32)p[i] << 16);
}

// MIS: rows may start off a kCfAlign boundary (T % kCfAlign != 0).  EDGES: a block
// can hold tokens of two rows (T % 8 != 0).
template <int TT, bool MIS, bool EDGES>
__global__ __launch_bounds__(256) void residual_gate_cf(CFParams p, u32 tiles, u32 tiles_t,
                                                        u32 tiles_b) {
    constexpr int kLead = MIS ? (int)kCfAlign : 0;  // tokens held before the tile's first
    constexpr int kRow = TT + kLead;                 // tokens held per hidden row
    constexpr int kStride = lds_stride(kRow);        // bytes
    constexpr int kBlocks = TT / 64;                 // blocks per lane and hidden row
    constexpr int kItems = kRow / 2 * 8;             // phase-1 items: token pair x chunk
    constexpr int kIter = (kItems + 255) / 256;
    __shared__ __align__(16) u32 lds[kTile * kStride / 4];

    const u32 bid = blockIdx.x;
    const u32 tile = (bid & 7u) * ((tiles + 7u) / 8u) + (bid >> 3);
    if (tile >= tiles) return;  // the grid's round-up to a multiple of eight
    const u32 bq = tile / tiles_b;
    const u32 rem = tile - bq * tiles_b;
    const u32 hq = rem / tiles_t;
    const int64_t b = bq;
    const int64_t h0 = (int64_t)hq * kTile;
    const int64_t jt = (int64_t)(rem - hq * tiles_t) * TT;  // the tile's first token
    const int64_t g0 = jt - kLead;                          // token of LDS column 0
    const int tid = threadIdx.x;

    // phase-1 loads: item tid + 256*it is tokens g0 + 2u, g0 + 2u + 1 (u = item / 8) of
    // hidden chunk hc = tid % 8
    const int hc = tid & 7;
    const int64_t hg = h0 + 8 * hc;
    const bool h_in = hg < p.H;
    const uint4 gv = ld16(h_in ? p.gate + b * p.gate_bs + hg : p.gate);
    // every load is issued unconditionally (a token or hidden chunk outside the tensor
    // reads the tensor's first block instead, and its values are never used), so no
    // load result shares registers with a default value and the waits stay exact; the
    // gate first, then update, then res, so that phase 1 waits for neither res nor a
    // later load
    uint4 ua[kIter], uc[kIter];
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
        const int u = (tid + 256 * it) >> 3;
        const int64_t t0 = g0 + 2 * u;
        const bool ok = h_in && (kItems % 256 == 0 || tid + 256 * it < kItems);
        const bool ok0 = ok && t0 >= 0 && t0 < p.T, ok1 = ok && t0 + 1 >= 0 && t0 + 1 < p.T;
        const uint16_t* a0 = ok0 ? p.update + (b * p.T + t0) * p.H + hg : p.update;
        const uint16_t* a1 = ok1 ? p.update + (b * p.T + t0 + 1) * p.H + hg : p.update;
        ua[it] = MIS ? ld16(a0) : ld16_nt(a0);
        uc[it] = MIS ? ld16(a1) : ld16_nt(a1);
    }

    // residual blocks: hidden row hl = tid/8 + 32*it, block k = tid%8 + 8*m.  A block
    // holding tokens of two rows is still loaded whole (the other row's halfwords are
    // not used); only the block reaching past the end of the tensor (the last block of
    // a launch, when B*H*T % 8 != 0) is gathered element by element, after the barrier
    const int64_t total = p.B * p.H * p.T;
    uint4 rv[2][kBlocks];
    int64_t row[2];          // flat index of token 0 of the row
    int64_t tb[2][kBlocks];  // token of the block's first element
    int col[2][kBlocks];     // LDS column of that element; -1: no block
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int64_t h = h0 + (tid >> 3) + 32 * it;
        row[it] = (b * p.H + h) * p.T;
        const int mis = MIS ? (int)((u32)row[it] & (u32)(kCfAlign - 1)) : 0;
#pragma unroll
        for (int m = 0; m < kBlocks; ++m) {
            const int k = (tid & 7) + 8 * m;
            const int64_t t = jt - mis + 8 * k;
            const bool live = h < p.H && t < p.T && t + 8 > 0;
            const bool fits = !EDGES || row[it] + t + 8 <= total;
            tb[it][m] = t;
            col[it][m] = live ? kLead - mis + 8 * k : -1;
            rv[it][m] = ld16_nt(live && fits ? p.res + row[it] + t : p.res);
        }
    }

    // phase 1: g = bf16(gate * update), rows of hidden, two tokens per word
    float gf[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        gf[2 * q] = bf_lo(word(gv, q));
        gf[2 * q + 1] = bf_hi(word(gv, q));
    }
    u32* lrow = lds + 8 * hc * (kStride / 4);
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
        if (kItems % 256 != 0 && tid + 256 * it >= kItems) break;
        const int u = (tid + 256 * it) >> 3;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32 a = word(ua[it], q), c = word(uc[it], q);
            lrow[(2 * q) * (kStride / 4) + u] = pack_bf16(gf[2 * q] * bf_lo(a), gf[2 * q] * bf_lo(c));
            lrow[(2 * q + 1) * (kStride / 4) + u] =
                pack_bf16(gf[2 * q + 1] * bf_hi(a), gf[2 * q + 1] * bf_hi(c));
        }
    }
    __syncthreads();

    // phase 2: sums of the residual blocks and the gated values of their tokens
    const uint16_t* l16 = reinterpret_cast<const uint16_t*>(lds);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int hl = (tid >> 3) + 32 * it;
#pragma unroll
        for (int m = 0; m < kBlocks; ++m) {
            if (col[it][m] < 0) continue;
            const uint16_t* g = l16 + hl * (kStride / 2) + col[it][m];
            const int64_t t = tb[it][m];
            uint4 v = rv[it][m];
            if (EDGES && row[it] + t + 8 > total) {
                u32 w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (t + e < p.T)
                        w[e >> 1] |= (u32)__builtin_nontemporal_load(p.res + row[it] + t + e)
                                     << (16 * (e & 1));
                v = make_uint4(w[0], w[1], w[2], w[3]);
            }
            u32 o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                o[q] = pack_bf16(bf_lo(word(v, q)) + bf_at(g, 2 * q),   // bf16(res + g)
                                 bf_hi(word(v, q)) + bf_at(g, 2 * q + 1));
            if (!EDGES || (t >= 0 && t + 8 <= p.T)) {
                st16_nt(p.out + row[it] + t, make_uint4(o[0], o[1], o[2], o[3]));
            } else {
                // the block shared with the previous or next row: only this row's tokens
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (t + e >= 0 && t + e < p.T)
                        __builtin_nontemporal_store((uint16_t)(o[e >> 1] >> (16 * (e & 1))),
                                                    p.out + row[it] + t + e);
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
    const int64_t tiles_t = cf_tiles_t(p.T);
    const int64_t tiles_b = tiles_t * ((p.H + 63) / 64);
    void (*fn)(CFParams, u32, u32, u32) =
        p.T % kCfAlign == 0 ? residual_gate_cf<kCfTokens, false, false>
        : p.T % 8 == 0      ? residual_gate_cf<kCfTokens, true, false>
                            : residual_gate_cf<kCfTokens, true, true>;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(256), 0, stream, p, (u32)tiles,
                       (u32)tiles_t, (u32)tiles_b);
    return hipGetLastError();
}

}  // namespace adaln
