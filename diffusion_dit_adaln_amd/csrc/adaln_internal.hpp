// adaln_internal.hpp -- interface between the C-ABI layer (adaln_api.cpp) and the
// HIP launchers (adaln_kernels.hip) of libadaln.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace adaln {

// LN: LayerNorm + modulate; RMS: RMSNorm + scale/shift; RG: residual gate then
// RMSNorm + scale/shift; RGLN: residual gate then LayerNorm + modulate; LNQ:
// LayerNorm + modulate + static FP8 (E4M3) quantisation of the output.
enum Op : int { OP_LN = 0, OP_RMS = 1, OP_RG = 2, OP_RGLN = 3, OP_LNQ = 4 };
constexpr bool op_gated(int op) { return op == OP_RG || op == OP_RGLN; }
constexpr bool op_layernorm(int op) { return op == OP_LN || op == OP_RGLN || op == OP_LNQ; }
constexpr bool op_fp8(int op) { return op == OP_LNQ; }

// Arguments of one launch, already validated by the C-ABI layer.
struct Params {
    const uint16_t* x;       // norm input (LN, RMS) or the gated update (RG, RGLN), [rows, H]
    const uint16_t* res;     // RG, RGLN: residual stream [rows, H]
    const uint16_t* gate;    // RG, RGLN: per-batch gate, row b at gate + b*gate_bs
    const uint16_t* weight;  // RMS / RG: [H] or NULL
    const uint16_t* scale;   // per-batch, row b at scale + b*scale_bs
    const uint16_t* shift;   // per-batch, row b at shift + b*shift_bs
    uint16_t* y;             // [rows, H] (not LNQ)
    uint8_t* q;              // LNQ: E4M3 codes [rows, H]
    const float* qscale;     // LNQ: the static quantisation scale (one float, device)
    uint16_t* r;             // RG, RGLN: [rows, H]
    int64_t rows;            // B*T > 0
    int64_t T;               // rows per batch entry
    int64_t H;
    int64_t gate_bs, scale_bs, shift_bs;
    float eps;
    int64_t groups;          // row groups: a wave (H < 2048) or a workgroup of 2 or 4 waves
    // The rows fall into blocks of blk_rows rows (the last may be short), each with
    // gpb groups: group g works in block g / gpb as its (g % gpb)-th group.
    int64_t gpb;             // groups per block (< 2^31)
    int64_t blk_rows;        // rows per block (T or rows)
    int64_t group_stride;    // a group's first row is its block's first + (g % gpb) * group_stride
    int64_t step;            // rows between a group's consecutive rows
    int64_t span;            // a group's rows lie below first row + span (and its block's end)
};

// Reduction layout of H (the numerics contract): waves per row, lanes, chunks.
struct Layout {
    int waves, lanes, chunks;
    bool ragged;  // H % (8 * lanes) != 0: the last chunk is partial
};
Layout layout_of(int64_t H);

// Per-head QK RMSNorm + interleaved RoPE (head_dim 128), validated by the C-ABI layer.
struct QKParams {
    const uint16_t* q;         // token t, head h at q + t*q_tstride + h*128
    const uint16_t* k;         // likewise with k_tstride
    const uint16_t* q_weight;  // [128] or NULL (one)
    const uint16_t* k_weight;  // [128] or NULL
    const float* cos_sin;      // [tokens, 128]: cos of pairs 0..63, then sin
    uint16_t* q_out;           // [tokens, heads_q, 128]
    uint16_t* k_out;           // [tokens, heads_k, 128]
    int64_t tokens, heads_q, heads_k, q_tstride, k_tstride;
    float eps;
    // set by launch_qk: a task is eight heads of Q or of K of one token; waves is a
    // multiple of tasks_per_token, and wave w takes the tasks w, w + waves, ...
    int64_t q_tasks, tasks_per_token, waves;
};
hipError_t launch_qk(const QKParams& p, hipStream_t stream);

// Residual gating on the channel-first layout, validated by the C-ABI layer.
struct CFParams {
    const uint16_t* res;     // [B, H, T]
    const uint16_t* update;  // [B, T, H]
    const uint16_t* gate;    // row b at gate + b*gate_bs
    uint16_t* out;           // [B, H, T] (may be res)
    int64_t B, T, H, gate_bs;
};
hipError_t launch_cf(const CFParams& p, hipStream_t stream);
// Workgroups of the channel-first launch: one per tile of 64 hidden rows x kCfTokens
// tokens of the residual rows.  A row's blocks start on a kCfAlign-element boundary
// of the flat tensor, up to kCfAlign - 1 tokens before the tile's first token, so
// unless every row starts on such a boundary (T % kCfAlign == 0) the tiles of a row
// cover T + kCfAlign - 1 tokens.  The grid is rounded up to a multiple of eight so
// that consecutive tiles land on one XCD.
#ifndef ADALN_CF_TOKENS
#define ADALN_CF_TOKENS 64  // tokens per tile (64 or 128; launch tuning)
#endif
#ifndef ADALN_CF_ALIGN
#define ADALN_CF_ALIGN 64  // block alignment in elements (64: 128-byte lines, or 8)
#endif
constexpr int64_t kCfTokens = ADALN_CF_TOKENS;
constexpr int64_t kCfAlign = ADALN_CF_ALIGN;
inline int64_t cf_tiles_t(int64_t T) {
    const int64_t span = T % kCfAlign == 0 ? T : T + kCfAlign - 1;
    return (span + kCfTokens - 1) / kCfTokens;
}
inline int64_t cf_tiles(int64_t B, int64_t H, int64_t T) {
    return B * ((H + 63) / 64) * cf_tiles_t(T);
}
inline int64_t cf_grid(int64_t tiles) { return (tiles + 7) / 8 * 8; }

// Resident workgroups of `block` threads per CU for a kernel on the current device,
// and the CU count (cached per kernel and device, thread-safe).
bool occupancy(const void* fn, int block, int* blocks_per_cu, int* cus);

// How a launch of the fused kernel splits `rows` rows over row groups, given how
// many groups fit on the device at once for the deep-ring kernel (resident) and
// for the one-slot ring (resident_shallow; 0 if it is not available).  Group g
// takes the rows g*group_stride + i*step below min(g*group_stride + span, rows)
// (within its block of rows: see Params).  Large launches take a one-shot grid
// with more groups than fit at once.
struct Plan {
    bool shallow;          // the one-slot ring kernel (ring 1)
    int slots;             // ring depth S
    int ring;              // the kernel instantiation: 0 default depth, 1 one slot,
                           // 2 two rows
    int64_t groups, gpb, blk_rows, group_stride, step, span;
    int64_t blocks;        // workgroups launched
    int block_threads;     // threads per workgroup
};
// resident_two: resident groups of the two-slot ring kernel (0: not available);
// cus: compute units (0: unknown; the two-slot choice needs it)
Plan plan_launch(Op op, int64_t rows, int64_t H, int64_t T, int64_t resident,
                 int64_t resident_shallow, int64_t resident_two = 0, int64_t cus = 0);

// Launch the fused kernel for `op`; returns the HIP error of the launch.
hipError_t launch(Op op, const Params& p, hipStream_t stream);

// The plan of a launch from what fits on the device at once: resident[0..2] row
// groups with the default ring, the one-slot ring and the two-row ring (0: not
// available), and the CU count.
Plan decide(Op op, int64_t rows, int64_t H, int64_t T, const int64_t resident[3], int64_t cus);
// The same plan with the resident counts of the current device (occupancy queries,
// cached); false when a query fails.
bool device_plan(Op op, int64_t rows, int64_t H, int64_t T, bool weight, Plan* pl,
                 int64_t resident[3], int64_t* cus);

hipError_t launch_diag_round(const float* in, uint16_t* out, int64_t n, hipStream_t stream);
hipError_t launch_diag_finalize(const float* in, float* out, int64_t n, int64_t H, float eps,
                                hipStream_t stream);
// Streaming measurement kernels (adaln_stream.hip): copy src to dst, read src (the
// XOR fold of each wave's data lands in dst, stream_sink_bytes(n16, per) bytes),
// or fill dst; per: 16-byte vectors per thread (1, 2, 4, 8 or 16).
enum StreamKind : int { STREAM_COPY = 0, STREAM_READ = 1, STREAM_FILL = 2 };
hipError_t launch_stream(int kind, const void* src, void* dst, int64_t n16, int per,
                         hipStream_t stream);
int64_t stream_sink_bytes(int64_t n16, int per);
hipError_t launch_diag_quant(const float* in, uint8_t* out, int64_t n, const float* qscale,
                             hipStream_t stream);

}  // namespace adaln
