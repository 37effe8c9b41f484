// adaln_device.hpp -- device helpers shared by the kernels of libadaln (gfx950):
// bf16 <-> binary32 conversions, raw buffer descriptors with non-temporal 16-byte
// accesses, the E4M3 quantisation step, DPP and row-swap cross-lane moves, and the
// correctly rounded finalize (general, and the exact shortcut for in-range waves).
// Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// bf16(v) widened back to binary32 in one instruction: with a zero low slot,
// v_cvt_pk_bf16_f32 leaves bf16(v) in the high half, and that register read as
// binary32 is exactly the bf16 value (the low half bf16(+0) is all zero bits).
__device__ __forceinline__ float round_bf16(float v) { return __uint_as_float(pack_bf16(0.0f, v)); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Small per-batch vectors: ordinary cached loads (shared by every row of a batch).
__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}
// Activations are touched once: non-temporal (nt) 16-byte buffer loads and stores
// through a descriptor that spans exactly the rows being accessed.  An access at
// an offset past the descriptor's range reads zeros and writes nothing, without
// memory traffic; the kernels use that to issue every load and store of their
// loops unconditionally (refills past the last row, lanes past a ragged row end),
// so the compiler can count outstanding memory operations exactly and never waits
// on a prefetch it does not need yet.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) buffer, gfx9-family descriptor word 3
constexpr int kOutOfRange = 0x7FFFFFF0;  // any offset >= the descriptor's byte range
constexpr int kNonTemporal = 2;          // cache-policy bit nt

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ uint4 ld16_stream(rsrc_t r, int off) {
    const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal);
    return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void st16_stream(rsrc_t r, int off, uint4 v) {
    const u32x4 t = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(t, r, off, 0, kNonTemporal);
}

// Non-temporal 16-byte accesses through plain pointers (callers check bounds).
__device__ __forceinline__ uint4 ld16_nt(const uint16_t* p) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void st16_nt(uint16_t* p, uint4 v) {
    const u32x4 t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4*>(p));
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st8_stream(rsrc_t r, int off, u32 lo, u32 hi) {
    const u32x2 t = {lo, hi};
    __builtin_amdgcn_raw_buffer_store_b64(t, r, off, 0, kNonTemporal);
}

// Static FP8 quantisation of four values already multiplied by 1/scale: clamp to
// [-448, 448] with IEEE-754-2019 maximum/minimum (v_maximum3/v_minimum3: a NaN stays
// NaN), then v_cvt_pk_fp8_f32, which rounds to nearest-even into the OCP E4M3 format
// on gfx950.  Byte k of the result is value k.
__device__ __forceinline__ float clamp448(float v) {
    return __builtin_elementwise_minimum(__builtin_elementwise_maximum(v, -448.0f), 448.0f);
}
// The same with the clamp as one median of three: exact for every input except a
// NaN (which the median does not keep), so only for values known not to be NaN.
__device__ __forceinline__ u32 quant4_no_nan(float a, float b, float c, float d) {
    const u32 lo = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, -448.0f, 448.0f),
                                                   __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f), 0,
                                                   false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(c, -448.0f, 448.0f),
                                           __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f), lo, true);
}
__device__ __forceinline__ u32 quant4(float a, float b, float c, float d) {
    const u32 lo = __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), lo, true);
}

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

// Every lane's source lies inside its own row, so bound_ctrl changes no value; it
// lets the compiler fold the move into the instruction that consumes it.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
// DPP into the lanes of the banks (groups of 4 lanes of a 16-lane row) set in
// BANKS; the other lanes keep v.
template <int CTRL, int BANKS>
__device__ __forceinline__ float dpp_banks(float v) {
    const int i = __builtin_bit_cast(int, v);
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(i, i, CTRL, 0xF, BANKS, false));
}
// The butterfly partners at distance K (1, 2, 4, 8) in their fixed order: lo is
// the value of lane t & ~K, hi that of lane t | K, in every lane.
template <int K>
__device__ __forceinline__ float partner_lo(float v) {
    if constexpr (K == 1) return dpp<0xA0>(v);             // quad_perm [0,0,2,2]
    else if constexpr (K == 2) return dpp<0x44>(v);        // quad_perm [0,1,0,1]
    else if constexpr (K == 4) return dpp_banks<0x114, 0xA>(v);  // row_shr:4 into banks 1, 3
    else return dpp_banks<0x118, 0xC>(v);                  // row_shr:8 into banks 2, 3
}
template <int K>
__device__ __forceinline__ float partner_hi(float v) {
    if constexpr (K == 1) return dpp<0xF5>(v);             // quad_perm [1,1,3,3]
    else if constexpr (K == 2) return dpp<0xEE>(v);        // quad_perm [2,3,2,3]
    else if constexpr (K == 4) return dpp_banks<0x104, 0x5>(v);  // row_shl:4 into banks 0, 2
    else return dpp_banks<0x108, 0x3>(v);                  // row_shl:8 into banks 0, 1
}
// Distances 16 and 32 when every 16-lane row (every 32-lane half) holds one value:
// v_permlane16_swap exchanges the odd rows of its first operand with the even rows
// of its second, v_permlane32_swap the upper half of the first with the lower half
// of the second, so that from two copies of v every lane gets the value of the lower
// row (half) of its pair in lo and of the upper one in hi.  The leading s_nop covers
// the wait states the swap needs after a VALU write of its operands.
__device__ __forceinline__ void pair16(float v, float& lo, float& hi) {
    lo = v;
    hi = v;
    asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
}
__device__ __forceinline__ void pair32(float v, float& lo, float& hi) {
    lo = v;
    hi = v;
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(lo), "+v"(hi));
}
__device__ __forceinline__ float readlane(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// rstd = RN(1 / RN(sqrt(RN(stat + eps)))), correctly rounded steps.
__device__ __forceinline__ float finalize(float stat, float eps) {
    const float v = stat + eps;
    const float root = __builtin_sqrtf(v);
    return 1.0f / root;
}

// rstd = RN(1 / RN(sqrt(RN(RN(S / H) + eps)))) for a row's statistic S (sum of
// squares or M2) over H elements, rH = RN(1 / H); the same bits as finalize(S / H,
// eps).  When every active lane of the wave is in the range below, shorter exact
// sequences replace the general divide and square root (one uniform branch; the
// general path only when some lane is outside it):
//  - S / H: q0 = RN(S * rH) is within 1.5 ulp of S / H, its remainder S - q0 * H is
//    exact (a multiple of ulp(q0) below 2^14 ulp(q0)), and one correction
//    RN(q0 + r * rH) gives RN(S / H) (checked exhaustively on the CPU for every
//    significand of S and every H = 8, 16, ..., 8192; the steps scale with S by
//    powers of two while S stays in [2^-64, 2^64]; for S = 0 every step is 0);
//  - sqrt: the hardware root s, then the neighbour below or above it when the
//    exact residual v - (s -/+ ulp) * s says the root lies beyond the midpoint
//    (checked on the CPU for every v in [1, 4) with s off by up to one ulp either
//    way; scales by powers of four for v in [2^-100, 2^100]);
//  - 1 / s: one Newton step from the hardware reciprocal, y0 + y0 * (1 - s * y0),
//    which rounds correctly from any faithful y0 except for a significand of all
//    ones (checked on the CPU for every significand), so that case keeps the
//    general divide.
// (The host checks are tests/test_rstd_steps.py; the device's own results are
// compared over every non-negative S by the GPU finalize tests.)
// POW2: H is a power of two (S * rH is then exact).
template <bool POW2>
__device__ __forceinline__ float row_rstd(float S, float H, float rH, float eps) {
    // every step computed unconditionally, then one uniform test
    float q = S * rH;
    if (!POW2) {
        const float r = __builtin_fmaf(-q, H, S);
        q = __builtin_fmaf(r, rH, q);
    }
    const float v = q + eps;
    const float s0 = __builtin_amdgcn_sqrtf(v);
    const float lo = __uint_as_float(__float_as_uint(s0) - 1u);
    const float hi = __uint_as_float(__float_as_uint(s0) + 1u);
    const float t = __builtin_fmaf(-lo, s0, v) <= 0.0f ? lo : s0;
    const float s = __builtin_fmaf(-hi, s0, v) > 0.0f ? hi : t;  // RN(sqrt(v))
    const float y0 = __builtin_amdgcn_rcpf(s);
    const float e = __builtin_fmaf(-s, y0, 1.0f);
    const float y = __builtin_fmaf(e, y0, y0);  // RN(1 / s)
    const bool ok = ((S == 0.0f) | ((S >= 0x1p-64f) & (S <= 0x1p64f))) & (v >= 0x1p-100f) &
                    (v <= 0x1p100f) & ((__float_as_uint(s) & 0x7FFFFFu) != 0x7FFFFFu);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(!ok) != 0, 0)) return finalize(S / H, eps);
    return y;
}

}  // namespace
}  // namespace adaln
