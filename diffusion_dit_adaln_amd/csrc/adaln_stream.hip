// adaln_stream.hip -- measurement kernels of libadaln: the attainable streaming
// rates of the device for the fused kernels' access style (16-byte non-temporal
// loads and stores), timed beside them as ceilings.  Not on the path.
//
//  - copy: each thread loads PER 16-byte vectors, then stores them (loads first,
//    so that PER vectors per thread are in flight; the accesses of a whole block
//    are unconditional, since a guarded load would be waited for before the next);
//  - read: each thread loads PER vectors and folds them with XOR; lane 0 of each
//    wave stores the wave's fold (4 bytes per 1024*PER bytes read), so no load
//    can be removed;
//  - fill: each thread stores PER vectors of a constant pattern.
// One-shot grids of 256-thread workgroups; the last workgroup is partial.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "adaln_device.hpp"
#include "adaln_internal.hpp"

namespace adaln {
namespace {

template <int PER>
__global__ __launch_bounds__(256) void stream_copy(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, int64_t n16) {
    const int64_t base = (int64_t)blockIdx.x * 256 * PER + threadIdx.x;
    u32x4 v[PER];
    if ((int64_t)(blockIdx.x + 1) * 256 * PER <= n16) {
        // a whole block: unconditional accesses, so every load is in flight before
        // the first wait
#pragma unroll
        for (int k = 0; k < PER; ++k) v[k] = __builtin_nontemporal_load(src + base + k * 256);
        __builtin_amdgcn_sched_barrier(0);  // every load issued before the first store
#pragma unroll
        for (int k = 0; k < PER; ++k) __builtin_nontemporal_store(v[k], dst + base + k * 256);
        return;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int64_t i = base + (int64_t)k * 256;
        if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
    }
}

template <int PER>
__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ src,
                                                   u32* __restrict__ sink, int64_t n16) {
    const int64_t base = (int64_t)blockIdx.x * 256 * PER + threadIdx.x;
    u32 acc = 0;
    if ((int64_t)(blockIdx.x + 1) * 256 * PER <= n16) {
        u32x4 v[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) v[k] = __builtin_nontemporal_load(src + base + k * 256);
        __builtin_amdgcn_sched_barrier(0);  // every load issued before the first fold
#pragma unroll
        for (int k = 0; k < PER; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    } else {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int64_t i = base + (int64_t)k * 256;
            if (i < n16) {
                const u32x4 t = __builtin_nontemporal_load(src + i);
                acc ^= t.x ^ t.y ^ t.z ^ t.w;
            }
        }
    }
    // fold over the wave (any order: XOR), lane 0 keeps the wave's value
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d, 64);
    if ((threadIdx.x & 63) == 0) sink[(int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

template <int PER>
__global__ __launch_bounds__(256) void stream_fill(u32x4* __restrict__ dst, int64_t n16,
                                                   u32 pattern) {
    const int64_t base = (int64_t)blockIdx.x * 256 * PER + threadIdx.x;
    const u32x4 v = {pattern, pattern ^ 0x9E3779B9u, pattern, pattern ^ 0x9E3779B9u};
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int64_t i = base + (int64_t)k * 256;
        if (i < n16) __builtin_nontemporal_store(v, dst + i);
    }
}

template <int PER>
hipError_t launch_stream_per(int kind, const void* src, void* dst, int64_t n16,
                             hipStream_t stream) {
    const int64_t per_block = 256 * PER;
    const int64_t blocks = (n16 + per_block - 1) / per_block;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks), block(256);
    if (kind == STREAM_COPY)
        hipLaunchKernelGGL(stream_copy<PER>, grid, block, 0, stream,
                           static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
    else if (kind == STREAM_READ)
        hipLaunchKernelGGL(stream_read<PER>, grid, block, 0, stream,
                           static_cast<const u32x4*>(src), static_cast<u32*>(dst), n16);
    else
        hipLaunchKernelGGL(stream_fill<PER>, grid, block, 0, stream, static_cast<u32x4*>(dst),
                           n16, 0x3F803F80u);
    return hipGetLastError();
}

}  // namespace

int64_t stream_sink_bytes(int64_t n16, int per) {
    // one 4-byte word per wave of 64 threads, four waves per workgroup
    const int64_t blocks = (n16 + 256 * (int64_t)per - 1) / (256 * (int64_t)per);
    return blocks * 16;
}

hipError_t launch_stream(int kind, const void* src, void* dst, int64_t n16, int per,
                         hipStream_t stream) {
    switch (per) {
        case 1: return launch_stream_per<1>(kind, src, dst, n16, stream);
        case 2: return launch_stream_per<2>(kind, src, dst, n16, stream);
        case 4: return launch_stream_per<4>(kind, src, dst, n16, stream);
        case 8: return launch_stream_per<8>(kind, src, dst, n16, stream);
        case 16: return launch_stream_per<16>(kind, src, dst, n16, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace adaln
