// Streaming copy kernel for gfx950: the read+write bandwidth ceiling that the row
// normalization kernels are measured against (include/stream_probe.h).
//
// It has the normalization kernels' access pattern without their arithmetic: 16-byte
// accesses, lane t of a workgroup on chunks t, t + B, ... of a tile (1 KiB per wavefront
// access), every load of a tile issued before its first store, optional non-temporal
// (streaming) cache policy.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "stream_probe.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int B, int V, bool NT>
__global__ __launch_bounds__(B) void stream_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        int64_t n, int64_t tiles) {
    constexpr int64_t TILE = static_cast<int64_t>(B) * V;
    for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const int64_t base = tile * TILE + threadIdx.x;
        u32x4 v[V];
        if (base + (V - 1) * B < n) {  // whole tile for this lane: no per-chunk test
#pragma unroll
            for (int i = 0; i < V; ++i) v[i] = NT ? __builtin_nontemporal_load(src + base + i * B) : src[base + i * B];
            __builtin_amdgcn_sched_barrier(0);  // all loads issued before the first store
#pragma unroll
            for (int i = 0; i < V; ++i) {
                if (NT) {
                    __builtin_nontemporal_store(v[i], dst + base + i * B);
                } else {
                    dst[base + i * B] = v[i];
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i)
                if (base + i * B < n) dst[base + i * B] = src[base + i * B];
        }
    }
}

template <int B, int V, bool NT>
hipError_t go(const void* src, void* dst, int64_t n, int64_t grid, hipStream_t s) {
    const int64_t tiles = (n + static_cast<int64_t>(B) * V - 1) / (static_cast<int64_t>(B) * V);
    int64_t g = grid <= 0 ? tiles : (grid < tiles ? grid : tiles);
    if (g > (int64_t(1) << 30)) g = int64_t(1) << 30;
    hipLaunchKernelGGL((stream_copy_kernel<B, V, NT>), dim3(static_cast<unsigned>(g)), dim3(B), 0, s,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n, tiles);
    return hipGetLastError();
}

template <int B, bool NT>
hipError_t by_v(int V, const void* src, void* dst, int64_t n, int64_t grid, hipStream_t s) {
    switch (V) {
    case 1: return go<B, 1, NT>(src, dst, n, grid, s);
    case 2: return go<B, 2, NT>(src, dst, n, grid, s);
    case 4: return go<B, 4, NT>(src, dst, n, grid, s);
    case 8: return go<B, 8, NT>(src, dst, n, grid, s);
    default: return hipErrorInvalidValue;
    }
}

template <bool NT>
hipError_t by_b(int B, int V, const void* src, void* dst, int64_t n, int64_t grid, hipStream_t s) {
    switch (B) {
    case 256: return by_v<256, NT>(V, src, dst, n, grid, s);
    case 512: return by_v<512, NT>(V, src, dst, n, grid, s);
    case 1024: return by_v<1024, NT>(V, src, dst, n, grid, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int rn_probe_copy(const void* src, void* dst, int64_t bytes,
                                                                     int chunks_per_lane, int block_threads,
                                                                     int64_t grid, int nontemporal, hipStream_t stream) {
    if (src == nullptr || dst == nullptr) return 1;
    if (bytes < 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(dst) % 16 != 0)
        return 2;
    if ((chunks_per_lane != 1 && chunks_per_lane != 2 && chunks_per_lane != 4 && chunks_per_lane != 8) ||
        (block_threads != 256 && block_threads != 512 && block_threads != 1024))
        return 3;
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    if (bytes > 0 && a < b + static_cast<uintptr_t>(bytes) && b < a + static_cast<uintptr_t>(bytes)) return 4;
    if (bytes == 0) return 0;
    const int64_t n = bytes / 16;
    const hipError_t e = nontemporal ? by_b<true>(block_threads, chunks_per_lane, src, dst, n, grid, stream)
                                     : by_b<false>(block_threads, chunks_per_lane, src, dst, n, grid, stream);
    return e == hipSuccess ? 0 : 6;
}
