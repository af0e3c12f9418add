/* stream_probe.h - a streaming copy kernel for gfx950 (MI355X), built as libstreamprobe.so.
 *
 * Measurement support, not part of the normalization path: it moves the same kind of
 * traffic as a row normalization (every byte of a tensor read once from HBM, every byte of
 * another written once, 16-byte coalesced accesses) with no arithmetic at all, so its
 * throughput at a given size is the practical read+write ceiling that the normalization
 * kernels are compared against. The pages frame these kernels by the bandwidth wall and a
 * roofline ("05 LLM Ops" lesson, smarter.xin, basic concepts: bandwidth wall and roofline)
 * and time them on hot and cold caches ("CUDA fused RMSNorm kernel", diycv.top, section 6);
 * this kernel gives the same timing protocol a reference point measured on this GPU rather
 * than a published peak.
 *
 * Plain C ABI: device pointers, byte counts, a hipStream_t. Nothing is allocated, freed or
 * synchronized; the launch is enqueued on `stream`.
 */
#ifndef STREAM_PROBE_H
#define STREAM_PROBE_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Copies `bytes` bytes from device memory `src` to device memory `dst` (both 16-byte
 * aligned, not overlapping; `bytes` a multiple of 16).
 *
 * Geometry: workgroups of `block_threads` lanes (256, 512 or 1024); each lane moves
 * `chunks_per_lane` 16-byte chunks (1, 2, 4 or 8) per tile, issuing every load of the tile
 * before its first store; a tile is block_threads * chunks_per_lane chunks, and lane t of a
 * workgroup takes chunks t, t + block_threads, ... of the tile, so each wavefront access
 * covers 1 KiB of contiguous memory. `grid` workgroups loop over the tiles (grid <= 0: one
 * workgroup per tile). `nontemporal` != 0 marks the loads and stores as streaming
 * (non-temporal).
 *
 * Returns 0 on success; 1 for a null pointer, 2 for a size or alignment that is not a
 * multiple of 16 bytes, 3 for an unsupported geometry, 4 for overlapping buffers (all
 * detected before anything is enqueued); 6 when the launch fails (hipGetLastError). */
int rn_probe_copy(const void* src, void* dst, int64_t bytes, int chunks_per_lane, int block_threads,
                  int64_t grid, int nontemporal, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* STREAM_PROBE_H */
