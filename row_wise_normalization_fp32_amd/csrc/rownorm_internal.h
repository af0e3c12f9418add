// Internal interface between the C-ABI host code (rownorm_capi.cpp) and the kernels
// (rownorm_kernels.hip). Not installed; the public interface is include/rownorm.h.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace rn {

enum Op { OP_LN = 0, OP_RMS = 1, OP_FUSED = 2 };
enum Dt { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };
enum Variant { V_AUTO = 0, V_WAVE = 1, V_WORKGROUP = 2, V_GENERAL = 3 };

// Kernel arguments, passed by value. Pointers are device pointers; nullable ones are
// documented in include/rownorm.h.
struct Params {
    const void* x;
    const void* residual;
    const void* gamma;  // gamma (LayerNorm) or weight (RMSNorm ops)
    const void* beta;
    void* y;
    void* residual_out;
    float* mean;
    float* rstd;
    int64_t rows;
    int64_t N;
    int64_t C;  // 16-byte chunks per row (vectorized variants)
    float eps;
};

// Launch geometry chosen on the host.
struct Plan {
    int variant;         // V_WAVE, V_WORKGROUP or V_GENERAL
    int waves_per_row;   // W
    int rows_per_block;  // rows one workgroup handles per loop iteration
    int chunks_per_lane; // V (vectorized variants)
    int block_threads;
    int64_t grid;
};

// Largest per-lane chunk count and row-group width the vectorized kernels are built for.
constexpr int kMaxChunksPerLane = 16;
constexpr int kWaveRowsPerBlock = 4;   // wave variant: 4 rows (4 wavefronts) per workgroup
constexpr int kGroupWaves = 4;         // workgroup variant: 4 wavefronts share one row
constexpr int kGeneralThreads = 256;   // general variant: 256 lanes per row
constexpr int64_t kMaxGrid = 1 << 20;  // grid cap; kernels loop over the remaining rows

// Enqueue the planned kernel. Returns the HIP error of the launch.
hipError_t launch(int op, int dtype, const Plan& plan, const Params& p, hipStream_t stream);

}  // namespace rn
