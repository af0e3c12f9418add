// Internal interface between the C-ABI host code (rownorm_capi.cpp) and the kernels
// (rownorm_kernels.hpp, instantiated in rownorm_kernels_<dtype>.hip and
// rownorm_kernels_<dtype>_persistent.hip). Not installed; the public interface is
// include/rownorm.h.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace rn {

enum Op { OP_LN = 0, OP_RMS = 1, OP_FUSED = 2, OP_FUSED_LN = 3, OP_SOFTMAX = 4 };
enum Dt { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };
enum Variant { V_AUTO = 0, V_WAVE = 1, V_WORKGROUP = 2, V_GENERAL = 3, V_ELEMENT = 4, V_WIDE = 5, V_WIDE_ELEM = 6 };

// Kernel arguments, passed by value. Pointers are device pointers; nullable ones are
// documented in include/rownorm.h.
struct Params {
    const void* x;
    const void* residual;
    const void* gamma;  // gamma (LayerNorm ops) or weight (RMSNorm ops)
    const void* beta;
    void* y;
    void* residual_out;
    float* mean;  // softmax: the row maximum
    float* rstd;  // softmax: the row's sum of exp(x - max)
    int64_t rows;
    int64_t N;
    int64_t C;    // 16-byte chunks per row (vectorized variants)
    int64_t ldx, ldr, ldy, ldro;  // row strides in elements of x, residual, y, residual_out
    int64_t cx, cr, cy, cro;      // the same in 16-byte chunks (vectorized variants)
    float eps;
    float inv_n;  // 1 / N rounded to fp32
};

// Split-row (wide) launches: the caller's workspace of [rows][S] float4 segment records.
struct WideArgs {
    void* ws;
    int S;  // segments per row
    // one-pass launches: [0] ticket counter, [1] count of records computed by waiting
    // workgroups (zeroed before launch), then records of four 64-bit words
    // (tag << 32 | fp32 bits) per (row, segment)
    unsigned* sync;
    unsigned long long* rec64;
    int P;           // row blocks
    int R;           // rows per block (one ticket = one block of one segment) ...
    int P1;          // ... for the first P1 blocks; the rest have R2 rows (the last one fewer)
    int R2;
    int wait_polls;  // polls of a missing record before the waiting workgroup computes it
};

// Backward row kernel arguments (rownorm_backward.hpp).
struct BwdParams {
    const void* dy;
    const void* x;
    const void* gamma;  // gamma / weight, nullable (1)
    const float* mean;  // LayerNorm only
    const float* rstd;
    void* dx;           // nullable: parameter gradients only
    float* ws;          // [2][P][N] fp32 column partials; nullable when no parameter gradient is wanted
    int64_t rows;
    int64_t N;
    int64_t C;          // 16-byte chunks per row (vectorized kernel)
    float inv_n;
    int parts;          // P = gridDim.x of the row kernel
    // split rows (rows longer than one workgroup holds)
    float* rec;         // [rows][S] records of two floats: the segment's sum g and sum g * xhat
    int S;              // segments per row
    int vec;            // rows, tensors and segments are whole 16-byte groups
    // one-pass split rows: [0] ticket counter, [1] count of records a waiting workgroup
    // computed itself (zeroed before launch); records of two 64-bit words
    // (tag << 32 | fp32 bits) per (row, segment)
    unsigned* sync;
    unsigned long long* rec64;
    int R;              // rows per row block (one ticket = one block of one segment)
    int wait_polls;     // polls of a missing record before the waiting workgroup computes it
};

// Backward column-sum kernel arguments.
struct BwdColParams {
    const float* ws;    // [2][P][N]
    void* dgamma;       // nullable
    void* dbeta;        // nullable
    int64_t N;
    int parts;
};

// Launch geometry chosen on the host.
struct Plan {
    int variant;          // a Variant other than V_AUTO
    int waves_per_row;    // W: wavefronts that share one row
    int rows_per_block;   // RPB: row groups per workgroup
    int chunks_per_lane;  // V: 16-byte chunks (vectorized variants) or elements (element
                          // variant) each lane holds
    int block_threads;    // 64 * W * RPB
    int64_t grid;         // workgroups (for persistent launches: an upper bound, capped at launch)
    bool exact;           // C == 64 * W * V: no tail handling needed
    bool persistent;      // parameters staged on chip once, grid sized to resident capacity
    int lds_bytes;        // dynamic LDS of a persistent launch
    bool pairs;           // element variant, 16-bit: slots of two adjacent elements (pair kernel)
    bool ragged = false;  // vectorized variants, persistent: rows addressed by byte (row starts,
                          // tensors or row lengths that are not whole 16-byte chunks)
    // Caller-chosen launch (rn_forward_tuned / rn_plan_tuned); the automatic plan leaves these
    // at their defaults.
    int64_t grid_force = 0;  // persistent vectorized launches: workgroups to launch (0: the grid rule)
    int prefetch = -1;       // persistent vectorized launches: 1 the prefetching instance, 0 the
                             // looping one, -1 the grid rule's choice
    bool dry = false;        // resolve the kernel instance only, with no HIP call: hipSuccess if
                             // it is built, hipErrorNotSupported if not
};

// Shapes the vectorized kernels are built for.
constexpr int kMaxWaveChunks = 16;     // wave variant: up to 16 chunks per lane (1024 per row)
constexpr int kMaxGroupWaves = 16;     // workgroup variant: up to 16 waves per row ...
constexpr int kMaxGroupChunks = 4;     // ... holding up to 4 chunks per lane (4096 per row)
constexpr int kMaxBigChunks = 8;       // RMSNorm: 16 waves x 8 chunks per lane (rows up to 128 KiB)
constexpr int kMaxSoftmaxChunks = 16;  // fp32 softmax: 16 waves x 16 chunks per lane (rows up to 256 KiB)
constexpr int kTargetChunks = 4;       // automatic choice: about 4 chunks per lane
constexpr int kGeneralThreads = 256;   // general variant: 256 lanes per row
constexpr int kElemTarget = 8;         // element variant: about 8 elements per lane ...
constexpr int kElemMaxPerLane = 16;    // ... at most 16 (with 16 waves: rows up to 16384)
constexpr int kPairTarget = 8;         // pair kernel: about 8 two-element slots per lane ...
constexpr int kPairMaxPerLane = 8;     // ... at most 8 (with 16 waves: rows up to 16384)
constexpr int kSoftmaxElemMaxPerLane = 64;  // softmax rows (no parameters in registers): up to 64
constexpr int kSoftmaxPairMaxPerLane = 32;  // elements / 32 pairs per lane, rows up to 65536
constexpr int kElemCuRowBytes = 32768; // element kernels, persistent: row bytes held per CU
constexpr int kLoopWorkgroupsPerCu = 8;  // looping-only persistent launches (1024-lane workgroups): grid per CU
constexpr int64_t kLoopCuRowBytes = 40960;  // looping persistent launches with parameters: row bytes in flight per CU
constexpr int64_t kMaxGrid = 1 << 20;  // grid cap; kernels loop over the remaining rows
constexpr int64_t kPersistentBlocks = 2048;  // element / pair kernels: persistent launch from this many workgroups
constexpr int64_t kPersistentVecBlocks = 256;  // vectorized kernels: persistent launch from this many workgroups
constexpr int kWideSegChunks = 2048;   // split-row variant: 16-byte chunks per segment (one workgroup)
constexpr int kWideElemSeg = 8192;     // split-row element variant: elements per segment (one workgroup)
constexpr int kBwdMaxParts = 1024;     // backward: at most this many partial column rows (workspace bound)
constexpr int kBwdSegLanes = 512;      // backward split rows: 512 lanes ...
constexpr int kBwdSegPerLane = 16;     // ... of 16 elements: 8192-element segments
constexpr int kBwdSeg = kBwdSegLanes * kBwdSegPerLane;
constexpr int kBwdWideMaxGroups = 2048;  // backward split rows: at most this many segment workgroups
constexpr int kBwdWaitPolls = 1 << 12;   // one-pass split rows: polls of a missing record (about 1-2 us
                                         // each) before the waiting workgroup computes it itself
constexpr int kBwdOnePassMaxSeg = 256;   // one-pass split rows: at most this many segments per row
constexpr int kWideOnePassMaxSeg = 256;  // forward one-pass split rows: at most this many segments per row
constexpr int kWideWaitPolls = 1 << 12;  // forward one-pass split rows: polls of a missing record
constexpr int kWideOnePassRows = 8;      // forward one-pass split rows: rows per ticket (row block)
constexpr int kBwdTargetChunks = 2;    // backward: about 2 chunks of x and of dy per lane (1 measured slower)

// Enqueue the planned kernel for one I/O dtype (one translation unit per dtype and mode).
hipError_t launch_f32(int op, const Plan& plan, const Params& p, hipStream_t stream);
hipError_t launch_f16(int op, const Plan& plan, const Params& p, hipStream_t stream);
hipError_t launch_bf16(int op, const Plan& plan, const Params& p, hipStream_t stream);
hipError_t launch_f32_persistent(int op, const Plan& plan, const Params& p, hipStream_t stream);
hipError_t launch_f16_persistent(int op, const Plan& plan, const Params& p, hipStream_t stream);
hipError_t launch_bf16_persistent(int op, const Plan& plan, const Params& p, hipStream_t stream);
hipError_t launch_wide_f32(int op, const Plan& plan, const Params& p, const WideArgs& wa, hipStream_t stream);
hipError_t launch_wide_f16(int op, const Plan& plan, const Params& p, const WideArgs& wa, hipStream_t stream);
hipError_t launch_wide_bf16(int op, const Plan& plan, const Params& p, const WideArgs& wa, hipStream_t stream);
hipError_t launch_bwd_f32(int op, const Plan& plan, const BwdParams& p, const BwdColParams& cp, hipStream_t stream);
hipError_t launch_bwd_f16(int op, const Plan& plan, const BwdParams& p, const BwdColParams& cp, hipStream_t stream);
hipError_t launch_bwd_bf16(int op, const Plan& plan, const BwdParams& p, const BwdColParams& cp, hipStream_t stream);

}  // namespace rn
