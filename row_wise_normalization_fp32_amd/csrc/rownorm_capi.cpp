// C ABI of librownorm.so: argument validation, kernel-variant planning and launch.
// The contract (argument meaning, layout, ownership, aliasing, errors) is documented in
// include/rownorm.h. Everything here runs on the host; nothing is dereferenced, allocated
// or synchronized. The pages' PyTorch-extension boundary (device / contiguity / shape /
// dtype checks, dtype dispatch, device guard, current stream, launch check: "CUDA fused
// RMSNorm kernel", diycv.top, section 5) maps to: the Python binding checks devices and
// contiguity and passes torch's current stream; this file checks the rest and reports the
// launch's own HIP error.

#include <math.h>
#include <stdint.h>

#include "../../include/rownorm.h"
#include "rownorm_internal.h"

namespace {

using rn::Params;
using rn::Plan;

constexpr int kVersion = 10000;  // 1.0.0

struct Buf {
    const void* p;
    int64_t bytes;
    bool out;
    int role;  // 0 x, 1 residual, 2 gamma, 3 beta, 4 y, 5 residual_out, 6 mean, 7 rstd
};

enum { R_X, R_RES, R_G, R_B, R_Y, R_RO, R_MEAN, R_RSTD };

bool overlaps(const Buf& a, const Buf& b) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + static_cast<uintptr_t>(b.bytes) && b0 < a0 + static_cast<uintptr_t>(a.bytes);
}

// Exact aliasing that the kernels support: an output row element is written by the lane
// that read the same element of the input, after it read it.
bool exact_alias_allowed(const Buf& out, const Buf& other) {
    if (out.p != other.p || out.bytes != other.bytes) return false;
    if (out.role == R_Y) return other.role == R_X || other.role == R_RES;
    if (out.role == R_RO) return other.role == R_X || other.role == R_RES;
    return false;
}

int next_pow2(int64_t v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

int validate_and_plan(int op, const void* x, const void* residual, const void* gamma, const void* beta,
                      const void* y, const void* residual_out, const void* mean, const void* rstd, int64_t rows,
                      int64_t N, float eps, int dtype, int variant, Plan* plan, int64_t* chunks) {
    if (dtype != RN_F32 && dtype != RN_F16 && dtype != RN_BF16) return RN_ERR_DTYPE;
    if (op != RN_OP_LAYER_NORM && op != RN_OP_RMS_NORM && op != RN_OP_FUSED_ADD_RMS_NORM) return RN_ERR_SHAPE;
    if (variant < RN_VARIANT_AUTO || variant > RN_VARIANT_GENERAL) return RN_ERR_UNSUPPORTED;
    const int64_t s = dtype == RN_F32 ? 4 : 2;
    if (rows < 0 || N <= 0) return RN_ERR_SHAPE;
    if (!(eps >= 0.f) || !isfinite(eps)) return RN_ERR_SHAPE;
    if (rows > 0 && N > INT64_MAX / s / rows) return RN_ERR_SHAPE;
    if (N > (int64_t(1) << 40)) return RN_ERR_SHAPE;
    const bool fused = op == RN_OP_FUSED_ADD_RMS_NORM;
    plan->variant = rn::V_GENERAL;
    plan->waves_per_row = 0;
    plan->rows_per_block = 0;
    plan->chunks_per_lane = 0;
    plan->block_threads = 0;
    plan->grid = 0;
    plan->exact = false;
    plan->persistent = false;
    plan->lds_bytes = 0;
    *chunks = 0;
    if (rows == 0) return RN_OK;

    if (!x || !y) return RN_ERR_NULL;
    if (fused && (!residual || !residual_out)) return RN_ERR_NULL;
    if (op != RN_OP_LAYER_NORM) {
        beta = nullptr;  // not part of these ops
        mean = nullptr;
    }
    if (!fused) {
        residual = nullptr;
        residual_out = nullptr;
    }

    const int64_t mat = rows * N * s;
    const Buf bufs[] = {
        {x, mat, false, R_X},           {residual, mat, false, R_RES}, {gamma, N * s, false, R_G},
        {beta, N * s, false, R_B},      {y, mat, true, R_Y},           {residual_out, mat, true, R_RO},
        {mean, rows * 4, true, R_MEAN}, {rstd, rows * 4, true, R_RSTD},
    };
    const int nb = sizeof(bufs) / sizeof(bufs[0]);
    for (int i = 0; i < nb; ++i) {
        if (!bufs[i].p) continue;
        const uintptr_t a = reinterpret_cast<uintptr_t>(bufs[i].p);
        const int64_t need = (bufs[i].role == R_MEAN || bufs[i].role == R_RSTD) ? 4 : s;
        if (a % static_cast<uintptr_t>(need) != 0) return RN_ERR_ALIGN;
    }
    for (int i = 0; i < nb; ++i) {
        if (!bufs[i].p || !bufs[i].out) continue;
        for (int j = 0; j < nb; ++j) {
            if (j == i || !bufs[j].p) continue;
            if (overlaps(bufs[i], bufs[j]) && !exact_alias_allowed(bufs[i], bufs[j])) return RN_ERR_ALIAS;
        }
    }

    // Vectorized variants need whole 16-byte chunks per row and 16-byte aligned tensors.
    bool vec_ok = (N * s) % 16 == 0;
    for (int i = 0; i < nb && vec_ok; ++i) {
        if (!bufs[i].p || bufs[i].role == R_MEAN || bufs[i].role == R_RSTD) continue;
        if (reinterpret_cast<uintptr_t>(bufs[i].p) % 16 != 0) vec_ok = false;
    }
    const int64_t C = vec_ok ? (N * s) / 16 : 0;
    const int64_t wave_cap = int64_t(64) * rn::kMaxWaveChunks;                         // 1024 chunks
    const int64_t group_cap = int64_t(64) * rn::kMaxGroupWaves * rn::kMaxGroupChunks;  // 4096 chunks

    // Automatic row-group width: enough waves that each lane holds about kTargetChunks
    // chunks (measured on MI355X: 4 chunks per lane balances bytes in flight against VGPRs).
    int w_auto = next_pow2((C + 64 * rn::kTargetChunks - 1) / (64 * rn::kTargetChunks));
    if (w_auto > rn::kMaxGroupWaves) w_auto = rn::kMaxGroupWaves;

    int v = variant;
    if (v == RN_VARIANT_AUTO) {
        if (!vec_ok || C > group_cap)
            v = RN_VARIANT_GENERAL;
        else
            v = w_auto == 1 ? RN_VARIANT_WAVE : RN_VARIANT_WORKGROUP;
    }
    int W = 0;
    if (v == RN_VARIANT_WAVE) {
        if (!vec_ok || C > wave_cap) return RN_ERR_UNSUPPORTED;
        W = 1;
        plan->variant = rn::V_WAVE;
    } else if (v == RN_VARIANT_WORKGROUP) {
        if (!vec_ok || C > group_cap) return RN_ERR_UNSUPPORTED;
        W = w_auto < 2 ? 2 : w_auto;
        plan->variant = rn::V_WORKGROUP;
    } else {
        plan->variant = rn::V_GENERAL;
    }
    if (plan->variant == rn::V_GENERAL) {
        plan->waves_per_row = rn::kGeneralThreads / 64;
        plan->rows_per_block = 1;
        plan->chunks_per_lane = 0;
        plan->block_threads = rn::kGeneralThreads;
    } else {
        plan->waves_per_row = W;
        plan->rows_per_block = W <= 4 ? 4 / W : 1;
        plan->chunks_per_lane = next_pow2((C + 64 * W - 1) / (64 * W));
        plan->block_threads = 64 * W * plan->rows_per_block;
    }
    const int64_t blocks = (rows + plan->rows_per_block - 1) / plan->rows_per_block;
    plan->grid = blocks < rn::kMaxGrid ? blocks : rn::kMaxGrid;
    plan->exact = plan->variant != rn::V_GENERAL && C == int64_t(64) * W * plan->chunks_per_lane;
    // Persistent launch: for exact shapes with parameters and enough rows that workgroups
    // would otherwise be launched many times over (measured: it pays from about 2048
    // workgroups up). Parameters go to LDS once per workgroup; LayerNorm with both keeps
    // gamma in VGPRs and stages only beta, so the LDS need is at most one row (64 KiB).
    const bool has_g = gamma != nullptr;
    const bool has_b = op == RN_OP_LAYER_NORM && beta != nullptr;
    plan->persistent = plan->exact && (has_g || has_b) && blocks >= rn::kPersistentBlocks;
    plan->lds_bytes = 0;
    if (plan->persistent) plan->lds_bytes = static_cast<int>(C * 16);  // one parameter vector in LDS
    *chunks = C;
    return RN_OK;
}

int run(int op, const void* x, const void* residual, const void* gamma, const void* beta, void* y,
        void* residual_out, float* mean, float* rstd, int64_t rows, int64_t N, float eps, int dtype,
        hipStream_t stream, int variant) {
    Plan plan;
    int64_t C = 0;
    const int st = validate_and_plan(op, x, residual, gamma, beta, y, residual_out, mean, rstd, rows, N, eps, dtype,
                                     variant, &plan, &C);
    if (st != RN_OK || rows == 0) return st;
    Params p;
    p.x = x;
    p.residual = op == RN_OP_FUSED_ADD_RMS_NORM ? residual : nullptr;
    p.gamma = gamma;
    p.beta = op == RN_OP_LAYER_NORM ? beta : nullptr;
    p.y = y;
    p.residual_out = op == RN_OP_FUSED_ADD_RMS_NORM ? residual_out : nullptr;
    p.mean = op == RN_OP_LAYER_NORM ? mean : nullptr;
    p.rstd = rstd;
    p.rows = rows;
    p.N = N;
    p.C = C;
    p.eps = eps;
    p.inv_n = static_cast<float>(1.0 / static_cast<double>(N));
    hipError_t e = hipErrorInvalidValue;
    switch (dtype) {
    case RN_F32: e = plan.persistent ? rn::launch_f32_persistent(op, plan, p, stream)
                                     : rn::launch_f32(op, plan, p, stream); break;
    case RN_F16: e = plan.persistent ? rn::launch_f16_persistent(op, plan, p, stream)
                                     : rn::launch_f16(op, plan, p, stream); break;
    case RN_BF16: e = plan.persistent ? rn::launch_bf16_persistent(op, plan, p, stream)
                                      : rn::launch_bf16(op, plan, p, stream); break;
    default: break;
    }
    return e == hipSuccess ? RN_OK : RN_ERR_HIP;
}

}  // namespace

extern "C" {

int ln_forward(const void* x, const void* gamma, const void* beta, void* y, float* mean, float* rstd, int64_t rows,
               int64_t N, float eps, int dtype, hipStream_t stream) {
    return run(RN_OP_LAYER_NORM, x, nullptr, gamma, beta, y, nullptr, mean, rstd, rows, N, eps, dtype, stream,
               RN_VARIANT_AUTO);
}

int rms_norm(const void* x, const void* weight, void* y, float* rstd, int64_t rows, int64_t N, float eps, int dtype,
             hipStream_t stream) {
    return run(RN_OP_RMS_NORM, x, nullptr, weight, nullptr, y, nullptr, nullptr, rstd, rows, N, eps, dtype, stream,
               RN_VARIANT_AUTO);
}

int fused_add_rms_norm(const void* x, const void* residual, const void* weight, void* y, void* residual_out,
                       float* rstd, int64_t rows, int64_t N, float eps, int dtype, hipStream_t stream) {
    return run(RN_OP_FUSED_ADD_RMS_NORM, x, residual, weight, nullptr, y, residual_out, nullptr, rstd, rows, N, eps,
               dtype, stream, RN_VARIANT_AUTO);
}

int ln_forward_variant(const void* x, const void* gamma, const void* beta, void* y, float* mean, float* rstd,
                       int64_t rows, int64_t N, float eps, int dtype, hipStream_t stream, int variant) {
    return run(RN_OP_LAYER_NORM, x, nullptr, gamma, beta, y, nullptr, mean, rstd, rows, N, eps, dtype, stream,
               variant);
}

int rms_norm_variant(const void* x, const void* weight, void* y, float* rstd, int64_t rows, int64_t N, float eps,
                     int dtype, hipStream_t stream, int variant) {
    return run(RN_OP_RMS_NORM, x, nullptr, weight, nullptr, y, nullptr, nullptr, rstd, rows, N, eps, dtype, stream,
               variant);
}

int fused_add_rms_norm_variant(const void* x, const void* residual, const void* weight, void* y, void* residual_out,
                               float* rstd, int64_t rows, int64_t N, float eps, int dtype, hipStream_t stream,
                               int variant) {
    return run(RN_OP_FUSED_ADD_RMS_NORM, x, residual, weight, nullptr, y, residual_out, nullptr, rstd, rows, N, eps,
               dtype, stream, variant);
}

int rn_plan(int op, const void* x, const void* residual, const void* gamma, const void* beta, const void* y,
            const void* residual_out, const void* mean, const void* rstd, int64_t rows, int64_t N, float eps,
            int dtype, int variant, rn_plan_info* out) {
    Plan plan;
    int64_t C = 0;
    const int st = validate_and_plan(op, x, residual, gamma, beta, y, residual_out, mean, rstd, rows, N, eps, dtype,
                                     variant, &plan, &C);
    if (out) {
        out->variant = plan.variant;
        out->waves_per_row = plan.waves_per_row;
        out->rows_per_block = plan.rows_per_block;
        out->block_threads = plan.block_threads;
        out->chunks_per_lane = plan.chunks_per_lane;
        out->grid_blocks = plan.grid;
        out->exact = plan.exact ? 1 : 0;
        out->persistent = plan.persistent ? 1 : 0;
        out->lds_bytes = plan.lds_bytes;
    }
    return st;
}

const char* rn_status_string(int status) {
    switch (status) {
    case RN_OK: return "RN_OK";
    case RN_ERR_NULL: return "RN_ERR_NULL";
    case RN_ERR_SHAPE: return "RN_ERR_SHAPE";
    case RN_ERR_DTYPE: return "RN_ERR_DTYPE";
    case RN_ERR_ALIAS: return "RN_ERR_ALIAS";
    case RN_ERR_UNSUPPORTED: return "RN_ERR_UNSUPPORTED";
    case RN_ERR_HIP: return "RN_ERR_HIP";
    case RN_ERR_ALIGN: return "RN_ERR_ALIGN";
    default: return "unknown status";
    }
}

int rn_version(void) { return kVersion; }

}  // extern "C"
