// Row-wise LayerNorm / RMSNorm / fused residual-add + RMSNorm kernels for gfx950 (MI355X).
//
// The operations are defined in include/rownorm.h. All three are bandwidth-bound: a few
// fp32 operations per element against 2-4 bytes moved per element (the LayerNorm CUDA
// walkthrough, lpnh.cn/news/2756757, section 1, counts about 5 FLOP per 4-byte element;
// "CUDA fused RMSNorm kernel", diycv.top, section 1, calls RMSNorm memory-bound). So the
// design goal is: read every input byte from HBM once, write every output byte once, with
// 16-byte coalesced accesses and enough bytes in flight per CU; the arithmetic only has to
// stay off the critical path.
//
// Vectorized kernel (rownorm_vec_kernel), used when a row is a whole number of 16-byte
// chunks and all pointers are 16-byte aligned:
//   * W wavefronts (64 lanes each) own one row; W = 1 is the "wave per row" variant, W > 1
//     the "workgroup per row" variant. Lane t of the row group holds chunks t, t + 64W,
//     t + 128W, ... (V chunks at most), so each load instruction of a wavefront reads 1 KiB
//     of contiguous row. The whole row stays in VGPRs between the statistics and the
//     normalization: x is read from HBM exactly once (the walkthrough's sections 3-4 show
//     a second read of x costing +50% traffic; its shared-memory row cache becomes a
//     register-resident row here).
//   * Cross-lane sums use DPP (quad_perm, row_half_mirror, row_mirror: each step adds a
//     lane's value to its partner's, and every partner pair is symmetric, so all 16 lanes
//     of a DPP row end with the same bits), then readlane of lanes 0/16/32/48 adds the
//     four row sums in a fixed order. The result is wave-uniform and deterministic.
//   * W > 1: each wavefront produces a (count, mean, M2) triple for its share of the row;
//     the triples meet in LDS after one barrier and every lane folds them in the same
//     fixed order with the pairwise Welford combine (count = na + nb, delta = mb - ma,
//     mean = ma + delta * nb / n, M2 = M2a + M2b + delta^2 * na * nb / n; the "05 LLM Ops"
//     lesson, smarter.xin, section "Welford combine function").
//   * LayerNorm statistics are shifted: K = x[row, 0] is subtracted from every element
//     before the sums (exact when K and x are within a factor of two, Sterbenz), so the
//     mean and the squared deviations are taken of small numbers. On rows whose mean is
//     large next to their spread (the cancellation case of the walkthrough's section 6),
//     plain fp32 sums lose the 1e-4 accuracy bar; the shift keeps about 1e-6.
//
// General kernel (rownorm_general_kernel): any N and any element-aligned pointers. One
// 256-lane workgroup per row; it reads the row up to three times (statistics, centered
// squares, normalization), element by element. Correct everywhere, not tuned.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rownorm_internal.h"

namespace rn {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <typename To, typename From>
__device__ __forceinline__ To bit_cast(From v) {
    return __builtin_bit_cast(To, v);
}

// ---------------------------------------------------------------------------------------
// I/O element types: widen 16-byte chunks to fp32 and narrow fp32 back (round to nearest
// even; the hardware conversions v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32 do this).
// ---------------------------------------------------------------------------------------

template <int DT>
struct Io;

template <>
struct Io<DT_F32> {
    static constexpr int E = 4;  // elements per 16-byte chunk
    static constexpr int BYTES = 4;
    __device__ static __forceinline__ void unpack(const u32x4& v, float* f) {
        f[0] = bit_cast<float>(v.x);
        f[1] = bit_cast<float>(v.y);
        f[2] = bit_cast<float>(v.z);
        f[3] = bit_cast<float>(v.w);
    }
    __device__ static __forceinline__ u32x4 pack(const float* f) {
        return u32x4{bit_cast<unsigned>(f[0]), bit_cast<unsigned>(f[1]), bit_cast<unsigned>(f[2]),
                     bit_cast<unsigned>(f[3])};
    }
    __device__ static __forceinline__ float first(const u32x4& v) { return bit_cast<float>(v.x); }
    __device__ static __forceinline__ float load1(const void* p, int64_t i) {
        return static_cast<const float*>(p)[i];
    }
    __device__ static __forceinline__ void store1(void* p, int64_t i, float v) { static_cast<float*>(p)[i] = v; }
    __device__ static __forceinline__ float round(float v) { return v; }
};

template <>
struct Io<DT_F16> {
    static constexpr int E = 8;
    static constexpr int BYTES = 2;
    __device__ static __forceinline__ f32x2 widen2(unsigned u) {
        return __builtin_convertvector(bit_cast<f16x2>(u), f32x2);
    }
    __device__ static __forceinline__ unsigned narrow2(float a, float b) {
        return bit_cast<unsigned>(__builtin_convertvector((f32x2{a, b}), f16x2));
    }
    __device__ static __forceinline__ void unpack(const u32x4& v, float* f) {
        f32x2 p0 = widen2(v.x), p1 = widen2(v.y), p2 = widen2(v.z), p3 = widen2(v.w);
        f[0] = p0.x; f[1] = p0.y; f[2] = p1.x; f[3] = p1.y;
        f[4] = p2.x; f[5] = p2.y; f[6] = p3.x; f[7] = p3.y;
    }
    __device__ static __forceinline__ u32x4 pack(const float* f) {
        return u32x4{narrow2(f[0], f[1]), narrow2(f[2], f[3]), narrow2(f[4], f[5]), narrow2(f[6], f[7])};
    }
    __device__ static __forceinline__ float first(const u32x4& v) { return widen2(v.x).x; }
    __device__ static __forceinline__ float load1(const void* p, int64_t i) {
        return static_cast<float>(static_cast<const _Float16*>(p)[i]);
    }
    __device__ static __forceinline__ void store1(void* p, int64_t i, float v) {
        static_cast<_Float16*>(p)[i] = static_cast<_Float16>(v);
    }
    __device__ static __forceinline__ float round(float v) { return static_cast<float>(static_cast<_Float16>(v)); }
};

template <>
struct Io<DT_BF16> {
    static constexpr int E = 8;
    static constexpr int BYTES = 2;
    // bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits.
    __device__ static __forceinline__ float lo(unsigned u) { return bit_cast<float>(u << 16); }
    __device__ static __forceinline__ float hi(unsigned u) { return bit_cast<float>(u & 0xffff0000u); }
    __device__ static __forceinline__ unsigned narrow2(float a, float b) {
        return bit_cast<unsigned>(__builtin_convertvector((f32x2{a, b}), bf16x2));
    }
    __device__ static __forceinline__ void unpack(const u32x4& v, float* f) {
        f[0] = lo(v.x); f[1] = hi(v.x); f[2] = lo(v.y); f[3] = hi(v.y);
        f[4] = lo(v.z); f[5] = hi(v.z); f[6] = lo(v.w); f[7] = hi(v.w);
    }
    __device__ static __forceinline__ u32x4 pack(const float* f) {
        return u32x4{narrow2(f[0], f[1]), narrow2(f[2], f[3]), narrow2(f[4], f[5]), narrow2(f[6], f[7])};
    }
    __device__ static __forceinline__ float first(const u32x4& v) { return lo(v.x); }
    __device__ static __forceinline__ float load1(const void* p, int64_t i) {
        return lo(static_cast<const unsigned short*>(p)[i]);
    }
    __device__ static __forceinline__ void store1(void* p, int64_t i, float v) {
        static_cast<__bf16*>(p)[i] = static_cast<__bf16>(v);
    }
    __device__ static __forceinline__ float round(float v) { return static_cast<float>(static_cast<__bf16>(v)); }
};

// ---------------------------------------------------------------------------------------
// Wavefront reductions. Must be called with all 64 lanes active.
// ---------------------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return bit_cast<float>(__builtin_amdgcn_update_dpp(0, bit_cast<int>(v), CTRL, 0xF, 0xF, true));
}

// Sum over the 64 lanes; every lane returns the same bits.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]: partner lane ^ 1
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]: partner lane ^ 2 -> quad-uniform
    v += dpp<0x141>(v);  // row_half_mirror: lane i <- 7 - i, the other quad -> 8-uniform
    v += dpp<0x140>(v);  // row_mirror: lane i <- 15 - i, the other 8 lanes -> 16-uniform
    const float r0 = bit_cast<float>(__builtin_amdgcn_readlane(bit_cast<int>(v), 0));
    const float r1 = bit_cast<float>(__builtin_amdgcn_readlane(bit_cast<int>(v), 16));
    const float r2 = bit_cast<float>(__builtin_amdgcn_readlane(bit_cast<int>(v), 32));
    const float r3 = bit_cast<float>(__builtin_amdgcn_readlane(bit_cast<int>(v), 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float uniform(float v) {
    return bit_cast<float>(__builtin_amdgcn_readfirstlane(bit_cast<int>(v)));
}

// (count, mean, M2) of a part of a row; mean is relative to the row's shift K.
struct Moments {
    float n, m, m2;
};

// Pairwise Welford combine; an empty side returns the other side unchanged.
__device__ __forceinline__ Moments combine(const Moments& a, const Moments& b) {
    if (b.n == 0.f) return a;
    if (a.n == 0.f) return b;
    const float n = a.n + b.n;
    const float d = b.m - a.m;
    const float f = b.n / n;
    return Moments{n, a.m + d * f, a.m2 + b.m2 + d * d * a.n * f};
}

__device__ __forceinline__ float inv_sqrt(float v) { return 1.0f / sqrtf(v); }

// ---------------------------------------------------------------------------------------
// Vectorized kernel.
// ---------------------------------------------------------------------------------------

template <int DT, int OP, int W, int V, int RPB>
__global__ __launch_bounds__(64 * W * RPB) void rownorm_vec_kernel(Params p) {
    static_assert(W == 1 || RPB == 1, "a row group spanning waves owns the whole workgroup");
    using IO = Io<DT>;
    constexpr int E = IO::E;
    constexpr int LANES = 64 * W;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rg = wave / W;           // row slot of this wave in the workgroup
    const int wr = wave - rg * W;      // wave index inside the row group
    const int t = wr * 64 + lane;      // lane index inside the row group
    const int64_t C = p.C;
    const int Ci = static_cast<int>(C);  // chunks per row fit in 32 bits here (C <= 64 * W * V)
    const float nf = static_cast<float>(p.N);
    const bool has_g = p.gamma != nullptr;
    const bool has_b = p.beta != nullptr;

    // Per-wave partial moments for the cross-wave combine (double-buffered by iteration).
    __shared__ float part[2][W > 1 ? W : 1][3];
    int buf = 0;

    for (int64_t base = static_cast<int64_t>(blockIdx.x) * RPB; base < p.rows;
         base += static_cast<int64_t>(gridDim.x) * RPB) {
        const int64_t row = base + rg;
        if (W == 1 && row >= p.rows) break;  // wave-uniform; no barrier in this variant

        const u32x4* xr = static_cast<const u32x4*>(p.x) + row * C;

        // ---- a1: issue every load of the row (and of the residual / parameters) first.
        u32x4 xv[V];
        u32x4 rv[OP == OP_FUSED ? V : 1];
        u32x4 gv[V];
        u32x4 bv[OP == OP_LN ? V : 1];
        bool valid[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int c = i * LANES + t;
            valid[i] = c < Ci;
            const int cc = valid[i] ? c : Ci - 1;  // in-bounds address for idle lanes
            xv[i] = xr[cc];
            if constexpr (OP == OP_FUSED) rv[i] = (static_cast<const u32x4*>(p.residual) + row * C)[cc];
        }
        if (has_g) {
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const int c = i * LANES + t;
                gv[i] = static_cast<const u32x4*>(p.gamma)[valid[i] ? c : Ci - 1];
            }
        }
        if constexpr (OP == OP_LN) {
            if (has_b) {
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    const int c = i * LANES + t;
                    bv[i] = static_cast<const u32x4*>(p.beta)[valid[i] ? c : Ci - 1];
                }
            }
        }

        // ---- widen to fp32 (a2: fused add, rounded to the I/O dtype and stored).
        float v[V][E];
        if constexpr (OP == OP_FUSED) {
            u32x4* ro = static_cast<u32x4*>(p.residual_out) + row * C;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float a[E], b[E];
                IO::unpack(xv[i], a);
                IO::unpack(rv[i], b);
#pragma unroll
                for (int e = 0; e < E; ++e) a[e] += b[e];
                const u32x4 tv = IO::pack(a);  // t = round(x + residual)
                if (valid[i]) ro[i * LANES + t] = tv;
                IO::unpack(tv, v[i]);          // the rounded value is what gets normalized
            }
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) IO::unpack(xv[i], v[i]);
        }
#pragma unroll
        for (int i = 0; i < V; ++i) {
            if (!valid[i]) {
#pragma unroll
                for (int e = 0; e < E; ++e) v[i][e] = 0.f;
            }
        }

        float scale;   // rstd
        float center;  // LayerNorm: mean relative to K; unused for RMSNorm
        float K = 0.f;
        if constexpr (OP == OP_LN) {
            // ---- a3/a4: shifted moments of this wave's part of the row.
            if constexpr (W == 1) {
                K = uniform(IO::first(xv[0]));  // lane 0 holds chunk 0
            } else {
                K = IO::load1(p.x, row * p.N);
            }
            float s1 = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    v[i][e] = valid[i] ? v[i][e] - K : 0.f;
                    s1 += v[i][e];
                }
            }
            float n_w;
            if constexpr (W == 1) {
                n_w = nf;
            } else {
                int cnt = 0;  // valid chunks of this wave
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    const int first = i * LANES + wr * 64;
                    const int k = Ci - first;
                    cnt += k <= 0 ? 0 : (k >= 64 ? 64 : k);
                }
                n_w = static_cast<float>(cnt * E);
            }
            const float S1 = wave_sum(s1);
            const float m_w = n_w > 0.f ? S1 / n_w : 0.f;
            float s2 = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float d = v[i][e] - m_w;
                    s2 += valid[i] ? d * d : 0.f;
                }
            }
            Moments mo{n_w, m_w, wave_sum(s2)};
            if constexpr (W > 1) {
                // ---- a5: cross-wave combine of (n, mean, M2) in LDS.
                if (lane == 0) {
                    part[buf][wr][0] = mo.n;
                    part[buf][wr][1] = mo.m;
                    part[buf][wr][2] = mo.m2;
                }
                __syncthreads();
                Moments acc{part[buf][0][0], part[buf][0][1], part[buf][0][2]};
#pragma unroll
                for (int w = 1; w < W; ++w) acc = combine(acc, Moments{part[buf][w][0], part[buf][w][1], part[buf][w][2]});
                mo = acc;
                buf ^= 1;
            }
            // ---- a6: finalize.
            center = mo.m;
            scale = inv_sqrt(mo.m2 / nf + p.eps);
            if (t == 0) {
                if (p.mean) p.mean[row] = K + center;
                if (p.rstd) p.rstd[row] = scale;
            }
        } else {
            // ---- RMSNorm statistics: sum of squares.
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) {
#pragma unroll
                for (int e = 0; e < E; ++e) s += v[i][e] * v[i][e];
            }
            float S = wave_sum(s);
            if constexpr (W > 1) {
                if (lane == 0) part[buf][wr][0] = S;
                __syncthreads();
                S = part[buf][0][0];
#pragma unroll
                for (int w = 1; w < W; ++w) S += part[buf][w][0];
                buf ^= 1;
            }
            center = 0.f;
            scale = inv_sqrt(S / nf + p.eps);
            if (t == 0 && p.rstd) p.rstd[row] = scale;
        }

        // ---- a7: normalize from registers, apply the affine parameters, store.
        u32x4* yr = static_cast<u32x4*>(p.y) + row * C;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float g[E], b[E];
            if (has_g) {
                IO::unpack(gv[i], g);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) g[e] = 1.f;
            }
            if constexpr (OP == OP_LN) {
                if (has_b) {
                    IO::unpack(bv[i], b);
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) b[e] = 0.f;
                }
            }
            float o[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                if constexpr (OP == OP_LN) {
                    o[e] = (v[i][e] - center) * scale * g[e] + b[e];
                } else {
                    o[e] = v[i][e] * scale * g[e];
                }
            }
            if (valid[i]) yr[i * LANES + t] = IO::pack(o);
        }
    }
}

// ---------------------------------------------------------------------------------------
// General kernel: any N, element-aligned pointers.
// ---------------------------------------------------------------------------------------

template <int NWAVES>
__device__ __forceinline__ float block_sum(float v, float* slots) {
    const float w = wave_sum(v);
    if ((threadIdx.x & 63) == 0) slots[threadIdx.x >> 6] = w;
    __syncthreads();
    float s = slots[0];
#pragma unroll
    for (int i = 1; i < NWAVES; ++i) s += slots[i];
    return s;
}

template <int DT, int OP>
__global__ __launch_bounds__(kGeneralThreads) void rownorm_general_kernel(Params p) {
    using IO = Io<DT>;
    constexpr int NW = kGeneralThreads / 64;
    __shared__ float slots[2][NW];
    const int tid = threadIdx.x;
    const int64_t N = p.N;
    const float nf = static_cast<float>(N);
    for (int64_t row = blockIdx.x; row < p.rows; row += gridDim.x) {
        const int64_t off = row * N;
        float center = 0.f, scale, K = 0.f;
        if constexpr (OP == OP_LN) {
            K = IO::load1(p.x, off);
            float s1 = 0.f;
            for (int64_t j = tid; j < N; j += kGeneralThreads) s1 += IO::load1(p.x, off + j) - K;
            center = block_sum<NW>(s1, slots[0]) / nf;
            float s2 = 0.f;
            for (int64_t j = tid; j < N; j += kGeneralThreads) {
                const float d = (IO::load1(p.x, off + j) - K) - center;
                s2 += d * d;
            }
            scale = inv_sqrt(block_sum<NW>(s2, slots[1]) / nf + p.eps);
            if (tid == 0) {
                if (p.mean) p.mean[row] = K + center;
                if (p.rstd) p.rstd[row] = scale;
            }
        } else {
            float s = 0.f;
            for (int64_t j = tid; j < N; j += kGeneralThreads) {
                float v;
                if constexpr (OP == OP_FUSED) {
                    v = IO::round(IO::load1(p.x, off + j) + IO::load1(p.residual, off + j));
                    IO::store1(p.residual_out, off + j, v);
                } else {
                    v = IO::load1(p.x, off + j);
                }
                s += v * v;
            }
            scale = inv_sqrt(block_sum<NW>(s, slots[0]) / nf + p.eps);
            if (tid == 0 && p.rstd) p.rstd[row] = scale;
        }
        for (int64_t j = tid; j < N; j += kGeneralThreads) {
            const float g = p.gamma ? IO::load1(p.gamma, j) : 1.f;
            float o;
            if constexpr (OP == OP_LN) {
                const float b = p.beta ? IO::load1(p.beta, j) : 0.f;
                o = ((IO::load1(p.x, off + j) - K) - center) * scale * g + b;
            } else if constexpr (OP == OP_FUSED) {
                // this lane's own residual_out element, written above
                o = IO::load1(p.residual_out, off + j) * scale * g;
            } else {
                o = IO::load1(p.x, off + j) * scale * g;
            }
            IO::store1(p.y, off + j, o);
        }
        __syncthreads();  // slots are reused by the next row
    }
}

// ---------------------------------------------------------------------------------------
// Dispatch from runtime (op, dtype, plan) to a template instance.
// ---------------------------------------------------------------------------------------

template <typename K>
static hipError_t go(K kernel, const Plan& plan, const Params& p, hipStream_t stream) {
    Params args = p;
    void* argv[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<unsigned>(plan.grid)),
                           dim3(static_cast<unsigned>(plan.block_threads)), argv, 0, stream);
}

template <int DT, int OP, int W, int RPB>
static hipError_t launch_vec(const Plan& plan, const Params& p, hipStream_t s) {
    switch (plan.chunks_per_lane) {
    case 1: return go(rownorm_vec_kernel<DT, OP, W, 1, RPB>, plan, p, s);
    case 2: return go(rownorm_vec_kernel<DT, OP, W, 2, RPB>, plan, p, s);
    case 4: return go(rownorm_vec_kernel<DT, OP, W, 4, RPB>, plan, p, s);
    case 8: return go(rownorm_vec_kernel<DT, OP, W, 8, RPB>, plan, p, s);
    case 16: return go(rownorm_vec_kernel<DT, OP, W, 16, RPB>, plan, p, s);
    default: return hipErrorInvalidValue;
    }
}

template <int DT, int OP>
static hipError_t launch_op(const Plan& plan, const Params& p, hipStream_t s) {
    if (plan.variant == V_WAVE) {
        if (plan.waves_per_row == 1 && plan.rows_per_block == kWaveRowsPerBlock)
            return launch_vec<DT, OP, 1, kWaveRowsPerBlock>(plan, p, s);
    } else if (plan.variant == V_WORKGROUP) {
        if (plan.waves_per_row == kGroupWaves && plan.rows_per_block == 1)
            return launch_vec<DT, OP, kGroupWaves, 1>(plan, p, s);
    } else if (plan.variant == V_GENERAL) {
        return go(rownorm_general_kernel<DT, OP>, plan, p, s);
    }
    return hipErrorInvalidValue;
}

template <int DT>
static hipError_t launch_dt(int op, const Plan& plan, const Params& p, hipStream_t s) {
    switch (op) {
    case OP_LN: return launch_op<DT, OP_LN>(plan, p, s);
    case OP_RMS: return launch_op<DT, OP_RMS>(plan, p, s);
    case OP_FUSED: return launch_op<DT, OP_FUSED>(plan, p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch(int op, int dtype, const Plan& plan, const Params& p, hipStream_t stream) {
    switch (dtype) {
    case DT_F32: return launch_dt<DT_F32>(op, plan, p, stream);
    case DT_F16: return launch_dt<DT_F16>(op, plan, p, stream);
    case DT_BF16: return launch_dt<DT_BF16>(op, plan, p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace rn
