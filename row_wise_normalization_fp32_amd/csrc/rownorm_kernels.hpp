// Row-wise LayerNorm / RMSNorm / fused residual-add + RMSNorm kernels for gfx950 (MI355X).
//
// The operations are defined in include/rownorm.h. All three are bandwidth-bound: a few
// fp32 operations per element against 2-4 bytes moved per element (the LayerNorm CUDA
// walkthrough, lpnh.cn/news/2756757, section 1, counts about 5 FLOP per 4-byte element;
// "CUDA fused RMSNorm kernel", diycv.top, section 1, calls RMSNorm memory-bound). The
// design goal: read every input byte from HBM once, write every output byte once, with
// 16-byte coalesced accesses and enough bytes in flight per CU, while keeping the VALU
// work per element small. The last point matters on this chip: without packed-fp32
// instructions a CU retires 64 fp32 lane-operations per clock, which at the HBM rate is
// only about 20 operations per bf16 element of a LayerNorm (2 B in + 2 B out).
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
//   * EXACT instances (the row is exactly V passes of the row group, true for every
//     power-of-two width) carry no tail masking at all; the others clamp idle lanes'
//     addresses into the row and zero their values.
//   * Every load of a row is issued before any of its values is used (a scheduling
//     barrier keeps the compiler from interleaving the first uses with the loads).
//   * Cross-lane sums use DPP (quad_perm, row_half_mirror, row_mirror: each step adds a
//     lane's value to its partner's, and every partner pair is symmetric, so all 16 lanes
//     of a DPP row end with the same bits), then readlane of lanes 0/16/32/48 adds the
//     four row sums in a fixed order. The result is wave-uniform and deterministic.
//   * LayerNorm statistics: corrected two-pass (see VecRow::norm_row). A rough mean comes
//     from a first pass (v_dot2 of packed fp16 / bf16 pairs with 1.0; for fp32 a pass
//     shifted by K = x[row, 0]), one centered pass then gives the exact mean and M2.
//   * W > 1: each wavefront produces a (count, mean - K, M2) triple for its share of the
//     row; the triples meet in LDS after one barrier and every lane folds them in the same
//     fixed pairwise tree (count = na + nb, delta = mb - ma, mean = ma + delta * nb / n,
//     M2 = M2a + M2b + delta^2 * na * nb / n; the "05 LLM Ops" lesson, smarter.xin, section
//     "Welford combine function"). With equal parts every scaling is by exactly 1/2.
//   * gamma / beta / weight presence is a compile-time property (AFF flags), so absent
//     parameters cost nothing.
//   * Two launch modes. Grid per row: one workgroup per RPB rows, parameters loaded with
//     each row. Persistent (many rows): a grid sized to the resident capacity, each
//     workgroup loops over rows; the parameters are staged once (gamma in VGPRs and beta in
//     LDS for LayerNorm, the weight in LDS otherwise), rows stream with non-temporal
//     accesses, and LayerNorm keeps only the loaded row between statistics and output.
//
// General kernel (rownorm_general_kernel): any N and any element-aligned pointers. One
// 256-lane workgroup per row; it reads the row up to three times (statistics, centered
// squares, normalization), element by element. Correct everywhere, not tuned.
#pragma once

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
    __device__ static __forceinline__ float elem(const u32x4& v, int e) { return bit_cast<float>(v[e]); }
    // acc + the sum of the chunk's elements / of their squares
    __device__ static __forceinline__ float sum(const u32x4& v, float acc) {
        return acc + (bit_cast<float>(v.x) + bit_cast<float>(v.y)) + (bit_cast<float>(v.z) + bit_cast<float>(v.w));
    }
    __device__ static __forceinline__ float sumsq(const u32x4& v, float acc) {
        float f[4];
        unpack(v, f);
        return fmaf(f[3], f[3], fmaf(f[2], f[2], fmaf(f[1], f[1], fmaf(f[0], f[0], acc))));
    }
    __device__ static __forceinline__ float load1(const void* p, int64_t i) {
        return static_cast<const float*>(p)[i];
    }
    __device__ static __forceinline__ void store1(void* p, int64_t i, float v) { static_cast<float*>(p)[i] = v; }
    __device__ static __forceinline__ float round(float v) { return v; }
};

template <>
struct Io<DT_F16> {
    static constexpr int E = 8;
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
    __device__ static __forceinline__ float elem(const u32x4& v, int e) {
        return static_cast<float>(bit_cast<f16x2>(v[e >> 1])[e & 1]);
    }
    // v_dot2_f32_f16: products of fp16 values with 1.0 or with themselves are exact in fp32.
    __device__ static __forceinline__ float dot(unsigned a, unsigned b, float acc) {
        return __builtin_amdgcn_fdot2(bit_cast<f16x2>(a), bit_cast<f16x2>(b), acc, false);
    }
    __device__ static __forceinline__ float sum(const u32x4& v, float acc) {
        constexpr unsigned one = 0x3c003c00u;  // (1.0, 1.0)
        return dot(v.w, one, dot(v.z, one, dot(v.y, one, dot(v.x, one, acc))));
    }
    __device__ static __forceinline__ float sumsq(const u32x4& v, float acc) {
        return dot(v.w, v.w, dot(v.z, v.z, dot(v.y, v.y, dot(v.x, v.x, acc))));
    }
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
    __device__ static __forceinline__ float elem(const u32x4& v, int e) { return (e & 1) ? hi(v[e >> 1]) : lo(v[e >> 1]); }
    // v_dot2_f32_bf16: products of bf16 values with 1.0 or with themselves are exact in fp32.
    __device__ static __forceinline__ float dot(unsigned a, unsigned b, float acc) {
        return __builtin_amdgcn_fdot2_f32_bf16(bit_cast<bf16x2>(a), bit_cast<bf16x2>(b), acc, false);
    }
    __device__ static __forceinline__ float sum(const u32x4& v, float acc) {
        constexpr unsigned one = 0x3f803f80u;  // (1.0, 1.0)
        return dot(v.w, one, dot(v.z, one, dot(v.y, one, dot(v.x, one, acc))));
    }
    __device__ static __forceinline__ float sumsq(const u32x4& v, float acc) {
        return dot(v.w, v.w, dot(v.z, v.z, dot(v.y, v.y, dot(v.x, v.x, acc))));
    }
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

// 1 / sqrt(v) with the hardware reciprocal square root (error within about 1 ulp).
__device__ __forceinline__ float inv_sqrt(float v) { return __builtin_amdgcn_rsqf(v); }

// Pairwise combine of two parts of equal size n: mean = (ma + mb) / 2,
// M2 = M2a + M2b + (mb - ma)^2 * n / 2. Every scaling is by a power of two, so the only
// roundings are those of the additions.
__device__ __forceinline__ Moments combine_equal(const Moments& a, const Moments& b) {
    const float d = b.m - a.m;
    return Moments{a.n + b.n, 0.5f * (a.m + b.m), a.m2 + b.m2 + d * d * (0.5f * a.n)};
}

// Compile-time presence of the affine parameters.
enum { AFF_G = 1, AFF_B = 2 };

// Compile-time memory-access choices of the vectorized kernel.
enum {
    FL_NT_STORE = 2,     // non-temporal (streaming) stores of y / residual_out
    FL_NT_LOAD = 4,      // non-temporal loads of x / residual
    FL_NOFLOAT = 8,      // LayerNorm: keep only the loaded row between the statistics and the
                         // normalization (re-widen / re-center it there) instead of an fp32 copy
    FL_PARAMS_LDS = 16,  // stage gamma / beta / weight in LDS once per workgroup, not VGPRs
    FL_GAMMA_REG = 32,   // with FL_PARAMS_LDS and both parameters: gamma stays in VGPRs (loaded
                         // once per workgroup), only beta is staged in LDS (half the LDS)
};

template <int FL>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
    if constexpr ((FL & FL_NT_LOAD) != 0) return __builtin_nontemporal_load(p);
    return *p;
}

template <int FL>
__device__ __forceinline__ void st(u32x4* p, const u32x4& v) {
    if constexpr ((FL & FL_NT_STORE) != 0) {
        __builtin_nontemporal_store(v, p);
    } else {
        *p = v;
    }
}

// ---------------------------------------------------------------------------------------
// Vectorized kernels: one row group of W wavefronts holds a row in VGPRs.
// ---------------------------------------------------------------------------------------

template <int DT, int OP, int W, int V, bool EXACT, int AFF, int FL>
struct VecRow {
    using IO = Io<DT>;
    static constexpr int E = IO::E;
    static constexpr int LANES = 64 * W;
    static constexpr int WS = W > 1 ? W : 1;
    static constexpr bool HG = (AFF & AFF_G) != 0;                 // gamma / weight present
    static constexpr bool HB = OP == OP_LN && (AFF & AFF_B) != 0;  // beta present
    static constexpr int NR = OP == OP_FUSED ? V : 1;              // residual registers
    static constexpr int NG = HG ? V : 1;
    static constexpr int NB = HB ? V : 1;

    // Chunk of slot i for lane t, clamped into the row for idle lanes of a ragged tail.
    __device__ static __forceinline__ int chunk(int i, int t, int Ci) {
        const int c = i * LANES + t;
        return EXACT ? c : (c < Ci ? c : Ci - 1);
    }
    __device__ static __forceinline__ bool valid(int i, int t, int Ci) { return EXACT || i * LANES + t < Ci; }

    // LayerNorm's common reference point K = x[row, 0] is loaded with the row when the row
    // spans several waves (with one wave, lane 0 already holds it).
    static constexpr bool LOAD_K = OP == OP_LN && W > 1;

    // a1: issue every load of the row (and of the residual, and K).
    __device__ static __forceinline__ void load_row(const Params& p, int64_t row, int t, int Ci, u32x4 (&xv)[V],
                                                    u32x4 (&rv)[NR], float& K) {
        if constexpr (LOAD_K) K = IO::load1(p.x, row * p.N);
        const u32x4* xr = static_cast<const u32x4*>(p.x) + row * p.C;
#pragma unroll
        for (int i = 0; i < V; ++i) xv[i] = ld<FL>(xr + chunk(i, t, Ci));
        if constexpr (OP == OP_FUSED) {
            const u32x4* rr = static_cast<const u32x4*>(p.residual) + row * p.C;
#pragma unroll
            for (int i = 0; i < V; ++i) rv[i] = ld<FL>(rr + chunk(i, t, Ci));
        }
    }

    __device__ static __forceinline__ void load_params(const Params& p, int t, int Ci, u32x4 (&gv)[NG],
                                                       u32x4 (&bv)[NB]) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
            if constexpr (HG) gv[i] = static_cast<const u32x4*>(p.gamma)[chunk(i, t, Ci)];
            if constexpr (HB) bv[i] = static_cast<const u32x4*>(p.beta)[chunk(i, t, Ci)];
        }
    }

    // Where the epilogue takes gamma / beta / weight from.
    enum { PARAMS_REG = 0, PARAMS_LDS = 2 };

    // a2-a7 for one row whose chunks are in xv / rv. `part` is the workgroup's LDS
    // exchange area (double-buffered by `buf`), used when W > 1. Parameters come from gv /
    // bv (PARAMS_REG) or are read from LDS at `lds` (PARAMS_LDS: gamma chunks then beta
    // chunks; with FL_GAMMA_REG gamma comes from gv and LDS holds only beta).
    //
    // LayerNorm statistics use the corrected two-pass form (Chan, Golub and LeVeque): a
    // rough mean a = sum(x) / n from a first pass (for fp16 / bf16 one v_dot2 per element
    // pair, no widening), then one centered pass that accumulates c = sum(x - a) and
    // q = sum((x - a)^2): mean = a + c / n and M2 = q - c^2 / n, exact for any a and
    // accurate when a is near the mean. Only the centered values x - a stay in registers.
    // Across the waves of a row group the per-wave moments are made relative to a common
    // point K = x[row, 0] and combined pairwise (Welford), as the walkthrough's section 6
    // and the LLM-ops lesson's combine function describe.
    template <int PSRC>
    __device__ static __forceinline__ void norm_row(const Params& p, int64_t row, int lane, int wr, int t, int Ci,
                                                    const u32x4 (&xv)[V], const u32x4 (&rv)[NR], float K,
                                                    u32x4 (&gv)[NG], u32x4 (&bv)[NB], const u32x4* lds,
                                                    float (*part)[WS][3], int& buf) {
        const float nf = static_cast<float>(p.N);
        // Chunk i as the kernel sees it: the input, or for the fused op the rounded sum.
        u32x4 src[V];
        if constexpr (OP == OP_FUSED) {
            // ---- a2: t = round(x + residual), stored as residual_out; t is what gets normalized.
            u32x4* ro = static_cast<u32x4*>(p.residual_out) + row * p.C;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float a[E], b[E];
                IO::unpack(xv[i], a);
                IO::unpack(rv[i], b);
#pragma unroll
                for (int e = 0; e < E; ++e) a[e] += b[e];
                src[i] = IO::pack(a);
                if (valid(i, t, Ci)) st<FL>(ro + i * LANES + t, src[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) src[i] = xv[i];
        }
        if constexpr (!EXACT) {
#pragma unroll
            for (int i = 0; i < V; ++i)
                if (!valid(i, t, Ci)) src[i] = u32x4{0u, 0u, 0u, 0u};  // idle lanes contribute zeros
        }
        float n_w;  // elements held by this wave
        if constexpr (W == 1) {
            n_w = nf;
        } else if constexpr (EXACT) {
            n_w = static_cast<float>(V * 64 * E);
        } else {
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const int k = Ci - (i * LANES + wr * 64);
                cnt += k <= 0 ? 0 : (k >= 64 ? 64 : k);
            }
            n_w = static_cast<float>(cnt * E);
        }

        // NOFLOAT: the widened row is not kept; the epilogue widens the packed row again.
        constexpr bool NOFLOAT = (FL & FL_NOFLOAT) != 0 && OP == OP_LN;
        float v[NOFLOAT ? 1 : V][NOFLOAT ? 1 : E];  // LayerNorm: x - a; RMSNorm: x
        float scale;    // rstd
        float offset = 0.f;
        float a_keep = 0.f;  // LayerNorm: the rough mean a
        if constexpr (OP == OP_LN) {
            // ---- a3/a4, first pass: rough mean of this wave's part. The common reference
            // K = x[row, 0] is needed by the cross-wave combine and, for fp32 rows, shifts
            // this pass so that a constant row gives a == K exactly (for fp16 / bf16 rows
            // the plain sums of a constant are exact already).
            if constexpr (DT == DT_F32 && W == 1) K = uniform(IO::first(src[0]));  // lane 0 holds chunk 0
            float s1 = 0.f;
            if constexpr (DT == DT_F32) {
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    float f[E];
                    IO::unpack(src[i], f);
#pragma unroll
                    for (int e = 0; e < E; ++e) s1 += valid(i, t, Ci) ? f[e] - K : 0.f;
                }
            } else {
#pragma unroll
                for (int i = 0; i < V; ++i) s1 = IO::sum(src[i], s1);
            }
            const float inv_w = W == 1 ? p.inv_n : (n_w > 0.f ? 1.0f / n_w : 0.f);  // constant when EXACT
            const float mw = wave_sum(s1) * inv_w;
            const float a = DT == DT_F32 ? K + mw : mw;
            // ---- centered pass.
            float c = 0.f, q = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float f[E];
                IO::unpack(src[i], f);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float d = valid(i, t, Ci) ? f[e] - a : 0.f;
                    if constexpr (!NOFLOAT) v[i][e] = d;
                    c += d;
                    q = fmaf(d, d, q);
                }
            }
            a_keep = a;
            const float Cw = wave_sum(c);
            const float Qw = wave_sum(q);
            float rel;  // mean - a
            float m2;   // sum of squared deviations
            if constexpr (W == 1) {
                rel = Cw * p.inv_n;
                m2 = fmaxf(Qw - Cw * rel, 0.f);
                if (t == 0 && p.mean) p.mean[row] = a + rel;
            } else {
                // ---- a5: per-wave (n, mean - K, M2), combined across the row group in LDS.
                const float cw = Cw * inv_w;
                Moments mo{n_w, (a - K) + cw, fmaxf(Qw - Cw * cw, 0.f)};
                if (lane == 0) {
                    part[buf][wr][0] = mo.n;
                    part[buf][wr][1] = mo.m;
                    part[buf][wr][2] = mo.m2;
                }
                __syncthreads();
                Moments acc;
                if constexpr (EXACT && (W & (W - 1)) == 0) {
                    // equal parts: a fixed pairwise tree, (0,1) (2,3) ... then pairs of pairs
                    Moments m[W];
#pragma unroll
                    for (int w = 0; w < W; ++w) m[w] = Moments{part[buf][w][0], part[buf][w][1], part[buf][w][2]};
#pragma unroll
                    for (int step = 1; step < W; step *= 2) {
#pragma unroll
                        for (int w = 0; w + step < W; w += 2 * step) m[w] = combine_equal(m[w], m[w + step]);
                    }
                    acc = m[0];
                } else {
                    acc = Moments{part[buf][0][0], part[buf][0][1], part[buf][0][2]};
#pragma unroll
                    for (int w = 1; w < W; ++w) acc = combine(acc, Moments{part[buf][w][0], part[buf][w][1], part[buf][w][2]});
                }
                buf ^= 1;
                rel = acc.m - (a - K);  // row mean relative to this wave's a
                m2 = acc.m2;
                if (t == 0 && p.mean) p.mean[row] = K + acc.m;
            }
            // ---- a6: finalize.
            scale = inv_sqrt(fmaf(m2, p.inv_n, p.eps));
            offset = -rel * scale;
            if (t == 0 && p.rstd) p.rstd[row] = scale;
        } else {
            // ---- RMSNorm statistics: sum of squares.
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) s = IO::sumsq(src[i], s);
            float S = wave_sum(s);
            if constexpr (W > 1) {
                if (lane == 0) part[buf][wr][0] = S;
                __syncthreads();
                S = part[buf][0][0];
#pragma unroll
                for (int w = 1; w < W; ++w) S += part[buf][w][0];
                buf ^= 1;
            }
            scale = inv_sqrt(fmaf(S, p.inv_n, p.eps));
            if (t == 0 && p.rstd) p.rstd[row] = scale;
#pragma unroll
            for (int i = 0; i < V; ++i) IO::unpack(src[i], v[i]);
        }

        // ---- a7: normalize from registers, apply the affine parameters, store.
        if constexpr (NOFLOAT) {
            // Make the packed registers opaque so the widening below is recomputed here
            // rather than kept alive (as fp32 values) since the centered pass.
#pragma unroll
            for (int i = 0; i < V; ++i) asm volatile("" : "+v"(src[i]));
        }
        u32x4* yr = static_cast<u32x4*>(p.y) + row * p.C;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float g[E], b[E], o[E];
            float w[E];  // NOFLOAT: x - a of this chunk
            if constexpr (NOFLOAT) {
                IO::unpack(src[i], w);
#pragma unroll
                for (int e = 0; e < E; ++e) w[e] -= a_keep;
            }
            if constexpr (PSRC == PARAMS_LDS) {
                const int c = chunk(i, t, Ci);
                constexpr bool GREG = (FL & FL_GAMMA_REG) != 0 && HG && HB;
                if constexpr (GREG) {
                    IO::unpack(gv[i], g);
                    IO::unpack(lds[c], b);
                } else {
                    if constexpr (HG) IO::unpack(lds[c], g);
                    if constexpr (HB) IO::unpack(lds[(HG ? Ci : 0) + c], b);
                }
            } else {
                if constexpr (HG) IO::unpack(gv[i], g);
                if constexpr (HB) IO::unpack(bv[i], b);
            }
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float z;
                if constexpr (NOFLOAT) {
                    z = fmaf(w[e], scale, offset);
                } else {
                    z = OP == OP_LN ? fmaf(v[i][e], scale, offset) : v[i][e] * scale;
                }
                if constexpr (HG && HB) {
                    z = fmaf(z, g[e], b[e]);
                } else if constexpr (HG) {
                    z = z * g[e];
                } else if constexpr (HB) {
                    z = z + b[e];
                }
                o[e] = z;
            }
            if (valid(i, t, Ci)) st<FL>(yr + i * LANES + t, IO::pack(o));
        }
    }
};

// One row group per row, rows assigned round-robin over the grid (grid-stride loop). With
// FL_PARAMS_LDS the workgroup first stages gamma / beta / weight in LDS, once, and all its
// row groups read them from there for every row; the grid is then sized to the device's
// resident capacity so that each workgroup handles many rows.
template <int DT, int OP, int W, int V, int RPB, bool EXACT, int AFF, int FL>
__global__ __launch_bounds__(64 * W * RPB) void rownorm_vec_kernel(Params p) {
    using R = VecRow<DT, OP, W, V, EXACT, AFF, FL>;
    constexpr bool PLDS = (FL & FL_PARAMS_LDS) != 0 && (R::HG || R::HB);
    constexpr int PSRC = PLDS ? R::PARAMS_LDS : R::PARAMS_REG;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rg = wave / W;       // row slot of this wave in the workgroup
    const int wr = wave - rg * W;  // wave index inside the row group
    const int t = wr * 64 + lane;  // lane index inside the row group
    const int Ci = static_cast<int>(p.C);  // chunks per row fit in 32 bits here (C <= 64 * W * V)
    __shared__ float part[RPB][2][R::WS][3];
    extern __shared__ u32x4 prm[];  // PLDS: gamma chunks [C], then beta chunks [C]
    constexpr bool GREG = PLDS && (FL & FL_GAMMA_REG) != 0 && R::HG && R::HB;
    u32x4 gkeep[GREG ? V : 1];  // GREG: this lane's gamma chunks, for all rows
    if constexpr (PLDS) {
        for (int c = threadIdx.x; c < Ci; c += 64 * W * RPB) {
            if constexpr (GREG) {
                prm[c] = static_cast<const u32x4*>(p.beta)[c];
            } else {
                if constexpr (R::HG) prm[c] = static_cast<const u32x4*>(p.gamma)[c];
                if constexpr (R::HB) prm[(R::HG ? Ci : 0) + c] = static_cast<const u32x4*>(p.beta)[c];
            }
        }
        if constexpr (GREG) {
#pragma unroll
            for (int i = 0; i < V; ++i) gkeep[i] = static_cast<const u32x4*>(p.gamma)[R::chunk(i, t, Ci)];
        }
        __syncthreads();
    }
    int buf = 0;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * RPB; base < p.rows;
         base += static_cast<int64_t>(gridDim.x) * RPB) {
        const int64_t row = base + rg;
        if (row >= p.rows) {
            if constexpr (W == 1) break;  // wave-uniform; no barrier in this variant
            // a row group without a row still takes part in the workgroup barrier
            __syncthreads();
            buf ^= 1;
            continue;
        }
        u32x4 xv[V], rv[R::NR], gv[R::NG], bv[R::NB];
        float K = 0.f;
        R::load_row(p, row, t, Ci, xv, rv, K);
        if constexpr (PSRC == R::PARAMS_REG) R::load_params(p, t, Ci, gv, bv);
        if constexpr (GREG) {
#pragma unroll
            for (int i = 0; i < V; ++i) gv[i] = gkeep[i];
        }
        __builtin_amdgcn_sched_barrier(0);  // every load of the row is issued before any use
        R::template norm_row<PSRC>(p, row, lane, wr, t, Ci, xv, rv, K, gv, bv, prm, part[rg], buf);
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
// Dispatch from a runtime plan to a template instance. Instantiated per dtype and mode in
// rownorm_kernels_<dtype>.hip (grid-per-row launches and the general kernel) and
// rownorm_kernels_<dtype>_persistent.hip (persistent launches).
// ---------------------------------------------------------------------------------------

// Row groups per workgroup for a row-group width: 256-lane workgroups up to W = 4.
constexpr int rows_per_block_for(int W) { return W <= 4 ? 4 / W : 1; }

// Memory-access flags of the persistent mode: non-temporal streaming of the rows,
// parameters staged once per workgroup (gamma in VGPRs and beta in LDS when LayerNorm has
// both), and no fp32 copy of the LayerNorm row (more workgroups resident per CU).
template <int OP, int AFF>
constexpr int persistent_flags() {
    int fl = FL_NT_LOAD | FL_NT_STORE | FL_PARAMS_LDS;
    if (OP == OP_LN) fl |= FL_NOFLOAT;
    if (OP == OP_LN && AFF == (AFF_G | AFF_B)) fl |= FL_GAMMA_REG;
    return fl;
}

template <typename K>
inline hipError_t go(K kernel, const Plan& plan, const Params& p, hipStream_t stream) {
    Params args = p;
    void* argv[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<unsigned>(plan.grid)),
                           dim3(static_cast<unsigned>(plan.block_threads)), argv, 0, stream);
}

constexpr int kMaxDevices = 64;

// Persistent launch: as many workgroups as the current device keeps resident (queried once
// per kernel instance and device), at most one per row group of work.
template <typename K>
inline hipError_t go_persistent(K kernel, const Plan& plan, const Params& p, hipStream_t stream) {
    static int per_cu_cache[kMaxDevices];  // 0: not yet known; a benign race writes the same value
    static int cus_cache[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int per_cu = dev < kMaxDevices ? __atomic_load_n(&per_cu_cache[dev], __ATOMIC_RELAXED) : 0;
    int cus = dev < kMaxDevices ? __atomic_load_n(&cus_cache[dev], __ATOMIC_RELAXED) : 0;
    if (per_cu <= 0 || cus <= 0) {
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel),
                                                         plan.block_threads, static_cast<size_t>(plan.lds_bytes));
        if (e != hipSuccess) return e;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (per_cu < 1) per_cu = 1;
        if (dev < kMaxDevices) {
            __atomic_store_n(&per_cu_cache[dev], per_cu, __ATOMIC_RELAXED);
            __atomic_store_n(&cus_cache[dev], cus, __ATOMIC_RELAXED);
        }
    }
    int64_t grid = static_cast<int64_t>(cus) * per_cu;
    if (grid > plan.grid) grid = plan.grid;
    Params args = p;
    void* argv[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(static_cast<unsigned>(grid)),
                           dim3(static_cast<unsigned>(plan.block_threads)), argv,
                           static_cast<size_t>(plan.lds_bytes), stream);
}

template <int DT, int OP, int W, bool EXACT, int AFF, bool PERS>
inline hipError_t launch_v(const Plan& plan, const Params& p, hipStream_t s) {
    constexpr int RPB = rows_per_block_for(W);
    constexpr int FL = PERS ? persistent_flags<OP, AFF>() : 0;
    if (plan.rows_per_block != RPB) return hipErrorInvalidValue;
#define RN_GO(VV) \
    (PERS ? go_persistent(rownorm_vec_kernel<DT, OP, W, VV, RPB, EXACT, AFF, FL>, plan, p, s) \
          : go(rownorm_vec_kernel<DT, OP, W, VV, RPB, EXACT, AFF, FL>, plan, p, s))
    switch (plan.chunks_per_lane) {
    case 1: return RN_GO(1);
    case 2: return RN_GO(2);
    case 4: return RN_GO(4);
    default: break;
    }
    if constexpr (W == 1) {
        switch (plan.chunks_per_lane) {
        case 8: return RN_GO(8);
        case 16: return RN_GO(16);
        default: break;
        }
    }
#undef RN_GO
    return hipErrorInvalidValue;
}

template <int DT, int OP, bool EXACT, int AFF, bool PERS>
inline hipError_t launch_w(const Plan& plan, const Params& p, hipStream_t s) {
    switch (plan.waves_per_row) {
    case 1: return launch_v<DT, OP, 1, EXACT, AFF, PERS>(plan, p, s);
    case 2: return launch_v<DT, OP, 2, EXACT, AFF, PERS>(plan, p, s);
    case 4: return launch_v<DT, OP, 4, EXACT, AFF, PERS>(plan, p, s);
    case 8: return launch_v<DT, OP, 8, EXACT, AFF, PERS>(plan, p, s);
    case 16: return launch_v<DT, OP, 16, EXACT, AFF, PERS>(plan, p, s);
    default: return hipErrorInvalidValue;
    }
}

template <int DT, int OP, int AFF, bool PERS>
inline hipError_t launch_e(const Plan& plan, const Params& p, hipStream_t s) {
    if constexpr (PERS) {
        // persistent launches are planned only for exact shapes with parameters
        if (!plan.exact || AFF == 0) return hipErrorInvalidValue;
        if constexpr (AFF != 0) return launch_w<DT, OP, true, AFF, true>(plan, p, s);
        return hipErrorInvalidValue;
    } else {
        return plan.exact ? launch_w<DT, OP, true, AFF, false>(plan, p, s)
                          : launch_w<DT, OP, false, AFF, false>(plan, p, s);
    }
}

template <int DT, int OP, bool PERS>
inline hipError_t launch_op(const Plan& plan, const Params& p, hipStream_t s) {
    if (plan.variant == V_GENERAL) {
        if constexpr (PERS) return hipErrorInvalidValue;
        return go(rownorm_general_kernel<DT, OP>, plan, p, s);
    }
    if (plan.variant != V_WAVE && plan.variant != V_WORKGROUP) return hipErrorInvalidValue;
    const int aff = (p.gamma ? AFF_G : 0) | (OP == OP_LN && p.beta ? AFF_B : 0);
    switch (aff) {
    case 0: return launch_e<DT, OP, 0, PERS>(plan, p, s);
    case AFF_G: return launch_e<DT, OP, AFF_G, PERS>(plan, p, s);
    default: break;
    }
    if constexpr (OP == OP_LN) {
        if (aff == AFF_B) return launch_e<DT, OP, AFF_B, PERS>(plan, p, s);
        return launch_e<DT, OP, AFF_G | AFF_B, PERS>(plan, p, s);
    }
    return hipErrorInvalidValue;
}

template <int DT, bool PERS>
inline hipError_t launch_dtype(int op, const Plan& plan, const Params& p, hipStream_t s) {
    switch (op) {
    case OP_LN: return launch_op<DT, OP_LN, PERS>(plan, p, s);
    case OP_RMS: return launch_op<DT, OP_RMS, PERS>(plan, p, s);
    case OP_FUSED: return launch_op<DT, OP_FUSED, PERS>(plan, p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace rn
