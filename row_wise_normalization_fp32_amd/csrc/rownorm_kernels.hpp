// Row-wise LayerNorm / RMSNorm / fused residual-add + RMSNorm / fused residual-add +
// LayerNorm / softmax kernels for gfx950 (MI355X).
//
// The operations are defined in include/rownorm.h. All of them are bandwidth-bound: a few
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
// Element kernel (rownorm_elem_kernel) and pair kernel (rownorm_pair_kernel): rows that are
// not whole 16-byte chunks or tensors that are only element-aligned, rows of up to 16384
// elements. The same register-resident structure at element granularity, through buffer
// resources bounded by the row; 16-bit rows move as 4-byte element pairs when all row
// tensors sit at the same position within 4-byte words.
//
// Split-row kernels (rownorm_wide_* and rownorm_wide_elem_*): rows longer than a workgroup's
// registers, cut into segments; a statistics launch writes one record per segment to a
// caller workspace, a second launch combines the row's records and normalizes.
//
// General kernel (rownorm_general_kernel): any N and any element-aligned pointers, for long
// rows without a workspace. One 256-lane workgroup per row; it reads the row up to three
// times (statistics, centered squares, normalization), element by element. Correct
// everywhere, not tuned.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// Buffer resources for element-granular rows: a descriptor in SGPRs (base, byte size) and
// 32-bit byte offsets in VGPRs. Loads beyond the size return 0 and stores beyond it are
// dropped by the hardware (raw buffer addressing), so a row needs neither clamped indices
// nor branches around its accesses, and no 64-bit address per element.
using Rsrc = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // 32-bit data format, no swizzle (untyped accesses)

//
// Every resource here describes memory of one row (or segment, or parameter vector) that the
// whole wave works on: base and size are the same on every lane. They are taken from the
// first active lane so that the compiler keeps the descriptor in SGPRs even where it cannot
// prove it uniform (a value defined inside a loop that lanes leave at different times counts
// as divergent after it); a descriptor in VGPRs would wrap each access in a loop over the
// distinct descriptors of the lanes.
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, static_cast<short>(0), static_cast<int>(n), kRsrcWord3);
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
    template <int CP = 0>
    __device__ static __forceinline__ float bload(Rsrc r, uint32_t j) {
        return bit_cast<float>(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(j * 4), 0, CP));
    }
    template <int CP = 0>
    __device__ static __forceinline__ void bstore(Rsrc r, uint32_t j, float v) {
        __builtin_amdgcn_raw_buffer_store_b32(bit_cast<unsigned>(v), r, static_cast<int>(j * 4), 0, CP);
    }
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
    template <int CP = 0>
    __device__ static __forceinline__ float bload(Rsrc r, uint32_t j) {
        return static_cast<float>(
            bit_cast<_Float16>(__builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(j * 2), 0, CP)));
    }
    template <int CP = 0>
    __device__ static __forceinline__ void bstore(Rsrc r, uint32_t j, float v) {
        __builtin_amdgcn_raw_buffer_store_b16(bit_cast<unsigned short>(static_cast<_Float16>(v)), r,
                                              static_cast<int>(j * 2), 0, CP);
    }
    // two adjacent elements held in one 32-bit word, the lower-addressed one in the low half
    __device__ static __forceinline__ f32x2 widen_pair(unsigned u) { return widen2(u); }
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
    // Scalar conversions go through the packed hardware conversion (v_cvt_pk_bf16_f32,
    // round to nearest even) instead of a scalar software rounding sequence.
    __device__ static __forceinline__ void store1(void* p, int64_t i, float v) {
        static_cast<unsigned short*>(p)[i] = static_cast<unsigned short>(narrow2(v, v));
    }
    __device__ static __forceinline__ float round(float v) { return lo(narrow2(v, v)); }
    template <int CP = 0>
    __device__ static __forceinline__ float bload(Rsrc r, uint32_t j) {
        return lo(__builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(j * 2), 0, CP));
    }
    template <int CP = 0>
    __device__ static __forceinline__ void bstore(Rsrc r, uint32_t j, float v) {
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(narrow2(v, v)), r, static_cast<int>(j * 2),
                                              0, CP);
    }
    __device__ static __forceinline__ f32x2 widen_pair(unsigned u) { return f32x2{lo(u), hi(u)}; }
};

// 32-bit and 16-bit buffer accesses at a byte offset (out of range: loads read 0, stores
// are dropped). CP is the instruction's cache-policy field (2: non-temporal).
template <int CP = 0>
__device__ __forceinline__ unsigned bload32(Rsrc r, uint32_t off) {
    return static_cast<unsigned>(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, CP));
}
template <int CP = 0>
__device__ __forceinline__ void bstore32(Rsrc r, uint32_t off, unsigned v) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, static_cast<int>(off), 0, CP);
}
template <int CP = 0>
__device__ __forceinline__ void bstore16(Rsrc r, uint32_t off, unsigned v) {
    __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(v), r, static_cast<int>(off), 0, CP);
}

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

// Maximum of two values that is NaN if either is (v_maximum3_f32), unlike fmaxf, which
// returns the other operand. Softmax takes its maxima this way so that a NaN logit makes its
// row NaN (0 / 0 in the final scale) instead of silently dropping out of the row; -inf
// (masked) entries still drop out, as max(-inf, x) = x.
__device__ __forceinline__ float max_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Maximum over the 64 lanes, by the same exchange pattern (NaN if any lane holds NaN).
__device__ __forceinline__ float wave_max(float v) {
    v = max_nan(v, dpp<0xB1>(v));
    v = max_nan(v, dpp<0x4E>(v));
    v = max_nan(v, dpp<0x141>(v));
    v = max_nan(v, dpp<0x140>(v));
    const float r0 = bit_cast<float>(__builtin_amdgcn_readlane(bit_cast<int>(v), 0));
    const float r1 = bit_cast<float>(__builtin_amdgcn_readlane(bit_cast<int>(v), 16));
    const float r2 = bit_cast<float>(__builtin_amdgcn_readlane(bit_cast<int>(v), 32));
    const float r3 = bit_cast<float>(__builtin_amdgcn_readlane(bit_cast<int>(v), 48));
    return max_nan(max_nan(r0, r1), max_nan(r2, r3));
}

__device__ __forceinline__ float uniform(float v) {
    return bit_cast<float>(__builtin_amdgcn_readfirstlane(bit_cast<int>(v)));
}

// (count, mean, M2) of a part of a row; mean is relative to a reference point common to
// the parts being combined.
struct Moments {
    float n, m, m2;
};

// Pairwise Welford combine; an empty side returns the other side unchanged. The weight
// nb / n uses the hardware reciprocal (about 1 ulp; a correctly rounded division costs about
// ten instructions, per part and row). Equal means (d == 0) combine exactly either way.
__device__ __forceinline__ Moments combine(const Moments& a, const Moments& b) {
    if (b.n == 0.f) return a;
    if (a.n == 0.f) return b;
    const float n = a.n + b.n;
    const float d = b.m - a.m;
    const float f = b.n * __builtin_amdgcn_rcpf(n);
    return Moments{n, a.m + d * f, a.m2 + b.m2 + d * d * a.n * f};
}

// 1 / sqrt(v) with the hardware reciprocal square root (error within about 1 ulp).
__device__ __forceinline__ float inv_sqrt(float v) { return __builtin_amdgcn_rsqf(v); }

// 2^v with the hardware exponential (v_exp_f32).
__device__ __forceinline__ float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }
constexpr float kLog2e = 1.44269504088896340736f;           // log2(e) rounded to fp32
constexpr float kLog2eLo = 1.92596298909109e-8f;            // log2(e) - kLog2e

// e^u for u <= 0 (softmax's x - max), with a relative error of a few ulps for every u.
// The hardware exponential takes a base-2 argument; its error, and the rounding of
// u * log2(e), grow with the argument's magnitude (about |u| * 2^-23 relative). So the
// product is formed exactly as hi + lo (fma for the rounding error of hi, plus the part of
// log2(e) that fp32 drops), its integer part n is split off exactly, 2^(fraction) comes
// from v_exp_f32 on [-0.5, 0.5], and ldexp applies 2^n without rounding (down to the
// subnormal range). Arguments below -200 (including -inf, an empty part's maximum) give 0,
// and so does NaN (-inf - (-inf) for a part holding only masked entries); a NaN logit
// reaches the result through the row's maximum instead (see max_nan).
__device__ __forceinline__ float exp_neg(float u) {
    // No contraction: every kernel that inlines this gets the same roundings (the segment
    // records of a split row must have the same bits whichever kernel forms them).
#pragma clang fp contract(off)
    u = fmaxf(u, -200.f);
    const float hi = u * kLog2e;
    const float lo = fmaf(u, kLog2e, -hi) + u * kLog2eLo;
    const float n = rintf(hi);
    const float f = (hi - n) + lo;
    return ldexpf(exp2_hw(f), static_cast<int>(n));
}

// Pairwise combine of two parts of equal size n: mean = (ma + mb) / 2,
// M2 = M2a + M2b + (mb - ma)^2 * n / 2. Every scaling is by a power of two, so the only
// roundings are those of the additions.
__device__ __forceinline__ Moments combine_equal(const Moments& a, const Moments& b) {
    const float d = b.m - a.m;
    return Moments{a.n + b.n, 0.5f * (a.m + b.m), a.m2 + b.m2 + d * d * (0.5f * a.n)};
}

// Softmax partial state of a part of a row: its maximum and sum of exp(x - max).
// Combining two parts rescales both sums to the larger maximum (the "05 LLM Ops" lesson,
// smarter.xin, sections "Online Softmax denominator correction" and "merging (max, sum)
// with decay").
__device__ __forceinline__ void softmax_combine(float& m, float& s, float mb, float sb) {
    // No contraction: both products are rounded, so combining (a, b) and (b, a) gives the same
    // bits (the butterflies rely on it) in every kernel that inlines this.
#pragma clang fp contract(off)
    const float M = max_nan(m, mb);
    s = s * exp_neg(m - M) + sb * exp_neg(mb - M);
    m = M;
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
    FL_PREFETCH = 64,    // grid-stride loop: the next row's loads are issued before the current
                         // row's reductions and stores (two rows of registers per lane)
    FL_RAGGED = 128,     // rows addressed by byte: row starts and tensors need only element
                         // alignment, and the row's last chunk may be partial (see VecRow)
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

// Properties of an operation.
template <int OP>
struct OpTraits {
    static constexpr bool LN = OP == OP_LN || OP == OP_FUSED_LN;    // mean-centred statistics
    static constexpr bool RES = OP == OP_FUSED || OP == OP_FUSED_LN;  // residual add first
    static constexpr bool SM = OP == OP_SOFTMAX;
    static constexpr bool RMS = OP == OP_RMS || OP == OP_FUSED;
};

// Per-wave LDS record of a row group: LayerNorm (n, rough mean a, mean - a, M2);
// RMSNorm (sum of squares); softmax (max, sum).
struct WavePart {
    float v[4];
};

// ---------------------------------------------------------------------------------------
// Row-group statistics shared by the vectorized and the element kernels. Each wave has
// reduced its own part of the row; these combine the W parts after one workgroup barrier
// (W == 1: nothing to combine). `part` is this row group's LDS area, double-buffered by
// `buf` so that consecutive rows need one barrier each.
// ---------------------------------------------------------------------------------------

// LayerNorm: wave part (n_w, a_w, cw = mean_w - a_w, M2_w). Returns the row's mean relative
// to this wave's a (rel), M2 and the row mean. The parts are put on a common reference
// R = a_0 (wave 0's rough mean): m_w = (a_w - R) + cw, where a_w - R is exact whenever the
// rough means are within a factor of two of each other (Sterbenz), then combined in a fixed
// pairwise tree (equal parts) or left to right.
template <int W, bool EQUAL>
__device__ __forceinline__ void group_moments(WavePart (*part)[W > 1 ? W : 1], int& buf, int lane, int wr, float n_w,
                                              float a_w, float cw, float m2w, float& rel, float& m2, float& mean) {
    if constexpr (W == 1) {
        rel = cw;
        m2 = m2w;
        mean = a_w + cw;
    } else {
        if (lane == 0) {
            WavePart& q = part[buf][wr];
            q.v[0] = n_w;
            q.v[1] = a_w;
            q.v[2] = cw;
            q.v[3] = m2w;
        }
        __syncthreads();
        const float R = part[buf][0].v[1];
        auto load = [&](int w) {
            const WavePart q = part[buf][w];
            return Moments{q.v[0], (q.v[1] - R) + q.v[2], q.v[3]};
        };
        Moments acc;
        if constexpr (EQUAL && (W & (W - 1)) == 0 && W <= 16) {
            // The fixed pairwise tree ((0,1),(2,3)),((4,5),(6,7)),... across lanes: lane l
            // holds part l, and at step s lane l combines with lane l + s (DPP: quad_perm
            // for s = 1, 2, row_shl for s = 4, 8). Lane 0 ends with the row's moments.
            const WavePart q = part[buf][lane < W ? lane : 0];
            Moments m{q.v[0], (q.v[1] - R) + q.v[2], q.v[3]};
            auto step = [&](auto ctrl) {
                constexpr int C = decltype(ctrl)::value;
                const Moments o{dpp<C>(m.n), dpp<C>(m.m), dpp<C>(m.m2)};
                m = combine_equal(m, o);
            };
            step(std::integral_constant<int, 0xB1>{});                      // lane + 1
            if constexpr (W > 2) step(std::integral_constant<int, 0x4E>{});  // lane + 2
            if constexpr (W > 4) step(std::integral_constant<int, 0x104>{}); // row_shl:4
            if constexpr (W > 8) step(std::integral_constant<int, 0x108>{}); // row_shl:8
            acc = Moments{uniform(m.n), uniform(m.m), uniform(m.m2)};
        } else {
            acc = load(0);
#pragma unroll
            for (int w = 1; w < W; ++w) acc = combine(acc, load(w));
        }
        buf ^= 1;
        rel = acc.m - (a_w - R);
        m2 = acc.m2;
        mean = R + acc.m;
    }
}

template <int W>
__device__ __forceinline__ float group_sum(WavePart (*part)[W > 1 ? W : 1], int& buf, int lane, int wr, float s) {
    if constexpr (W == 1) {
        return s;
    } else {
        if (lane == 0) part[buf][wr].v[0] = s;
        __syncthreads();
        float S = part[buf][0].v[0];
#pragma unroll
        for (int w = 1; w < W; ++w) S += part[buf][w].v[0];
        buf ^= 1;
        return S;
    }
}

// Softmax: combine the waves' (max, sum) pairs, left to right; returns the row's max and sum.
template <int W>
__device__ __forceinline__ void group_softmax(WavePart (*part)[W > 1 ? W : 1], int& buf, int lane, int wr, float mw,
                                              float sw, float& M, float& S) {
    if constexpr (W == 1) {
        M = mw;
        S = sw;
    } else {
        if (lane == 0) {
            part[buf][wr].v[0] = mw;
            part[buf][wr].v[1] = sw;
        }
        __syncthreads();
        M = part[buf][0].v[0];
        S = part[buf][0].v[1];
#pragma unroll
        for (int w = 1; w < W; ++w) softmax_combine(M, S, part[buf][w].v[0], part[buf][w].v[1]);
        buf ^= 1;
    }
}

// ---------------------------------------------------------------------------------------
// Vectorized kernels: one row group of W wavefronts holds a row in VGPRs.
// ---------------------------------------------------------------------------------------

template <int DT, int OP, int W, int V, bool EXACT, int AFF, int FL>
struct VecRow {
    using IO = Io<DT>;
    using OT = OpTraits<OP>;
    static constexpr int E = IO::E;
    static constexpr int LANES = 64 * W;
    static constexpr int WS = W > 1 ? W : 1;
    static constexpr bool HG = !OT::SM && (AFF & AFF_G) != 0;  // gamma / weight present
    static constexpr bool HB = OT::LN && (AFF & AFF_B) != 0;   // beta present
    static constexpr int NR = OT::RES ? V : 1;                 // residual registers
    static constexpr int NG = HG ? V : 1;
    static constexpr int NB = HB ? V : 1;

    // FL_RAGGED: row r of a row tensor starts at byte r * ld * s, at any element-aligned
    // address. The lane layout stays the aligned one (chunk c holds elements E c to E c + E - 1),
    // and every chunk moves as one 16-byte access, which the hardware performs at any alignment,
    // through a buffer resource that ends with the row. The hardware checks such a resource's
    // range per dword (a dword of an access moves only if all of its 4 bytes lie inside), so
    // the row's partial last chunk (N not a multiple of E) moves its whole dwords and reads 0
    // for the rest, and nothing past the row is touched. What is left is the row's last element
    // when a 16-bit row has an odd length: the low half of a dword that straddles the row's
    // end. One 2-byte access moves it (issued by the waves holding that chunk, with an offset
    // past the row on every lane but its own), and it joins the chunk where the row is first
    // used, so that no load waits inside the row's batch of loads. The partial chunk's missing
    // elements are masked out of the statistics.
    static constexpr bool RAG = (FL & FL_RAGGED) != 0;
    static constexpr int SB = 16 / E;                            // bytes per element
    static constexpr int CPL = (FL & FL_NT_LOAD) != 0 ? 2 : 0;   // buffer cache policy: non-temporal
    static constexpr int CPS = (FL & FL_NT_STORE) != 0 ? 2 : 0;
    struct Rag {
        uint32_t rb;  // bytes of the row
        int te;       // elements of the partial chunk (0: none)
        int ti;       // its slot (-1: none)
        int tt;       // its lane in the row group
        int hd;       // 16-bit rows of odd length: the partial chunk's dword holding the last
                      // element in its low half; -1 otherwise
    };
    __device__ static __forceinline__ Rag rag(const Params& p) {
        Rag g;
        const int n = static_cast<int>(p.N);  // N <= 64 * W * V * E fits in 32 bits here
        const int full = n / E;
        g.rb = static_cast<uint32_t>(n) * SB;
        g.te = n - full * E;
        g.ti = g.te != 0 ? full / LANES : -1;
        g.tt = full % LANES;
        g.hd = SB == 2 && (n & 1) != 0 ? (g.te - 1) >> 1 : -1;
        return g;
    }
    // The waves that hold the partial chunk's lane (the 2-byte access is issued by them only).
    __device__ static __forceinline__ bool tail_wave(const Rag& g, int t) {
        return g.hd >= 0 && __builtin_amdgcn_readfirstlane(t >> 6) == (g.tt >> 6);
    }
    // The last element of an odd-length 16-bit row, in the low half (0 on other lanes).
    template <int CP>
    __device__ static __forceinline__ unsigned tail_half(Rsrc r, const Rag& g, int t) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(t == g.tt ? g.rb - 2u : g.rb), 0, CP);
    }
    __device__ static __forceinline__ u32x4 with_half(u32x4 v, unsigned h, const Rag& g) {
        v.x |= g.hd == 0 ? h : 0u;
        v.y |= g.hd == 1 ? h : 0u;
        v.z |= g.hd == 2 ? h : 0u;
        v.w |= g.hd == 3 ? h : 0u;
        return v;
    }
    // The row at byte address `base`: its chunks into v, the last element of an odd-length
    // 16-bit row into th on the lane that holds it (th is read only on that lane).
    __device__ static __forceinline__ void rag_load_row(const char* base, const Rag& g, int t, int Ci, u32x4 (&v)[V],
                                                        u32x4& th) {
        const Rsrc r = make_rsrc(base, g.rb);
#pragma unroll
        for (int i = 0; i < V; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, chunk(i, t, Ci) * 16, 0, CPL);
        if (tail_wave(g, t)) th.x = tail_half<CPL>(r, g, t);
    }
    __device__ static __forceinline__ void rag_store_row(char* base, const Rag& g, int i, int t, int Ci,
                                                         const u32x4& v) {
        const Rsrc r = make_rsrc(base, g.rb);
        if (valid(i, t, Ci))  // the partial chunk: its whole dwords
            __builtin_amdgcn_raw_buffer_store_b128(v, r, (i * LANES + t) * 16, 0, CPS);
        if (tail_slot(i, g) && tail_wave(g, t)) {  // and the half dword of an odd-length 16-bit row
            const unsigned h = g.hd == 0 ? v.x : g.hd == 1 ? v.y : g.hd == 2 ? v.z : v.w;
            bstore16<CPS>(r, t == g.tt ? g.rb - 2u : g.rb, h);
        }
    }
    // Chunk c of a parameter vector (element-aligned, N elements).
    __device__ static __forceinline__ u32x4 param_chunk(const void* base, int c, const Rag& g) {
        if constexpr (!RAG) {
            return static_cast<const u32x4*>(base)[c];
        } else {
            const Rsrc r = make_rsrc(base, g.rb);
            u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, c * 16, 0, 0);
            if (g.hd >= 0 && c == g.ti * LANES + g.tt)
                v = with_half(v, __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(g.rb - 2u), 0, 0), g);
            return v;
        }
    }

    // Chunk of slot i for lane t, clamped into the row for idle lanes of a ragged tail.
    __device__ static __forceinline__ int chunk(int i, int t, int Ci) {
        const int c = i * LANES + t;
        return EXACT ? c : (c < Ci ? c : Ci - 1);
    }
    __device__ static __forceinline__ bool valid(int i, int t, int Ci) { return EXACT || i * LANES + t < Ci; }
    // Uniform slot classes of a row of Ci chunks (chunk-exact rows: every slot full). A full
    // slot holds a chunk of the row on every lane, a live one on some lane.
    __device__ static __forceinline__ bool full_slot(int i, int Ci) { return EXACT || (i + 1) * LANES <= Ci; }
    __device__ static __forceinline__ bool live_slot(int i, int Ci) { return EXACT || i * LANES < Ci; }
    // RAG: slot i holds the row's partial last chunk. In chunk-exact rows that chunk is the last
    // slot's, so the test is a constant false for the other slots.
    __device__ static __forceinline__ bool tail_slot(int i, const Rag& g) {
        if constexpr (!RAG)
            return false;
        else
            return (!EXACT || i == V - 1) && i == g.ti;
    }

    // a1: issue every load of the row (and of the residual). Row strides are in chunks.
    __device__ static __forceinline__ void load_row(const Params& p, int64_t row, int t, int Ci, u32x4 (&xv)[V],
                                                    u32x4 (&rv)[NR], u32x4& xt, u32x4& rt) {
        if constexpr (RAG) {
            const Rag g = rag(p);
            rag_load_row(static_cast<const char*>(p.x) + row * p.ldx * SB, g, t, Ci, xv, xt);
            if constexpr (OT::RES) rag_load_row(static_cast<const char*>(p.residual) + row * p.ldr * SB, g, t, Ci, rv, rt);
            return;
        }
        const u32x4* xr = static_cast<const u32x4*>(p.x) + row * p.cx;
#pragma unroll
        for (int i = 0; i < V; ++i) xv[i] = ld<FL>(xr + chunk(i, t, Ci));
        if constexpr (OT::RES) {
            const u32x4* rr = static_cast<const u32x4*>(p.residual) + row * p.cr;
#pragma unroll
            for (int i = 0; i < V; ++i) rv[i] = ld<FL>(rr + chunk(i, t, Ci));
        }
    }

    __device__ static __forceinline__ void load_params(const Params& p, int t, int Ci, u32x4 (&gv)[NG],
                                                       u32x4 (&bv)[NB]) {
        const Rag g = RAG ? rag(p) : Rag{};
#pragma unroll
        for (int i = 0; i < V; ++i) {
            if constexpr (HG) gv[i] = param_chunk(p.gamma, chunk(i, t, Ci), g);
            if constexpr (HB) bv[i] = param_chunk(p.beta, chunk(i, t, Ci), g);
        }
    }

    // Where the epilogue takes gamma / beta / weight from.
    enum { PARAMS_REG = 0, PARAMS_LDS = 2 };

    // a2-a7 for one row whose chunks are in xv / rv. Parameters come from gv / bv
    // (PARAMS_REG) or are read from LDS at `lds` (PARAMS_LDS: gamma chunks then beta
    // chunks; with FL_GAMMA_REG gamma comes from gv and LDS holds only beta).
    //
    // LayerNorm statistics use the corrected two-pass form (Chan, Golub and LeVeque): a
    // rough mean a = sum(x) / n from a first pass (for fp16 / bf16 one v_dot2 per element
    // pair, no widening; for fp32 a pass shifted by the wave's first element, so that a
    // constant row gives a exactly), then one centered pass that accumulates c = sum(x - a)
    // and q = sum((x - a)^2): mean = a + c / n and M2 = q - c^2 / n, exact for any a and
    // accurate when a is near the mean. Only the centered values x - a stay in registers.
    // Across the waves of a row group the per-wave moments are combined pairwise (Welford),
    // as the walkthrough's section 6 and the LLM-ops lesson's combine function describe.
    //
    // Softmax: per wave the maximum, then the sum of exp(x - max) with the exponentials kept
    // in registers; the waves' (max, sum) pairs are combined with the rescaling of the online
    // form; the output is exp(x - max_w) * (exp(max_w - max) / sum).
    template <int PSRC>
    __device__ static __forceinline__ void norm_row(const Params& p, int64_t row, int lane, int wr, int t, int Ci,
                                                    const u32x4 (&xv)[V], const u32x4 (&rv)[NR], const u32x4& xt,
                                                    const u32x4& rt, u32x4 (&gv)[NG], u32x4 (&bv)[NB],
                                                    const u32x4* lds, WavePart (*part)[WS], int& buf) {
        const Rag g = RAG ? rag(p) : Rag{};
        // RAG: the partial chunk joins its slot here, at the row's first use.
        auto xin = [&](int i) {
            u32x4 v = xv[i];
            if constexpr (RAG) {
                if (tail_slot(i, g) && g.hd >= 0 && t == g.tt) v = with_half(v, xt.x, g);
            }
            return v;
        };
        auto rin = [&](int i) {
            u32x4 v = rv[OT::RES ? i : 0];
            if constexpr (RAG) {
                if (tail_slot(i, g) && g.hd >= 0 && t == g.tt) v = with_half(v, rt.x, g);
            }
            return v;
        };
        // RAG: in the slot that holds the partial chunk (a uniform branch), its missing
        // elements take the value `fill` on the lane that holds it, so that they add exactly 0
        // to a sum of (f - fill) terms; the other slots are left alone
        auto fill_tail = [&](int i, float(&f)[E], float fill) {
            if constexpr (RAG) {
                if (tail_slot(i, g)) {
                    const bool me = t == g.tt;
#pragma unroll
                    for (int e = 0; e < E; ++e) f[e] = (me && e >= g.te) ? fill : f[e];
                }
            }
        };
        // element e of slot i is part of the row
        auto ok = [&](int i, int e) {
            if constexpr (RAG)
                return valid(i, t, Ci) && !(tail_slot(i, g) && t == g.tt && e >= g.te);
            else
                return valid(i, t, Ci);
        };
        // Slot i needs no per-element mask (a uniform branch): every lane holds a whole chunk
        // of the row there (fp32: the partial chunk's missing elements are filled instead).
        auto plain = [&](int i) { return full_slot(i, Ci) && (DT == DT_F32 || !tail_slot(i, g)); };
        // Chunk i as the kernel sees it: the input, or for the fused ops the rounded sum.
        u32x4 src[V];
        if constexpr (OT::RES) {
            // ---- a2: t = round(x + residual), stored as residual_out; t is what gets normalized.
            u32x4* ro = static_cast<u32x4*>(p.residual_out) + row * p.cro;
            char* rob = static_cast<char*>(p.residual_out) + row * p.ldro * SB;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                if (!live_slot(i, Ci)) {  // (uniform) no lane holds a chunk of the row here
                    src[i] = u32x4{0u, 0u, 0u, 0u};
                    continue;
                }
                float a[E], b[E];
                IO::unpack(xin(i), a);
                IO::unpack(rin(i), b);
#pragma unroll
                for (int e = 0; e < E; ++e) a[e] += b[e];
                src[i] = IO::pack(a);
                if constexpr (RAG)
                    rag_store_row(rob, g, i, t, Ci, src[i]);
                else if (valid(i, t, Ci))
                    st<FL>(ro + i * LANES + t, src[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) src[i] = xin(i);
        }
        if constexpr (!EXACT && !OT::SM) {
#pragma unroll
            for (int i = 0; i < V; ++i)
                if (!full_slot(i, Ci) && !valid(i, t, Ci)) src[i] = u32x4{0u, 0u, 0u, 0u};  // idle lanes: zeros
        }
        float n_w;  // elements held by this wave
        if constexpr (W == 1) {
            n_w = static_cast<float>(p.N);
        } else if constexpr (EXACT) {
            n_w = static_cast<float>(V * 64 * E);
            if constexpr (RAG) {
                if (g.ti >= 0 && (g.tt >> 6) == wr) n_w -= static_cast<float>(E - g.te);  // the partial chunk's wave
            }
        } else {
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const int k = Ci - (i * LANES + wr * 64);
                cnt += k <= 0 ? 0 : (k >= 64 ? 64 : k);
            }
            if constexpr (RAG) {
                if (g.ti >= 0 && (g.tt >> 6) == wr) cnt = cnt * E - (E - g.te);  // the partial chunk's wave
                else cnt *= E;
                n_w = static_cast<float>(cnt);
            } else {
                n_w = static_cast<float>(cnt * E);
            }
        }

        // NOFLOAT: the widened row is not kept; the epilogue widens the packed row again.
        constexpr bool NOFLOAT = (FL & FL_NOFLOAT) != 0 && OT::LN;
        float v[NOFLOAT ? 1 : V][NOFLOAT ? 1 : E];  // LayerNorm: x - a; RMSNorm: x; softmax: exp
        float scale;    // rstd, or 1 / sum for softmax
        float offset = 0.f;
        float a_keep = 0.f;  // LayerNorm: the rough mean a
        if constexpr (OT::LN) {
            // ---- a3/a4, first pass: rough mean of this wave's part.
            float K = 0.f;
            float s1 = 0.f;
            if constexpr (DT == DT_F32) {
                K = uniform(IO::first(src[0]));  // lane 0 holds the wave's first chunk
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    float f[E];
                    IO::unpack(src[i], f);
                    fill_tail(i, f, K);
                    if (plain(i)) {
#pragma unroll
                        for (int e = 0; e < E; ++e) s1 += f[e] - K;
                    } else {
                        const bool vl = valid(i, t, Ci);
#pragma unroll
                        for (int e = 0; e < E; ++e) s1 += vl ? f[e] - K : 0.f;
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < V; ++i) s1 = IO::sum(src[i], s1);
            }
            const float inv_w = W == 1 ? p.inv_n : (n_w > 0.f ? 1.0f / n_w : 0.f);  // constant when EXACT
            const float a = K + wave_sum(s1) * inv_w;
            // ---- centered pass.
            float c = 0.f, q = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float f[E];
                IO::unpack(src[i], f);
                if constexpr (DT == DT_F32) fill_tail(i, f, a);  // (16-bit rows: fewer VGPRs masked)
                if (plain(i)) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float d = f[e] - a;
                        if constexpr (!NOFLOAT) v[i][e] = d;
                        c += d;
                        q = fmaf(d, d, q);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float d = (DT == DT_F32 ? valid(i, t, Ci) : ok(i, e)) ? f[e] - a : 0.f;
                        if constexpr (!NOFLOAT) v[i][e] = d;
                        c += d;
                        q = fmaf(d, d, q);
                    }
                }
            }
            a_keep = a;
            const float Cw = wave_sum(c);
            const float Qw = wave_sum(q);
            const float cw = Cw * inv_w;
            // ---- a5: per-wave (n, a, mean - a, M2), combined across the row group in LDS.
            float rel, m2, mean;
            // (ragged rows: the partial chunk's wave holds fewer elements, so the general combine)
            group_moments<W, EXACT && !RAG>(part, buf, lane, wr, n_w, a, cw, fmaxf(Qw - Cw * cw, 0.f), rel, m2, mean);
            if (t == 0 && p.mean) p.mean[row] = mean;
            // ---- a6: finalize.
            scale = inv_sqrt(fmaf(m2, p.inv_n, p.eps));
            offset = -rel * scale;
            if (t == 0 && p.rstd) p.rstd[row] = scale;
        } else if constexpr (OT::SM) {
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float f[E];
                IO::unpack(src[i], f);
                if (full_slot(i, Ci) && !tail_slot(i, g)) {
#pragma unroll
                    for (int e = 0; e < E; ++e) mx = max_nan(mx, f[e]);
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) mx = ok(i, e) ? max_nan(mx, f[e]) : mx;
                }
            }
            const float mw = wave_max(mx);
            // exp(x - m_w): x - m_w is exact for the elements near the maximum.
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float f[E];
                IO::unpack(src[i], f);
                if (full_slot(i, Ci) && !tail_slot(i, g)) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float ex = exp_neg(f[e] - mw);
                        v[i][e] = ex;
                        s += ex;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float ex = ok(i, e) ? exp_neg(f[e] - mw) : 0.f;
                        v[i][e] = ex;
                        s += ex;
                    }
                }
            }
            float M, S;
            group_softmax<W>(part, buf, lane, wr, mw, wave_sum(s), M, S);
            scale = exp_neg(mw - M) / S;
            if (t == 0 && p.mean) p.mean[row] = M;
            if (t == 0 && p.rstd) p.rstd[row] = S;
        } else {
            // ---- RMSNorm statistics: sum of squares.
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) s = IO::sumsq(src[i], s);
            const float S = group_sum<W>(part, buf, lane, wr, wave_sum(s));
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
            // likewise the packed parameters: widen them here, not since their load
#pragma unroll
            for (int i = 0; i < V; ++i) {
                if constexpr (HG && PSRC == PARAMS_REG) asm volatile("" : "+v"(gv[i]));
                if constexpr (HB && PSRC == PARAMS_REG) asm volatile("" : "+v"(bv[i]));
            }
        }
        u32x4* yr = static_cast<u32x4*>(p.y) + row * p.cy;
        char* yb = static_cast<char*>(p.y) + row * p.ldy * SB;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            if (!live_slot(i, Ci)) continue;  // (uniform) nothing of the row to store here
            float gm[E], b[E], o[E];
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
                    IO::unpack(gv[i], gm);
                    IO::unpack(lds[c], b);
                } else {
                    if constexpr (HG) IO::unpack(lds[c], gm);
                    if constexpr (HB) IO::unpack(lds[(HG ? Ci : 0) + c], b);
                }
            } else {
                if constexpr (HG) IO::unpack(gv[i], gm);
                if constexpr (HB) IO::unpack(bv[i], b);
            }
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float z;
                if constexpr (NOFLOAT) {
                    z = fmaf(w[e], scale, offset);
                } else {
                    z = OT::LN ? fmaf(v[i][e], scale, offset) : v[i][e] * scale;
                }
                if constexpr (HG && HB) {
                    z = fmaf(z, gm[e], b[e]);
                } else if constexpr (HG) {
                    z = z * gm[e];
                } else if constexpr (HB) {
                    z = z + b[e];
                }
                o[e] = z;
            }
            if constexpr (RAG)
                rag_store_row(yb, g, i, t, Ci, IO::pack(o));
            else if (valid(i, t, Ci))
                st<FL>(yr + i * LANES + t, IO::pack(o));
        }
    }
};

// One row group per row, rows assigned round-robin over the grid (grid-stride loop). With
// FL_PARAMS_LDS the workgroup first stages gamma / beta / weight in LDS, once, and all its
// row groups read them from there for every row; the grid is then sized to the device's
// resident capacity so that each workgroup handles many rows.
//
// FL_PREFETCH keeps two rows per row group in flight: row r + stride is loaded into a second
// register set before row r is reduced and stored, and the two sets alternate (the loop is
// unrolled by two so that no registers are copied).
template <int DT, int OP, int W, int V, int RPB, bool EXACT, int AFF, int FL>
__global__ __launch_bounds__(64 * W * RPB) void rownorm_vec_kernel(Params p) {
    using R = VecRow<DT, OP, W, V, EXACT, AFF, FL>;
    constexpr bool PLDS = (FL & FL_PARAMS_LDS) != 0 && (R::HG || R::HB);
    constexpr int PSRC = PLDS ? R::PARAMS_LDS : R::PARAMS_REG;
    constexpr bool PF = (FL & FL_PREFETCH) != 0;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (SGPR)
    const int rg = wave / W;       // row slot of this wave in the workgroup
    const int wr = wave - rg * W;  // wave index inside the row group
    const int t = wr * 64 + lane;  // lane index inside the row group
    const int Ci = static_cast<int>(p.C);  // chunks per row fit in 32 bits here (C <= 64 * W * V)
    __shared__ WavePart part[RPB][2][R::WS];
    extern __shared__ u32x4 prm[];  // PLDS: gamma chunks [C], then beta chunks [C]
    constexpr bool GREG = PLDS && (FL & FL_GAMMA_REG) != 0 && R::HG && R::HB;
    u32x4 gkeep[GREG ? V : 1];  // GREG: this lane's gamma chunks, for all rows
    const int64_t stride = static_cast<int64_t>(gridDim.x) * RPB;
    int64_t base = static_cast<int64_t>(blockIdx.x) * RPB;
    // Row registers: xa / ra hold the row being processed; with FL_PREFETCH, xb / rb the next.
    u32x4 xa[V], ra[R::NR], xb[PF ? V : 1], rb[PF ? R::NR : 1];
    u32x4 xta, rta, xtb, rtb;  // FL_RAGGED: the partial chunk of the rows in xa / ra and xb / rb
    if constexpr (PLDS) {
        const typename R::Rag g = R::RAG ? R::rag(p) : typename R::Rag{};
        for (int c = threadIdx.x; c < Ci; c += 64 * W * RPB) {
            if constexpr (GREG) {
                prm[c] = R::param_chunk(p.beta, c, g);
            } else {
                if constexpr (R::HG) prm[c] = R::param_chunk(p.gamma, c, g);
                if constexpr (R::HB) prm[(R::HG ? Ci : 0) + c] = R::param_chunk(p.beta, c, g);
            }
        }
        if constexpr (GREG) {
#pragma unroll
            for (int i = 0; i < V; ++i) gkeep[i] = R::param_chunk(p.gamma, R::chunk(i, t, Ci), g);
        }
        __syncthreads();
    }
    int buf = 0;
    if constexpr (!PF) {
        for (; base < p.rows; base += stride) {
            const int64_t row = base + rg;
            if (row >= p.rows) {
                if constexpr (W == 1) break;  // wave-uniform; no barrier in this variant
                // a row group without a row still takes part in the workgroup barrier
                __syncthreads();
                buf ^= 1;
                continue;
            }
            // Per-lane addresses are recomputed for every row (a few VALU operations) rather than
            // hoisted out of the loop, where they would hold two VGPRs each for the whole kernel.
            int tl = t;
            asm volatile("" : "+v"(tl));
            u32x4 gv[R::NG], bv[R::NB];
            R::load_row(p, row, tl, Ci, xa, ra, xta, rta);
            if constexpr (PSRC == R::PARAMS_REG) R::load_params(p, tl, Ci, gv, bv);
            if constexpr (GREG) {
#pragma unroll
                for (int i = 0; i < V; ++i) gv[i] = gkeep[i];
            }
            __builtin_amdgcn_sched_barrier(0);  // every load of the row is issued before any use
            R::template norm_row<PSRC>(p, row, lane, wr, tl, Ci, xa, ra, xta, rta, gv, bv, prm, part[rg], buf);
        }
    } else {
        static_assert(PSRC == R::PARAMS_LDS || !(R::HG || R::HB), "the prefetching loop stages the parameters");
        {
            int tl = t;
            asm volatile("" : "+v"(tl));
            if (base + rg < p.rows) R::load_row(p, base + rg, tl, Ci, xa, ra, xta, rta);
        }
        // One row: its registers (xc, rc) are already loaded; the row one stride further is
        // loaded into (xn, rn) first.
        auto one = [&](int64_t row, u32x4(&xc)[V], u32x4(&rc)[R::NR], u32x4& xtc, u32x4& rtc, u32x4(&xn)[V],
                       u32x4(&rn)[R::NR], u32x4& xtn, u32x4& rtn) {
            int tl = t;
            asm volatile("" : "+v"(tl));
            if (row + stride < p.rows) R::load_row(p, row + stride, tl, Ci, xn, rn, xtn, rtn);
            u32x4 gv[R::NG], bv[R::NB];
            if constexpr (GREG) {
#pragma unroll
                for (int i = 0; i < V; ++i) gv[i] = gkeep[i];
            }
            __builtin_amdgcn_sched_barrier(0);
            if (row < p.rows) {
                R::template norm_row<PSRC>(p, row, lane, wr, tl, Ci, xc, rc, xtc, rtc, gv, bv, prm, part[rg], buf);
            } else if constexpr (W > 1) {
                __syncthreads();  // a row group without a row still takes part in the barrier
                buf ^= 1;
            }
        };
        while (base < p.rows) {
            one(base + rg, xa, ra, xta, rta, xb, rb, xtb, rtb);
            base += stride;
            if (base >= p.rows) break;
            one(base + rg, xb, rb, xtb, rtb, xa, ra, xta, rta);
            base += stride;
        }
    }
}

// ---------------------------------------------------------------------------------------
// Element kernel: rows that are not whole 16-byte chunks, or tensors that are only
// element-aligned. The same register-resident structure with one element per slot: lane t
// of a row group of W waves holds elements t, t + 64W, ... (V of them), loaded with
// element-sized coalesced accesses, so the row is still read from HBM once.
// ---------------------------------------------------------------------------------------

template <int DT, int OP, int W, int V, int RPB, int AFF>
__global__ __launch_bounds__(64 * W * RPB) void rownorm_elem_kernel(Params p) {
    using IO = Io<DT>;
    using OT = OpTraits<OP>;
    constexpr int LANES = 64 * W;
    constexpr int S = DT == DT_F32 ? 4 : 2;  // bytes per element
    constexpr bool HG = !OT::SM && (AFF & AFF_G) != 0;
    constexpr bool HB = OT::LN && (AFF & AFF_B) != 0;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (SGPR)
    const int rg = wave / W;
    const int wr = wave - rg * W;
    const unsigned t = static_cast<unsigned>(wr * 64 + lane);
    const unsigned N = static_cast<unsigned>(p.N);  // N <= 64 * W * V fits in 32 bits
    const uint32_t row_bytes = N * S;
    __shared__ WavePart part_all[RPB][2][W > 1 ? W : 1];
    WavePart(*part)[W > 1 ? W : 1] = part_all[rg];
    // elements of this wave: slot i holds column i * LANES + wr * 64 + lane
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int k = static_cast<int>(N) - (i * LANES + wr * 64);
        cnt += k <= 0 ? 0 : (k >= 64 ? 64 : k);
    }
    const float n_w = static_cast<float>(cnt);
    const float inv_w = n_w > 0.f ? 1.0f / n_w : 0.f;
    // The lane's columns are the same for every row: its parameters are loaded once
    // (columns beyond N read as 0).
    float g[HG ? V : 1], b[HB ? V : 1];
    {
        const Rsrc gr = make_rsrc(p.gamma, HG ? row_bytes : 0);
        const Rsrc br = make_rsrc(p.beta, HB ? row_bytes : 0);
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const unsigned j = static_cast<unsigned>(i * LANES) + t;
            if constexpr (HG) g[i] = IO::bload(gr, j);
            if constexpr (HB) b[i] = IO::bload(br, j);
        }
    }
    int buf = 0;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * RPB; base < p.rows;
         base += static_cast<int64_t>(gridDim.x) * RPB) {
        const int64_t row = base + rg;
        if (row >= p.rows) {
            if constexpr (W == 1) break;
            __syncthreads();
            buf ^= 1;
            continue;
        }
        // One buffer resource per row and tensor (row bases are wave-uniform): loads beyond
        // the row read 0, so idle slots need no masking; stores beyond it are dropped.
        const Rsrc xr = make_rsrc(static_cast<const char*>(p.x) + row * p.ldx * S, row_bytes);
        float f[V], r[OT::RES ? V : 1];
        // a1 (+ a2): load the row; the fused ops form, store and keep t = round(x + r)
#pragma unroll
        for (int i = 0; i < V; ++i) f[i] = IO::bload(xr, static_cast<unsigned>(i * LANES) + t);
        if constexpr (OT::RES) {
            const Rsrc rr = make_rsrc(static_cast<const char*>(p.residual) + row * p.ldr * S, row_bytes);
#pragma unroll
            for (int i = 0; i < V; ++i) r[i] = IO::bload(rr, static_cast<unsigned>(i * LANES) + t);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (OT::RES) {
            const Rsrc orr = make_rsrc(static_cast<char*>(p.residual_out) + row * p.ldro * S, row_bytes);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                f[i] = IO::round(f[i] + r[i]);  // 0 + 0 = 0 in idle slots
                IO::bstore(orr, static_cast<unsigned>(i * LANES) + t, f[i]);
            }
        }
        float scale, offset = 0.f;
        if constexpr (OT::LN) {
            const float K = uniform(f[0]);  // the wave's first element (0 if it holds none)
            float s1 = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) s1 += static_cast<unsigned>(i * LANES) + t < N ? f[i] - K : 0.f;
            const float a = K + wave_sum(s1) * inv_w;
            float c = 0.f, q = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                f[i] = static_cast<unsigned>(i * LANES) + t < N ? f[i] - a : 0.f;
                c += f[i];
                q = fmaf(f[i], f[i], q);
            }
            const float Cw = wave_sum(c);
            const float Qw = wave_sum(q);
            const float cw = Cw * inv_w;
            float rel, m2, mean;
            group_moments<W, false>(part, buf, lane, wr, n_w, a, cw, fmaxf(Qw - Cw * cw, 0.f), rel, m2, mean);
            if (t == 0 && p.mean) p.mean[row] = mean;
            scale = inv_sqrt(fmaf(m2, p.inv_n, p.eps));
            offset = -rel * scale;
            if (t == 0 && p.rstd) p.rstd[row] = scale;
        } else if constexpr (OT::SM) {
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < V; ++i) mx = static_cast<unsigned>(i * LANES) + t < N ? max_nan(mx, f[i]) : mx;
            const float mw = wave_max(mx);
            float sm = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                f[i] = static_cast<unsigned>(i * LANES) + t < N ? exp_neg(f[i] - mw) : 0.f;
                sm += f[i];
            }
            float M, Ssum;
            group_softmax<W>(part, buf, lane, wr, mw, wave_sum(sm), M, Ssum);
            scale = exp_neg(mw - M) / Ssum;
            if (t == 0 && p.mean) p.mean[row] = M;
            if (t == 0 && p.rstd) p.rstd[row] = Ssum;
        } else {
            float sq = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) sq = fmaf(f[i], f[i], sq);  // idle slots hold 0
            const float Ssq = group_sum<W>(part, buf, lane, wr, wave_sum(sq));
            scale = inv_sqrt(fmaf(Ssq, p.inv_n, p.eps));
            if (t == 0 && p.rstd) p.rstd[row] = scale;
        }
        // a7: normalize, apply the parameters, store (stores beyond the row are dropped).
        const Rsrc yr = make_rsrc(static_cast<char*>(p.y) + row * p.ldy * S, row_bytes);
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float z = OT::LN ? fmaf(f[i], scale, offset) : f[i] * scale;
            if constexpr (HG && HB) {
                z = fmaf(z, g[i], b[i]);
            } else if constexpr (HG) {
                z = z * g[i];
            } else if constexpr (HB) {
                z = z + b[i];
            }
            IO::bstore(yr, static_cast<unsigned>(i * LANES) + t, z);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Pair kernel: 16-bit rows that are not whole 16-byte chunks (ragged N, padded or unaligned
// rows). A lane slot holds two adjacent elements and moves them with one 4-byte access:
// half the memory instructions of the element kernel, each moving twice the bytes. Slots
// sit on 4-byte boundaries, so a row that starts in the upper half of a word has head
// h = 1 and slot position q holds element q - h. The at most two positions outside the row
// (one before it, one after it, each in a word that also holds row data, so never on
// another page) are read but masked out of the statistics, and never written: a wave's slot
// that does not lie wholly inside the row is written with 2-byte stores. Every row tensor
// of the call has the same head on a given row (checked by the planner).
// ---------------------------------------------------------------------------------------
template <int DT, int OP, int W, int VP, int RPB, int AFF>
__global__ __launch_bounds__(64 * W * RPB) void rownorm_pair_kernel(Params p) {
    using IO = Io<DT>;
    using OT = OpTraits<OP>;
    constexpr int LANES = 64 * W;
    constexpr int NE = 2 * VP;  // elements per lane
    constexpr bool HG = !OT::SM && (AFF & AFF_G) != 0;
    constexpr bool HB = OT::LN && (AFF & AFF_B) != 0;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rg = wave / W;
    const int wr = wave - rg * W;
    const int t = wr * 64 + lane;
    const int N = static_cast<int>(p.N);  // 2 * 64 * W * VP > N: 32-bit offsets
    __shared__ WavePart part_all[RPB][2][W > 1 ? W : 1];
    WavePart(*part)[W > 1 ? W : 1] = part_all[rg];
    float g[HG ? NE : 1], b[HB ? NE : 1];
    int hp = -1;  // the head that the parameters and n_w were set up for
    float n_w = 0.f, inv_w = 0.f;
    int buf = 0;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * RPB; base < p.rows;
         base += static_cast<int64_t>(gridDim.x) * RPB) {
        const int64_t row = base + rg;
        if (row >= p.rows) {
            if constexpr (W == 1) break;
            __syncthreads();
            buf ^= 1;
            continue;
        }
        const char* xrow = static_cast<const char*>(p.x) + row * p.ldx * 2;
        const int h = static_cast<int>((reinterpret_cast<uintptr_t>(xrow) >> 1) & 1);
        // a0 + 2 * i * LANES (+ 1) is the element in slot i's low (high) half
        const int a0 = 2 * t - h;
        if (h != hp) {  // wave-uniform; once per row group when its rows share a head
            hp = h;
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < VP; ++i) {
                const int s0 = 2 * (i * LANES + wr * 64);  // the wave's first position in slot i
                const int k = N + h - s0;
                cnt += (k <= 0 ? 0 : (k >= 128 ? 128 : k)) - (s0 == 0 ? h : 0);
            }
            n_w = static_cast<float>(cnt);
            inv_w = cnt > 0 ? 1.0f / n_w : 0.f;
            const Rsrc gr = make_rsrc(p.gamma, HG ? static_cast<uint32_t>(2 * N) : 0);
            const Rsrc br = make_rsrc(p.beta, HB ? static_cast<uint32_t>(2 * N) : 0);
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                const int j = a0 + 2 * (e >> 1) * LANES + (e & 1);
                const uint32_t jj = j >= 0 ? static_cast<uint32_t>(j) : static_cast<uint32_t>(N);  // N: reads 0
                if constexpr (HG) g[e] = IO::bload(gr, jj);
                if constexpr (HB) b[e] = IO::bload(br, jj);
            }
        }
        // Element e of the lane (slot e / 2, half e % 2) is in the row iff
        // 0 <= a0 + 2 * (e / 2) * LANES + e % 2 < N; only e = 0 can fall below 0. The test
        // is one compare against a constant; `av` is made opaque before each use so that
        // the compiler recomputes the tests instead of holding 2 * VP masks in SGPRs.
        int av = a0;
        auto ok = [&](int e) {
            return e == 0 ? static_cast<unsigned>(av) < static_cast<unsigned>(N)
                          : av < N - 2 * (e >> 1) * LANES - (e & 1);
        };
        const uint32_t wbytes = static_cast<uint32_t>(((N + h + 1) >> 1) * 4);  // words holding row data
        // stores of slot i's word: whole when the wave's 64 words lie in the row, else halves
        auto store_slot = [&](char* rowp, int i, unsigned w) {
            const int s0 = 2 * (i * LANES + wr * 64);
            if (s0 >= h && s0 + 128 <= N + h) {
                bstore32(make_rsrc(rowp - 2 * h, wbytes), static_cast<uint32_t>(4 * (i * LANES + t)), w);
            } else {
                const Rsrc r16 = make_rsrc(rowp, static_cast<uint32_t>(2 * N));
                const int e0 = a0 + 2 * i * LANES;
                bstore16(r16, static_cast<uint32_t>(ok(2 * i) ? 2 * e0 : 2 * N), w & 0xffffu);
                bstore16(r16, static_cast<uint32_t>(ok(2 * i + 1) ? 2 * e0 + 2 : 2 * N), w >> 16);
            }
        };
        unsigned u[VP], ur[OT::RES ? VP : 1];
        {
            const Rsrc xr = make_rsrc(xrow - 2 * h, wbytes);
#pragma unroll
            for (int i = 0; i < VP; ++i) u[i] = bload32(xr, static_cast<uint32_t>(4 * (i * LANES + t)));
        }
        if constexpr (OT::RES) {
            const char* rrow = static_cast<const char*>(p.residual) + row * p.ldr * 2;
            const Rsrc rr = make_rsrc(rrow - 2 * h, wbytes);
#pragma unroll
            for (int i = 0; i < VP; ++i) ur[i] = bload32(rr, static_cast<uint32_t>(4 * (i * LANES + t)));
        }
        __builtin_amdgcn_sched_barrier(0);
        float f[NE];
#pragma unroll
        for (int i = 0; i < VP; ++i) {
            const f32x2 v = IO::widen_pair(u[i]);
            f[2 * i] = v.x;
            f[2 * i + 1] = v.y;
        }
        if constexpr (OT::RES) {
            char* orow = static_cast<char*>(p.residual_out) + row * p.ldro * 2;
#pragma unroll
            for (int i = 0; i < VP; ++i) {
                const f32x2 r = IO::widen_pair(ur[i]);
                const unsigned w = IO::narrow2(f[2 * i] + r.x, f[2 * i + 1] + r.y);  // t = round(x + r)
                store_slot(orow, i, w);
                const f32x2 v = IO::widen_pair(w);
                f[2 * i] = v.x;
                f[2 * i + 1] = v.y;
            }
        }
        float scale, offset = 0.f;
        if constexpr (OT::LN) {
            const float K = uniform(ok(1) ? f[1] : 0.f);  // a shift near the wave's data
            float s1 = 0.f;
            asm volatile("" : "+v"(av));
#pragma unroll
            for (int e = 0; e < NE; ++e) s1 += ok(e) ? f[e] - K : 0.f;
            const float a = K + wave_sum(s1) * inv_w;
            float c = 0.f, q = 0.f;
            asm volatile("" : "+v"(av));
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                f[e] = ok(e) ? f[e] - a : 0.f;
                c += f[e];
                q = fmaf(f[e], f[e], q);
            }
            const float Cw = wave_sum(c);
            const float Qw = wave_sum(q);
            const float cw = Cw * inv_w;
            float rel, m2, mean;
            group_moments<W, false>(part, buf, lane, wr, n_w, a, cw, fmaxf(Qw - Cw * cw, 0.f), rel, m2, mean);
            if (t == 0 && p.mean) p.mean[row] = mean;
            scale = inv_sqrt(fmaf(m2, p.inv_n, p.eps));
            offset = -rel * scale;
            if (t == 0 && p.rstd) p.rstd[row] = scale;
        } else if constexpr (OT::SM) {
            float mx = -INFINITY;
            asm volatile("" : "+v"(av));
#pragma unroll
            for (int e = 0; e < NE; ++e) mx = ok(e) ? max_nan(mx, f[e]) : mx;
            const float mw = wave_max(mx);
            float sm = 0.f;
            asm volatile("" : "+v"(av));
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                f[e] = ok(e) ? exp_neg(f[e] - mw) : 0.f;
                sm += f[e];
            }
            float M, Ssum;
            group_softmax<W>(part, buf, lane, wr, mw, wave_sum(sm), M, Ssum);
            scale = exp_neg(mw - M) / Ssum;
            if (t == 0 && p.mean) p.mean[row] = M;
            if (t == 0 && p.rstd) p.rstd[row] = Ssum;
        } else {
            float sq = 0.f;
#pragma unroll
            for (int e = 0; e < NE; ++e) sq = ok(e) ? fmaf(f[e], f[e], sq) : sq;
            const float Ssq = group_sum<W>(part, buf, lane, wr, wave_sum(sq));
            scale = inv_sqrt(fmaf(Ssq, p.inv_n, p.eps));
            if (t == 0 && p.rstd) p.rstd[row] = scale;
        }
        char* yrow = static_cast<char*>(p.y) + row * p.ldy * 2;
        asm volatile("" : "+v"(av));
#pragma unroll
        for (int i = 0; i < VP; ++i) {
            float z[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int e = 2 * i + k;
                z[k] = OT::LN ? fmaf(f[e], scale, offset) : f[e] * scale;
                if constexpr (HG && HB) {
                    z[k] = fmaf(z[k], g[e], b[e]);
                } else if constexpr (HG) {
                    z[k] = z[k] * g[e];
                } else if constexpr (HB) {
                    z[k] = z[k] + b[e];
                }
            }
            store_slot(yrow, i, IO::narrow2(z[0], z[1]));
        }
    }
}

// The S segment records of a split row, combined by one wave: lane k takes records k, k + 64,
// ... in that order, then the 64 lane results meet in a butterfly whose every step combines
// (lower lane, upper lane) in that order. All lanes, waves and workgroups of the row so get
// the same bits, and the records are read in parallel (one load per lane for S <= 64)
// instead of one after another.
//   LayerNorm records (n, R, mean - R, M2): returns (R0, mean - R0, M2, n) with R0 = record 0's R.
//   Softmax records (max, sum): returns (max, sum).  RMSNorm records (sum of squares): (sum).
template <int OP>
__device__ __forceinline__ float4 combine_records(const float4* rec, int S, int lane) {
    using OT = OpTraits<OP>;
    if constexpr (OT::LN) {
        const float R0 = rec[0].y;
        Moments acc{0.f, 0.f, 0.f};
        for (int k = lane; k < S; k += 64) {
            const float4 r = rec[k];
            acc = combine(acc, Moments{r.x, (r.y - R0) + r.z, r.w});
        }
#pragma unroll
        for (int step = 1; step < 64; step <<= 1) {
            const Moments o{__shfl_xor(acc.n, step), __shfl_xor(acc.m, step), __shfl_xor(acc.m2, step)};
            acc = (lane & step) ? combine(o, acc) : combine(acc, o);
        }
        return make_float4(R0, acc.m, acc.m2, acc.n);
    } else if constexpr (OT::SM) {
        float m = -INFINITY, s = 0.f;
        for (int k = lane; k < S; k += 64) {
            const float4 r = rec[k];
            softmax_combine(m, s, r.x, r.y);
        }
#pragma unroll
        for (int step = 1; step < 64; step <<= 1) {
            const float mo = __shfl_xor(m, step), so = __shfl_xor(s, step);
            softmax_combine(m, s, mo, so);  // symmetric in its two sides, bit for bit
        }
        return make_float4(m, s, 0.f, 0.f);
    } else {
        float q = 0.f;
        for (int k = lane; k < S; k += 64) q += rec[k].x;
#pragma unroll
        for (int step = 1; step < 64; step <<= 1) q += __shfl_xor(q, step);  // a + b == b + a
        return make_float4(q, 0.f, 0.f, 0.f);
    }
}

// ---------------------------------------------------------------------------------------
// Split-row kernels: rows too long for one workgroup's registers (the walkthrough's
// section 1.1 case of a row that outgrows one block), with 16-byte chunks. A row is cut into
// S segments of kWideChunks chunks, one workgroup (kWideW waves, kWideV chunks per lane) per
// segment, in two launches:
//   1. rownorm_wide_stats_kernel: the segment's statistics (LayerNorm: count, a reference
//      point R_s and the mean relative to it, M2; RMSNorm: sum of squares; softmax: max and
//      sum of exp(x - max)) into the workspace, one float4 per segment. The fused ops also
//      write residual_out here.
//   2. rownorm_wide_norm_kernel: every workgroup of the row combines the S records in the
//      same fixed order (so all get the same bits), re-reads its segment (x, or residual_out
//      for the fused ops) and writes y.
// x is read twice; when the tensor fits the 256 MiB memory-side cache the second read is
// served from it.
// ---------------------------------------------------------------------------------------

constexpr int kWideW = 8;
constexpr int kWideV = 4;
constexpr int kWideLanes = 64 * kWideW;
constexpr int kWideChunks = kWideLanes * kWideV;  // 2048 chunks = 32 KiB per segment
static_assert(kWideChunks == kWideSegChunks, "segment size shared with the planner");

// The statistics record of one segment (Cs chunks; lane t holds chunks t, t + 512, ... of it):
// LayerNorm (count, this wave's rough mean a, the segment mean relative to a, M2), written by
// wave 0 so relative to its a; softmax (max, sum of exp(x - max)); RMSNorm (sum of squares).
// get(i) returns the lane's chunk i (x, or the rounded residual sum for the fused ops); it is
// called once per pass (twice for LayerNorm and softmax), so it may read memory again. Every
// wave takes part (one barrier). The two-launch statistics kernel, the one-pass kernel and a
// workgroup that computes another segment's record in its place all go through this, so the
// records have the same bits.
// The partial last chunk of a byte-addressed split row's last segment: its slot, its lane and
// its element count (ti = -1: the segment ends with a whole chunk).
struct WideTail {
    int ti = -1;
    int tt = 0;
    int te = 0;
};

template <int DT, int OP, bool EXACT, class Get>
__device__ __forceinline__ float4 wide_record(Get get, int Cs, int t, int lane, int wr, WavePart (*part)[kWideW],
                                              int& buf, const WideTail& tl = WideTail{}) {
    using IO = Io<DT>;
    using OT = OpTraits<OP>;
    constexpr int E = IO::E;
    constexpr int V = kWideV;
    auto valid = [&](int i) { return EXACT || i * kWideLanes + t < Cs; };
    // element e of slot i is part of the row (the partial chunk's missing elements read 0)
    auto ok = [&](int i, int e) { return valid(i) && !(i == tl.ti && t == tl.tt && e >= tl.te); };
    int cnt = 0;  // chunks of this wave
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int k = Cs - (i * kWideLanes + wr * 64);
        cnt += k <= 0 ? 0 : (k >= 64 ? 64 : k);
    }
    const int missing = tl.ti >= 0 ? E - tl.te : 0;  // elements the partial chunk lacks
    const float n_w = static_cast<float>(cnt * E - ((tl.tt >> 6) == wr ? missing : 0));
    if constexpr (OT::LN) {
        const float K = uniform(IO::first(get(0)));
        float s1 = 0.f;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float f[E];
            IO::unpack(get(i), f);
#pragma unroll
            for (int e = 0; e < E; ++e) s1 += ok(i, e) ? f[e] - K : 0.f;
        }
        const float inv_w = n_w > 0.f ? 1.0f / n_w : 0.f;
        const float a = K + wave_sum(s1) * inv_w;
        float c = 0.f, q = 0.f;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float f[E];
            IO::unpack(get(i), f);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float d = ok(i, e) ? f[e] - a : 0.f;
                c += d;
                q = fmaf(d, d, q);
            }
        }
        const float Cw = wave_sum(c), Qw = wave_sum(q);
        const float cw = Cw * inv_w;
        float rel, m2, mean;
        group_moments<kWideW, false>(part, buf, lane, wr, n_w, a, cw, fmaxf(Qw - Cw * cw, 0.f), rel, m2, mean);
        // relative to wave 0's rough mean R: rel is the mean minus this wave's a, so
        // mean - R = rel + (a - R); wave 0 (a == R) writes the record
        return make_float4(static_cast<float>(Cs * E - missing), a, rel, m2);
    } else if constexpr (OT::SM) {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float f[E];
            IO::unpack(get(i), f);
#pragma unroll
            for (int e = 0; e < E; ++e) mx = ok(i, e) ? max_nan(mx, f[e]) : mx;
        }
        const float mw = wave_max(mx);
        float sm = 0.f;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float f[E];
            IO::unpack(get(i), f);
#pragma unroll
            for (int e = 0; e < E; ++e) sm += ok(i, e) ? exp_neg(f[e] - mw) : 0.f;
        }
        float M, Ssum;
        group_softmax<kWideW>(part, buf, lane, wr, mw, wave_sum(sm), M, Ssum);
        return make_float4(M, Ssum, 0.f, 0.f);
    } else {
        float sq = 0.f;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float f[E];
            IO::unpack(get(i), f);
#pragma unroll
            for (int e = 0; e < E; ++e) sq = valid(i) ? fmaf(f[e], f[e], sq) : sq;
        }
        return make_float4(group_sum<kWideW>(part, buf, lane, wr, wave_sum(sq)), 0.f, 0.f, 0.f);
    }
}

template <int DT, int OP, bool EXACT>
__global__ __launch_bounds__(kWideLanes) void rownorm_wide_stats_kernel(Params p, WideArgs wa) {
    using IO = Io<DT>;
    using OT = OpTraits<OP>;
    constexpr int E = IO::E;
    constexpr int V = kWideV;
    const int lane = threadIdx.x & 63;
    const int wr = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (SGPR)
    const int t = threadIdx.x;
    __shared__ WavePart part[2][kWideW];
    int buf = 0;
    const int64_t total = p.rows * wa.S;
    for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
        const int64_t row = b / wa.S;
        const int seg = static_cast<int>(b - row * wa.S);
        const int64_t c0 = static_cast<int64_t>(seg) * kWideChunks;
        const int Cs = static_cast<int>(p.C - c0 < kWideChunks ? p.C - c0 : kWideChunks);  // chunks here
        auto valid = [&](int i) { return EXACT || i * kWideLanes + t < Cs; };
        auto chunk = [&](int i) {
            const int c = i * kWideLanes + t;
            return c0 + (EXACT ? c : (c < Cs ? c : Cs - 1));
        };
        // Ordinary (temporal) loads and stores here: the second launch reads the same bytes
        // again, from the memory-side cache when they are still there.
        u32x4 src[V];
        const u32x4* xr = static_cast<const u32x4*>(p.x) + row * p.cx;
#pragma unroll
        for (int i = 0; i < V; ++i) src[i] = xr[chunk(i)];
        if constexpr (OT::RES) {
            const u32x4* rr = static_cast<const u32x4*>(p.residual) + row * p.cr;
            u32x4 rv[V];
#pragma unroll
            for (int i = 0; i < V; ++i) rv[i] = __builtin_nontemporal_load(rr + chunk(i));
            u32x4* ro = static_cast<u32x4*>(p.residual_out) + row * p.cro;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float a[E], c[E];
                IO::unpack(src[i], a);
                IO::unpack(rv[i], c);
#pragma unroll
                for (int e = 0; e < E; ++e) a[e] += c[e];
                src[i] = IO::pack(a);
                if (valid(i)) ro[chunk(i)] = src[i];
            }
        }
        const float4 rec = wide_record<DT, OP, EXACT>([&](int i) { return src[i]; }, Cs, t, lane, wr, part, buf);
        if (t == 0) static_cast<float4*>(wa.ws)[row * wa.S + seg] = rec;
    }
}

// The row's normalization from its combined records (combine_records): LayerNorm subtracts
// R0 and scales by rstd with the offset -(mean - R0) * rstd; softmax scales exp(x - max) by
// 1 / sum; RMSNorm scales by rstd. Shared by the split-row normalize steps.
struct WideScale {
    float R0, scale, offset;
};

template <int OP>
__device__ __forceinline__ WideScale wide_scale(const float4& tot, const Params& p) {
    using OT = OpTraits<OP>;
    WideScale w{0.f, 0.f, 0.f};
    if constexpr (OT::LN) {
        w.R0 = tot.x;
        w.scale = inv_sqrt(fmaf(tot.z, p.inv_n, p.eps));
        w.offset = -tot.y * w.scale;
    } else if constexpr (OT::SM) {
        w.R0 = tot.x;
        w.scale = 1.0f / tot.y;
    } else {
        w.scale = inv_sqrt(fmaf(tot.x, p.inv_n, p.eps));
    }
    return w;
}

// The row statistics the caller asked for (the segment-0 workgroup stores them).
template <int OP>
__device__ __forceinline__ void wide_store_stats(const Params& p, int64_t row, const float4& tot, const WideScale& w) {
    using OT = OpTraits<OP>;
    if constexpr (OT::LN) {
        if (p.mean) p.mean[row] = w.R0 + tot.y;
        if (p.rstd) p.rstd[row] = w.scale;
    } else if constexpr (OT::SM) {
        if (p.mean) p.mean[row] = tot.x;
        if (p.rstd) p.rstd[row] = tot.y;
    } else {
        if (p.rstd) p.rstd[row] = w.scale;
    }
}

// One output chunk: the normalized source chunk with the affine parameters, rounded once.
template <int DT, int OP, bool HG, bool HB>
__device__ __forceinline__ u32x4 wide_out(const u32x4& src, const u32x4& gv, const u32x4& bv, const WideScale& w) {
    using IO = Io<DT>;
    using OT = OpTraits<OP>;
    constexpr int E = IO::E;
    float f[E], g[E], bb[E], o[E];
    IO::unpack(src, f);
    if constexpr (HG) IO::unpack(gv, g);
    if constexpr (HB) IO::unpack(bv, bb);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        float z;
        if constexpr (OT::LN) {
            z = fmaf(f[e] - w.R0, w.scale, w.offset);
        } else if constexpr (OT::SM) {
            z = exp_neg(f[e] - w.R0) * w.scale;
        } else {
            z = f[e] * w.scale;
        }
        if constexpr (HG && HB) {
            z = fmaf(z, g[e], bb[e]);
        } else if constexpr (HG) {
            z = z * g[e];
        } else if constexpr (HB) {
            z = z + bb[e];
        }
        o[e] = z;
    }
    return IO::pack(o);
}

template <int DT, int OP, bool EXACT, int AFF>
__global__ __launch_bounds__(kWideLanes) void rownorm_wide_norm_kernel(Params p, WideArgs wa) {
    using OT = OpTraits<OP>;
    constexpr int V = kWideV;
    constexpr bool HG = !OT::SM && (AFF & AFF_G) != 0;
    constexpr bool HB = OT::LN && (AFF & AFF_B) != 0;
    const int t = threadIdx.x;
    const int64_t total = p.rows * wa.S;
    for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
        const int64_t row = b / wa.S;
        const int seg = static_cast<int>(b - row * wa.S);
        const int64_t c0 = static_cast<int64_t>(seg) * kWideChunks;
        const int Cs = static_cast<int>(p.C - c0 < kWideChunks ? p.C - c0 : kWideChunks);
        auto valid = [&](int i) { return EXACT || i * kWideLanes + t < Cs; };
        auto chunk = [&](int i) {
            const int c = i * kWideLanes + t;
            return c0 + (EXACT ? c : (c < Cs ? c : Cs - 1));
        };
        // the segment's data (x, or residual_out for the fused ops) and parameters
        const u32x4* sr = OT::RES ? static_cast<const u32x4*>(p.residual_out) + row * p.cro
                                  : static_cast<const u32x4*>(p.x) + row * p.cx;
        u32x4 src[V], gv[HG ? V : 1], bv[HB ? V : 1];
#pragma unroll
        for (int i = 0; i < V; ++i) {
            src[i] = __builtin_nontemporal_load(sr + chunk(i));
            if constexpr (HG) gv[i] = static_cast<const u32x4*>(p.gamma)[chunk(i)];
            if constexpr (HB) bv[i] = static_cast<const u32x4*>(p.beta)[chunk(i)];
        }
        // combine the row's segment records (same bits in every workgroup of the row)
        const float4 tot = combine_records<OP>(static_cast<const float4*>(wa.ws) + row * wa.S, wa.S, t & 63);
        const WideScale w = wide_scale<OP>(tot, p);
        if (seg == 0 && t == 0) wide_store_stats<OP>(p, row, tot, w);
        u32x4* yr = static_cast<u32x4*>(p.y) + row * p.cy;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const u32x4 o = wide_out<DT, OP, HG, HB>(src[i], gv[HG ? i : 0], bv[HB ? i : 0], w);
            if (valid(i)) __builtin_nontemporal_store(o, yr + chunk(i));
        }
    }
}

// ---------------------------------------------------------------------------------------
// One-pass split rows (whole 16-byte chunks): x (for the fused ops, x and the residual) is
// read once, the walkthrough's single-read layout (sections 3-4) carried over to a row that
// outgrows one workgroup (section 1.1). The rows are cut into P blocks, P1 of R rows and
// then blocks of R2 rows; a ticket is one (block, segment) pair, ticket = block * S + segment,
// and workgroups take tickets from a counter in the workspace in increasing order. For each row of its block the workgroup
// holding a ticket keeps its segment in registers, forms the segment's statistics record
// (wide_record, as the two-launch path does) and publishes it as four 64-bit words (tag 1 in
// the upper half, the float's bits in the lower half; single-copy atomic, device scope), loads
// the row after next, posts the next row, and then waits (one wave, one lane per record)
// until all S records of the row carry the tag. The S records are combined in the same fixed
// order in every workgroup of the row (combine_records, so all get the same bits, the same as
// the two-launch path's), and the segment is normalized from its registers. A record still
// missing after a bounded wait (wait_polls polls) is computed by the waiting workgroup itself
// from that segment's data with wide_record, so nothing waits on a workgroup that is not
// running and the result does not depend on timing. The segment's gamma / beta are staged in
// LDS once per ticket. The counter, a count of records computed by waiting workgroups (a
// diagnostic) and the records are zeroed by rownorm_wide_clear_kernel before each launch (a
// kernel, not a memset, so that the call can be captured in a graph).
// ---------------------------------------------------------------------------------------

template <int DT>  // one instance per dtype's translation unit
__global__ __launch_bounds__(256) void rownorm_wide_clear_kernel(u32x4* p, int64_t n16) {
    const u32x4 z{0u, 0u, 0u, 0u};
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n16;
         i += static_cast<int64_t>(gridDim.x) * 256)
        p[i] = z;
}

// RAG: rows addressed by byte (rows, tensors or strides that are not whole 16-byte chunks):
// each segment of a row moves through a buffer resource that ends with the segment (the last
// one with the row), in 16-byte accesses at element alignment; the row's partial last chunk
// moves by its whole dwords (the hardware checks the range per dword) and, for an odd-length
// 16-bit row, its last element by one 2-byte access (the low half of `h` on the lane that holds
// that chunk), merged into the chunk where the segment is first used.
template <int DT, int OP, bool EXACT, int AFF, bool RAG = false>
__global__ __launch_bounds__(kWideLanes) void rownorm_wide_onepass_kernel(Params p, WideArgs wa) {
    using IO = Io<DT>;
    using OT = OpTraits<OP>;
    constexpr int E = IO::E;
    constexpr int V = kWideV;
    constexpr int SB = 16 / E;  // bytes per element
    constexpr bool HG = !OT::SM && (AFF & AFF_G) != 0;
    constexpr bool HB = OT::LN && (AFF & AFF_B) != 0;
    constexpr int NR = OT::RES ? V : 1;
    constexpr int POLLER = kWideW - 1;             // the wave that waits for the records
    constexpr int RPL = kWideOnePassMaxSeg / 64;   // records per lane of that wave
    const int lane = threadIdx.x & 63;
    const int wr = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (SGPR)
    const int t = threadIdx.x;
    __shared__ WavePart part[2][kWideW];
    __shared__ u32x4 prm[(HG ? kWideChunks : 0) + (HB ? kWideChunks : 0) + 1];  // gamma, then beta
    // per row, double-buffered by row parity: one barrier separates a row's reads from the
    // writes of the row after the next
    __shared__ float4 s_rec[2][kWideOnePassMaxSeg];  // the row's records
    __shared__ int s_need[2];                        // some record is computed here
    __shared__ unsigned char s_miss[kWideOnePassMaxSeg];
    __shared__ unsigned s_ticket;
    int buf = 0;
    const int S = wa.S;
    const unsigned total = static_cast<unsigned>(wa.P) * static_cast<unsigned>(S);
    // chunks per segment: 2048; byte-addressed rows split evenly instead (ceil(C / S) each, at
    // most 2048), so that a row's last segment is not a sliver whose workgroup idles while
    // the row waits for its record
    const int64_t L = RAG ? (p.C + S - 1) / S : kWideChunks;
    for (;;) {
        if (t == 0) s_ticket = __hip_atomic_fetch_add(wa.sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const unsigned ticket = s_ticket;  // read before the first barrier of the block's rows
        if (ticket >= total) break;        // uniform over the workgroup
        const int64_t blk = ticket / static_cast<unsigned>(S);
        const int seg = static_cast<int>(ticket % static_cast<unsigned>(S));
        const int64_t c0 = static_cast<int64_t>(seg) * L;
        const int Cs = static_cast<int>(p.C - c0 < L ? p.C - c0 : L);
        auto valid = [&](int i) { return EXACT || i * kWideLanes + t < Cs; };
        auto chunk = [&](int i) {
            const int c = i * kWideLanes + t;
            return c0 + (EXACT ? c : (c < Cs ? c : Cs - 1));
        };
        // RAG geometry of segment s: its first byte in the row, its bytes, its partial chunk
        const int64_t row_bytes = p.N * SB;
        auto seg_bytes = [&](int s_) {
            const int64_t b0 = static_cast<int64_t>(s_) * L * 16;
            const int64_t rem = row_bytes - b0;
            return static_cast<uint32_t>(rem < L * 16 ? rem : L * 16);
        };
        auto seg_tail = [&](int s_) {
            WideTail tl;
            const int te = static_cast<int>(p.N % E);
            if (RAG && te != 0 && s_ == S - 1) {
                const int idx = static_cast<int>(p.C - 1 - static_cast<int64_t>(s_) * L);
                tl.ti = idx / kWideLanes;
                tl.tt = idx % kWideLanes;
                tl.te = te;
            }
            return tl;
        };
        const uint32_t sb = seg_bytes(seg);
        const WideTail tail = seg_tail(seg);
        const bool odd16 = RAG && SB == 2 && (p.N & 1) != 0;  // a last element to move by 2 bytes
        const bool hseg = odd16 && tail.ti >= 0;               // ... in this segment
        const int hd = (tail.te - 1) >> 1;                      // the dword holding it (low half)
        // (the half's wave and lane; the waves without it issue nothing for it)
        auto half_wave = [&]() { return hseg && wr == (tail.tt >> 6); };
        auto with_half = [&](u32x4 v, unsigned h) {
            v.x |= hd == 0 ? h : 0u;
            v.y |= hd == 1 ? h : 0u;
            v.z |= hd == 2 ? h : 0u;
            v.w |= hd == 3 ? h : 0u;
            return v;
        };
        auto rsrc_seg = [&](const void* base, int64_t ld, int64_t row) {
            return make_rsrc(static_cast<const char*>(base) + (row * ld + c0 * E) * SB, sb);
        };
        // the segment's parameters, for all the block's rows (read after the first row's
        // wait, which is past at least one barrier)
        for (int c = t; c < kWideChunks; c += kWideLanes) {
            const int64_t cc = c0 + (c < Cs ? c : Cs - 1);
            if constexpr (RAG) {
                const int cl = c < Cs ? c : Cs - 1;
                auto pchunk = [&](const void* base) {
                    const Rsrc r = rsrc_seg(base, 0, 0);
                    u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, cl * 16, 0, 0);
                    if (hseg && cl == tail.ti * kWideLanes + tail.tt)
                        v = with_half(v, __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(sb - 2u), 0, 0));
                    return v;
                };
                if constexpr (HG) prm[c] = pchunk(p.gamma);
                if constexpr (HB) prm[(HG ? kWideChunks : 0) + c] = pchunk(p.beta);
            } else {
                if constexpr (HG) prm[c] = static_cast<const u32x4*>(p.gamma)[cc];
                if constexpr (HB) prm[(HG ? kWideChunks : 0) + c] = static_cast<const u32x4*>(p.beta)[cc];
            }
        }
        // xh / rh: RAG, the last element of an odd-length 16-bit row (see above)
        auto load = [&](int64_t row, u32x4(&xv)[V], u32x4(&rv)[NR], unsigned& xh, unsigned& rh) {
            if constexpr (RAG) {
                const Rsrc rx = rsrc_seg(p.x, p.ldx, row);
#pragma unroll
                for (int i = 0; i < V; ++i)
                    xv[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, static_cast<int>((chunk(i) - c0) * 16), 0, 2);
                if (half_wave())
                    xh = __builtin_amdgcn_raw_buffer_load_b16(rx, static_cast<int>(t == tail.tt ? sb - 2u : sb), 0, 2);
                if constexpr (OT::RES) {
                    const Rsrc rr = rsrc_seg(p.residual, p.ldr, row);
#pragma unroll
                    for (int i = 0; i < V; ++i)
                        rv[i] = __builtin_amdgcn_raw_buffer_load_b128(rr, static_cast<int>((chunk(i) - c0) * 16), 0, 2);
                    if (half_wave())
                        rh = __builtin_amdgcn_raw_buffer_load_b16(rr, static_cast<int>(t == tail.tt ? sb - 2u : sb), 0,
                                                                  2);
                }
                return;
            }
            const u32x4* xr = static_cast<const u32x4*>(p.x) + row * p.cx;
#pragma unroll
            for (int i = 0; i < V; ++i) xv[i] = __builtin_nontemporal_load(xr + chunk(i));
            if constexpr (OT::RES) {
                const u32x4* rr = static_cast<const u32x4*>(p.residual) + row * p.cr;
#pragma unroll
                for (int i = 0; i < V; ++i) rv[i] = __builtin_nontemporal_load(rr + chunk(i));
            }
        };
        // one output chunk of the segment (RAG: the partial chunk's whole dwords, then the half)
        auto store_seg = [&](void* base, int64_t ld, int64_t row, int i, const u32x4& v) {
            if constexpr (RAG) {
                const Rsrc r = rsrc_seg(base, ld, row);
                if (valid(i)) __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>((chunk(i) - c0) * 16), 0, 2);
                if (i == tail.ti && half_wave()) {
                    const unsigned hv = hd == 0 ? v.x : hd == 1 ? v.y : hd == 2 ? v.z : v.w;
                    bstore16<2>(r, t == tail.tt ? sb - 2u : sb, hv);
                }
            } else {
                if (valid(i)) __builtin_nontemporal_store(v, static_cast<u32x4*>(base) + row * (ld * SB / 16) + chunk(i));
            }
        };
        auto publish = [&](int64_t row, int sgm, const float4& rec) {
            if (t == 0) {
                unsigned long long* w = wa.rec64 + 4 * (row * S + sgm);
                const unsigned long long tag = 1ull << 32;
                __hip_atomic_store(w, tag | bit_cast<unsigned>(rec.x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(w + 1, tag | bit_cast<unsigned>(rec.y), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(w + 2, tag | bit_cast<unsigned>(rec.z), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(w + 3, tag | bit_cast<unsigned>(rec.w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        };
        // this workgroup's segment of one row: the fused ops form the rounded sum (kept in xv)
        // and store residual_out; then the record, published as record `seg` of the row
        // (RAG: the row's last element of an odd-length 16-bit row joins its chunk here)
        auto post = [&](int64_t row, u32x4(&xv)[V], u32x4(&rv)[NR], unsigned xh, unsigned rh) {
            if constexpr (RAG) {
                if (hseg && t == tail.tt) {
#pragma unroll
                    for (int i = 0; i < V; ++i) {
                        if (i == tail.ti) {
                            xv[i] = with_half(xv[i], xh);
                            if constexpr (OT::RES) rv[i] = with_half(rv[i], rh);
                        }
                    }
                }
            }
            if constexpr (OT::RES) {
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    float a[E], c[E];
                    IO::unpack(xv[i], a);
                    IO::unpack(rv[i], c);
#pragma unroll
                    for (int e = 0; e < E; ++e) a[e] += c[e];
                    xv[i] = IO::pack(a);
                    store_seg(p.residual_out, p.ldro, row, i, xv[i]);
                }
            }
            const float4 rec =
                wide_record<DT, OP, EXACT>([&](int i) { return xv[i]; }, Cs, t, lane, wr, part, buf, tail);
            publish(row, seg, rec);
        };
        // segment s2's record of one row, computed here from memory, one chunk per tensor at a
        // time (the rows in flight keep their registers)
        auto other_record = [&](int64_t row, int s2) {
            const int64_t c2 = static_cast<int64_t>(s2) * L;
            const int Cs2 = static_cast<int>(p.C - c2 < L ? p.C - c2 : L);
            const WideTail tl2 = seg_tail(s2);
            const uint32_t sb2 = seg_bytes(s2);
            // RAG: the segment's resource, and the byte offset of its 2-byte last element
            // (sb2 - 2 on the lane holding that chunk, past the segment elsewhere)
            const Rsrc rx2 = make_rsrc(static_cast<const char*>(p.x) + (row * p.ldx + c2 * E) * SB, sb2);
            const Rsrc rr2 = make_rsrc(OT::RES ? static_cast<const char*>(p.residual) + (row * p.ldr + c2 * E) * SB
                                               : nullptr,
                                       OT::RES ? sb2 : 0u);
            const bool h2 = odd16 && tl2.ti >= 0;
            const int hd2 = (tl2.te - 1) >> 1;
            const u32x4* xr = static_cast<const u32x4*>(p.x) + row * p.cx + c2;
            const u32x4* rr = OT::RES ? static_cast<const u32x4*>(p.residual) + row * p.cr + c2 : nullptr;
            auto ld2 = [&](const u32x4* gp, Rsrc r, int cc, int i) {
                if constexpr (RAG) {
                    u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, cc * 16, 0, 0);
                    if (h2 && i == tl2.ti) {
                        const unsigned h = __builtin_amdgcn_raw_buffer_load_b16(
                            r, static_cast<int>(t == tl2.tt ? sb2 - 2u : sb2), 0, 0);
                        v.x |= hd2 == 0 ? h : 0u;
                        v.y |= hd2 == 1 ? h : 0u;
                        v.z |= hd2 == 2 ? h : 0u;
                        v.w |= hd2 == 3 ? h : 0u;
                    }
                    return v;
                } else {
                    return gp[cc];
                }
            };
            auto get = [&](int i) {
                const int c = i * kWideLanes + t;
                const int cc = EXACT ? c : (c < Cs2 ? c : Cs2 - 1);
                u32x4 v = ld2(xr, rx2, cc, i);
                if constexpr (OT::RES) {
                    const u32x4 r = ld2(rr, rr2, cc, i);
                    float a[E], b[E];
                    IO::unpack(v, a);
                    IO::unpack(r, b);
#pragma unroll
                    for (int e = 0; e < E; ++e) a[e] += b[e];
                    v = IO::pack(a);
                }
                asm volatile("" ::: "memory");  // one chunk per tensor in flight
                return v;
            };
            return wide_record<DT, OP, EXACT>(get, Cs2, t, lane, wr, part, buf, tl2);
        };
        const int64_t r0 = blk < wa.P1 ? blk * wa.R
                                       : static_cast<int64_t>(wa.P1) * wa.R + (blk - wa.P1) * wa.R2;
        const int64_t rn = r0 + (blk < wa.P1 ? wa.R : wa.R2);
        const int64_t r1 = rn < p.rows ? rn : p.rows;
        // three rows in flight: row (record posted, waiting), row + 1 (posted before the wait
        // for row), row + 2 (loads issued before that wait)
        u32x4 cx[V], cr[NR], nx[V], nr[NR];
        unsigned cxh = 0, crh = 0, nxh = 0, nrh = 0;  // RAG: the rows' 2-byte last elements
        load(r0, cx, cr, cxh, crh);
        if (r0 + 1 < r1) load(r0 + 1, nx, nr, nxh, nrh);
        post(r0, cx, cr, cxh, crh);
        for (int64_t row = r0; row < r1; ++row) {
            const int par = static_cast<int>(row & 1);
            u32x4 mx[V], mr[NR];
            unsigned mxh = 0, mrh = 0;
            if (row + 2 < r1) load(row + 2, mx, mr, mxh, mrh);
            if (row + 1 < r1) post(row + 1, nx, nr, nxh, nrh);
            if (wr == POLLER) {
                const unsigned long long* w = wa.rec64 + 4 * row * S;
                unsigned miss = 0;
#pragma unroll
                for (int j = 0; j < RPL; ++j) {
                    const int k = lane + 64 * j;
                    if (k < S) {
                        bool got = false;
                        // wait_polls 0: no wait at all, every record of the row is computed here
                        for (int n = 0; wa.wait_polls > 0; ++n) {
                            const unsigned long long w0 = __hip_atomic_load(w + 4 * k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            const unsigned long long w1 = __hip_atomic_load(w + 4 * k + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            const unsigned long long w2 = __hip_atomic_load(w + 4 * k + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            const unsigned long long w3 = __hip_atomic_load(w + 4 * k + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            if (((w0 & w1 & w2 & w3) >> 32) != 0) {
                                s_rec[par][k] = make_float4(bit_cast<float>(static_cast<unsigned>(w0)),
                                                            bit_cast<float>(static_cast<unsigned>(w1)),
                                                            bit_cast<float>(static_cast<unsigned>(w2)),
                                                            bit_cast<float>(static_cast<unsigned>(w3)));
                                got = true;
                                break;
                            }
                            if (n >= wa.wait_polls) break;
                            __builtin_amdgcn_s_sleep(8);
                        }
                        if (!got) miss |= 1u << j;
                        s_miss[k] = got ? 0 : 1;
                    }
                }
                const bool any = __any(miss != 0);  // all 64 lanes active here
                if (lane == 0) s_need[par] = any ? 1 : 0;
            }
            __syncthreads();
            if (s_need[par] != 0) {  // uniform: compute the missing records here
                int computed = 0;
                for (int s2 = 0; s2 < S; ++s2) {
                    if (s_miss[s2] == 0) continue;  // uniform
                    const float4 rec = other_record(row, s2);
                    publish(row, s2, rec);
                    if (t == 0) s_rec[par][s2] = rec;
                    ++computed;
                }
                if (t == 0)
                    __hip_atomic_fetch_add(wa.sync + 1, static_cast<unsigned>(computed), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                __syncthreads();
            }
            // combine the row's records (same bits in every workgroup of the row) and normalize
            const float4 tot = combine_records<OP>(s_rec[par], S, lane);
            const WideScale ws = wide_scale<OP>(tot, p);
            if (seg == 0 && t == 0) wide_store_stats<OP>(p, row, tot, ws);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const int c = i * kWideLanes + t;
                const int cl = EXACT ? c : (c < Cs ? c : Cs - 1);
                const u32x4 gv = HG ? prm[cl] : u32x4{0u, 0u, 0u, 0u};
                const u32x4 bv = HB ? prm[(HG ? kWideChunks : 0) + cl] : u32x4{0u, 0u, 0u, 0u};
                const u32x4 o = wide_out<DT, OP, HG, HB>(cx[i], gv, bv, ws);
                store_seg(p.y, p.ldy, row, i, o);
            }
#pragma unroll
            for (int i = 0; i < V; ++i) {
                cx[i] = nx[i];
                nx[i] = mx[i];
                if constexpr (OT::RES) {
                    cr[i] = nr[i];
                    nr[i] = mr[i];
                }
            }
            nxh = mxh;
            nrh = mrh;
        }
    }
}

// ---------------------------------------------------------------------------------------
// Split-row element kernels: the same two launches for long rows that are not whole 16-byte
// chunks (ragged N, unaligned tensors, strides that are not whole chunks). A segment is
// kWideElemSeg elements, one per register slot (kWideEV slots per lane, element i * 512 + t
// of the segment); every tensor of the segment is read and written through a buffer
// resource bounded by the segment, so slots past the row's end read 0 and write nothing.
// ---------------------------------------------------------------------------------------

constexpr int kWideEV = kWideElemSeg / kWideLanes;  // 16 elements per lane
static_assert(kWideEV * kWideLanes == kWideElemSeg, "element segment = 512 lanes x kWideEV");

template <int DT, int OP>
__global__ __launch_bounds__(kWideLanes) void rownorm_wide_elem_stats_kernel(Params p, WideArgs wa) {
    using IO = Io<DT>;
    using OT = OpTraits<OP>;
    constexpr int V = kWideEV;
    constexpr int S = DT == DT_F32 ? 4 : 2;
    const int lane = threadIdx.x & 63;
    const int wr = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = threadIdx.x;
    __shared__ WavePart part[2][kWideW];
    int buf = 0;
    const int64_t total = p.rows * wa.S;
    for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
        const int64_t row = b / wa.S;
        const int seg = static_cast<int>(b - row * wa.S);
        const int64_t e0 = static_cast<int64_t>(seg) * kWideElemSeg;
        const int Ns = static_cast<int>(p.N - e0 < kWideElemSeg ? p.N - e0 : kWideElemSeg);  // elements here
        const uint32_t nb = static_cast<uint32_t>(Ns * S);
        auto valid = [&](int i) { return i * kWideLanes + t < Ns; };
        // temporal loads and stores: the second launch reads the same bytes again
        const Rsrc xr = make_rsrc(static_cast<const char*>(p.x) + (row * p.ldx + e0) * S, nb);
        float f[V];
#pragma unroll
        for (int i = 0; i < V; ++i) f[i] = IO::bload(xr, static_cast<uint32_t>(i * kWideLanes + t));
        if constexpr (OT::RES) {
            const Rsrc rr = make_rsrc(static_cast<const char*>(p.residual) + (row * p.ldr + e0) * S, nb);
            float r[V];
#pragma unroll
            for (int i = 0; i < V; ++i) r[i] = IO::bload(rr, static_cast<uint32_t>(i * kWideLanes + t));
            const Rsrc orr = make_rsrc(static_cast<char*>(p.residual_out) + (row * p.ldro + e0) * S, nb);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                f[i] = IO::round(f[i] + r[i]);
                IO::bstore(orr, static_cast<uint32_t>(i * kWideLanes + t), f[i]);
            }
        }
        int cnt = 0;  // elements of this wave
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int k = Ns - (i * kWideLanes + wr * 64);
            cnt += k <= 0 ? 0 : (k >= 64 ? 64 : k);
        }
        const float n_w = static_cast<float>(cnt);
        float4 rec;
        if constexpr (OT::LN) {
            const float K = uniform(f[0]);  // 0 when the wave holds no element
            float s1 = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) s1 += valid(i) ? f[i] - K : 0.f;
            const float inv_w = n_w > 0.f ? 1.0f / n_w : 0.f;
            const float a = K + wave_sum(s1) * inv_w;
            float c = 0.f, q = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const float d = valid(i) ? f[i] - a : 0.f;
                c += d;
                q = fmaf(d, d, q);
            }
            const float Cw = wave_sum(c), Qw = wave_sum(q);
            const float cw = Cw * inv_w;
            float rel, m2, mean;
            group_moments<kWideW, false>(part, buf, lane, wr, n_w, a, cw, fmaxf(Qw - Cw * cw, 0.f), rel, m2, mean);
            rec = make_float4(static_cast<float>(Ns), a, rel, m2);  // wave 0 (a == R) writes it
        } else if constexpr (OT::SM) {
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < V; ++i) mx = valid(i) ? max_nan(mx, f[i]) : mx;
            const float mw = wave_max(mx);
            float sm = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) sm += valid(i) ? exp_neg(f[i] - mw) : 0.f;
            float M, Ssum;
            group_softmax<kWideW>(part, buf, lane, wr, mw, wave_sum(sm), M, Ssum);
            rec = make_float4(M, Ssum, 0.f, 0.f);
        } else {
            float sq = 0.f;
#pragma unroll
            for (int i = 0; i < V; ++i) sq = fmaf(f[i], f[i], sq);  // slots past the row hold 0
            rec = make_float4(group_sum<kWideW>(part, buf, lane, wr, wave_sum(sq)), 0.f, 0.f, 0.f);
        }
        if (t == 0) static_cast<float4*>(wa.ws)[row * wa.S + seg] = rec;
    }
}

template <int DT, int OP, int AFF>
__global__ __launch_bounds__(kWideLanes) void rownorm_wide_elem_norm_kernel(Params p, WideArgs wa) {
    using IO = Io<DT>;
    using OT = OpTraits<OP>;
    constexpr int V = kWideEV;
    constexpr int S = DT == DT_F32 ? 4 : 2;
    constexpr bool HG = !OT::SM && (AFF & AFF_G) != 0;
    constexpr bool HB = OT::LN && (AFF & AFF_B) != 0;
    const int t = threadIdx.x;
    const int64_t total = p.rows * wa.S;
    for (int64_t it = blockIdx.x; it < total; it += gridDim.x) {
        // last rows first: the statistics launch read them last, so they may still be in
        // the memory-side cache (fp32 LayerNorm 1024 x 65537: 37.6% -> 42.1% of HBM peak;
        // the whole-chunk split rows measured no better this way)
        const int64_t b = total - 1 - it;
        const int64_t row = b / wa.S;
        const int seg = static_cast<int>(b - row * wa.S);
        const int64_t e0 = static_cast<int64_t>(seg) * kWideElemSeg;
        const int Ns = static_cast<int>(p.N - e0 < kWideElemSeg ? p.N - e0 : kWideElemSeg);
        const uint32_t nb = static_cast<uint32_t>(Ns * S);
        // the segment's data (x, or residual_out for the fused ops) and parameters
        const Rsrc sr = OT::RES ? make_rsrc(static_cast<const char*>(p.residual_out) + (row * p.ldro + e0) * S, nb)
                                : make_rsrc(static_cast<const char*>(p.x) + (row * p.ldx + e0) * S, nb);
        const Rsrc gr = make_rsrc(HG ? static_cast<const char*>(p.gamma) + e0 * S : nullptr, HG ? nb : 0);
        const Rsrc br = make_rsrc(HB ? static_cast<const char*>(p.beta) + e0 * S : nullptr, HB ? nb : 0);
        float f[V], g[HG ? V : 1], bb[HB ? V : 1];
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const uint32_t j = static_cast<uint32_t>(i * kWideLanes + t);
            f[i] = IO::bload(sr, j);
            if constexpr (HG) g[i] = IO::bload(gr, j);
            if constexpr (HB) bb[i] = IO::bload(br, j);
        }
        // combine the row's segment records (same bits in every workgroup of the row)
        const float4 tot = combine_records<OP>(static_cast<const float4*>(wa.ws) + row * wa.S, wa.S, t & 63);
        float scale, offset = 0.f, R0 = 0.f;
        if constexpr (OT::LN) {
            R0 = tot.x;
            scale = inv_sqrt(fmaf(tot.z, p.inv_n, p.eps));
            offset = -tot.y * scale;
            if (seg == 0 && t == 0) {
                if (p.mean) p.mean[row] = R0 + tot.y;
                if (p.rstd) p.rstd[row] = scale;
            }
        } else if constexpr (OT::SM) {
            R0 = tot.x;
            scale = 1.0f / tot.y;
            if (seg == 0 && t == 0) {
                if (p.mean) p.mean[row] = tot.x;
                if (p.rstd) p.rstd[row] = tot.y;
            }
        } else {
            scale = inv_sqrt(fmaf(tot.x, p.inv_n, p.eps));
            if (seg == 0 && t == 0 && p.rstd) p.rstd[row] = scale;
        }
        const Rsrc yr = make_rsrc(static_cast<char*>(p.y) + (row * p.ldy + e0) * S, nb);
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float z;
            if constexpr (OT::LN) {
                z = fmaf(f[i] - R0, scale, offset);
            } else if constexpr (OT::SM) {
                z = exp_neg(f[i] - R0) * scale;
            } else {
                z = f[i] * scale;
            }
            if constexpr (HG && HB) {
                z = fmaf(z, g[i], bb[i]);
            } else if constexpr (HG) {
                z = z * g[i];
            } else if constexpr (HB) {
                z = z + bb[i];
            }
            IO::bstore(yr, static_cast<uint32_t>(i * kWideLanes + t), z);
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

template <int NWAVES>
__device__ __forceinline__ float block_max(float v, float* slots) {
    const float w = wave_max(v);
    if ((threadIdx.x & 63) == 0) slots[threadIdx.x >> 6] = w;
    __syncthreads();
    float s = slots[0];
#pragma unroll
    for (int i = 1; i < NWAVES; ++i) s = max_nan(s, slots[i]);
    return s;
}

template <int DT, int OP>
__global__ __launch_bounds__(kGeneralThreads) void rownorm_general_kernel(Params p) {
    using IO = Io<DT>;
    using OT = OpTraits<OP>;
    constexpr int NW = kGeneralThreads / 64;
    __shared__ float slots[3][NW];
    const int tid = threadIdx.x;
    const int64_t N = p.N;
    const float nf = static_cast<float>(N);
    for (int64_t row = blockIdx.x; row < p.rows; row += gridDim.x) {
        const int64_t xo = row * p.ldx, ro = row * p.ldr, yo = row * p.ldy, oo = row * p.ldro;
        // The row's source values: x, or for the fused ops residual_out (written by the
        // same lane in the first sweep, so re-reading it is safe under exact aliasing).
        float center = 0.f, scale = 1.f, K = 0.f;
        if constexpr (OT::RES) {
            if constexpr (OT::LN) K = IO::round(IO::load1(p.x, xo) + IO::load1(p.residual, ro));
            __syncthreads();  // K is read before any lane overwrites x / residual in place
            float s = 0.f;
            for (int64_t j = tid; j < N; j += kGeneralThreads) {
                const float v = IO::round(IO::load1(p.x, xo + j) + IO::load1(p.residual, ro + j));
                IO::store1(p.residual_out, oo + j, v);
                s += OT::LN ? v - K : v * v;
            }
            if constexpr (OT::LN) {
                center = block_sum<NW>(s, slots[0]) / nf;
            } else {
                scale = inv_sqrt(block_sum<NW>(s, slots[0]) / nf + p.eps);
            }
        } else if constexpr (OT::LN) {
            K = IO::load1(p.x, xo);
            float s1 = 0.f;
            for (int64_t j = tid; j < N; j += kGeneralThreads) s1 += IO::load1(p.x, xo + j) - K;
            center = block_sum<NW>(s1, slots[0]) / nf;
        } else if constexpr (OT::SM) {
            float m = -INFINITY;
            for (int64_t j = tid; j < N; j += kGeneralThreads) m = max_nan(m, IO::load1(p.x, xo + j));
            K = block_max<NW>(m, slots[0]);
            float s = 0.f;
            for (int64_t j = tid; j < N; j += kGeneralThreads)
                s += exp_neg(IO::load1(p.x, xo + j) - K);
            const float S = block_sum<NW>(s, slots[1]);
            scale = 1.0f / S;
            if (tid == 0) {
                if (p.mean) p.mean[row] = K;
                if (p.rstd) p.rstd[row] = S;
            }
        } else {
            float s = 0.f;
            for (int64_t j = tid; j < N; j += kGeneralThreads) {
                const float v = IO::load1(p.x, xo + j);
                s += v * v;
            }
            scale = inv_sqrt(block_sum<NW>(s, slots[0]) / nf + p.eps);
        }
        const void* src = OT::RES ? static_cast<const void*>(p.residual_out) : p.x;
        const int64_t so = OT::RES ? oo : xo;
        if constexpr (OT::LN) {
            float s2 = 0.f;
            for (int64_t j = tid; j < N; j += kGeneralThreads) {
                const float d = (IO::load1(src, so + j) - K) - center;
                s2 += d * d;
            }
            scale = inv_sqrt(block_sum<NW>(s2, slots[1]) / nf + p.eps);
            if (tid == 0) {
                if (p.mean) p.mean[row] = K + center;
                if (p.rstd) p.rstd[row] = scale;
            }
        } else if constexpr (!OT::SM) {
            if (tid == 0 && p.rstd) p.rstd[row] = scale;
        }
        for (int64_t j = tid; j < N; j += kGeneralThreads) {
            const float v = IO::load1(src, so + j);
            float o;
            if constexpr (OT::LN) {
                const float g = p.gamma ? IO::load1(p.gamma, j) : 1.f;
                const float b = p.beta ? IO::load1(p.beta, j) : 0.f;
                o = ((v - K) - center) * scale * g + b;
            } else if constexpr (OT::SM) {
                o = exp_neg(v - K) * scale;
            } else {
                const float g = p.gamma ? IO::load1(p.gamma, j) : 1.f;
                o = v * scale * g;
            }
            IO::store1(p.y, yo + j, o);
        }
        __syncthreads();  // slots are reused by the next row
    }
}

// ---------------------------------------------------------------------------------------
// Dispatch from a runtime plan to a template instance. Instantiated per dtype and mode in
// rownorm_kernels_<dtype>.hip (grid-per-row launches, the element and the general kernel)
// and rownorm_kernels_<dtype>_persistent.hip (persistent launches).
// ---------------------------------------------------------------------------------------

// Row groups per workgroup for a row-group width: 256-lane workgroups up to W = 4.
constexpr int rows_per_block_for(int W) { return W <= 4 ? 4 / W : 1; }

// Memory-access flags of the persistent mode: non-temporal streaming of the rows,
// parameters staged once per workgroup (gamma in VGPRs and beta in LDS when LayerNorm has
// both), and no fp32 copy of the LayerNorm row (more workgroups resident per CU).
template <int OP, int AFF>
constexpr int persistent_flags() {
    int fl = FL_NT_LOAD | FL_NT_STORE | FL_PARAMS_LDS;
    if (OpTraits<OP>::LN) fl |= FL_NOFLOAT;
    if (OpTraits<OP>::LN && AFF == (AFF_G | AFF_B)) fl |= FL_GAMMA_REG;
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
// per kernel instance and device: the kernel is a template argument, so each instance has
// its own cache), capped as below, at most one per row group of work.
// Resident capacity of a kernel instance: CUs and workgroups per CU at this block size and
// dynamic LDS, queried once per device (per instance: each template instance has its own
// cache; a benign race writes the same values).
template <auto KERNEL>
inline hipError_t resident(int block_threads, int lds_bytes, int* cus_out, int* per_cu_out) {
    static int per_cu_cache[kMaxDevices];  // 0: not yet known
    static int cus_cache[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int per_cu = dev < kMaxDevices ? __atomic_load_n(&per_cu_cache[dev], __ATOMIC_RELAXED) : 0;
    int cus = dev < kMaxDevices ? __atomic_load_n(&cus_cache[dev], __ATOMIC_RELAXED) : 0;
    if (per_cu <= 0 || cus <= 0) {
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(KERNEL), block_threads,
                                                         static_cast<size_t>(lds_bytes));
        if (e != hipSuccess) return e;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (per_cu < 1) per_cu = 1;
        if (dev < kMaxDevices) {
            __atomic_store_n(&per_cu_cache[dev], per_cu, __ATOMIC_RELAXED);
            __atomic_store_n(&cus_cache[dev], cus, __ATOMIC_RELAXED);
        }
    }
    *cus_out = cus;
    *per_cu_out = per_cu;
    return hipSuccess;
}

// grid > 0: that many workgroups (at most the row blocks) instead of the resident count.
template <auto KERNEL>
inline hipError_t go_persistent(const Plan& plan, const Params& p, hipStream_t stream, int row_bytes_per_wave = 0,
                                int64_t grid_set = 0) {
    if (grid_set > 0) {
        Params args = p;
        void* argv[] = {&args};
        return hipLaunchKernel(reinterpret_cast<const void*>(KERNEL),
                               dim3(static_cast<unsigned>(grid_set < plan.grid ? grid_set : plan.grid)),
                               dim3(static_cast<unsigned>(plan.block_threads)), argv,
                               static_cast<size_t>(plan.lds_bytes), stream);
    }
    int cus = 0, per_cu = 0;
    hipError_t e = resident<KERNEL>(plan.block_threads, plan.lds_bytes, &cus, &per_cu);
    if (e != hipSuccess) return e;
    // Vectorized workgroups that stage parameters and hold 4 chunks per lane: at most two
    // per CU (more rows per workgroup, measured better for fused add + LayerNorm 8192 x 4096:
    // 68.3% -> 70.0%, neutral for the others); smaller rows, and launches without parameters
    // (softmax: 54-64% -> 63-69% for 16-bit rows of 4096-16384 uncapped), keep the full
    // resident count for bytes in flight.
    // The element kernels (row_bytes_per_wave > 0: the row bytes one wave holds) keep about
    // kElemCuRowBytes of row data per CU (measured on MI355X, persistent grids of 1 to 6
    // workgroups per CU: 16 waves of 2 KiB or 32 of 1 KiB are the best or within noise of
    // it; fp32 LayerNorm 8192 x 4095: 60% resident-limited -> 68%).
    // Rows shorter than half of kLoopCuRowBytes keep more workgroups, so that a CU still has
    // about that many row bytes in flight (measured on MI355X, cold cache, graph replays:
    // byte-addressed LayerNorm bf16 8192 x 4608, rows of 9 KiB on 4 waves, 51.1 us on two
    // workgroups per CU, 37.5 on four, 35.2 on six; rows of 16 KiB and more measured best on
    // two).
    int cap = per_cu;
    if (row_bytes_per_wave > 0) {
        const int waves = kElemCuRowBytes / row_bytes_per_wave;
        const int wg = waves / (plan.block_threads / 64);
        cap = wg < 1 ? 1 : (wg < per_cu ? wg : per_cu);
    } else if (plan.chunks_per_lane >= 4 && per_cu > 2 && plan.lds_bytes > 0) {
        const int64_t rb = p.C * 16 * plan.rows_per_block;  // row bytes per workgroup
        const int64_t want = rb > 0 ? kLoopCuRowBytes / rb : 2;
        cap = want <= 2 ? 2 : (want < per_cu ? static_cast<int>(want) : per_cu);
    }
    int64_t grid = static_cast<int64_t>(cus) * cap;
    if (grid > plan.grid) grid = plan.grid;
    Params args = p;
    void* argv[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void*>(KERNEL), dim3(static_cast<unsigned>(grid)),
                           dim3(static_cast<unsigned>(plan.block_threads)), argv,
                           static_cast<size_t>(plan.lds_bytes), stream);
}

// Persistent vectorized launches: parameters staged on chip, streaming accesses, and a grid
// set by R = blocks / (CUs x resident workgroups per CU of the prefetching instance), where a
// block is the RPB rows one workgroup takes at a time:
//   R <= A: one workgroup per block, so that every row of the launch is in flight at once
//           (A = 3/4 for the fused ops, which read two row tensors; just under 1 for the
//           others, and 1 for 16-bit LayerNorm);
//   R <= 3: half as many workgroups, each loading its second block while it reduces and
//           stores the first (FL_PREFETCH);
//   R >  3: one workgroup per block again (the hardware starts a workgroup whenever one ends,
//           which keeps rows in flight without holding a second row in registers), except
//           for rows of 4 or more waves with parameters. Of those, LayerNorm and RMSNorm rows,
//           whose staged parameters are as large as the block or larger, loop over the rows
//           on two workgroups per CU without prefetching, staging the parameters once; the
//           fused ops (two row tensors in, two out) keep one workgroup per block, with the
//           looping instance from 8 waves per row (whose prefetching instance holds two rows
//           in fewer registers per lane).
// The thresholds come from a sweep on MI355X (cold cache, device time per launch of replayed
// HIP graphs) over LayerNorm, RMSNorm, fused add + RMSNorm / LayerNorm and softmax, 256 to
// 65536 rows of 1024 to 16384 elements, at grids of 1 to 8 workgroups per CU, half and full:
// the rule is within 0.5% of the fastest measured grid on average (at most 5% off), where
// the earlier fixed grid of two looping workgroups per CU was 6% off on average and up to
// 29%. Examples against that grid: LayerNorm bf16 2048 x 4096 8.82 -> 7.63 us, 4096 x 4096
// 14.14 -> 11.97 us, 32768 x 4096 89.75 -> 86.81 us; fused add + RMSNorm fp16 2048 x 4096
// 13.74 -> 11.64 us, 32768 x 4096 184.1 -> 174.2 us; RMSNorm fp16 2048 x 4096 8.01 -> 6.96
// us; fused add + LayerNorm bf16 32768 x 4096 184.8 -> 171.8 us; softmax fp32 32768 x 4096
// 182.1 -> 169.9 us; LayerNorm bf16 4096 x 16384 unchanged at 46.3 us.
// Measured on MI355X for the R > 3 exceptions (cold cache, device time per launch; every
// alternative in the launch-plan sweep of the benchmark): LayerNorm bf16 4096 x 16384 looping
// on 512 workgroups 46.4 us, prefetching one per block 49.5 us; LayerNorm bf16 16384 x 8192
// 88.3 against 90.5 us; fused add + LayerNorm bf16 16384 x 8192 prefetching one per block
// 171.9 us, looping on 512 182.2 us; fused add + RMSNorm fp16 16384 x 8192 174.5 against
// 182.8 us; fused add + LayerNorm bf16 4096 x 16384 (8 waves) looping one per block 90.7 us,
// prefetching one per block 94.5 us, looping on the resident grid 94.2 us.
// Byte-addressed 16-bit LayerNorm rows of 1 or 2 waves keep half as many workgroups for R > 3
// as well (their accesses at 2-byte alignment take longer, and a second row in flight per
// workgroup covers that): LayerNorm bf16 16384 x 4095 54.3 -> 51.2 us (one per block 54.5).
struct GridRule {
    bool two_tensors;  // fused ops: x and the residual
    bool ln16;         // LayerNorm of 16-bit rows
    bool loop_wide;    // R > 3: the looping instance on the resident grid
    bool loop_blocks;  // R > 3: the looping instance, one workgroup per block
    bool half_many;    // R > 3: half as many workgroups, prefetching
};

// The grid of a persistent vectorized launch and its instance: *loop_out selects the looping
// instance, on *grid_out workgroups, or on the resident grid when *grid_out is 0.
template <auto PF_KERNEL>
inline hipError_t persistent_grid(const Plan& plan, const GridRule& rule, int* grid_out, bool* loop_out) {
    int cus = 0, per_cu = 0;
    hipError_t e = resident<PF_KERNEL>(plan.block_threads, plan.lds_bytes, &cus, &per_cu);
    if (e != hipSuccess) return e;
    const int64_t blocks = plan.grid;
    const int64_t res = static_cast<int64_t>(cus) * per_cu;  // resident workgroups
    const bool one_round = rule.two_tensors ? 4 * blocks <= 3 * res : (rule.ln16 ? blocks <= res : blocks < res);
    int64_t grid = blocks;
    bool loop = false;
    if (!one_round) {
        if (blocks <= 3 * res) {
            grid = (blocks + 1) / 2;
        } else if (rule.loop_wide) {
            loop = true;
            grid = 0;
        } else if (rule.half_many) {
            grid = (blocks + 1) / 2;
        } else {
            loop = rule.loop_blocks;
        }
    }
    if (grid > kMaxGrid) grid = kMaxGrid;
    *grid_out = static_cast<int>(grid);
    *loop_out = loop;
    return hipSuccess;
}

template <auto KERNEL>
inline hipError_t launch_grid(const Plan& plan, const Params& p, hipStream_t stream, int64_t grid) {
    Params args = p;
    void* argv[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void*>(KERNEL), dim3(static_cast<unsigned>(grid)),
                           dim3(static_cast<unsigned>(plan.block_threads)), argv,
                           static_cast<size_t>(plan.lds_bytes), stream);
}

// One vectorized launch: persistent (the prefetching instance, or the looping one for wide
// rows with parameters when R > 3) or grid per row.
template <int DT, int OP, int W, int V, bool EXACT, int AFF, bool PERS, bool RAG = false>
inline hipError_t go_v(const Plan& plan, const Params& p, hipStream_t s) {
    constexpr int RPB = rows_per_block_for(W);
    if constexpr (PERS) {
        constexpr int FL = persistent_flags<OP, AFF>() | (RAG ? FL_RAGGED : 0);
        // 1024-lane workgroups have no registers for a second row, nor have one-wave rows of 8
        // or more chunks per lane (reached only by forcing the wave variant): they loop
        // without prefetching, as do wide rows with parameters when R > 2.
        constexpr bool NOPF = W >= 16 || (W == 1 && V >= 8);
        constexpr bool WIDE_PARAMS = W >= 4 && AFF != 0 && !OpTraits<OP>::SM;
        // A caller-chosen instance (plan.prefetch 0 / 1) must be one that is built: the looping
        // instance exists for NOPF shapes and wide rows with parameters only.
        if constexpr (NOPF) {
            if (plan.prefetch == 1) return hipErrorNotSupported;
            if (plan.dry) return hipSuccess;
            constexpr auto K = rownorm_vec_kernel<DT, OP, W, V, RPB, EXACT, AFF, FL>;
            int64_t grid = plan.grid_force;
            if (grid <= 0) {
                // Up to kLoopWorkgroupsPerCu workgroups per CU, more than stay resident: each
                // loops over fewer rows, and the hardware hands the later ones to whichever
                // CU finishes first, which evens out the CUs' finishing times. Measured on
                // MI355X against two looping workgroups per CU (cold cache, graph replays):
                // RMSNorm fp32 4096 x 16384 92.7 -> 89.1 us, 4096 x 16383 (byte-addressed)
                // 99.5 -> 95.8 us, LayerNorm fp32 4096 x 16384 91.0 -> 89.8 us, softmax bf16
                // 4096 x 32768 115.2 -> 112.1 us.
                int cus = 0, per_cu = 0;
                hipError_t e = resident<K>(plan.block_threads, plan.lds_bytes, &cus, &per_cu);
                if (e != hipSuccess) return e;
                grid = static_cast<int64_t>(cus) * kLoopWorkgroupsPerCu;
            }
            return go_persistent<K>(plan, p, s, 0, grid);
        } else {
            if (plan.prefetch == 0 && !WIDE_PARAMS) return hipErrorNotSupported;
            if (plan.dry) return hipSuccess;
            constexpr auto PFK = rownorm_vec_kernel<DT, OP, W, V, RPB, EXACT, AFF, FL | FL_PREFETCH>;
            constexpr bool RES = OpTraits<OP>::RES;
            constexpr GridRule rule{RES, OP == OP_LN && DT != DT_F32, WIDE_PARAMS && !RES,
                                    WIDE_PARAMS && RES && W >= 8, RAG && OP == OP_LN && DT != DT_F32};
            int grid = 0;
            bool loop = false;
            hipError_t e = persistent_grid<PFK>(plan, rule, &grid, &loop);
            if (e != hipSuccess) return e;
            if (plan.prefetch >= 0) loop = plan.prefetch == 0;
            if (plan.grid_force > 0) grid = static_cast<int>(plan.grid_force < plan.grid ? plan.grid_force : plan.grid);
            if constexpr (WIDE_PARAMS) {
                if (loop) return go_persistent<rownorm_vec_kernel<DT, OP, W, V, RPB, EXACT, AFF, FL>>(plan, p, s, 0, grid);
            }
            if (grid <= 0) grid = static_cast<int>(plan.grid);  // the prefetching instance chosen over a looping rule
            return launch_grid<PFK>(plan, p, s, grid);
        }
    } else {
        if (plan.dry) return hipSuccess;
        // 1024-lane workgroups have 128 VGPRs per lane: LayerNorm rows there keep no fp32 copy.
        constexpr int FL = (W >= 16 && OpTraits<OP>::LN ? FL_NOFLOAT : 0) | (RAG ? FL_RAGGED : 0);
        return go(rownorm_vec_kernel<DT, OP, W, V, RPB, EXACT, AFF, FL>, plan, p, s);
    }
}

template <int DT, int OP, int W, bool EXACT, int AFF, bool PERS, bool RAG = false>
inline hipError_t launch_v(const Plan& plan, const Params& p, hipStream_t s) {
    constexpr int RPB = rows_per_block_for(W);
    if (plan.rows_per_block != RPB) return hipErrorInvalidValue;
#define RN_GO(VV) go_v<DT, OP, W, VV, EXACT, AFF, PERS, RAG>(plan, p, s)
    // Ragged rows: persistent, the planner's shapes, about 4 chunks per lane (fewer only for
    // one-wave rows); grid per row, softmax rows of more than 4096 chunks on one 16-wave
    // workgroup (8 chunks per lane, fp32 up to 16).
    if constexpr (RAG && !PERS) {
        if constexpr (W == 16 && OP == OP_SOFTMAX) {
            if (plan.chunks_per_lane == 8) return RN_GO(8);
            if constexpr (DT == DT_F32) {
                if (plan.chunks_per_lane == 16) return RN_GO(16);
            }
        }
        return hipErrorNotSupported;
    } else if constexpr (RAG) {
        if (plan.chunks_per_lane == 4) return RN_GO(4);
        if constexpr (W == 1) {
            switch (plan.chunks_per_lane) {
            case 1: return RN_GO(1);
            case 2: return RN_GO(2);
            default: break;
            }
        }
        return hipErrorNotSupported;
    } else {
    // The planner gives rows of 8 and 16 waves 4 chunks per lane (or 8 / 16 for the one-
    // workgroup rows below); fewer chunks per lane occur only with 1, 2 and 4 waves.
    if constexpr (W <= 4) {
        switch (plan.chunks_per_lane) {
        case 1: return RN_GO(1);
        case 2: return RN_GO(2);
        default: break;
        }
    }
    if (plan.chunks_per_lane == 4) return RN_GO(4);
    // Rows of 64 * W * o chunks, o odd from 3 to 15, held exactly (persistent launches only;
    // rows of 16 waves: o = 3, of 8 waves up to 7; the rest exceed 4096 chunks)
    if constexpr (PERS && EXACT) {
        if (plan.chunks_per_lane == 3) return RN_GO(3);
        if constexpr (W <= 8) {
            if (plan.chunks_per_lane == 5) return RN_GO(5);
            if (plan.chunks_per_lane == 7) return RN_GO(7);
        }
        if constexpr (W <= 4) {
            if (plan.chunks_per_lane == 9) return RN_GO(9);
            if (plan.chunks_per_lane == 11) return RN_GO(11);
            if (plan.chunks_per_lane == 13) return RN_GO(13);
            if (plan.chunks_per_lane == 15) return RN_GO(15);
        }
    }
    if constexpr (W == 1) {
        switch (plan.chunks_per_lane) {
        case 8: return RN_GO(8);
        case 16: return RN_GO(16);
        default: break;
        }
    }
    // softmax and RMSNorm rows of up to 128 KiB, one workgroup each (measured against the
    // split-row path); LayerNorm and fused add + RMSNorm rows too when no workspace allows
    // split rows (the fused add + LayerNorm instance would spill)
    if constexpr (W == 16 && !PERS && (OP == OP_SOFTMAX || OP == OP_RMS || OP == OP_LN || OP == OP_FUSED)) {
        if (plan.chunks_per_lane == 8) return RN_GO(8);
    }
    if constexpr (W == 16 && !PERS && OP == OP_SOFTMAX && DT == DT_F32) {  // fp32 softmax rows up to 256 KiB
        if (plan.chunks_per_lane == 16) return RN_GO(16);
    }
    return hipErrorNotSupported;  // no instance of this shape is built
    }
#undef RN_GO
}

template <int DT, int OP, bool EXACT, int AFF, bool PERS, bool RAG = false>
inline hipError_t launch_w(const Plan& plan, const Params& p, hipStream_t s) {
    switch (plan.waves_per_row) {
    case 1: return launch_v<DT, OP, 1, EXACT, AFF, PERS, RAG>(plan, p, s);
    case 2: return launch_v<DT, OP, 2, EXACT, AFF, PERS, RAG>(plan, p, s);
    case 4: return launch_v<DT, OP, 4, EXACT, AFF, PERS, RAG>(plan, p, s);
    case 8: return launch_v<DT, OP, 8, EXACT, AFF, PERS, RAG>(plan, p, s);
    case 16: return launch_v<DT, OP, 16, EXACT, AFF, PERS, RAG>(plan, p, s);
    default: return hipErrorNotSupported;
    }
}

template <int DT, int OP, int AFF, bool PERS>
inline hipError_t launch_e(const Plan& plan, const Params& p, hipStream_t s) {
    if constexpr (PERS) {
        // persistent launches are planned for exact shapes and for ragged rows (byte-addressed
        // rows; exact when the row's chunks, the last one partial, fill the row group)
        if (plan.ragged)
            return plan.exact ? launch_w<DT, OP, true, AFF, true, true>(plan, p, s)
                              : launch_w<DT, OP, false, AFF, true, true>(plan, p, s);
        if (!plan.exact) return hipErrorNotSupported;
        return launch_w<DT, OP, true, AFF, true>(plan, p, s);
    } else {
        // grid per row: byte-addressed softmax rows of more than 4096 chunks (the instance
        // that is not chunk-exact serves every such row)
        if (plan.ragged) {
            if constexpr (OP == OP_SOFTMAX)
                return launch_w<DT, OP, false, AFF, false, true>(plan, p, s);
            else
                return hipErrorNotSupported;
        }
        return plan.exact ? launch_w<DT, OP, true, AFF, false>(plan, p, s)
                          : launch_w<DT, OP, false, AFF, false>(plan, p, s);
    }
}

// Element kernel instances: W = 1 with 1-8 elements per lane; W = 2, 4, 8 with 8; W = 16
// with 8 or 16 (rows of up to 16384 elements). Many rows: a persistent grid (the kernel
// loops over rows either way; its parameters stay in registers across rows).
template <int DT, int OP>
inline hipError_t launch_pair(const Plan& plan, const Params& p, hipStream_t s) {
    const int W = plan.waves_per_row, V = plan.chunks_per_lane;
    const int aff = (p.gamma ? AFF_G : 0) | (OpTraits<OP>::LN && p.beta ? AFF_B : 0);
    if (plan.rows_per_block != rows_per_block_for(W)) return hipErrorInvalidValue;
#define RN_PR(WW, VV, A)                                                                      \
    (plan.persistent ? go_persistent<rownorm_pair_kernel<DT, OP, WW, VV, rows_per_block_for(WW), A>>(plan, p, s, 256 * VV) \
                     : go(rownorm_pair_kernel<DT, OP, WW, VV, rows_per_block_for(WW), A>, plan, p, s))
#define RN_PR_AFF(WW, VV)                                                     \
    do {                                                                      \
        if constexpr (OpTraits<OP>::SM) {                                     \
            return RN_PR(WW, VV, 0);                                          \
        } else {                                                              \
            if (aff == 0) return RN_PR(WW, VV, 0);                            \
            if (aff == AFF_G) return RN_PR(WW, VV, AFF_G);                    \
            if constexpr (OpTraits<OP>::LN) {                                 \
                if (aff == AFF_B) return RN_PR(WW, VV, AFF_B);                \
                return RN_PR(WW, VV, AFF_G | AFF_B);                          \
            }                                                                 \
            return hipErrorInvalidValue;                                      \
        }                                                                     \
    } while (0)
    // the shapes the planner produces: W = 1 with 1..8 words per lane, else 8 words per lane
    if (W == 1) {
        switch (V) {
        case 1: RN_PR_AFF(1, 1);
        case 2: RN_PR_AFF(1, 2);
        case 4: RN_PR_AFF(1, 4);
        case 8: RN_PR_AFF(1, 8);
        default: return hipErrorInvalidValue;
        }
    }
    if constexpr (OpTraits<OP>::SM) {  // rows of up to 65536 elements
        if (W == 16 && V == 16) RN_PR_AFF(16, 16);
        if (W == 16 && V == 32) RN_PR_AFF(16, 32);
    }
    if (V != 8) return hipErrorInvalidValue;
    switch (W) {
    case 2: RN_PR_AFF(2, 8);
    case 4: RN_PR_AFF(4, 8);
    case 8: RN_PR_AFF(8, 8);
    case 16: RN_PR_AFF(16, 8);
    default: return hipErrorInvalidValue;
    }
#undef RN_PR_AFF
#undef RN_PR
}

template <int DT, int OP>
inline hipError_t launch_elem(const Plan& plan, const Params& p, hipStream_t s) {
    const int W = plan.waves_per_row, V = plan.chunks_per_lane;
    const int aff = (p.gamma ? AFF_G : 0) | (OpTraits<OP>::LN && p.beta ? AFF_B : 0);
    if (plan.pairs) {
        if constexpr (DT == DT_F32) {
            return hipErrorInvalidValue;
        } else {
            return launch_pair<DT, OP>(plan, p, s);
        }
    }
    if (plan.rows_per_block != rows_per_block_for(W)) return hipErrorInvalidValue;
#define RN_EL(WW, VV, A)                                                                      \
    (plan.persistent ? go_persistent<rownorm_elem_kernel<DT, OP, WW, VV, rows_per_block_for(WW), A>>(plan, p, s, 64 * VV * (DT == DT_F32 ? 4 : 2)) \
                     : go(rownorm_elem_kernel<DT, OP, WW, VV, rows_per_block_for(WW), A>, plan, p, s))
#define RN_EL_AFF(WW, VV)                                                     \
    do {                                                                      \
        if constexpr (OpTraits<OP>::SM) {                                     \
            return RN_EL(WW, VV, 0);                                          \
        } else {                                                              \
            if (aff == 0) return RN_EL(WW, VV, 0);                            \
            if (aff == AFF_G) return RN_EL(WW, VV, AFF_G);                    \
            if constexpr (OpTraits<OP>::LN) {                                 \
                if (aff == AFF_B) return RN_EL(WW, VV, AFF_B);                \
                return RN_EL(WW, VV, AFF_G | AFF_B);                          \
            }                                                                 \
            return hipErrorInvalidValue;                                      \
        }                                                                     \
    } while (0)
    if (W == 1) {
        switch (V) {
        case 1: RN_EL_AFF(1, 1);
        case 2: RN_EL_AFF(1, 2);
        case 4: RN_EL_AFF(1, 4);
        case 8: RN_EL_AFF(1, 8);
        default: return hipErrorInvalidValue;
        }
    }
    if (W == 2 && V == 8) RN_EL_AFF(2, 8);
    if (W == 4 && V == 8) RN_EL_AFF(4, 8);
    if (W == 8 && V == 8) RN_EL_AFF(8, 8);
    if (W == 16 && V == 8) RN_EL_AFF(16, 8);
    if (W == 16 && V == 16) RN_EL_AFF(16, 16);
    if constexpr (OpTraits<OP>::SM) {  // rows of up to 65536 elements
        if (W == 16 && V == 32) RN_EL_AFF(16, 32);
        if (W == 16 && V == 64) RN_EL_AFF(16, 64);
    }
#undef RN_EL_AFF
#undef RN_EL
    return hipErrorInvalidValue;
}

template <int DT, int OP, bool PERS>
inline hipError_t launch_op(const Plan& plan, const Params& p, hipStream_t s) {
    if (plan.variant == V_GENERAL || plan.variant == V_ELEMENT) {
        if constexpr (PERS) {
            return hipErrorInvalidValue;
        } else {
            if (plan.variant == V_ELEMENT) return launch_elem<DT, OP>(plan, p, s);
            return go(rownorm_general_kernel<DT, OP>, plan, p, s);
        }
    }
    if (plan.variant != V_WAVE && plan.variant != V_WORKGROUP) return hipErrorInvalidValue;
    if constexpr (OpTraits<OP>::SM) {
        return launch_e<DT, OP, 0, PERS>(plan, p, s);
    } else {
        const int aff = (p.gamma ? AFF_G : 0) | (OpTraits<OP>::LN && p.beta ? AFF_B : 0);
        switch (aff) {
        case 0: return launch_e<DT, OP, 0, PERS>(plan, p, s);
        case AFF_G: return launch_e<DT, OP, AFF_G, PERS>(plan, p, s);
        default: break;
        }
        if constexpr (OpTraits<OP>::LN) {
            if (aff == AFF_B) return launch_e<DT, OP, AFF_B, PERS>(plan, p, s);
            return launch_e<DT, OP, AFF_G | AFF_B, PERS>(plan, p, s);
        }
        return hipErrorInvalidValue;
    }
}

// Split-row launches: statistics, then normalization, on the same stream.
// A split-row launch: one workgroup per (row, segment) work item up to the grid cap (a grid
// of only what the device keeps resident, looping over the work items, measured 5-10%
// slower on MI355X).
template <auto KERNEL>
inline hipError_t go_wide(const Plan& plan, const Params& p, const WideArgs& wa, hipStream_t s) {
    const int64_t grid = plan.grid;
    Params pa = p;
    WideArgs wb = wa;
    void* argv[] = {&pa, &wb};
    return hipLaunchKernel(reinterpret_cast<const void*>(KERNEL), dim3(static_cast<unsigned>(grid)), dim3(kWideLanes),
                           argv, 0, s);
}

template <int DT, int OP>
inline hipError_t launch_wide_elem_op(const Plan& plan, const Params& p, const WideArgs& wa, hipStream_t s) {
    hipError_t e = go_wide<rownorm_wide_elem_stats_kernel<DT, OP>>(plan, p, wa, s);
    if (e != hipSuccess) return e;
    const int aff = (OpTraits<OP>::SM ? 0 : (p.gamma ? AFF_G : 0)) | (OpTraits<OP>::LN && p.beta ? AFF_B : 0);
#define RN_WEN(A) go_wide<rownorm_wide_elem_norm_kernel<DT, OP, A>>(plan, p, wa, s)
    if constexpr (OpTraits<OP>::SM) {
        return RN_WEN(0);
    } else {
        if (aff == 0) return RN_WEN(0);
        if (aff == AFF_G) return RN_WEN(AFF_G);
        if constexpr (OpTraits<OP>::LN) {
            if (aff == AFF_B) return RN_WEN(AFF_B);
            return RN_WEN(AFF_G | AFF_B);
        }
        return hipErrorInvalidValue;
    }
#undef RN_WEN
}

// One-pass split rows (rows of whole chunks, a workspace that holds the one-pass layout):
// the clear launch, then the one-pass kernel on min(resident, P * S) workgroups over P row
// blocks (at most 256 segments and room for two workgroups per segment on the device;
// otherwise, or for lack of the layout, the two launches). Returns hipErrorNotSupported when
// the one pass does not apply.
template <int DT, int OP, bool EXACT, int AFF, bool RAG = false>
inline hipError_t go_wide_onepass(const Plan& plan, const Params& p, const WideArgs& wa0, hipStream_t s) {
    constexpr auto K = rownorm_wide_onepass_kernel<DT, OP, EXACT, AFF, RAG>;
    if (wa0.sync == nullptr || wa0.rec64 == nullptr || wa0.S > kWideOnePassMaxSeg) return hipErrorNotSupported;
    int cus = 0, per_cu = 0;
    hipError_t e = resident<K>(kWideLanes, 0, &cus, &per_cu);
    if (e != hipSuccess) return e;
    const int64_t res = static_cast<int64_t>(cus) * per_cu;
    if (res < 2 * static_cast<int64_t>(wa0.S)) return hipErrorNotSupported;
    // Blocks of about kWideOnePassRows rows (at least enough blocks to fill the resident
    // grid). Measured on MI355X with the single-row tail below, rows per block 4 / 8:
    // LayerNorm fp32 x 65536, 512 rows 61.8 / 61.1 us, 1024 rows 106.2 / 107.6 us, 2048 rows
    // 200.7 / 200.6 us; LayerNorm bf16 1024 x 131072 119.9 / 114.9 us; fused add + RMSNorm
    // fp16 1024 x 65536 116.1 / 97.8 us (6 and 12 rows: 5-16% slower). Without the tail,
    // LayerNorm fp32 1024 x 65536: 16 rows per block 114.3 us, 8 109.0, 4 107.9. Rejected (same shapes): three rows loaded ahead instead of two (1024 rows:
    // 112.9 us), each workgroup on one segment for the whole launch with per-segment block
    // counters (134 us: a row's segments were no longer processed together), and tickets
    // claimed a row ahead with the row pipeline running across tickets (112.6 us).
    WideArgs wa = wa0;
    int64_t P = (p.rows + kWideOnePassRows - 1) / kWideOnePassRows;
    if (P < res / wa.S) P = res / wa.S;
    if (P > p.rows) P = p.rows;
    const int64_t R = (p.rows + P - 1) / P;
    P = (p.rows + R - 1) / R;
    // The last rows, about one round of the resident grid (res / S, at most a quarter of
    // the rows), in tickets of one row, so that the workgroups run out of work together:
    // measured on MI355X, LayerNorm fp32 x 65536: 512 rows 63.3 -> 61.5 us, 1024 rows 109.2 ->
    // 106.6 us, 2048 rows 204.4 -> 201.3 us (tails of 128-256 rows in 2-row tickets: 0-2 us).
    int64_t P1 = P;
    const int64_t R2 = 1;
    const int64_t tail = res / wa.S < p.rows / 4 ? res / wa.S : p.rows / 4;
    if (R > 1 && tail > 0) {
        P1 = (p.rows - tail) / R;
        P = P1 + (p.rows - P1 * R + R2 - 1) / R2;
    }
    if (P * wa.S > INT32_MAX) return hipErrorNotSupported;  // tickets come from a 32-bit counter
    wa.P = static_cast<int>(P);
    wa.R = static_cast<int>(R);
    wa.P1 = static_cast<int>(P1);
    wa.R2 = static_cast<int>(R2);
    // header (counter, count) and records: 256 + rows * S * 32 bytes
    const int64_t n16 = (256 + p.rows * wa.S * 32) / 16;
    int64_t gc = (n16 + 255) / 256;
    if (gc > 1024) gc = 1024;
    u32x4* clr = reinterpret_cast<u32x4*>(wa.sync);
    void* zargv[] = {&clr, const_cast<int64_t*>(&n16)};
    e = hipLaunchKernel(reinterpret_cast<const void*>(rownorm_wide_clear_kernel<DT>), dim3(static_cast<unsigned>(gc)),
                        dim3(256), zargv, 0, s);
    if (e != hipSuccess) return e;
    const int64_t tickets = P * wa.S;
    const int64_t g = res < tickets ? res : tickets;
    Params pa = p;
    void* argv[] = {&pa, &wa};
    return hipLaunchKernel(reinterpret_cast<const void*>(K), dim3(static_cast<unsigned>(g)), dim3(kWideLanes), argv, 0,
                           s);
}

template <int DT, int OP, bool EXACT, bool RAG = false>
inline hipError_t launch_wide_onepass(const Plan& plan, const Params& p, const WideArgs& wa, hipStream_t s) {
    if constexpr (OpTraits<OP>::SM) {
        return go_wide_onepass<DT, OP, EXACT, 0, RAG>(plan, p, wa, s);
    } else {
        const int aff = (p.gamma ? AFF_G : 0) | (OpTraits<OP>::LN && p.beta ? AFF_B : 0);
        if (aff == 0) return go_wide_onepass<DT, OP, EXACT, 0, RAG>(plan, p, wa, s);
        if (aff == AFF_G) return go_wide_onepass<DT, OP, EXACT, AFF_G, RAG>(plan, p, wa, s);
        if constexpr (OpTraits<OP>::LN) {
            if (aff == AFF_B) return go_wide_onepass<DT, OP, EXACT, AFF_B, RAG>(plan, p, wa, s);
            return go_wide_onepass<DT, OP, EXACT, AFF_G | AFF_B, RAG>(plan, p, wa, s);
        }
        return hipErrorInvalidValue;
    }
}

template <int DT, int OP>
inline hipError_t launch_wide_op(const Plan& plan, const Params& p, const WideArgs& wa, hipStream_t s) {
    if (plan.variant == V_WIDE_ELEM) return launch_wide_elem_op<DT, OP>(plan, p, wa, s);
    if (plan.ragged) {
        // byte-addressed rows: the one-pass kernel, or (when the device cannot hold it) the
        // element-granular two launches over the same workspace, which the planner sized for both
        const hipError_t e1 = launch_wide_onepass<DT, OP, false, true>(plan, p, wa, s);
        if (e1 != hipErrorNotSupported) return e1;
        Plan pe = plan;
        pe.variant = V_WIDE_ELEM;
        pe.ragged = false;
        const int64_t S2 = (p.N + kWideElemSeg - 1) / kWideElemSeg;
        pe.grid = p.rows * S2 < kMaxGrid ? p.rows * S2 : kMaxGrid;
        pe.exact = p.N % kWideElemSeg == 0;
        WideArgs we = wa;
        we.S = static_cast<int>(S2);
        we.sync = nullptr;
        we.rec64 = nullptr;
        return launch_wide_elem_op<DT, OP>(pe, p, we, s);
    }
    {
        const hipError_t e1 = plan.exact ? launch_wide_onepass<DT, OP, true>(plan, p, wa, s)
                                         : launch_wide_onepass<DT, OP, false>(plan, p, wa, s);
        if (e1 != hipErrorNotSupported) return e1;
    }
    hipError_t e = plan.exact ? go_wide<rownorm_wide_stats_kernel<DT, OP, true>>(plan, p, wa, s)
                              : go_wide<rownorm_wide_stats_kernel<DT, OP, false>>(plan, p, wa, s);
    if (e != hipSuccess) return e;
    const int aff = (OpTraits<OP>::SM ? 0 : (p.gamma ? AFF_G : 0)) | (OpTraits<OP>::LN && p.beta ? AFF_B : 0);
#define RN_WN(A)                                                                    \
    (plan.exact ? go_wide<rownorm_wide_norm_kernel<DT, OP, true, A>>(plan, p, wa, s) \
                : go_wide<rownorm_wide_norm_kernel<DT, OP, false, A>>(plan, p, wa, s))
    if constexpr (OpTraits<OP>::SM) {
        return RN_WN(0);
    } else {
        if (aff == 0) return RN_WN(0);
        if (aff == AFF_G) return RN_WN(AFF_G);
        if constexpr (OpTraits<OP>::LN) {
            if (aff == AFF_B) return RN_WN(AFF_B);
            return RN_WN(AFF_G | AFF_B);
        }
        return hipErrorInvalidValue;
    }
#undef RN_WN
}

template <int DT>
inline hipError_t launch_wide(int op, const Plan& plan, const Params& p, const WideArgs& wa, hipStream_t s) {
    if ((plan.variant != V_WIDE && plan.variant != V_WIDE_ELEM) || wa.ws == nullptr || wa.S < 1)
        return hipErrorInvalidValue;
    switch (op) {
    case OP_LN: return launch_wide_op<DT, OP_LN>(plan, p, wa, s);
    case OP_RMS: return launch_wide_op<DT, OP_RMS>(plan, p, wa, s);
    case OP_FUSED: return launch_wide_op<DT, OP_FUSED>(plan, p, wa, s);
    case OP_FUSED_LN: return launch_wide_op<DT, OP_FUSED_LN>(plan, p, wa, s);
    case OP_SOFTMAX: return launch_wide_op<DT, OP_SOFTMAX>(plan, p, wa, s);
    default: return hipErrorInvalidValue;
    }
}

template <int DT, bool PERS>
inline hipError_t launch_dtype(int op, const Plan& plan, const Params& p, hipStream_t s) {
    switch (op) {
    case OP_LN: return launch_op<DT, OP_LN, PERS>(plan, p, s);
    case OP_RMS: return launch_op<DT, OP_RMS, PERS>(plan, p, s);
    case OP_FUSED: return launch_op<DT, OP_FUSED, PERS>(plan, p, s);
    case OP_FUSED_LN: return launch_op<DT, OP_FUSED_LN, PERS>(plan, p, s);
    case OP_SOFTMAX: return launch_op<DT, OP_SOFTMAX, PERS>(plan, p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace rn
