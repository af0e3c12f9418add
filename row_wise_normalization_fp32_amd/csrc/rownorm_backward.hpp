// Backward passes of row-wise LayerNorm and RMSNorm for gfx950 (MI355X).
//
// For one row, with xhat_j = (x_j - mean) * rstd (RMSNorm: x_j * rstd) and g_j = dy_j *
// gamma_j, the chain rule through the normalization gives
//     dx_j = rstd * (g_j - (1/N) sum_k g_k - xhat_j * (1/N) sum_k g_k xhat_k)
// (RMSNorm: without the (1/N) sum_k g_k term), and over all rows
//     dgamma_j = sum_r dy_rj * xhat_rj,    dbeta_j = sum_r dy_rj.
// This is the BatchNorm gradient of "BatchNorm CUDA implementation" (jianying88.com/news/
// 30214), section 3.1, turned by 90 degrees: the statistics run along a row, so gamma sits
// inside the row sums, and the parameter gradients become column sums over the rows. The
// same article's section 3.2 weighs organizations of the kernel; the one here reads x and
// dy once and writes dx once:
//
//   1. rownorm_bwd_vec_kernel (or rownorm_bwd_elem_kernel for rows that are not whole
//      16-byte chunks): a grid of P workgroups loops over the rows. A row group of W waves
//      holds a row of x and dy in VGPRs, reduces sum g and sum g * xhat across the row (DPP,
//      then LDS across waves), and writes dx. Each lane owns the same columns for every row,
//      so it also accumulates its columns' dgamma / dbeta terms in fp32 registers across
//      all the rows it visits. At the end the row groups of a workgroup add their column
//      sums in a fixed order through LDS, and the workgroup writes one fp32 partial row per
//      parameter to the workspace: [2][P][N].
//   2. rownorm_bwd_cols_kernel sums the P partial rows of each column in a fixed order and
//      rounds to the I/O dtype.
// Results are bitwise reproducible for a given P: every floating-point sum is formed in a
// fixed order, and none is accumulated with an atomic. P depends on the device's CU count
// and the kernels' occupancy (and, for split rows, on the segments per row). The one-pass
// split-row kernel below uses integer atomics only to hand out work (a ticket counter) and
// to publish its per-segment sums (tagged 64-bit words read in a fixed order).
#pragma once

#include <map>
#include <mutex>
#include <utility>

#include "rownorm_kernels.hpp"

namespace rn {

// Cache-policy operand of the buffer builtins: the non-temporal bit (gfx940 and later), for
// x, dy and dx, which each call touches once (LayerNorm bf16 1024 x 65536 split rows: 120.5
// -> 116.0 us; fp32 512 x 65536: 103 -> 94.7 us).
constexpr int kNonTemporal = 2;

// Sum of two per-wave values across the row group's waves (one barrier).
template <int W>
__device__ __forceinline__ void group_sum2(WavePart (*part)[W > 1 ? W : 1], int& buf, int lane, int wr, float& a,
                                           float& b) {
    if constexpr (W > 1) {
        if (lane == 0) {
            part[buf][wr].v[0] = a;
            part[buf][wr].v[1] = b;
        }
        __syncthreads();
        a = part[buf][0].v[0];
        b = part[buf][0].v[1];
#pragma unroll
        for (int w = 1; w < W; ++w) {
            a += part[buf][w].v[0];
            b += part[buf][w].v[1];
        }
        buf ^= 1;
    }
}

// Row groups of a workgroup add their per-lane column sums in order 0, 1, ..., RPB - 1
// through LDS (red: n floats), and the last writes the workgroup's partial row to `out`.
// `cols(i, e)` is the column of register slot (i, e); `ok(i, e)` whether it is in the row.
template <int RPB, int NS, typename ColF, typename OkF>
__device__ __forceinline__ void flush_columns(const float (&acc)[NS], float* red, int rg, float* out, ColF cols,
                                              OkF ok) {
    if constexpr (RPB == 1) {
#pragma unroll
        for (int k = 0; k < NS; ++k)
            if (ok(k)) out[cols(k)] = acc[k];
    } else {
        for (int r = 0; r < RPB; ++r) {
            if (rg == r) {
#pragma unroll
                for (int k = 0; k < NS; ++k) {
                    if (!ok(k)) continue;
                    const float v = r == 0 ? acc[k] : red[cols(k)] + acc[k];
                    if (r == RPB - 1)
                        out[cols(k)] = v;
                    else
                        red[cols(k)] = v;
                }
            }
            __syncthreads();
        }
    }
}

template <int DT, int OP, int W, int V, int RPB, bool EXACT, bool HG>
__global__ __launch_bounds__(64 * W * RPB) void rownorm_bwd_vec_kernel(BwdParams p) {
    using IO = Io<DT>;
    constexpr int E = IO::E;
    constexpr int LANES = 64 * W;
    constexpr bool LN = OP == OP_LN;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rg = wave / W;
    const int wr = wave - rg * W;
    const int t = wr * 64 + lane;
    const int Ci = static_cast<int>(p.C);
    __shared__ WavePart part_all[RPB][2][W > 1 ? W : 1];
    extern __shared__ float red[];  // RPB > 1: N floats
    WavePart(*part)[W > 1 ? W : 1] = part_all[rg];
    auto chunk = [&](int i) {
        const int c = i * LANES + t;
        return EXACT ? c : (c < Ci ? c : Ci - 1);
    };
    auto valid = [&](int i) { return EXACT || i * LANES + t < Ci; };
    const bool want_cols = p.ws != nullptr;

    u32x4 gk[HG ? V : 1];
    if constexpr (HG) {
#pragma unroll
        for (int i = 0; i < V; ++i) gk[i] = static_cast<const u32x4*>(p.gamma)[chunk(i)];
    }
    float adg[V * E], adb[LN ? V * E : 1];
#pragma unroll
    for (int k = 0; k < V * E; ++k) {
        adg[k] = 0.f;
        if constexpr (LN) adb[k] = 0.f;
    }
    int buf = 0;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * RPB; base < p.rows;
         base += static_cast<int64_t>(gridDim.x) * RPB) {
        const int64_t row = base + rg;
        if (row >= p.rows) {
            if constexpr (W > 1) {
                __syncthreads();
                buf ^= 1;
            }
            continue;
        }
        int tl = t;
        asm volatile("" : "+v"(tl));
        const u32x4* xr = static_cast<const u32x4*>(p.x) + row * p.C;
        const u32x4* dr = static_cast<const u32x4*>(p.dy) + row * p.C;
        u32x4 xv[V], dv[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int c = EXACT ? i * LANES + tl : (i * LANES + tl < Ci ? i * LANES + tl : Ci - 1);
            xv[i] = __builtin_nontemporal_load(xr + c);
            dv[i] = __builtin_nontemporal_load(dr + c);
        }
        const float mean = LN ? p.mean[row] : 0.f;
        const float rstd = p.rstd[row];
        __builtin_amdgcn_sched_barrier(0);
        // gamma stays packed; it is widened where used (not hoisted out of the row loop as
        // fp32 values, which would cost 4 VGPRs per chunk for the whole kernel)
        u32x4 gl[HG ? V : 1];
#pragma unroll
        for (int i = 0; i < (HG ? V : 0); ++i) {
            gl[i] = gk[i];
            asm volatile("" : "+v"(gl[i]));
        }
        float sg = 0.f, sgx = 0.f;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float xf[E], df[E], gf[E];
            IO::unpack(xv[i], xf);
            IO::unpack(dv[i], df);
            if constexpr (HG) IO::unpack(gl[i], gf);
            const bool ok = valid(i);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float xh = LN ? (xf[e] - mean) * rstd : xf[e] * rstd;
                const float d = ok ? df[e] : 0.f;
                const float g = HG ? d * gf[e] : d;
                sg += g;
                sgx = fmaf(g, xh, sgx);
                adg[i * E + e] = fmaf(d, xh, adg[i * E + e]);
                if constexpr (LN) adb[i * E + e] += d;
            }
        }
        float Sg = wave_sum(sg), Sgx = wave_sum(sgx);
        group_sum2<W>(part, buf, lane, wr, Sg, Sgx);
        const float c1 = LN ? Sg * p.inv_n : 0.f;
        const float c2 = Sgx * p.inv_n;
        if (p.dx) {
            u32x4* o = static_cast<u32x4*>(p.dx) + row * p.C;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float xf[E], df[E], gf[E], r[E];
                IO::unpack(xv[i], xf);
                IO::unpack(dv[i], df);
                if constexpr (HG) IO::unpack(gl[i], gf);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float xh = LN ? (xf[e] - mean) * rstd : xf[e] * rstd;
                    const float g = HG ? df[e] * gf[e] : df[e];
                    r[e] = rstd * ((g - c1) - xh * c2);
                }
                if (valid(i)) __builtin_nontemporal_store(IO::pack(r), o + i * LANES + tl);
            }
        }
    }
    if (!want_cols) return;  // uniform over the grid
    float* dg_out = p.ws + static_cast<int64_t>(blockIdx.x) * p.N;
    float* db_out = p.ws + (static_cast<int64_t>(p.parts) + blockIdx.x) * p.N;
    auto col = [&](int k) { return (k / E * LANES + t) * E + k % E; };
    auto okc = [&](int k) { return EXACT || (k / E) * LANES + t < Ci; };
    flush_columns<RPB>(adg, red, rg, dg_out, col, okc);
    if constexpr (LN) flush_columns<RPB>(adb, red, rg, db_out, col, okc);
}

// Rows that are not whole 16-byte chunks: one element per register slot (rows up to
// 16384 elements), the same computation.
template <int DT, int OP, int W, int V, int RPB, bool HG>
__global__ __launch_bounds__(64 * W * RPB) void rownorm_bwd_elem_kernel(BwdParams p) {
    using IO = Io<DT>;
    constexpr int LANES = 64 * W;
    constexpr int S = DT == DT_F32 ? 4 : 2;
    constexpr bool LN = OP == OP_LN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: row bases stay in SGPRs
    const int rg = wave / W;
    const int wr = wave - rg * W;
    const unsigned t = static_cast<unsigned>(wr * 64 + lane);
    const unsigned N = static_cast<unsigned>(p.N);
    __shared__ WavePart part_all[RPB][2][W > 1 ? W : 1];
    extern __shared__ float red[];
    WavePart(*part)[W > 1 ? W : 1] = part_all[rg];
    const uint32_t row_bytes = N * S;  // N <= 64 * W * V: 32-bit offsets
    // gamma lives in VGPRs across rows unless that would push the widest instance (16
    // slots per lane, 1024 threads, 128 VGPRs) into spills; then it is re-read per row
    // (an L1/L2 hit: every row reads the same N values).
    constexpr bool GREG = HG && V < 16;
    const Rsrc gr = make_rsrc(p.gamma, HG ? row_bytes : 0);
    float gv[HG ? V : 1];
    if constexpr (GREG) {
#pragma unroll
        for (int i = 0; i < V; ++i) gv[i] = IO::bload(gr, static_cast<unsigned>(i * LANES) + t);
    }
    float adg[V], adb[LN ? V : 1];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        adg[i] = 0.f;
        if constexpr (LN) adb[i] = 0.f;
    }
    int buf = 0;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * RPB; base < p.rows;
         base += static_cast<int64_t>(gridDim.x) * RPB) {
        const int64_t row = base + rg;
        if (row >= p.rows) {
            if constexpr (W > 1) {
                __syncthreads();
                buf ^= 1;
            }
            continue;
        }
        // buffer resources bounded by the row: slots beyond N read 0 (so they add nothing
        // to the sums or the column partials) and their dx stores are dropped
        const Rsrc xr = make_rsrc(static_cast<const char*>(p.x) + row * p.N * S, row_bytes);
        const Rsrc dr = make_rsrc(static_cast<const char*>(p.dy) + row * p.N * S, row_bytes);
        float xf[V], df[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const unsigned j = static_cast<unsigned>(i * LANES) + t;
            xf[i] = IO::template bload<kNonTemporal>(xr, j);
            df[i] = IO::template bload<kNonTemporal>(dr, j);
        }
        const float mean = LN ? p.mean[row] : 0.f;
        const float rstd = p.rstd[row];
        __builtin_amdgcn_sched_barrier(0);
        // gamma of slot i: held (GREG) or read where it is used, in this loop and again in
        // the dx loop, so that only dy stays in registers across the row's reduction
        auto gam = [&](int i) {
            if constexpr (GREG) return gv[i];
            return IO::bload(gr, static_cast<unsigned>(i * LANES) + t);
        };
        float sg = 0.f, sgx = 0.f;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            xf[i] = LN ? (xf[i] - mean) * rstd : xf[i] * rstd;  // xhat (0 where df is 0)
            adg[i] = fmaf(df[i], xf[i], adg[i]);
            if constexpr (LN) adb[i] += df[i];
            const float g = HG ? df[i] * gam(i) : df[i];
            sg += g;
            sgx = fmaf(g, xf[i], sgx);
        }
        float Sg = wave_sum(sg), Sgx = wave_sum(sgx);
        group_sum2<W>(part, buf, lane, wr, Sg, Sgx);
        const float c1 = LN ? Sg * p.inv_n : 0.f;
        const float c2 = Sgx * p.inv_n;
        if (p.dx) {
            const Rsrc o = make_rsrc(static_cast<char*>(p.dx) + row * p.N * S, row_bytes);
#pragma unroll
            for (int i = 0; i < V; ++i) {
                const float g = HG ? df[i] * gam(i) : df[i];
                IO::template bstore<kNonTemporal>(o, static_cast<unsigned>(i * LANES) + t, rstd * ((g - c1) - xf[i] * c2));
            }
        }
    }
    if (p.ws == nullptr) return;
    float* dg_out = p.ws + static_cast<int64_t>(blockIdx.x) * p.N;
    float* db_out = p.ws + (static_cast<int64_t>(p.parts) + blockIdx.x) * p.N;
    auto col = [&](int k) { return static_cast<int>(k * LANES + t); };
    auto okc = [&](int k) { return static_cast<unsigned>(k * LANES) + t < N; };
    flush_columns<RPB>(adg, red, rg, dg_out, col, okc);
    if constexpr (LN) flush_columns<RPB>(adb, red, rg, db_out, col, okc);
}

// dgamma_j (dbeta_j) = the sum of the P partial rows of column j: lane s of 16 sums rows
// b = s, s + 16, ... in order, then the 16 lane sums are added in order; rounded once to the
// I/O dtype. A workgroup covers 64 columns of one parameter (blockIdx.y: 0 dgamma, 1 dbeta):
// 16 column quads x 16 lanes, so one wavefront load reads four 256-byte runs of partial rows
// (16-byte loads when N is a multiple of 4 and the workspace is 16-byte aligned; element
// loads otherwise). The two parameters run in parallel workgroups. Runs of 256 bytes or more
// matter: 64-byte runs (16 columns per workgroup) took twice as long.
template <int DT>
__global__ __launch_bounds__(256) void rownorm_bwd_cols_kernel(BwdColParams p) {
    using IO = Io<DT>;
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    constexpr int L = 16;       // partial-row lanes
    constexpr int Q = 256 / L;  // column quads per workgroup
    constexpr int B = 8;        // loads in flight per lane
    __shared__ f32x4 sums[L][Q + 1];
    void* out = blockIdx.y == 0 ? p.dgamma : p.dbeta;
    if (out == nullptr) return;  // uniform over the workgroup
    const int q = threadIdx.x % Q;   // column quad within the tile
    const int s = threadIdx.x / Q;  // partial-row lane
    const int64_t j0 = static_cast<int64_t>(blockIdx.x) * (4 * Q) + 4 * q;
    const bool vec = (p.N & 3) == 0 && (reinterpret_cast<uintptr_t>(p.ws) & 15) == 0;
    const float* src = p.ws + static_cast<int64_t>(blockIdx.y) * p.parts * p.N;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    if (vec) {
        if (j0 < p.N) {  // then j0 + 3 < N as well
            int b = s;
            for (; b + L * (B - 1) < p.parts; b += L * B) {
                f32x4 v[B];
#pragma unroll
                for (int u = 0; u < B; ++u)
                    v[u] = *reinterpret_cast<const f32x4*>(src + static_cast<int64_t>(b + L * u) * p.N + j0);
#pragma unroll
                for (int u = 0; u < B; ++u) a += v[u];
            }
            for (; b < p.parts; b += L) a += *reinterpret_cast<const f32x4*>(src + static_cast<int64_t>(b) * p.N + j0);
        }
    } else {
        // element loads at clamped columns (values of columns past N are never stored), in
        // the same batches and order as above
        int64_t jc[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) jc[e] = j0 + e < p.N ? j0 + e : p.N - 1;
        int b = s;
        for (; b + L * (B - 1) < p.parts; b += L * B) {
            f32x4 v[B];
#pragma unroll
            for (int u = 0; u < B; ++u) {
                const float* r = src + static_cast<int64_t>(b + L * u) * p.N;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[u][e] = r[jc[e]];
            }
#pragma unroll
            for (int u = 0; u < B; ++u) a += v[u];
        }
        for (; b < p.parts; b += L) {
            const float* r = src + static_cast<int64_t>(b) * p.N;
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] += r[jc[e]];
        }
    }
    sums[s][q] = a;
    __syncthreads();
    if (s == 0) {
        f32x4 r = sums[0][q];
#pragma unroll
        for (int u = 1; u < L; ++u) r += sums[u][q];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (j0 + e < p.N) IO::store1(out, j0 + e, r[e]);
    }
}

// ---------------------------------------------------------------------------------------
// Split-row backward: rows longer than one workgroup holds (more than 16384 elements). A row
// is cut into S segments of kBwdSeg elements (512 lanes x 16). The one-pass kernel below
// (rownorm_bwd_wide_onepass_kernel) is the usual path; rows of more segments than half the
// workgroups the device keeps resident, 16-bit rows that are not whole 16-byte groups, and
// workspaces that are not 16-byte aligned take three launches instead:
//   1. rownorm_bwd_wide_stats_kernel: per (row, segment) the segment's sum of g = dy * gamma
//      and of g * xhat, one record of two floats per segment in the workspace;
//   2. rownorm_bwd_wide_dx_kernel: workgroup (q, s) owns segment s of rows q, q + Q, ...: it
//      adds the row's S records in a fixed order (so every workgroup of the row gets the
//      same bits), writes dx for its segment, and accumulates its columns' dgamma / dbeta
//      terms in fp32 registers across its rows; at the end it writes its columns of partial
//      row q to the workspace ([2][Q][N], the layout the column kernel reads);
//   3. rownorm_bwd_cols_kernel sums the Q partial rows.
// x and dy are read twice. Rows, tensors and segments that are whole 16-byte groups move
// in 16-byte accesses (lane t holds groups i * 512 + t of the segment); otherwise element by
// element (lane t holds elements k * 512 + t). Elements past the row read as 0, which adds
// nothing to any sum (dy = 0), and are never written.
// ---------------------------------------------------------------------------------------

template <int DT>
struct BwdSeg {
    using IO = Io<DT>;
    static constexpr int SB = DT == DT_F32 ? 4 : 2;  // bytes per element
    static constexpr int G = 16 / SB;                // elements per 16-byte group
    static constexpr int V = kBwdSegPerLane;

    __device__ static __forceinline__ void load(const void* base, uint32_t nbytes, bool vec, int t, float (&f)[V]) {
        const Rsrc r = make_rsrc(base, nbytes);
        if (vec) {
#pragma unroll
            for (int i = 0; i < V / G; ++i) {
                const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (i * kBwdSegLanes + t) * 16, 0, 0);
                IO::unpack(v, &f[i * G]);
            }
        } else {
#pragma unroll
            for (int k = 0; k < V; ++k) f[k] = IO::bload(r, static_cast<uint32_t>(k * kBwdSegLanes + t));
        }
    }

    // AUX: cache policy of the 16-byte stores (kNonTemporal for data not read again soon)
    template <int AUX = 0>
    __device__ static __forceinline__ void store(void* base, uint32_t nbytes, bool vec, int t, const float (&f)[V]) {
        const Rsrc r = make_rsrc(base, nbytes);
        if (vec) {
#pragma unroll
            for (int i = 0; i < V / G; ++i)
                __builtin_amdgcn_raw_buffer_store_b128(IO::pack(&f[i * G]), r, (i * kBwdSegLanes + t) * 16, 0, AUX);
        } else {
#pragma unroll
            for (int k = 0; k < V; ++k) IO::template bstore<AUX>(r, static_cast<uint32_t>(k * kBwdSegLanes + t), f[k]);
        }
    }

    // fp32 values at the segment's element positions (the partial column rows)
    __device__ static __forceinline__ void store_f32(float* base, uint32_t n, bool vec, int t, const float (&f)[V]) {
        const Rsrc r = make_rsrc(base, n * 4);
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const uint32_t j = vec ? static_cast<uint32_t>((k / G * kBwdSegLanes + t) * G + k % G)
                                   : static_cast<uint32_t>(k * kBwdSegLanes + t);
            Io<DT_F32>::bstore(r, j, f[k]);
        }
    }
};

template <int DT, int OP, bool HG>
__global__ __launch_bounds__(kBwdSegLanes) void rownorm_bwd_wide_stats_kernel(BwdParams p) {
    using SG = BwdSeg<DT>;
    constexpr int V = SG::V;
    constexpr bool LN = OP == OP_LN;
    const int lane = threadIdx.x & 63;
    const int wr = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = threadIdx.x;
    __shared__ WavePart part[2][kBwdSegLanes / 64];
    int buf = 0;
    const bool vec = p.vec != 0;
    const int64_t total = p.rows * p.S;
    for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
        const int64_t row = b / p.S;
        const int seg = static_cast<int>(b - row * p.S);
        const int64_t e0 = static_cast<int64_t>(seg) * kBwdSeg;
        const uint32_t nb = static_cast<uint32_t>((p.N - e0 < kBwdSeg ? p.N - e0 : kBwdSeg) * SG::SB);
        const int64_t off = (row * p.N + e0) * SG::SB;
        float xf[V], df[V], gf[HG ? V : 1];
        SG::load(static_cast<const char*>(p.x) + off, nb, vec, t, xf);
        SG::load(static_cast<const char*>(p.dy) + off, nb, vec, t, df);
        if constexpr (HG) SG::load(static_cast<const char*>(p.gamma) + e0 * SG::SB, nb, vec, t, gf);
        const float mean = LN ? p.mean[row] : 0.f;
        const float rstd = p.rstd[row];
        float sg = 0.f, sgx = 0.f;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const float xh = LN ? (xf[k] - mean) * rstd : xf[k] * rstd;
            const float g = HG ? df[k] * gf[k] : df[k];
            sg += g;
            sgx = fmaf(g, xh, sgx);
        }
        float Sg = wave_sum(sg), Sgx = wave_sum(sgx);
        group_sum2<kBwdSegLanes / 64>(part, buf, lane, wr, Sg, Sgx);
        if (t == 0) {
            p.rec[2 * (row * p.S + seg)] = Sg;
            p.rec[2 * (row * p.S + seg) + 1] = Sgx;
        }
    }
}

template <int DT, int OP, bool HG>
__global__ __launch_bounds__(kBwdSegLanes) void rownorm_bwd_wide_dx_kernel(BwdParams p) {
    using SG = BwdSeg<DT>;
    constexpr int V = SG::V;
    constexpr bool LN = OP == OP_LN;
    const int lane = threadIdx.x & 63;
    const int t = threadIdx.x;
    const bool vec = p.vec != 0;
    const int S = p.S;
    const int seg = static_cast<int>(blockIdx.x % static_cast<unsigned>(S));
    const int q = static_cast<int>(blockIdx.x / static_cast<unsigned>(S));
    const int Q = static_cast<int>(gridDim.x / static_cast<unsigned>(S));
    const int64_t e0 = static_cast<int64_t>(seg) * kBwdSeg;
    const int Ns = static_cast<int>(p.N - e0 < kBwdSeg ? p.N - e0 : kBwdSeg);
    const uint32_t nb = static_cast<uint32_t>(Ns * SG::SB);
    float gf[HG ? V : 1];
    if constexpr (HG) SG::load(static_cast<const char*>(p.gamma) + e0 * SG::SB, nb, vec, t, gf);
    float adg[V], adb[LN ? V : 1];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        adg[k] = 0.f;
        if constexpr (LN) adb[k] = 0.f;
    }
    for (int64_t rr = q; rr < p.rows; rr += Q) {
        // last rows first: the statistics launch read them last, so they may still be in
        // the memory-side cache (LayerNorm fp32 1024 x 65537: 34.0% -> 35.1% of HBM peak,
        // RMSNorm bf16 512 x 131072: 36.0% -> 37.1%)
        const int64_t row = p.rows - 1 - rr;
        const int64_t off = (row * p.N + e0) * SG::SB;
        float xf[V], df[V];
        SG::load(static_cast<const char*>(p.x) + off, nb, vec, t, xf);
        SG::load(static_cast<const char*>(p.dy) + off, nb, vec, t, df);
        // the row's sums: lane k adds records k, k + 64, ... in order, then a butterfly
        // whose every step adds two equal operand pairs (a + b == b + a): same bits in every
        // lane and every workgroup of the row
        const float* rec = p.rec + 2 * row * S;
        float Sg = 0.f, Sgx = 0.f;
        for (int k = lane; k < S; k += 64) {
            Sg += rec[2 * k];
            Sgx += rec[2 * k + 1];
        }
#pragma unroll
        for (int step = 1; step < 64; step <<= 1) {
            Sg += __shfl_xor(Sg, step);
            Sgx += __shfl_xor(Sgx, step);
        }
        const float mean = LN ? p.mean[row] : 0.f;
        const float rstd = p.rstd[row];
        const float c1 = LN ? Sg * p.inv_n : 0.f;
        const float c2 = Sgx * p.inv_n;
        float r[V];
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const float xh = LN ? (xf[k] - mean) * rstd : xf[k] * rstd;
            const float g = HG ? df[k] * gf[k] : df[k];
            r[k] = rstd * ((g - c1) - xh * c2);
            adg[k] = fmaf(df[k], xh, adg[k]);
            if constexpr (LN) adb[k] += df[k];
        }
        if (p.dx) SG::store(static_cast<char*>(p.dx) + off, nb, vec, t, r);
    }
    if (p.ws == nullptr) return;  // uniform over the grid
    SG::store_f32(p.ws + static_cast<int64_t>(q) * p.N + e0, static_cast<uint32_t>(Ns), vec, t, adg);
    if constexpr (LN) SG::store_f32(p.ws + (static_cast<int64_t>(Q) + q) * p.N + e0, static_cast<uint32_t>(Ns), vec, t, adb);
}

// ---------------------------------------------------------------------------------------
// One-pass split rows: x and dy are read once. The rows are cut into P blocks of R rows; a
// ticket is one (block, segment) pair, ticket = block * S + segment. Workgroups take
// tickets from a counter in the workspace in increasing order. For each row of its block,
// the workgroup holding a ticket:
//   - reduces its segment's sum g and sum g * xhat and publishes them as two 64-bit words
//     (tag 1 in the upper half, the float's bits in the lower half; single-copy atomic, so a
//     reader sees either the cleared word or the whole value);
//   - issues the loads of its next row;
//   - waits (one wave, one lane per record) until all S records of the row carry the tag,
//     adds them in a fixed order (the same bits in every workgroup of the row), and writes
//     dx for its segment, accumulating its columns' dgamma / dbeta terms in registers;
// then writes its columns of partial row `block` ([2][P][N], as the column kernel reads).
// Progress does not depend on which workgroups are resident or how many: the wait for a
// record is bounded (p.wait_polls polls), and a record still missing after it is computed by
// the waiting workgroup itself, from that segment's x, dy and gamma, with the same lanes,
// element positions and reduction order as its owner uses, so the sums have the same bits
// whichever workgroup computes them (it also publishes them, which is harmless: the owner
// stores the same words). A workgroup therefore never waits on another to be scheduled,
// and no result depends on timing. The count of records computed this way is added to
// sync[1] (a diagnostic; it is zero when the segments of a row run side by side).
// The counter, the count and the records are zeroed by rownorm_bwd_wide_clear_kernel before
// each launch (a kernel, not a memset, so that the call can be captured in a graph).
// ---------------------------------------------------------------------------------------

template <int DT>  // one instance per dtype's translation unit
__global__ __launch_bounds__(256) void rownorm_bwd_wide_clear_kernel(u32x4* p, int64_t n16) {
    const u32x4 z{0u, 0u, 0u, 0u};
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n16;
         i += static_cast<int64_t>(gridDim.x) * 256)
        p[i] = z;
}

// One row's segment as loaded: 16-byte groups kept packed (VEC), or single elements.
template <int DT, bool VEC>
struct SegRaw {
    using IO = Io<DT>;
    static constexpr int V = kBwdSegPerLane;
    static constexpr int G = IO::E;  // elements per 16-byte group
    u32x4 v[VEC ? V / G : 1];
    float f[VEC ? 1 : V];

    template <int AUX = 0>
    __device__ __forceinline__ void load(const void* base, uint32_t nbytes, int t) {
        const Rsrc r = make_rsrc(base, nbytes);
        if constexpr (VEC) {
#pragma unroll
            for (int i = 0; i < V / G; ++i) v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, (i * kBwdSegLanes + t) * 16, 0, AUX);
        } else {
#pragma unroll
            for (int k = 0; k < V; ++k) f[k] = IO::template bload<AUX>(r, static_cast<uint32_t>(k * kBwdSegLanes + t));
        }
    }
    // element k of the lane: the same positions as BwdSeg's load / store / store_f32
    __device__ __forceinline__ float operator[](int k) const {
        if constexpr (VEC)
            return IO::elem(v[k / G], k % G);
        else
            return f[k];
    }
};

// One element's terms of a segment record: g = dy * gamma (or dy), g * xhat. The record's
// owner and a workgroup that computes it in its place both go through this, in the same
// element order, so the sums have the same bits.
template <bool LN, bool HG>
__device__ __forceinline__ void record_terms(float x, float d, float gm, float mean, float rstd, float& sg,
                                             float& sgx) {
    const float xh = LN ? (x - mean) * rstd : x * rstd;
    const float g = HG ? d * gm : d;
    sg += g;
    sgx = fmaf(g, xh, sgx);
}

template <int DT, int OP, bool HG, bool VEC>
__global__ __launch_bounds__(kBwdSegLanes) void rownorm_bwd_wide_onepass_kernel(BwdParams p) {
    using SG = BwdSeg<DT>;
    using RW = SegRaw<DT, VEC>;
    constexpr int V = SG::V;
    constexpr bool LN = OP == OP_LN;
    const int lane = threadIdx.x & 63;
    const int wr = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t = threadIdx.x;
    __shared__ WavePart part[2][kBwdSegLanes / 64];
    // per row, double-buffered by row parity: one barrier separates a row's reads from the
    // writes of the row after the next
    __shared__ float rowsum[2][2];  // [parity][sum g, sum g * xhat] of the whole row
    __shared__ int s_need[2];       // [parity] some record of the row is computed here
    __shared__ unsigned char s_miss[kBwdOnePassMaxSeg];  // records to compute here
    __shared__ float s_rec[2][kBwdOnePassMaxSeg];        // the row's records (sum g, sum g * xhat)
    __shared__ unsigned s_ticket;
    // the columns' dgamma (and dbeta) terms, slot k of lane t at [k][t]: each lane owns its
    // slots, so they need no barrier; in LDS, not VGPRs, so that two workgroups fit a CU
    __shared__ float acc_s[LN ? 2 : 1][V][kBwdSegLanes];
    constexpr int POLLER = kBwdSegLanes / 64 - 1;  // the wave that waits for the records
    constexpr int RPL = kBwdOnePassMaxSeg / 64;      // records per lane of that wave
    int buf = 0;
    const int S = p.S;
    const unsigned total = static_cast<unsigned>(p.parts) * static_cast<unsigned>(S);
    const int64_t rowbytes = p.N * SG::SB;
    for (;;) {
        if (t == 0) s_ticket = __hip_atomic_fetch_add(p.sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const unsigned ticket = s_ticket;  // read before the first barrier of the block's rows
        if (ticket >= total) break;        // uniform over the workgroup
        const int64_t blk = ticket / static_cast<unsigned>(S);
        const int seg = static_cast<int>(ticket % static_cast<unsigned>(S));
        const int64_t e0 = static_cast<int64_t>(seg) * kBwdSeg;
        const int Ns = static_cast<int>(p.N - e0 < kBwdSeg ? p.N - e0 : kBwdSeg);
        const uint32_t nb = static_cast<uint32_t>(Ns * SG::SB);
        const char* xb = static_cast<const char*>(p.x) + e0 * SG::SB;
        const char* db = static_cast<const char*>(p.dy) + e0 * SG::SB;
        RW gr;
        if constexpr (HG) gr.load(static_cast<const char*>(p.gamma) + e0 * SG::SB, nb, t);
#pragma unroll
        for (int k = 0; k < V; ++k) {
            acc_s[0][k][t] = 0.f;
            if constexpr (LN) acc_s[LN ? 1 : 0][k][t] = 0.f;
        }
        // the sums g and g * xhat of this workgroup's segment of one row, from registers;
        // every wave takes part (one barrier)
        auto seg_sums = [&](int64_t row, const RW& x, const RW& d, float& Sg, float& Sgx) {
            const float mean = LN ? p.mean[row] : 0.f;
            const float rstd = p.rstd[row];
            float sg = 0.f, sgx = 0.f;
#pragma unroll
            for (int k = 0; k < V; ++k) record_terms<LN, HG>(x[k], d[k], HG ? gr[k] : 1.f, mean, rstd, sg, sgx);
            Sg = wave_sum(sg);
            Sgx = wave_sum(sgx);
            group_sum2<kBwdSegLanes / 64>(part, buf, lane, wr, Sg, Sgx);
        };
        // the same sums for another segment s2 of the row, read from memory one 16-byte group
        // (or element) per tensor at a time: the lanes and element order of seg_sums, and few
        // registers, since the rows in flight stay live around it
        auto other_seg_sums = [&](int64_t row, int s2, float& Sg, float& Sgx) {
            const int64_t e2 = static_cast<int64_t>(s2) * kBwdSeg;
            const uint32_t nb2 = static_cast<uint32_t>((p.N - e2 < kBwdSeg ? p.N - e2 : kBwdSeg) * SG::SB);
            const Rsrc rx = make_rsrc(static_cast<const char*>(p.x) + (row * p.N + e2) * SG::SB, nb2);
            const Rsrc rd = make_rsrc(static_cast<const char*>(p.dy) + (row * p.N + e2) * SG::SB, nb2);
            const Rsrc rg = make_rsrc(HG ? static_cast<const char*>(p.gamma) + e2 * SG::SB : nullptr, HG ? nb2 : 0u);
            const float mean = LN ? p.mean[row] : 0.f;
            const float rstd = p.rstd[row];
            float sg = 0.f, sgx = 0.f;
            if constexpr (VEC) {
                using IO = Io<DT>;
#pragma unroll 1
                for (int i = 0; i < V / RW::G; ++i) {
                    const int off = (i * kBwdSegLanes + t) * 16;
                    const u32x4 xv = __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0);
                    const u32x4 dv = __builtin_amdgcn_raw_buffer_load_b128(rd, off, 0, 0);
                    u32x4 gv = u32x4{0u, 0u, 0u, 0u};
                    if constexpr (HG) gv = __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0);
#pragma unroll
                    for (int e = 0; e < RW::G; ++e)
                        record_terms<LN, HG>(IO::elem(xv, e), IO::elem(dv, e), HG ? IO::elem(gv, e) : 1.f, mean, rstd,
                                             sg, sgx);
                    asm volatile("" ::: "memory");  // one group per tensor in flight
                }
            } else {
                using IO = Io<DT>;
#pragma unroll 1
                for (int k = 0; k < V; ++k) {
                    const uint32_t j = static_cast<uint32_t>(k * kBwdSegLanes + t);
                    const float xk = IO::bload(rx, j), dk = IO::bload(rd, j);
                    const float gk = HG ? IO::bload(rg, j) : 1.f;
                    record_terms<LN, HG>(xk, dk, gk, mean, rstd, sg, sgx);
                    asm volatile("" ::: "memory");
                }
            }
            Sg = wave_sum(sg);
            Sgx = wave_sum(sgx);
            group_sum2<kBwdSegLanes / 64>(part, buf, lane, wr, Sg, Sgx);
        };
        auto publish = [&](int64_t row, int sgm, float Sg, float Sgx) {
            if (t == 0) {
                unsigned long long* rec = p.rec64 + 2 * (row * S + sgm);
                const unsigned long long tag = 1ull << 32;
                __hip_atomic_store(rec, tag | bit_cast<unsigned>(Sg), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(rec + 1, tag | bit_cast<unsigned>(Sgx), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        };
        // this workgroup's segment of one row, published as the row's record `seg`
        auto post = [&](int64_t row, const RW& x, const RW& d) {
            float Sg, Sgx;
            seg_sums(row, x, d, Sg, Sgx);
            publish(row, seg, Sg, Sgx);
        };
        const int64_t r0 = blk * p.R;
        const int64_t r1 = r0 + p.R < p.rows ? r0 + p.R : p.rows;
        // three rows in flight: row (sums posted, waiting), row + 1 (sums posted before the
        // wait for row), row + 2 (loads issued before that wait)
        RW cx, cd, nx, nd;
        cx.template load<kNonTemporal>(xb + r0 * rowbytes, nb, t);
        cd.template load<kNonTemporal>(db + r0 * rowbytes, nb, t);
        if (r0 + 1 < r1) {
            nx.template load<kNonTemporal>(xb + (r0 + 1) * rowbytes, nb, t);
            nd.template load<kNonTemporal>(db + (r0 + 1) * rowbytes, nb, t);
        }
        post(r0, cx, cd);
        for (int64_t row = r0; row < r1; ++row) {
            const int par = static_cast<int>(row & 1);
            RW mx, md;
            if (row + 2 < r1) {
                mx.template load<kNonTemporal>(xb + (row + 2) * rowbytes, nb, t);
                md.template load<kNonTemporal>(db + (row + 2) * rowbytes, nb, t);
            }
            if (row + 1 < r1) post(row + 1, nx, nd);
            // The last wave polls: not wave 0, whose lane 0 has just stored the record (vector
            // memory counts retire in order, so its poll would also wait for those stores;
            // LayerNorm bf16 1024 x 65536: 123.9 -> 120.5 us). Lane l holds records l, l + 64,
            // ...; they are added in that order, then a butterfly whose every step adds two
            // equal operand pairs: the same bits in every workgroup of the row.
            // The records go to LDS (s_rec), whoever computed them; the poller adds them from
            // there.
            unsigned miss = 0;
            auto finish = [&]() {
                float a = 0.f, b = 0.f;
#pragma unroll
                for (int j = 0; j < RPL; ++j) {
                    if (lane + 64 * j < S) {
                        a += s_rec[0][lane + 64 * j];
                        b += s_rec[1][lane + 64 * j];
                    }
                }
#pragma unroll
                for (int step = 1; step < 64; step <<= 1) {
                    a += __shfl_xor(a, step);
                    b += __shfl_xor(b, step);
                }
                if (lane == 0) {
                    rowsum[par][0] = a;
                    rowsum[par][1] = b;
                }
            };
            if (wr == POLLER) {
                const unsigned long long* rec = p.rec64 + 2 * row * S;
#pragma unroll
                for (int j = 0; j < RPL; ++j) {
                    const int k = lane + 64 * j;
                    if (k < S) {
                        bool got = false;
                        for (int n = 0;; ++n) {
                            const unsigned long long w0 = __hip_atomic_load(rec + 2 * k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            const unsigned long long w1 = __hip_atomic_load(rec + 2 * k + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            if ((w0 >> 32) != 0 && (w1 >> 32) != 0) {
                                s_rec[0][k] = bit_cast<float>(static_cast<unsigned>(w0));
                                s_rec[1][k] = bit_cast<float>(static_cast<unsigned>(w1));
                                got = true;
                                break;
                            }
                            if (n >= p.wait_polls) break;
                            __builtin_amdgcn_s_sleep(8);
                        }
                        if (!got) miss |= 1u << j;
                        s_miss[k] = got ? 0 : 1;
                    }
                }
                const bool any = __any(miss != 0);  // all 64 lanes active here
                if (!any) finish();
                if (lane == 0) s_need[par] = any ? 1 : 0;
            }
            __syncthreads();
            if (s_need[par] != 0) {  // uniform: compute the missing records here
                int computed = 0;
                for (int s2 = 0; s2 < S; ++s2) {
                    if (s_miss[s2] == 0) continue;  // uniform
                    float Sg, Sgx;
                    other_seg_sums(row, s2, Sg, Sgx);
                    publish(row, s2, Sg, Sgx);
                    if (t == 0) {
                        s_rec[0][s2] = Sg;
                        s_rec[1][s2] = Sgx;
                    }
                    ++computed;
                }
                __syncthreads();
                if (wr == POLLER) {
                    finish();
                    if (lane == 0)
                        __hip_atomic_fetch_add(p.sync + 1, static_cast<unsigned>(computed), __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                }
                __syncthreads();
            }
            const float c1 = LN ? rowsum[par][0] * p.inv_n : 0.f;
            const float c2 = rowsum[par][1] * p.inv_n;
            const float mean = LN ? p.mean[row] : 0.f;
            const float rstd = p.rstd[row];
            float r[V];
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float xh = LN ? (cx[k] - mean) * rstd : cx[k] * rstd;
                const float g = HG ? cd[k] * gr[k] : cd[k];
                r[k] = rstd * ((g - c1) - xh * c2);
                acc_s[0][k][t] = fmaf(cd[k], xh, acc_s[0][k][t]);
                if constexpr (LN) acc_s[LN ? 1 : 0][k][t] += cd[k];
            }
            if (p.dx) SG::template store<kNonTemporal>(static_cast<char*>(p.dx) + (row * p.N + e0) * SG::SB, nb, VEC, t, r);
            cx = nx;
            cd = nd;
            nx = mx;
            nd = md;
        }
        if (p.ws == nullptr) continue;  // uniform over the grid
        float adg[V], adb[LN ? V : 1];
#pragma unroll
        for (int k = 0; k < V; ++k) {
            adg[k] = acc_s[0][k][t];
            if constexpr (LN) adb[k] = acc_s[LN ? 1 : 0][k][t];
        }
        SG::store_f32(p.ws + blk * p.N + e0, static_cast<uint32_t>(Ns), VEC, t, adg);
        if constexpr (LN)
            SG::store_f32(p.ws + (static_cast<int64_t>(p.parts) + blk) * p.N + e0, static_cast<uint32_t>(Ns), VEC, t, adb);
    }
}

constexpr int rows_per_block_bwd(int W) { return W >= 16 ? 1 : 16 / W; }  // 16-wave workgroups

using BwdKernel = void (*)(BwdParams);

// The row-kernel instance for a backward plan: V_WORKGROUP (vectorized) or V_ELEMENT.
template <int DT, int OP>
inline BwdKernel select_bwd(const Plan& plan, bool hg) {
    const int W = plan.waves_per_row, V = plan.chunks_per_lane;
    if (plan.rows_per_block != rows_per_block_bwd(W)) return nullptr;
#define RN_BV(WW, VV, EX)                                                                        \
    (hg ? static_cast<BwdKernel>(rownorm_bwd_vec_kernel<DT, OP, WW, VV, rows_per_block_bwd(WW), EX, true>) \
        : static_cast<BwdKernel>(rownorm_bwd_vec_kernel<DT, OP, WW, VV, rows_per_block_bwd(WW), EX, false>))
#define RN_BV_E(WW, VV) (plan.exact ? RN_BV(WW, VV, true) : RN_BV(WW, VV, false))
#define RN_BE(WW, VV)                                                                             \
    (hg ? static_cast<BwdKernel>(rownorm_bwd_elem_kernel<DT, OP, WW, VV, rows_per_block_bwd(WW), true>) \
        : static_cast<BwdKernel>(rownorm_bwd_elem_kernel<DT, OP, WW, VV, rows_per_block_bwd(WW), false>))
    if (plan.variant == V_WORKGROUP) {
        switch (W * 100 + V) {
        case 101: return RN_BV_E(1, 1);
        case 102: return RN_BV_E(1, 2);
        case 202: return RN_BV_E(2, 2);
        case 402: return RN_BV_E(4, 2);
        case 802: return RN_BV_E(8, 2);
        case 1602: return RN_BV_E(16, 2);
        default: return nullptr;
        }
    }
    if (plan.variant == V_ELEMENT) {
        switch (W * 100 + V) {
        case 101: return RN_BE(1, 1);
        case 102: return RN_BE(1, 2);
        case 104: return RN_BE(1, 4);
        case 108: return RN_BE(1, 8);
        case 208: return RN_BE(2, 8);
        case 408: return RN_BE(4, 8);
        case 808: return RN_BE(8, 8);
        case 1608: return RN_BE(16, 8);
        case 1616: return RN_BE(16, 16);
        default: return nullptr;
        }
    }
#undef RN_BE
#undef RN_BV_E
#undef RN_BV
    return nullptr;
}

// Resident workgroups per CU of a backward row-kernel instance and the CU count, queried
// once per (instance, LDS size, device) and cached (the host may call from several threads).
inline hipError_t bwd_resident(BwdKernel k, int dev, const Plan& plan, int* per_cu, int* cus) {
    struct Key {
        BwdKernel k;
        int dev, lds;
        bool operator<(const Key& o) const {
            if (k != o.k) return reinterpret_cast<uintptr_t>(k) < reinterpret_cast<uintptr_t>(o.k);
            if (dev != o.dev) return dev < o.dev;
            return lds < o.lds;
        }
    };
    static std::mutex mu;
    static std::map<Key, std::pair<int, int>> cache;
    const Key key{k, dev, plan.lds_bytes};
    {
        std::lock_guard<std::mutex> g(mu);
        auto it = cache.find(key);
        if (it != cache.end()) {
            *per_cu = it->second.first;
            *cus = it->second.second;
            return hipSuccess;
        }
    }
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, reinterpret_cast<const void*>(k),
                                                                plan.block_threads,
                                                                static_cast<size_t>(plan.lds_bytes));
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (*per_cu < 1) *per_cu = 1;
    std::lock_guard<std::mutex> g(mu);
    cache[key] = {*per_cu, *cus};
    return hipSuccess;
}

// Row kernel, then column kernel. The row kernel's grid P is what the device keeps resident
// (compute units x workgroups per unit for this instance, queried once per instance and
// device), capped by the plan: more workgroups would only add partial rows to sum.
// Split rows, when the device keeps at least 2 S one-pass workgroups resident (and the rows
// are fp32 or whole 16-byte groups, with a 16-byte aligned workspace): clear launch,
// one-pass launch (P row blocks, P = what the device keeps resident / S, capped by the
// plan's workspace bound; grid = min(resident, P S) workgroups), column launch. Otherwise:
// statistics launch, dx launch (Q workgroups per segment, bounded the same way), column
// launch.
template <int DT>
inline hipError_t launch_bwd_wide(int op, const Plan& plan, const BwdParams& p0, const BwdColParams& cp0,
                                  hipStream_t s) {
    BwdParams p = p0;
    BwdColParams cp = cp0;
    const bool hg = p.gamma != nullptr;
    const bool ln = op == OP_LN;
#define RN_BW(KER) \
    (ln ? (hg ? KER<DT, OP_LN, true> : KER<DT, OP_LN, false>) : (hg ? KER<DT, OP_RMS, true> : KER<DT, OP_RMS, false>))
    const BwdKernel ks = RN_BW(rownorm_bwd_wide_stats_kernel);
    const BwdKernel kd = RN_BW(rownorm_bwd_wide_dx_kernel);
#undef RN_BW
#define RN_B1(VV)                                                                                                  \
    (ln ? (hg ? rownorm_bwd_wide_onepass_kernel<DT, OP_LN, true, VV> : rownorm_bwd_wide_onepass_kernel<DT, OP_LN, false, VV>) \
        : (hg ? rownorm_bwd_wide_onepass_kernel<DT, OP_RMS, true, VV> : rownorm_bwd_wide_onepass_kernel<DT, OP_RMS, false, VV>))
    // 16-bit rows that are not whole 16-byte groups take three launches (below): their
    // element-layout one-pass instances are not built
    BwdKernel k1 = nullptr;
    if constexpr (DT == DT_F32) {
        k1 = p.vec ? RN_B1(true) : RN_B1(false);
    } else {
        k1 = p.vec ? RN_B1(true) : nullptr;
    }
#undef RN_B1
    if (p.S < 1 || p.rec == nullptr) return hipErrorInvalidValue;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int per_cu = 0, cus = 0;
    void* argv[] = {&p};
    int64_t resident = 0;
    if (k1 != nullptr) {
        e = bwd_resident(k1, dev, plan, &per_cu, &cus);
        if (e != hipSuccess) return e;
        resident = static_cast<int64_t>(cus) * per_cu;
    }
    // 16-bit rows that are not whole 16-byte groups (two-byte loads, one workgroup per CU)
    // measured faster in three launches (bf16 1024 x 65537: 154 us against 192 us one-pass;
    // fp32 1024 x 65537: 274 against 240, bf16 1024 x 65536 in 16-byte groups: 143 against 116)
    const bool onepass_rows = p.vec != 0 || DT == DT_F32;
    if (onepass_rows && k1 != nullptr && p.sync != nullptr && p.rec64 != nullptr &&
        resident >= 2 * static_cast<int64_t>(p.S) && p.S <= kBwdOnePassMaxSeg) {
        int64_t P = resident / p.S;
        if (P > plan.grid) P = plan.grid;
        const int64_t R = (p.rows + P - 1) / P;
        P = (p.rows + R - 1) / R;
        const int64_t tickets = P * p.S;
        // counter, count of locally computed records, and the records: 256 + rows * S * 16
        // bytes from p.sync
        const int64_t n16 = (256 + p.rows * p.S * 16) / 16;
        int64_t gc = (n16 + 255) / 256;
        if (gc > 1024) gc = 1024;
        u32x4* clr = reinterpret_cast<u32x4*>(p.sync);
        void* zargv[] = {&clr, const_cast<int64_t*>(&n16)};
        e = hipLaunchKernel(reinterpret_cast<const void*>(rownorm_bwd_wide_clear_kernel<DT>), dim3(static_cast<unsigned>(gc)),
                            dim3(256), zargv, 0, s);
        if (e != hipSuccess) return e;
        p.parts = static_cast<int>(P);
        p.R = static_cast<int>(R);
        const int64_t g = resident < tickets ? resident : tickets;
        e = hipLaunchKernel(reinterpret_cast<const void*>(k1), dim3(static_cast<unsigned>(g)), dim3(kBwdSegLanes), argv,
                            0, s);
        if (e != hipSuccess) return e;
    } else {
        e = bwd_resident(kd, dev, plan, &per_cu, &cus);
        if (e != hipSuccess) return e;
        int64_t Q = static_cast<int64_t>(cus) * per_cu / p.S;
        if (Q < 1) Q = 1;
        if (Q > plan.grid) Q = plan.grid;
        const int64_t total = p.rows * p.S;
        const unsigned g1 = static_cast<unsigned>(total < kMaxGrid ? total : kMaxGrid);
        e = hipLaunchKernel(reinterpret_cast<const void*>(ks), dim3(g1), dim3(kBwdSegLanes), argv, 0, s);
        if (e != hipSuccess) return e;
        p.parts = static_cast<int>(Q);
        e = hipLaunchKernel(reinterpret_cast<const void*>(kd), dim3(static_cast<unsigned>(Q * p.S)),
                            dim3(kBwdSegLanes), argv, 0, s);
        if (e != hipSuccess) return e;
    }
    if (cp.dgamma == nullptr && cp.dbeta == nullptr) return hipSuccess;
    cp.parts = p.parts;
    void* cargv[] = {&cp};
    const unsigned blocks = static_cast<unsigned>((cp.N + 63) / 64);
    return hipLaunchKernel(reinterpret_cast<const void*>(rownorm_bwd_cols_kernel<DT>),
                           dim3(blocks, cp.dbeta != nullptr ? 2u : 1u), dim3(256), cargv, 0, s);
}

template <int DT>
inline hipError_t launch_bwd_dtype(int op, const Plan& plan, const BwdParams& p0, const BwdColParams& cp0,
                                   hipStream_t s) {
    if (plan.variant == V_WIDE && p0.rows > 0) return launch_bwd_wide<DT>(op, plan, p0, cp0, s);
    BwdParams p = p0;
    BwdColParams cp = cp0;
    if (p.rows > 0 && (p.dx != nullptr || p.ws != nullptr)) {
        const bool hg = p.gamma != nullptr;
        BwdKernel k = op == OP_LN ? select_bwd<DT, OP_LN>(plan, hg) : select_bwd<DT, OP_RMS>(plan, hg);
        if (k == nullptr) return hipErrorInvalidValue;
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        int per_cu = 0, cus = 0;
        e = bwd_resident(k, dev, plan, &per_cu, &cus);
        if (e != hipSuccess) return e;
        int64_t parts = static_cast<int64_t>(cus) * per_cu;
        if (parts > plan.grid) parts = plan.grid;
        p.parts = static_cast<int>(parts);
        cp.parts = p.parts;
        void* argv[] = {&p};
        e = hipLaunchKernel(reinterpret_cast<const void*>(k), dim3(static_cast<unsigned>(parts)),
                            dim3(static_cast<unsigned>(plan.block_threads)), argv,
                            static_cast<size_t>(plan.lds_bytes), s);
        if (e != hipSuccess) return e;
    } else {
        cp.parts = 0;
    }
    if (cp.dgamma == nullptr && cp.dbeta == nullptr) return hipSuccess;
    void* argv[] = {&cp};
    const unsigned blocks = static_cast<unsigned>((cp.N + 63) / 64);
    return hipLaunchKernel(reinterpret_cast<const void*>(rownorm_bwd_cols_kernel<DT>),
                           dim3(blocks, cp.dbeta != nullptr ? 2u : 1u), dim3(256), argv, 0, s);
}

}  // namespace rn
