/*
 * rownorm.h -- C ABI of the MI355X (gfx950) row-wise normalization library, librownorm.so.
 *
 * Forward operations over a row-major [rows, N] tensor, each row processed on its own:
 *
 *   ln_forward            LayerNorm. mean = (1/N) sum x_j, var = (1/N) sum (x_j - mean)^2
 *                         (biased), rstd = 1/sqrt(var + eps), y_j = (x_j - mean) * rstd *
 *                         gamma_j + beta_j. Defined in the LayerNorm CUDA walkthrough
 *                         (lpnh.cn/news/2756757), section 1; the same formula is section 2.1
 *                         of "LayerNorm vs RMSNorm in LLM inference engines"
 *                         (lpnh.cn/news/2853107) and section 2 of the "05 LLM Ops" lesson
 *                         (smarter.xin/posts/cb29461c).
 *   rms_norm              RMSNorm. rstd = 1/sqrt((1/N) sum x_j^2 + eps), y_j = x_j * rstd * w_j.
 *                         Defined in "CUDA fused RMSNorm kernel"
 *                         (diycv.top/archives/cuda-fused-rmsnorm-kernel), sections 0.3 and 2.
 *   fused_add_rms_norm    residual_out = x + residual, rounded once to the I/O dtype; then
 *                         RMSNorm of that rounded value, which is also what gets squared.
 *                         Same article, sections 2 and 3.2.
 *   fused_add_layer_norm  the same residual add, then LayerNorm of the rounded value (the
 *                         pre-norm residual path of the same article, section 2, with the
 *                         walkthrough's LayerNorm).
 *   softmax_forward       y_j = exp(x_j - m) / sum_k exp(x_k - m), m = max_k x_k ("05 LLM Ops"
 *                         lesson, section 1 "Softmax"; the per-part (max, sum) pairs are
 *                         merged with the rescaling of its "Online Softmax" sections).
 *                         Entries of -inf (masked logits) give exactly 0; a row with no
 *                         entry above -inf gives NaN outputs, row max -inf and row sum 0.
 *
 * and the backward passes of LayerNorm and RMSNorm (ln_backward, rms_norm_backward).
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers (HIP device memory of the current device). x, residual,
 *     gamma / beta / weight, y and residual_out hold `dtype` elements; mean and rstd (softmax:
 *     row_max and row_sum) are fp32. Rows are dense (stride N elements) except through
 *     rn_forward_ex, which takes a row stride per [rows, N] tensor. gamma / beta / weight
 *     have N elements.
 *   - Arithmetic is fp32 for every dtype: fp16 / bf16 inputs are widened exactly, outputs
 *     are rounded once (round-to-nearest-even) to `dtype`.
 *   - The caller owns every buffer. The library never allocates, frees or synchronizes;
 *     work is enqueued on `stream` (0 = the null stream) and results are valid once the
 *     caller has synchronized that stream. The library keeps no per-call state (it only
 *     caches, per device, the occupancy of each kernel configuration it has launched) and may
 *     be called from several host threads at once.
 *   - Errors are reported by the return value (an rn_status). Argument errors are detected
 *     on the host before anything is enqueued, so an error leaves every output untouched.
 *   - rows == 0 is a successful no-op.
 *   - Aliasing: an output may be the exact same buffer as an input of the same shape and
 *     row stride (in place: y == x, residual_out == residual, residual_out == x,
 *     y == residual). Any other overlap between an output and any other buffer is
 *     RN_ERR_ALIAS (also when strided rows would interleave without touching: the check is
 *     on address ranges).
 *   - Every pointer must be aligned to its element size (RN_ERR_ALIGN otherwise). When N *
 *     sizeof(dtype) and every row stride in bytes are multiples of 16 and every [rows, N] /
 *     [N] pointer is 16-byte aligned, the vectorized kernels run: a row is held in registers
 *     by one 64-lane wavefront (rows of up to 4 KiB, or 16 KiB when forced) or by a group of
 *     up to 16 wavefronts (rows of up to 64 KiB: 16384 fp32 or 32768 fp16 / bf16 elements;
 *     softmax and RMSNorm rows of up to 128 KiB, and LayerNorm and fused add + RMSNorm rows
 *     of up to 128 KiB when no workspace is given). A row group of 2^k wavefronts holds
 *     16-byte chunks per lane in a power of two, or an odd number from 3 to 15 when that holds
 *     the row exactly (rows of 64 * 2^k * 3, 5, ..., 15 chunks, at least 256 row blocks).
 *     Other rows of up to 64 KiB (not whole chunks, or tensors / strides only element-
 *     aligned), when there are at least 256 row blocks, run the same vectorized kernel with
 *     rows addressed by byte: 16-byte accesses at element alignment through a buffer
 *     resource that ends with the row, the row's partial last chunk by its whole 4-byte
 *     words, and the last element of an odd-length 16-bit row by one 2-byte access; rows of
 *     whole chunks that do not fill their group of wavefronts exactly take it too (16-bit
 *     rows at odd 2-byte positions of the fused ops from 4 wavefronts per row and of
 *     RMSNorm from 8 keep the element / pair kernels, which measure faster there). Softmax
 *     rows of such kinds beyond 64 KiB, up to 256 KiB fp32 / 128 KiB 16-bit, are addressed
 *     by byte on one 16-wavefront workgroup per row, any number of rows.
 *     Otherwise rows of up to 16384 elements are held in registers one element per slot
 *     (the element kernel, still one read of x; 16-bit rows whose tensors share their
 *     position within 4-byte words move as element pairs). Longer rows take the split-row
 *     kernels (16-byte chunks, rows addressed by byte when they are not whole chunks; 16-bit
 *     rows at odd 2-byte positions and in-place calls: elements) when rn_forward_ex is given
 *     a workspace; without one (and beyond the 128 KiB rows above) they take a general
 *     kernel that reads the row up to three times.
 *   - Launches use the current HIP device (the device of the buffers and of `stream`). The
 *     first call of a kernel configuration on a device queries its occupancy once.
 */
#ifndef ROWNORM_H
#define ROWNORM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden symbol visibility; the entry points declared here are
 * the only symbols it exports. */
#pragma GCC visibility push(default)

/* I/O element type. */
typedef enum rn_dtype { RN_F32 = 0, RN_F16 = 1, RN_BF16 = 2 } rn_dtype;

/* Status codes returned by every entry point. */
typedef enum rn_status {
    RN_OK = 0,
    RN_ERR_NULL = 1,          /* a required pointer is NULL */
    RN_ERR_SHAPE = 2,         /* rows < 0, N <= 0, rows * N overflows, or eps < 0 / not finite */
    RN_ERR_DTYPE = 3,         /* dtype is not an rn_dtype */
    RN_ERR_ALIAS = 4,         /* an output overlaps another buffer other than by exact aliasing */
    RN_ERR_UNSUPPORTED = 5,   /* a forced kernel variant cannot run this shape / alignment */
    RN_ERR_HIP = 6,           /* the HIP runtime reported an error at launch */
    RN_ERR_ALIGN = 7,         /* a pointer is not aligned to its element size */
    RN_ERR_WORKSPACE = 8,     /* a required workspace is missing or smaller than
                                 rn_backward_workspace_bytes() / rn_forward_workspace_bytes() */
    RN_ERR_SCRATCH = 9        /* rn_forward_noalloc: the shape needs more scratch than the
                                 library's static array holds (RN_NOALLOC_SCRATCH_BYTES) */
} rn_status;

/* Kernel variants (for rn_*_variant entry points and rn_plan). */
typedef enum rn_variant {
    RN_VARIANT_AUTO = 0,      /* choose from N, dtype, alignment and rows (what the plain entry points do) */
    RN_VARIANT_WAVE = 1,      /* one 64-lane wavefront per row, row held in VGPRs (rows up to 16 KiB) */
    RN_VARIANT_WORKGROUP = 2, /* 2-16 wavefronts per row, partial moments combined in LDS (rows up to 64 KiB;
                                 softmax, RMSNorm and LayerNorm up to 128 KiB, fused add + RMSNorm
                                 too when no workspace is given) */
    RN_VARIANT_GENERAL = 3,   /* any N, any element-aligned pointers; re-reads the row */
    RN_VARIANT_ELEMENT = 4,   /* rows up to 16384 elements held in VGPRs one element per slot;
                                 any element-aligned pointers and strides */
    RN_VARIANT_WIDE = 5,      /* rows longer than RN_VARIANT_WORKGROUP holds: split into 32 KiB
                                 segments, one workgroup each, that exchange statistics through
                                 the workspace; x is read once (two launches, x read twice, for
                                 in-place calls or a workspace of only the two-launch size).
                                 Rows of whole 16-byte chunks; under RN_VARIANT_AUTO also other
                                 long rows (byte-addressed segments of ceil(C / S) chunks, C the
                                 row's chunks rounded up, S the segments of 32 KiB), out of
                                 place with a one-pass workspace, except 16-bit rows at odd
                                 2-byte positions; needs a workspace (rn_forward_ex) */
    RN_VARIANT_WIDE_ELEMENT = 6 /* rows of more than 16384 elements with any element-aligned
                                 pointers and strides: split into segments of 8192 elements (one
                                 per register slot), one workgroup each, in two launches; needs a
                                 workspace (rn_forward_ex) */
} rn_variant;

/* Operation codes (for rn_forward_ex and rn_plan). */
typedef enum rn_op {
    RN_OP_LAYER_NORM = 0,
    RN_OP_RMS_NORM = 1,
    RN_OP_FUSED_ADD_RMS_NORM = 2,
    RN_OP_FUSED_ADD_LAYER_NORM = 3,
    RN_OP_SOFTMAX = 4
} rn_op;

/* Row strides in elements of the [rows, N] tensors (row r starts at base + r * stride).
 * 0 means dense (N). A non-zero stride must be >= N. Unused entries are ignored. */
typedef struct rn_row_strides {
    int64_t x, residual, y, residual_out;
} rn_row_strides;

/*
 * LayerNorm forward.
 *   x      [rows, N] dtype, required.
 *   gamma  [N] dtype, nullable (NULL means 1).   beta [N] dtype, nullable (NULL means 0).
 *   y      [rows, N] dtype, required; may be x itself.
 *   mean   [rows] fp32, nullable: the row mean.  rstd [rows] fp32, nullable: 1/sqrt(var + eps).
 *   eps    >= 0, added to the variance inside the square root.
 */
int ln_forward(const void* x, const void* gamma, const void* beta, void* y, float* mean, float* rstd,
               int64_t rows, int64_t N, float eps, int dtype, hipStream_t stream);

/*
 * RMSNorm forward.
 *   x [rows, N] dtype, required.  weight [N] dtype, nullable (NULL means 1).
 *   y [rows, N] dtype, required; may be x itself.  rstd [rows] fp32, nullable:
 *   1/sqrt(mean(x^2) + eps).
 */
int rms_norm(const void* x, const void* weight, void* y, float* rstd, int64_t rows, int64_t N, float eps,
             int dtype, hipStream_t stream);

/*
 * Fused residual add + RMSNorm.
 *   x, residual [rows, N] dtype, required.  weight [N] dtype, nullable (NULL means 1).
 *   residual_out [rows, N] dtype, required: x + residual rounded to dtype (may be x or
 *   residual itself).  y [rows, N] dtype, required: RMSNorm(residual_out) * weight (may be
 *   x or residual itself, but not residual_out).  rstd [rows] fp32, nullable: the rstd of
 *   residual_out's row.
 */
int fused_add_rms_norm(const void* x, const void* residual, const void* weight, void* y, void* residual_out,
                       float* rstd, int64_t rows, int64_t N, float eps, int dtype, hipStream_t stream);

/*
 * Fused residual add + LayerNorm.
 *   x, residual [rows, N] dtype, required.  gamma, beta [N] dtype, nullable (1 and 0).
 *   residual_out [rows, N] dtype, required: x + residual rounded to dtype (may be x or
 *   residual itself).  y [rows, N] dtype, required: LayerNorm(residual_out) (may be x or
 *   residual itself, but not residual_out).  mean, rstd [rows] fp32, nullable: the
 *   statistics of residual_out's row.
 */
int fused_add_layer_norm(const void* x, const void* residual, const void* gamma, const void* beta, void* y,
                         void* residual_out, float* mean, float* rstd, int64_t rows, int64_t N, float eps,
                         int dtype, hipStream_t stream);

/*
 * Row-wise softmax.
 *   x [rows, N] dtype, required.  y [rows, N] dtype, required; may be x itself.
 *   row_max [rows] fp32, nullable: max_j x_j.  row_sum [rows] fp32, nullable:
 *   sum_j exp(x_j - row_max) (so log-sum-exp = row_max + log(row_sum)).
 *   Rows are expected to hold finite values.
 */
int softmax_forward(const void* x, void* y, float* row_max, float* row_sum, int64_t rows, int64_t N, int dtype,
                    hipStream_t stream);

/*
 * Any forward operation with explicit row strides, kernel variant and workspace.
 *   op         an rn_op; arguments the operation does not use are ignored (softmax: gamma,
 *              beta, residual, residual_out, eps; mean / rstd are row_max / row_sum).
 *   strides    nullable (all rows dense); see rn_row_strides.
 *   variant    an rn_variant; RN_VARIANT_AUTO chooses as the plain entry points do, except
 *              that rows too long for one workgroup's registers take RN_VARIANT_WIDE (whole
 *              16-byte chunks; other rows of more than 16384 elements when the workspace has
 *              the one-pass size, the call is out of place and, for 16-bit rows, no row
 *              tensor or stride sits at an odd 2-byte position) or RN_VARIANT_WIDE_ELEMENT
 *              (the remaining rows of more than 16384 elements) when a large enough
 *              workspace is given. A forced variant that cannot
 *              run the shape / alignment returns RN_ERR_UNSUPPORTED (the split-row variants
 *              without a large enough workspace: RN_ERR_WORKSPACE).
 *   workspace  nullable device memory of workspace_bytes, 16-byte aligned, owned by the
 *              caller, overlapping no other argument: per-segment statistics of the split-row
 *              path (rn_forward_workspace_bytes). Contents on entry do not matter; calls that
 *              share it must be ordered (same stream).
 * Unknown op codes return RN_ERR_SHAPE.
 *
 * Split rows (walkthrough section 1.1: a row that outgrows one block). Rows with up to 256
 * segments (whole 16-byte chunks, or under RN_VARIANT_AUTO the byte-addressed rows named at
 * RN_VARIANT_WIDE), called out of place with a workspace of
 * rn_forward_workspace_bytes, take one pass that reads x (and the residual) once: a small
 * kernel first clears a 256-byte header (a ticket counter; at byte offset 4 a 32-bit count of
 * records computed by waiting workgroups, left there as a diagnostic) and the records; the
 * workgroups then take (row block, segment) tickets in order, publish each segment's
 * statistics record as tagged 64-bit words, wait a bounded time for the row's other records
 * and compute any still missing themselves from the inputs, with the same bits, so the result
 * never depends on which workgroups run at the same time. The environment variable
 * RN_FWD_WAIT_POLLS (a non-negative integer, read at every call) sets the wait; 0 waits for
 * nothing and computes every record of a row in each of its workgroups. In-place calls (y == x, residual_out == residual, ...), rows
 * of more than 256 segments, and a workspace of only the two-launch size (rows * ceil(N /
 * 8192) * 16 bytes) take two launches: records, then normalization, which reads x (for the
 * fused ops: residual_out) a second time. Both forms give the same bits. Softmax, RMSNorm
 * and LayerNorm rows of whole chunks up to 128 KiB (fp32 softmax: 256 KiB) never split: one
 * 16-wave workgroup holds them. Without a workspace, fused add + RMSNorm rows of whole chunks
 * up to 128 KiB take one 16-wave workgroup too; other such rows take the general kernel.
 */
int rn_forward_ex(int op, const void* x, const void* residual, const void* gamma, const void* beta, void* y,
                  void* residual_out, float* mean, float* rstd, int64_t rows, int64_t N, float eps, int dtype,
                  const rn_row_strides* strides, int variant, void* workspace, size_t workspace_bytes,
                  hipStream_t stream);

/*
 * rn_forward_ex without a workspace argument and without any allocation, for callers that
 * cannot allocate device memory (work being captured into a HIP graph, serving loops that
 * must not call hipMalloc, harnesses that forbid it). Arguments, results and errors are
 * those of rn_forward_ex with variant RN_VARIANT_AUTO; the split-row workspace, when the
 * shape needs one (rn_forward_workspace_bytes > 0), is a static device array of the library,
 * RN_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, held from the library's first use on that GPU
 * until the process ends. A shape that needs more returns RN_ERR_SCRATCH before anything is
 * enqueued. The call itself allocates nothing and calls no allocating routine.
 * Every call on one GPU shares that GPU's array: calls that may run at the same time on one
 * GPU (different streams, or different host threads without ordering) race on it and must
 * not both take the split-row path; calls ordered on one stream are safe. Nothing is left in
 * the array that a later call depends on.
 */
#define RN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int rn_forward_noalloc(int op, const void* x, const void* residual, const void* gamma, const void* beta, void* y,
                       void* residual_out, float* mean, float* rstd, int64_t rows, int64_t N, float eps, int dtype,
                       const rn_row_strides* strides, hipStream_t stream);

/*
 * Launch choices that replace the planner's own (rn_forward_tuned, rn_plan_tuned): for
 * measuring the automatic plan against its alternatives on a given device, and for
 * autotuning. A field at its "automatic" value (0, or -1 where stated) changes nothing. They
 * apply to the vectorized variants (RN_VARIANT_WAVE / RN_VARIANT_WORKGROUP, or
 * RN_VARIANT_AUTO where it picks one of them); a tuning that changes anything for another
 * variant returns RN_ERR_UNSUPPORTED.
 */
typedef struct rn_tuning {
    int waves_per_row;    /* 1, 2, 4, 8 or 16 wavefronts per row (0: automatic); rows per workgroup
                             follow (4 / waves_per_row up to 4 waves, else 1) */
    int chunks_per_lane;  /* 16-byte chunks each lane holds, 64 * waves_per_row * chunks_per_lane
                             covering the row (0: the fewest power of two that covers it, or an
                             odd number from 3 to 15 when that many hold the row exactly and the
                             launch can be persistent); the odd counts are built for exact
                             persistent launches only */
    int persistent;       /* 1: persistent launch (rows that exactly fill the row group, up to 4096
                             chunks), 0: one workgroup per row block, -1: automatic */
    int prefetch;         /* persistent launches: 1 the instance that loads a workgroup's next row
                             before it reduces the current one, 0 the one that does not, -1: the
                             grid rule's choice. Rows of 16 waves, and one-wave rows of 8 or more
                             chunks per lane, have only the second; of the other shapes only rows
                             of 4 or more waves with parameters have both */
    int64_t grid_blocks;  /* workgroups to launch (at most one per row block; each loops over the
                             row blocks left), 0: automatic */
} rn_tuning;

/*
 * rn_forward_ex with a tuning (nullable: then exactly rn_forward_ex). Results are those of
 * rn_forward_ex, bit for bit, when only persistent, prefetch or grid_blocks change; another
 * row-group shape changes the order of the fp32 partial sums, not the tolerance the results
 * meet. RN_ERR_UNSUPPORTED when the library holds no kernel for the resulting shape (nothing
 * is enqueued then), or for a tuning outside the ranges above.
 */
int rn_forward_tuned(int op, const void* x, const void* residual, const void* gamma, const void* beta, void* y,
                     void* residual_out, float* mean, float* rstd, int64_t rows, int64_t N, float eps, int dtype,
                     const rn_row_strides* strides, int variant, const rn_tuning* tuning, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes rn_forward_ex needs for the split-row paths of this shape, 0 when N <= 16384
 * (such rows are never split). Otherwise the larger of the two-launch layout, rows *
 * ceil(N / 8192) * 16 bytes (16-byte records), and the one-pass layout, 256 + rows *
 * ceil(N * element_bytes / 32768) * 32 bytes (a header, then four 64-bit words per record):
 * enough for either split-row variant, whatever the alignment. */
size_t rn_forward_workspace_bytes(int op, int64_t rows, int64_t N, int dtype);

/* Same as the first three entry points above, with the kernel variant forced (RN_VARIANT_AUTO
 * behaves exactly like the plain entry point). A forced variant that cannot run the given
 * shape / alignment returns RN_ERR_UNSUPPORTED before anything is enqueued. Used by tests
 * to reach every kernel and by benchmarks to compare them. */
int ln_forward_variant(const void* x, const void* gamma, const void* beta, void* y, float* mean, float* rstd,
                       int64_t rows, int64_t N, float eps, int dtype, hipStream_t stream, int variant);
int rms_norm_variant(const void* x, const void* weight, void* y, float* rstd, int64_t rows, int64_t N, float eps,
                     int dtype, hipStream_t stream, int variant);
int fused_add_rms_norm_variant(const void* x, const void* residual, const void* weight, void* y,
                               void* residual_out, float* rstd, int64_t rows, int64_t N, float eps, int dtype,
                               hipStream_t stream, int variant);

/*
 * Backward passes. With xhat_j = (x_j - mean) * rstd (RMSNorm: x_j * rstd) and g_j = dy_j *
 * gamma_j, for each row
 *   dx_j = rstd * (g_j - (1/N) sum_k g_k - xhat_j * (1/N) sum_k g_k xhat_k)
 * (RMSNorm: without the (1/N) sum_k g_k term), and over all rows dgamma_j = sum_r dy_rj *
 * xhat_rj, dbeta_j = sum_r dy_rj: the normalization gradient of "BatchNorm CUDA
 * implementation" (jianying88.com/news/30214), section 3.1, with the reduction along the
 * row (gamma varies along the row, so it sits inside the row sums).
 *   dy, x        [rows, N] dtype (dense), required when rows > 0.
 *   gamma        [N] dtype, nullable (1).
 *   mean, rstd   [rows] fp32: the forward's statistics (ln_forward / rms_norm outputs), used
 *                as given; required when rows > 0 (RMSNorm: rstd only).
 *   dx           [rows, N] dtype, nullable (then only parameter gradients are computed); may
 *                be dy or x itself.
 *   dgamma, dbeta (RMSNorm: dweight)  [N] dtype, nullable; rows == 0 writes zeros.
 *   workspace    device memory of at least rn_backward_workspace_bytes(op, rows, N) bytes,
 *                4-byte aligned (16-byte alignment is faster), owned by the caller;
 *                required when a parameter gradient is requested or when rows are longer
 *                than 16384 elements (RN_ERR_WORKSPACE otherwise). Its contents on entry
 *                do not matter; on return they are unspecified. Calls that share a
 *                workspace must be ordered (same stream).
 * Rows of up to 16384 elements are held by one row group. Longer rows (any N) are split
 * into 8192-element segments (plan variant RN_VARIANT_WIDE). For fp32 rows and rows of
 * whole 16-byte groups, with a 16-byte aligned workspace and up to (workgroups the device
 * keeps resident) / 2 segments per row (at most 256), x and dy are read once: a small launch
 * clears a ticket counter and the segment records in the workspace, then workgroups take
 * (row block, segment) tickets in order (an integer atomic counter), publish each row's
 * per-segment sums of g and g * xhat in the workspace (64-bit atomic stores of tagged
 * words), wait for the row's other segments and write dx; the column sums follow. The wait
 * never fails and never depends on other workgroups being scheduled: after a bounded number
 * of polls (4096, about 5-10 ms; the environment variable RN_BWD_WAIT_POLLS, read at every
 * call, overrides it) the waiting workgroup computes a missing segment's sums itself, from
 * that segment's x, dy and gamma, with the same lanes and order as the segment's own
 * workgroup, so the result has the same bits either way. The number of records computed
 * that way is left in the workspace as a diagnostic: the 32-bit word at byte offset
 * rn_backward_workspace_bytes(op, rows, N) - 16 * rows * S - 252, S = ceil(N / 8192)
 * segments per row (zero when the segments of each row run side by side). Otherwise three
 * launches: per-segment sums into the workspace, dx with the parameter-gradient columns,
 * column sums (x and dy read twice).
 * Row and column sums are formed in fp32 in a fixed order; no floating-point value is ever
 * accumulated with an atomic, so results are bitwise reproducible on a given device.
 */
size_t rn_backward_workspace_bytes(int op, int64_t rows, int64_t N);
int ln_backward(const void* dy, const void* x, const void* gamma, const float* mean, const float* rstd, void* dx,
                void* dgamma, void* dbeta, int64_t rows, int64_t N, int dtype, void* workspace,
                size_t workspace_bytes, hipStream_t stream);
int rms_norm_backward(const void* dy, const void* x, const void* weight, const float* rstd, void* dx,
                      void* dweight, int64_t rows, int64_t N, int dtype, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Launch plan chosen for a call, computed on the host only (no HIP call is made), with the
 * same validation as the entry points. Pointers are only inspected for NULL, alignment and
 * overlap, never dereferenced. */
typedef struct rn_plan_info {
    int variant;           /* rn_variant actually used */
    int waves_per_row;     /* wavefronts cooperating on one row (split-row variant: on one segment) */
    int rows_per_block;    /* rows one workgroup processes per iteration */
    int block_threads;     /* workgroup size */
    int chunks_per_lane;   /* 16-byte chunks (vectorized variants: 1, 2, 4, 8, 16, or an odd number from
                              3 to 15 for rows of 64 * waves_per_row * that many chunks, persistent) or
                              elements (element variant) each lane holds */
    int64_t grid_blocks;   /* workgroups launched (persistent launches: an upper bound; the launch
                              caps it at what the current device keeps resident) */
    int exact;             /* 1 if a row is exactly chunks_per_lane passes of its row group */
    int persistent;        /* 1 if the grid is sized to what the device keeps resident and the
                              workgroups loop over many rows, with the parameters loaded on chip
                              once per workgroup */
    int lds_bytes;         /* dynamic LDS per workgroup of a persistent launch */
    int pairs;             /* element variant: 1 if each lane slot holds two adjacent 16-bit
                              elements moved as one 4-byte word (chunks_per_lane then counts
                              such slots) */
    int ragged;            /* vectorized variants: 1 if rows are addressed by byte (persistent
                              launches of many rows whose rows, row strides or tensors are not
                              whole 16-byte chunks, or whose rows do not fill the row group
                              exactly): 16-byte accesses at element alignment, the row's partial
                              last chunk moved by its whole dwords and, for an odd-length 16-bit
                              row, one 2-byte access; chunks_per_lane counts 16-byte chunks, the
                              last one partial, and exact is 1 when they fill the row group */
} rn_plan_info;

int rn_plan(int op, const void* x, const void* residual, const void* gamma, const void* beta, const void* y,
            const void* residual_out, const void* mean, const void* rstd, int64_t rows, int64_t N, float eps,
            int dtype, int variant, const rn_row_strides* strides, const void* workspace, size_t workspace_bytes,
            rn_plan_info* out);

/* rn_plan with a tuning (see rn_tuning), also host only: the plan rn_forward_tuned would launch
 * (grid_blocks: the tuning's grid when it sets one), and RN_ERR_UNSUPPORTED when the library
 * holds no kernel of that shape. */
int rn_plan_tuned(int op, const void* x, const void* residual, const void* gamma, const void* beta, const void* y,
                  const void* residual_out, const void* mean, const void* rstd, int64_t rows, int64_t N, float eps,
                  int dtype, int variant, const rn_row_strides* strides, const rn_tuning* tuning,
                  const void* workspace, size_t workspace_bytes, rn_plan_info* out);

/* The same for a backward call (op: RN_OP_LAYER_NORM or RN_OP_RMS_NORM); grid_blocks is the
 * row kernel's workgroup count before the launch caps it at what the device keeps resident
 * (split rows, RN_VARIANT_WIDE: the workgroups per segment at most; exact: 1 when rows move
 * in 16-byte groups). */
int rn_plan_backward(int op, const void* dy, const void* x, const void* gamma, const float* mean, const float* rstd,
                     const void* dx, const void* dgamma, const void* dbeta, int64_t rows, int64_t N, int dtype,
                     const void* workspace, size_t workspace_bytes, rn_plan_info* out);

/* Static string naming a status code ("RN_OK", ...); "unknown status" otherwise. */
const char* rn_status_string(int status);

/* Library version as major * 10000 + minor * 100 + patch. */
int rn_version(void);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif

#endif /* ROWNORM_H */
