/*
 * rownorm_oracle.c -- plain, slow, obviously correct fp64 CPU reference for row-wise
 * LayerNorm, RMSNorm, fused residual-add + RMSNorm / + LayerNorm, softmax, and the
 * backward passes of LayerNorm and RMSNorm.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library. The GPU product path never calls it, links it or shares
 * code with it: no headers, helpers, tables or constants are common to the two.
 *
 * Every quantity is computed in IEEE double precision, sequentially, row by row, in the
 * order the definitions state. Inputs arrive as raw I/O-dtype bit patterns (fp32, fp16
 * or bf16) and are decoded exactly; outputs are fp64 (y, mean, rstd) plus, for the fused
 * op, the residual stream rounded once to the I/O dtype.
 *
 * Sources (pages' titles and sections; see the function comments for which step follows
 * which passage):
 *   [WALK]  "LayerNorm CUDA walkthrough" (lpnh.cn/news/2756757): section 1 (definition of
 *           mean, biased variance, y), section 6 (two-pass or Welford for stability),
 *           section 2 / 7 (gamma and beta optional).
 *   [OPS]   "05 LLM Ops" lesson (smarter.xin/posts/cb29461c): section 2 LayerNorm and the
 *           "Welford recurrence" paragraph (delta, mean and M2 updates, var = M2/n);
 *           section 3 RMSNorm formula.
 *   [FUSED] "CUDA fused RMSNorm kernel" (diycv.top/archives/cuda-fused-rmsnorm-kernel):
 *           section 0.3 (RMSNorm = x / sqrt(mean(x^2) + eps), residual_out = x + residual),
 *           section 3.2 (fp32 accumulation; the sum x + residual is first rounded to the
 *           I/O dtype and the rounded value is the one squared and returned).
 *   [LLM]   "LayerNorm vs RMSNorm in LLM inference engines" (lpnh.cn/news/2853107),
 *           section 2.1 (y = gamma * (x - mean) / sqrt(var + eps) + beta;
 *           y = gamma * x / sqrt(mean(x^2) + eps)).
 *   [SMAX]  the same "05 LLM Ops" lesson, section 1 "Softmax" (softmax(x_i) =
 *           exp(x_i - m) / sum_j exp(x_j - m), m = max x) and "Online Softmax denominator
 *           correction" (running max and denominator, rescaled by exp(m_old - m_new)).
 *   [BN]    "BatchNorm CUDA implementation" (jianying88.com/news/30214), section 3.1:
 *           gradients of a normalization by the chain rule (d xhat = dy * gamma, then
 *           through the mean and the variance), dbeta = sum dy, dgamma = sum dy * xhat.
 *
 * Readings where the pages are silent (each is also listed in the design notes):
 *   - variance is the biased 1/N form; eps is added inside the square root;
 *   - rstd = 1 / sqrt(var + eps) for LayerNorm and 1 / sqrt(mean(x^2) + eps) for RMSNorm;
 *   - a null gamma / weight means 1, a null beta means 0;
 *   - rounding to fp16 / bf16 / fp32 is IEEE round-to-nearest, ties to even, with
 *     overflow to infinity (the pages do not name a rounding mode).
 *
 * Pins: tests/test_oracle.py checks this file against exact rational arithmetic on tiny
 * rows, torch's CPU float64 layer_norm / rms_norm, closed forms for N = 1 and N = 2, the
 * invariants of the definitions, and (for the codec) every fp16 / bf16 bit pattern;
 * softmax against 50-digit decimal arithmetic, scipy's float64 softmax and the logistic
 * closed form; the backward passes against central differences of this file's own fp64
 * forward rows, torch's float64 autograd, and the orthogonality invariants of dx.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* I/O dtype codes of this library (defined here, independently of the product). */
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

/* Error codes. */
enum { ORC_OK = 0, ORC_EARG = 1, ORC_EWELFORD = 2, ORC_ENOMEM = 3, ORC_EONLINE = 4 };

/* ---------------------------------------------------------------------------------- */
/* IEEE binary formats, from their definition: 1 sign bit, `e` exponent bits with bias */
/* 2^(e-1) - 1, `m` stored fraction bits; all-ones exponent encodes inf / NaN; zero    */
/* exponent encodes zero and subnormals with quantum 2^(1 - bias - m).                 */
/* ---------------------------------------------------------------------------------- */

static int fmt_bits(int dtype, int* m, int* e) {
    switch (dtype) {
    case ORC_F32: *m = 23; *e = 8; return 0;
    case ORC_F16: *m = 10; *e = 5; return 0;
    case ORC_BF16: *m = 7; *e = 8; return 0;
    default: return -1;
    }
}

static int dtype_size(int dtype) { return dtype == ORC_F32 ? 4 : 2; }

/* Exact value of a bit pattern. */
double orc_decode(int dtype, uint32_t bits) {
    int m, e;
    if (fmt_bits(dtype, &m, &e)) return NAN;
    const uint32_t emask = (1u << e) - 1u;
    const int bias = (1 << (e - 1)) - 1;
    const uint32_t sign = (bits >> (m + e)) & 1u;
    const uint32_t E = (bits >> m) & emask;
    const uint32_t M = bits & ((1u << m) - 1u);
    double v;
    if (E == emask) {
        v = (M == 0) ? INFINITY : NAN;
    } else if (E == 0) {
        v = ldexp((double)M, 1 - bias - m);
    } else {
        v = ldexp((double)M + ldexp(1.0, m), (int)E - bias - m);
    }
    return sign ? -v : v;
}

/* Round a double to the nearest representable value of the format, ties to even,
 * overflowing to infinity; return its bit pattern. One rounding step: the exact binary
 * value of `v` is scaled by a power of two so that the format's quantum at |v| becomes 1,
 * split into integer and fraction (both exact), and the integer part is bumped when the
 * fraction is above one half, or exactly one half with an odd integer part. */
uint32_t orc_encode(int dtype, double v) {
    int m, e;
    if (fmt_bits(dtype, &m, &e)) return 0;
    const uint32_t emask = (1u << e) - 1u;
    const int bias = (1 << (e - 1)) - 1;
    const int emin = 1 - bias; /* exponent of the smallest normal */
    const uint32_t sign = signbit(v) ? (1u << (m + e)) : 0u;
    if (isnan(v)) return sign | (emask << m) | (1u << (m - 1)); /* quiet NaN */
    double a = fabs(v);
    if (isinf(a)) return sign | (emask << m);
    if (a == 0.0) return sign;

    int ex;
    (void)frexp(a, &ex); /* a in [2^(ex-1), 2^ex) */
    int k = ex - 1;      /* binade exponent: a in [2^k, 2^(k+1)) */
    if (k < emin) k = emin; /* subnormal range: the quantum stays 2^(emin - m) */
    const double n = ldexp(a, m - k); /* a / quantum, exact */
    double r = floor(n);
    const double frac = n - r; /* exact */
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;

    const double one = ldexp(1.0, m); /* implicit leading bit */
    if (k == emin && r < one) {
        return sign | (uint32_t)r; /* subnormal (or zero) */
    }
    if (r == 2.0 * one) { /* rounded up into the next binade */
        r = one;
        k += 1;
    }
    const int E = k + bias;
    if (E >= (int)emask) return sign | (emask << m); /* overflow */
    return sign | ((uint32_t)E << m) | (uint32_t)(r - one);
}

static double load_elem(int dtype, const void* p, int64_t i) {
    if (dtype == ORC_F32) {
        uint32_t b;
        memcpy(&b, (const char*)p + 4 * i, 4);
        return orc_decode(dtype, b);
    }
    uint16_t h;
    memcpy(&h, (const char*)p + 2 * i, 2);
    return orc_decode(dtype, h);
}

static void store_elem(int dtype, void* p, int64_t i, uint32_t bits) {
    if (dtype == ORC_F32) {
        memcpy((char*)p + 4 * i, &bits, 4);
    } else {
        uint16_t h = (uint16_t)bits;
        memcpy((char*)p + 2 * i, &h, 2);
    }
}

void orc_decode_array(int dtype, const void* src, double* dst, int64_t n) {
    for (int64_t i = 0; i < n; ++i) dst[i] = load_elem(dtype, src, i);
}

void orc_encode_array(int dtype, const double* src, void* dst, int64_t n) {
    for (int64_t i = 0; i < n; ++i) store_elem(dtype, dst, i, orc_encode(dtype, src[i]));
}

/* ---------------------------------------------------------------------------------- */
/* Row statistics.                                                                     */
/* ---------------------------------------------------------------------------------- */

/* Two-pass moments ([WALK] section 1 and 6; [OPS] section 2 "naive" variant): the mean is
 * the plain sum over N, then the biased variance is the mean of squared deviations from
 * it. */
double orc_twopass_var(const double* x, int64_t n, double* mean_out) {
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += x[i];
    const double mean = s / (double)n;
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double d = x[i] - mean;
        ss += d * d;
    }
    if (mean_out) *mean_out = mean;
    return ss / (double)n;
}

/* Welford's online recurrence ([OPS] "Welford recurrence"): with delta = x_k - mean_{k-1},
 * mean_k = mean_{k-1} + delta / k and M2_k = M2_{k-1} + delta * (x_k - mean_k); the
 * variance is M2_n / n. */
double orc_welford_var(const double* x, int64_t n, double* mean_out) {
    double mean = 0.0, m2 = 0.0;
    for (int64_t k = 1; k <= n; ++k) {
        const double xk = x[k - 1];
        const double delta = xk - mean;
        mean += delta / (double)k;
        m2 += delta * (xk - mean);
    }
    if (mean_out) *mean_out = mean;
    return m2 / (double)n;
}

/* The two variance routes must agree; a disagreement means a bug (or an input outside
 * what fp64 can resolve) and the oracle refuses to answer. The bound is far above fp64
 * rounding (about N * 2^-53 relative) and far below any error a GPU kernel may make. */
static int variances_agree(double var_tp, double var_w, double mean) {
    if (var_tp == var_w) return 1;
    const double tol = 1e-9 * fabs(var_tp) + 1e-20 * mean * mean;
    return fabs(var_tp - var_w) <= tol;
}

/* ---------------------------------------------------------------------------------- */
/* Per-row operations.                                                                 */
/* ---------------------------------------------------------------------------------- */

enum { OP_LN = 0, OP_RMS = 1, OP_FUSED_RMS = 2, OP_FUSED_LN = 3, OP_SOFTMAX = 4 };

typedef struct {
    int op; /* OP_LN, OP_RMS, OP_FUSED_RMS, OP_FUSED_LN, OP_SOFTMAX */
    int dtype;
    const void* x;
    const void* residual;
    const void* gamma; /* gamma or weight; nullable */
    const void* beta;  /* nullable */
    int64_t rows, N;
    double eps;
    double* y;            /* [rows, N] fp64, nullable */
    double* mean;         /* [rows], nullable (LayerNorm); softmax: the row maximum */
    double* rstd;         /* [rows], nullable; softmax: the row's sum of exp(x - max) */
    void* residual_out;   /* [rows, N] I/O dtype, nullable (fused) */
    int64_t r0, r1;
    int status;
} job_t;

/* LayerNorm of one row ([WALK] section 1; [LLM] section 2.1):
 * mean = (1/N) sum x_j; var = (1/N) sum (x_j - mean)^2; rstd = 1/sqrt(var + eps);
 * y_j = (x_j - mean) * rstd * gamma_j + beta_j. */
static int ln_row(const job_t* jb, const double* xr, const double* g, const double* b, int64_t r) {
    const int64_t N = jb->N;
    double mean_tp, mean_w;
    const double var = orc_twopass_var(xr, N, &mean_tp);
    const double var_w = orc_welford_var(xr, N, &mean_w);
    if (!variances_agree(var, var_w, mean_tp)) return ORC_EWELFORD;
    const double rstd = 1.0 / sqrt(var + jb->eps);
    if (jb->mean) jb->mean[r] = mean_tp;
    if (jb->rstd) jb->rstd[r] = rstd;
    if (jb->y) {
        double* yr = jb->y + r * N;
        for (int64_t j = 0; j < N; ++j) {
            const double gj = g ? g[j] : 1.0;
            const double bj = b ? b[j] : 0.0;
            yr[j] = (xr[j] - mean_tp) * rstd * gj + bj;
        }
    }
    return ORC_OK;
}

/* RMSNorm of one row ([FUSED] section 0.3; [OPS] section 3; [LLM] section 2.1):
 * ms = (1/N) sum x_j^2; rstd = 1/sqrt(ms + eps); y_j = x_j * rstd * w_j. */
static void rms_row(const job_t* jb, const double* xr, const double* w, int64_t r) {
    const int64_t N = jb->N;
    double ss = 0.0;
    for (int64_t j = 0; j < N; ++j) ss += xr[j] * xr[j];
    const double rstd = 1.0 / sqrt(ss / (double)N + jb->eps);
    if (jb->rstd) jb->rstd[r] = rstd;
    if (jb->y) {
        double* yr = jb->y + r * N;
        for (int64_t j = 0; j < N; ++j) yr[j] = xr[j] * rstd * (w ? w[j] : 1.0);
    }
}


/* Softmax of one row ([SMAX] section 1): m = max_j x_j, d = sum_j exp(x_j - m),
 * y_j = exp(x_j - m) / d. Independently, the single-pass online form of the same section
 * ("denominator correction"): a running maximum m_k and denominator d_k, where a new
 * element x_k gives m_k = max(m_{k-1}, x_k) and d_k = d_{k-1} * exp(m_{k-1} - m_k) +
 * exp(x_k - m_k), starting from m = -inf, d = 0. Both must give the same maximum and, up
 * to fp64 rounding, the same denominator, or the oracle refuses to answer.
 * Entries of -inf (masked logits) have exp(x_j - m) = 0 and take no part; the online form
 * skips them (its rescaling is undefined while both maxima are -inf). A row with no entry
 * above -inf has no softmax: its maximum is -inf, its sum 0 and its outputs NaN. Other
 * entries are expected to be finite. */
static int softmax_row(const job_t* jb, const double* xr, int64_t r) {
    const int64_t N = jb->N;
    double m = -INFINITY;
    for (int64_t j = 0; j < N; ++j)
        if (xr[j] > m) m = xr[j];
    double* yr = jb->y ? jb->y + r * N : NULL;
    if (m == -INFINITY) {
        if (jb->mean) jb->mean[r] = m;
        if (jb->rstd) jb->rstd[r] = 0.0;
        if (yr)
            for (int64_t j = 0; j < N; ++j) yr[j] = NAN;
        return ORC_OK;
    }
    double d = 0.0;
    for (int64_t j = 0; j < N; ++j) d += exp(xr[j] - m);

    double mo = -INFINITY, dn = 0.0; /* online */
    for (int64_t k = 0; k < N; ++k) {
        if (xr[k] == -INFINITY) continue;
        const double mk = xr[k] > mo ? xr[k] : mo;
        dn = (mo == -INFINITY ? 0.0 : dn * exp(mo - mk)) + exp(xr[k] - mk);
        mo = mk;
    }
    if (mo != m || !(fabs(dn - d) <= 1e-12 * d)) return ORC_EONLINE;

    if (jb->mean) jb->mean[r] = m;
    if (jb->rstd) jb->rstd[r] = d;
    if (yr)
        for (int64_t j = 0; j < N; ++j) yr[j] = exp(xr[j] - m) / d;
    return ORC_OK;
}

static void* run_rows(void* arg) {
    job_t* jb = (job_t*)arg;
    const int64_t N = jb->N;
    double* xr = (double*)malloc(sizeof(double) * (size_t)N);
    const int fused = jb->op == OP_FUSED_RMS || jb->op == OP_FUSED_LN;
    double* rr = fused ? (double*)malloc(sizeof(double) * (size_t)N) : NULL;
    double* g = jb->gamma ? (double*)malloc(sizeof(double) * (size_t)N) : NULL;
    double* b = jb->beta ? (double*)malloc(sizeof(double) * (size_t)N) : NULL;
    if (!xr || (fused && !rr) || (jb->gamma && !g) || (jb->beta && !b)) {
        jb->status = ORC_ENOMEM;
        goto done;
    }
    if (g) orc_decode_array(jb->dtype, jb->gamma, g, N);
    if (b) orc_decode_array(jb->dtype, jb->beta, b, N);
    for (int64_t r = jb->r0; r < jb->r1; ++r) {
        orc_decode_array(jb->dtype, (const char*)jb->x + r * N * dtype_size(jb->dtype), xr, N);
        if (fused) {
            /* Fused ([FUSED] sections 0.3 and 3.2): residual_out = x + residual, the exact
             * sum rounded once to the I/O dtype; the normalization uses that rounded value. */
            orc_decode_array(jb->dtype, (const char*)jb->residual + r * N * dtype_size(jb->dtype), rr, N);
            for (int64_t j = 0; j < N; ++j) {
                const uint32_t t = orc_encode(jb->dtype, xr[j] + rr[j]);
                if (jb->residual_out) store_elem(jb->dtype, jb->residual_out, r * N + j, t);
                xr[j] = orc_decode(jb->dtype, t);
            }
        }
        int st = ORC_OK;
        if (jb->op == OP_LN || jb->op == OP_FUSED_LN) {
            st = ln_row(jb, xr, g, b, r);
        } else if (jb->op == OP_SOFTMAX) {
            st = softmax_row(jb, xr, r);
        } else {
            rms_row(jb, xr, g, r);
        }
        if (st != ORC_OK) {
            jb->status = st;
            goto done;
        }
    }
done:
    free(xr);
    free(rr);
    free(g);
    free(b);
    return NULL;
}

/* Split rows into contiguous ranges, one per thread (nthreads <= 1: the calling thread). */
static int run_job(const job_t* proto, int nthreads) {
    if (proto->rows < 0 || proto->N <= 0 || !proto->x || !(proto->eps >= 0.0)) return ORC_EARG;
    if (fmt_bits(proto->dtype, &(int){0}, &(int){0})) return ORC_EARG;
    if ((proto->op == OP_FUSED_RMS || proto->op == OP_FUSED_LN) && !proto->residual) return ORC_EARG;
    if (proto->rows == 0) return ORC_OK;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > proto->rows) nthreads = (int)proto->rows;
    job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return ORC_ENOMEM;
    }
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = *proto;
        jobs[t].r0 = proto->rows * t / nthreads;
        jobs[t].r1 = proto->rows * (t + 1) / nthreads;
        jobs[t].status = ORC_OK;
    }
    int started = 0;
    for (int t = 1; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, run_rows, &jobs[t]) != 0) break;
        started = t;
    }
    run_rows(&jobs[0]);
    /* Rows of threads that failed to start are done here, serially. */
    for (int t = started + 1; t < nthreads; ++t) run_rows(&jobs[t]);
    for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
    int st = ORC_OK;
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].status != ORC_OK) st = jobs[t].status;
    free(jobs);
    free(th);
    return st;
}

/* LayerNorm forward over x[rows, N]. y [rows, N], mean and rstd [rows] are fp64 and each
 * nullable; gamma / beta are I/O-dtype [N] and nullable. Returns an ORC_* code. */
int orc_layer_norm(int dtype, const void* x, const void* gamma, const void* beta, int64_t rows,
                   int64_t N, double eps, double* y, double* mean, double* rstd, int nthreads) {
    job_t jb = {0};
    jb.op = OP_LN; jb.dtype = dtype; jb.x = x; jb.gamma = gamma; jb.beta = beta;
    jb.rows = rows; jb.N = N; jb.eps = eps; jb.y = y; jb.mean = mean; jb.rstd = rstd;
    return run_job(&jb, nthreads);
}

/* RMSNorm forward over x[rows, N]; weight I/O-dtype [N], nullable. */
int orc_rms_norm(int dtype, const void* x, const void* weight, int64_t rows, int64_t N, double eps,
                 double* y, double* rstd, int nthreads) {
    job_t jb = {0};
    jb.op = OP_RMS; jb.dtype = dtype; jb.x = x; jb.gamma = weight;
    jb.rows = rows; jb.N = N; jb.eps = eps; jb.y = y; jb.rstd = rstd;
    return run_job(&jb, nthreads);
}

/* Fused residual add + RMSNorm; residual_out is I/O-dtype [rows, N], nullable. */
int orc_fused_add_rms_norm(int dtype, const void* x, const void* residual, const void* weight,
                           int64_t rows, int64_t N, double eps, double* y, void* residual_out,
                           double* rstd, int nthreads) {
    job_t jb = {0};
    jb.op = OP_FUSED_RMS; jb.dtype = dtype; jb.x = x; jb.residual = residual; jb.gamma = weight;
    jb.rows = rows; jb.N = N; jb.eps = eps; jb.y = y; jb.residual_out = residual_out; jb.rstd = rstd;
    return run_job(&jb, nthreads);
}


/* Fused residual add + LayerNorm: residual_out = round(x + residual) as for the fused
 * RMSNorm, then the LayerNorm of that rounded row (the pre-norm residual path of [FUSED]
 * section 2 with the normalization of [WALK] section 1). */
int orc_fused_add_layer_norm(int dtype, const void* x, const void* residual, const void* gamma,
                             const void* beta, int64_t rows, int64_t N, double eps, double* y,
                             void* residual_out, double* mean, double* rstd, int nthreads) {
    job_t jb = {0};
    jb.op = OP_FUSED_LN; jb.dtype = dtype; jb.x = x; jb.residual = residual; jb.gamma = gamma;
    jb.beta = beta; jb.rows = rows; jb.N = N; jb.eps = eps; jb.y = y; jb.residual_out = residual_out;
    jb.mean = mean; jb.rstd = rstd;
    return run_job(&jb, nthreads);
}

/* Row-wise softmax over x[rows, N]; y fp64 [rows, N], row_max and row_sum [rows] (the
 * maximum and the sum of exp(x - max)), each nullable. */
int orc_softmax(int dtype, const void* x, int64_t rows, int64_t N, double* y, double* row_max,
                double* row_sum, int nthreads) {
    job_t jb = {0};
    jb.op = OP_SOFTMAX; jb.dtype = dtype; jb.x = x; jb.rows = rows; jb.N = N; jb.y = y;
    jb.mean = row_max; jb.rstd = row_sum;
    return run_job(&jb, nthreads);
}

/* fp64 rows, for derivative checks: the forward formulas above applied to one row of
 * doubles (gamma / beta nullable). */
int orc_layer_norm_row_f64(const double* x, const double* gamma, const double* beta, int64_t N,
                           double eps, double* y) {
    job_t jb = {0};
    jb.op = OP_LN; jb.N = N; jb.eps = eps; jb.y = y;
    if (N <= 0) return ORC_EARG;
    return ln_row(&jb, x, gamma, beta, 0);
}

int orc_rms_norm_row_f64(const double* x, const double* weight, int64_t N, double eps, double* y) {
    job_t jb = {0};
    jb.op = OP_RMS; jb.N = N; jb.eps = eps; jb.y = y;
    if (N <= 0) return ORC_EARG;
    rms_row(&jb, x, weight, 0);
    return ORC_OK;
}

/* ---------------------------------------------------------------------------------- */
/* Backward passes.                                                                    */
/* ---------------------------------------------------------------------------------- */

/* LayerNorm backward over rows ([BN] section 3.1, with the reduction running along a row
 * instead of over a channel). With xhat_j = (x_j - mean) * rstd and y_j = xhat_j * gamma_j +
 * beta_j, the chain rule gives, for one row:
 *   g_j     = dy_j * gamma_j                        (gradient reaching xhat_j)
 *   dx_j    = rstd * (g_j - (1/N) sum_k g_k - xhat_j * (1/N) sum_k g_k * xhat_k)
 * and, over all rows, dgamma_j = sum_r dy_rj * xhat_rj, dbeta_j = sum_r dy_rj.
 * The gamma factor sits inside the row sums because gamma varies along the row (for a
 * batch normalization it is constant over the reduced set and factors out).
 * mean / rstd: the forward's fp32 statistics when given (their exact values are used), else
 * computed here in fp64 (two-pass). Outputs are fp64 and each nullable; the column sums run
 * sequentially over the rows in order. */
int orc_layer_norm_backward(int dtype, const void* dy, const void* x, const void* gamma,
                            const float* mean_in, const float* rstd_in, int64_t rows, int64_t N,
                            double eps, double* dx, double* dgamma, double* dbeta) {
    if (rows < 0 || N <= 0 || !dy || !x || !(eps >= 0.0)) return ORC_EARG;
    if (fmt_bits(dtype, &(int){0}, &(int){0})) return ORC_EARG;
    const size_t n = (size_t)N;
    double* xr = (double*)malloc(sizeof(double) * n);
    double* dr = (double*)malloc(sizeof(double) * n);
    double* g = (double*)malloc(sizeof(double) * n);
    int st = ORC_OK;
    if (!xr || !dr || !g) {
        st = ORC_ENOMEM;
        goto out;
    }
    for (int64_t j = 0; j < N; ++j) g[j] = gamma ? load_elem(dtype, gamma, j) : 1.0;
    if (dgamma) memset(dgamma, 0, sizeof(double) * n);
    if (dbeta) memset(dbeta, 0, sizeof(double) * n);
    for (int64_t r = 0; r < rows; ++r) {
        orc_decode_array(dtype, (const char*)x + r * N * dtype_size(dtype), xr, N);
        orc_decode_array(dtype, (const char*)dy + r * N * dtype_size(dtype), dr, N);
        double mean, rstd;
        if (mean_in && rstd_in) {
            mean = (double)mean_in[r];
            rstd = (double)rstd_in[r];
        } else {
            const double var = orc_twopass_var(xr, N, &mean);
            rstd = 1.0 / sqrt(var + eps);
        }
        double sg = 0.0, sgx = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            const double xh = (xr[j] - mean) * rstd;
            const double gj = dr[j] * g[j];
            sg += gj;
            sgx += gj * xh;
            if (dgamma) dgamma[j] += dr[j] * xh;
            if (dbeta) dbeta[j] += dr[j];
        }
        if (dx) {
            double* o = dx + r * N;
            for (int64_t j = 0; j < N; ++j) {
                const double xh = (xr[j] - mean) * rstd;
                o[j] = rstd * (dr[j] * g[j] - sg / (double)N - xh * (sgx / (double)N));
            }
        }
    }
out:
    free(xr);
    free(dr);
    free(g);
    return st;
}

/* RMSNorm backward over rows, by the same chain rule: xhat_j = x_j * rstd,
 * rstd = 1/sqrt((1/N) sum x^2 + eps), y_j = xhat_j * w_j:
 *   g_j  = dy_j * w_j
 *   dx_j = rstd * (g_j - xhat_j * (1/N) sum_k g_k * xhat_k)
 * and dw_j = sum_r dy_rj * xhat_rj. rstd: the forward's fp32 value when given, else fp64. */
int orc_rms_norm_backward(int dtype, const void* dy, const void* x, const void* weight,
                          const float* rstd_in, int64_t rows, int64_t N, double eps, double* dx,
                          double* dweight) {
    if (rows < 0 || N <= 0 || !dy || !x || !(eps >= 0.0)) return ORC_EARG;
    if (fmt_bits(dtype, &(int){0}, &(int){0})) return ORC_EARG;
    const size_t n = (size_t)N;
    double* xr = (double*)malloc(sizeof(double) * n);
    double* dr = (double*)malloc(sizeof(double) * n);
    double* w = (double*)malloc(sizeof(double) * n);
    int st = ORC_OK;
    if (!xr || !dr || !w) {
        st = ORC_ENOMEM;
        goto out;
    }
    for (int64_t j = 0; j < N; ++j) w[j] = weight ? load_elem(dtype, weight, j) : 1.0;
    if (dweight) memset(dweight, 0, sizeof(double) * n);
    for (int64_t r = 0; r < rows; ++r) {
        orc_decode_array(dtype, (const char*)x + r * N * dtype_size(dtype), xr, N);
        orc_decode_array(dtype, (const char*)dy + r * N * dtype_size(dtype), dr, N);
        double rstd;
        if (rstd_in) {
            rstd = (double)rstd_in[r];
        } else {
            double ss = 0.0;
            for (int64_t j = 0; j < N; ++j) ss += xr[j] * xr[j];
            rstd = 1.0 / sqrt(ss / (double)N + eps);
        }
        double sgx = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            const double xh = xr[j] * rstd;
            sgx += dr[j] * w[j] * xh;
            if (dweight) dweight[j] += dr[j] * xh;
        }
        if (dx) {
            double* o = dx + r * N;
            for (int64_t j = 0; j < N; ++j) o[j] = rstd * (dr[j] * w[j] - xr[j] * rstd * (sgx / (double)N));
        }
    }
out:
    free(xr);
    free(dr);
    free(w);
    return st;
}
