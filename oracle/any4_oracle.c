/*
 * any4 CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct reference for what the any4 weight-only
 * dequantize-GEMM computes.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library; the product path never
 * does.  It shares no code with the HIP library: no headers, helpers, tables or
 * constants.
 *
 * Sources (the pages this follows):
 *   [EXPL]  the 10100.com any4 explainer article:
 *           section 二 (the LUT: every weight is a 4-bit index into a 16-entry
 *           FP16/BF16 table kept per row), step 1 "分组缩放" (contiguous groups
 *           within a row, g = 128 typical, each with scale alpha and offset
 *           beta), step 2 "E-Step" / "M-Step" (weighted k-means that learns the
 *           per-row table), section 3 (overhead: 16 table entries per row),
 *           section 三 (the matmul runs at batch 1..16).
 *   [PAPER] "any4: Learned 4-bit Numeric Representation for LLMs" (the
 *           shd-paper.top summary), abstract: the same method at 3 and 2 bits
 *           (any3, any2).
 *   [ABS]   "any4: Learned 4-bit Numeric Representation for LLMs" (the
 *           shd-paper.top summary), abstract: a lookup-table GEMM for decode.
 *   [INT]   "量化技术应用：INT4/INT8对anything-llm的影响" (yongjin360.com),
 *           section "INT8：工业级部署的黄金标准" (Q = round(F/S + Z)) and
 *           "分组量化" (one S, Z per group of 128).
 *
 * Readings where the pages are silent (each is listed in the design doc):
 *   - dequant is w = alpha * LUT[idx] + beta, the inverse of the normalisation
 *     w_s = (w - beta) / alpha that [EXPL] step 2 names; it is evaluated as
 *     one correctly rounded fp32 fused multiply-add (the bf16 x bf16 product is
 *     exact in fp32) followed by round-to-nearest-even to bf16;
 *   - packed byte j of a row holds index 2j in bits 0..3 and 2j+1 in bits 4..7;
 *   - all arrays are dense row-major; alpha/beta[n][j] cover k in [j*g,(j+1)*g);
 *   - the GEMM reference is y[m][n] = sum_k x[m][k] * w[n][k] in fp64, k
 *     ascending, over the bf16 dequantised w;
 *   - the quantiser's group scale is asymmetric min-max onto [0, 15]; k-means
 *     starts from the identity table 0..15, ties go to the lower index, an
 *     empty (or zero-weight) cluster keeps its value, and it runs a fixed
 *     number of E/M rounds;
 *   - any3 / any2 ([PAPER]) are the same quantiser with Q = 8 / 4 table
 *     values: min-max onto [0, Q-1], start table 0..Q-1, indices 0..Q-1; the
 *     16-entry table row keeps the Q learned values first and zeros after
 *     them, so the 4-bit layouts and kernels run such layers unchanged.
 *
 * Build: gcc -O2 -fPIC -shared -ffp-contract=off -pthread (see build.py).
 */
#include <math.h>
#include <fenv.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* bf16 <-> fp32 / fp64                                                       */
/* ------------------------------------------------------------------------- */

/* bf16 is the upper half of an IEEE binary32: widening is a 16-bit shift. */
float orc_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> bf16, round to nearest, ties to even.  NaN stays NaN (quiet,
 * sign kept); infinities and overflow follow IEEE rounding. */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)           /* NaN */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16;                        /* truncated result      */
    uint32_t rest = u & 0xffffu;                    /* the 16 dropped bits   */
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u)))
        keep += 1u;                                 /* carries into exponent */
    return (uint16_t)keep;
}

void orc_f32_to_bf16_array(const float* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f32_to_bf16(in[i]);
}

/* binary64 -> bf16 with a single rounding (nearest, ties to even).  Used by the
 * quantiser, whose alpha, beta and table are computed in fp64. */
uint16_t orc_f64_to_bf16(double d)
{
    if (isnan(d))
        return signbit(d) ? 0xffc0u : 0x7fc0u;
    int neg = signbit(d) ? 1 : 0;
    double a = fabs(d);
    if (a == 0.0)
        return neg ? 0x8000u : 0x0000u;
    if (isinf(a))
        return neg ? 0xff80u : 0x7f80u;
    /* bf16 keeps 8 significant bits; below 2^-126 the quantum is 2^-133. */
    int e;
    frexp(a, &e);                        /* a = m * 2^e, m in [0.5, 1)          */
    int q = e - 8;                       /* quantum exponent for 8 bits         */
    if (q < -133)
        q = -133;                        /* subnormal range                     */
    int saved = fegetround();
    fesetround(FE_TONEAREST);
    double r = nearbyint(ldexp(a, -q));  /* integer multiple of the quantum     */
    fesetround(saved);
    double v = ldexp(r, q);              /* exact: r has <= 9 bits              */
    float f = (float)v;                  /* exact, or overflow to infinity      */
    if (isinf(f))
        return neg ? 0xff80u : 0x7f80u;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)((u >> 16) | (neg ? 0x8000u : 0u));
}

/* ------------------------------------------------------------------------- */
/* Nibble packing                                                             */
/* ------------------------------------------------------------------------- */

/* packed[n][j] = idx[n][2j] | idx[n][2j+1] << 4 (only the low 4 bits count). */
void orc_pack(const uint8_t* idx, uint8_t* packed, int64_t N, int64_t K)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j) {
            uint8_t lo = idx[n * K + 2 * j] & 15u;
            uint8_t hi = idx[n * K + 2 * j + 1] & 15u;
            packed[n * (K / 2) + j] = (uint8_t)(lo | (hi << 4));
        }
}

void orc_unpack(const uint8_t* packed, uint8_t* idx, int64_t N, int64_t K)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = packed[n * (K / 2) + k / 2];
            idx[n * K + k] = (k % 2 == 0) ? (uint8_t)(byte & 15u) : (uint8_t)(byte >> 4);
        }
}

/* ------------------------------------------------------------------------- */
/* Dequantisation ([EXPL] section 二 and step 1)                              */
/* ------------------------------------------------------------------------- */

/* w[n][k] = bf16( fp32( alpha[n][k/g] * LUT[n][idx[n][k]] + beta[n][k/g] ) ),
 * the inner expression rounded once to fp32 (fmaf is correctly rounded). */
uint16_t orc_dequant_one(uint16_t alpha, uint16_t lut_value, uint16_t beta)
{
    float s = fmaf(orc_bf16_to_f32(alpha), orc_bf16_to_f32(lut_value), orc_bf16_to_f32(beta));
    return orc_f32_to_bf16(s);
}

void orc_dequant(const uint8_t* packed, const uint16_t* lut, const uint16_t* alpha,
                 const uint16_t* beta, uint16_t* w, int64_t N, int64_t K, int64_t g)
{
    int64_t groups = K / g;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = packed[n * (K / 2) + k / 2];
            unsigned i = (k % 2 == 0) ? (byte & 15u) : (byte >> 4);
            int64_t j = k / g;
            w[n * K + k] = orc_dequant_one(alpha[n * groups + j], lut[n * 16 + i],
                                           beta[n * groups + j]);
        }
}

/* ------------------------------------------------------------------------- */
/* GEMM reference: y = x * W^T in fp64 ([EXPL] section 三: batch 1..16)         */
/* ------------------------------------------------------------------------- */

typedef struct {
    const uint16_t* x;
    const uint16_t* w;
    double* y;
    double* absdot;
    int64_t M, N, K, n_begin, n_end;
} gemm_job;

static void* gemm_worker(void* arg)
{
    gemm_job* j = (gemm_job*)arg;
    for (int64_t m = 0; m < j->M; ++m)
        for (int64_t n = j->n_begin; n < j->n_end; ++n) {
            double s = 0.0, a = 0.0;
            for (int64_t k = 0; k < j->K; ++k) {
                double p = (double)orc_bf16_to_f32(j->x[m * j->K + k]) *
                           (double)orc_bf16_to_f32(j->w[n * j->K + k]);
                s += p;
                a += fabs(p);
            }
            j->y[m * j->N + n] = s;
            if (j->absdot)
                j->absdot[m * j->N + n] = a;
        }
    return NULL;
}

/* y[m][n] = sum_k x[m][k] w[n][k], and absdot[m][n] = sum_k |x[m][k] w[n][k]|
 * (the scale of the GEMM tolerance).  Threads split n; each output is a
 * single sequential fp64 sum, so the thread count never changes a result. */
void orc_gemm(const uint16_t* x, const uint16_t* w, double* y, double* absdot,
              int64_t M, int64_t N, int64_t K, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > N)
        nthreads = N > 0 ? (int)N : 1;
    pthread_t th[256];
    gemm_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (gemm_job){x, w, y, absdot, M, N, K, N * t / nthreads, N * (t + 1) / nthreads};
        if (nthreads == 1)
            gemm_worker(&jobs[t]);
        else
            pthread_create(&th[t], NULL, gemm_worker, &jobs[t]);
    }
    if (nthreads > 1)
        for (int t = 0; t < nthreads; ++t)
            pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------- */
/* Quantiser ([EXPL] step 1 "分组缩放" and step 2 "E-Step" / "M-Step")          */
/* ------------------------------------------------------------------------- */

/* Group scale: beta = bf16(min), alpha = bf16((max - min) / 15) over each
 * contiguous group of g weights of a row, so that (w - beta) / alpha spans
 * [0, 15], the range of a 4-bit index. */
/* Group scale onto [0, levels - 1]: beta = bf16(min), alpha = bf16((max - min)
 * / (levels - 1)). */
void orc_group_scale_q(const double* W, int64_t N, int64_t K, int64_t g, int levels,
                       uint16_t* alpha, uint16_t* beta)
{
    int64_t groups = K / g;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < groups; ++j) {
            double lo = W[n * K + j * g], hi = lo;
            for (int64_t k = j * g; k < (j + 1) * g; ++k) {
                double v = W[n * K + k];
                if (v < lo)
                    lo = v;
                if (v > hi)
                    hi = v;
            }
            beta[n * groups + j] = orc_f64_to_bf16(lo);
            alpha[n * groups + j] = orc_f64_to_bf16((hi - lo) / (double)(levels - 1));
        }
}

void orc_group_scale(const double* W, int64_t N, int64_t K, int64_t g,
                     uint16_t* alpha, uint16_t* beta)
{
    orc_group_scale_q(W, N, K, g, 16, alpha, beta);
}

/* E-step: the index of the nearest of the Q table values (ties: the lower
 * index). */
static unsigned nearest(double v, const double* L, int Q)
{
    unsigned best = 0;
    double bd = fabs(v - L[0]);
    for (unsigned q = 1; q < (unsigned)Q; ++q) {
        double d = fabs(v - L[q]);
        if (d < bd) {
            bd = d;
            best = q;
        }
    }
    return best;
}

static double objective(const double* ws, const double* wt, const uint8_t* idx,
                        const double* L, int64_t K)
{
    double J = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double e = ws[k] - L[idx[k]];
        J += wt[k] * e * e;
    }
    return J;
}

/* Weighted k-means over one row in the normalised domain.
 *   ws[k]: normalised weight w_s, wt[k]: its importance alpha * E|x|.
 *   L[Q]: in = initial table, out = table after `iters` E/M rounds (fp64).
 *   idx[k]: out = assignment from the last E-step.
 *   trace (optional, 2*iters entries): objective after each E and each M step.
 * M-step: L_q = sum(wt * ws) / sum(wt) over the members of cluster q. */
void orc_kmeans_row_q(const double* ws, const double* wt, int64_t K, int iters, int Q,
                      double* L, uint8_t* idx, double* trace)
{
    for (int it = 0; it < iters; ++it) {
        for (int64_t k = 0; k < K; ++k)                     /* E-step */
            idx[k] = (uint8_t)nearest(ws[k], L, Q);
        if (trace)
            trace[2 * it] = objective(ws, wt, idx, L, K);
        double num[16] = {0}, den[16] = {0};                /* M-step */
        for (int64_t k = 0; k < K; ++k) {
            num[idx[k]] += wt[k] * ws[k];
            den[idx[k]] += wt[k];
        }
        for (int q = 0; q < Q; ++q)
            if (den[q] > 0.0)
                L[q] = num[q] / den[q];
        if (trace)
            trace[2 * it + 1] = objective(ws, wt, idx, L, K);
    }
    if (iters == 0)
        for (int64_t k = 0; k < K; ++k)
            idx[k] = (uint8_t)nearest(ws[k], L, Q);
}

void orc_kmeans_row(const double* ws, const double* wt, int64_t K, int iters,
                    double* L, uint8_t* idx, double* trace)
{
    orc_kmeans_row_q(ws, wt, K, iters, 16, L, idx, trace);
}

typedef struct {
    const double* W;
    const double* Ex;
    int64_t N, K, g, n_begin, n_end;
    int iters, Q;
    uint8_t* idx;
    uint16_t* lut;
    uint16_t* alpha;
    uint16_t* beta;
    int failed;
} quant_job;

static void* quant_worker(void* arg)
{
    quant_job* q = (quant_job*)arg;
    int64_t K = q->K, g = q->g, groups = K / g;
    double* ws = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    double* wt = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    if (!ws || !wt) {
        q->failed = 1;
        free(ws);
        free(wt);
        return NULL;
    }
    for (int64_t n = q->n_begin; n < q->n_end; ++n) {
        const double* row = q->W + n * K;
        uint16_t* a = q->alpha + n * groups;
        uint16_t* b = q->beta + n * groups;
        orc_group_scale_q(row, 1, K, g, q->Q, a, b);
        for (int64_t k = 0; k < K; ++k) {
            double al = (double)orc_bf16_to_f32(a[k / g]);
            double be = (double)orc_bf16_to_f32(b[k / g]);
            ws[k] = (al != 0.0) ? (row[k] - be) / al : 0.0;
            wt[k] = al * q->Ex[k];
        }
        double L[16];
        for (int i = 0; i < q->Q; ++i)
            L[i] = (double)i;                               /* uniform integer grid */
        uint8_t* id = q->idx + n * K;
        orc_kmeans_row_q(ws, wt, K, q->iters, q->Q, L, id, NULL);
        /* Store the table in bf16 (entries past Q: zero), then assign every
         * weight to the stored values so that the indices match what is kept. */
        double Lq[16];
        for (int i = 0; i < 16; ++i) {
            uint16_t h = i < q->Q ? orc_f64_to_bf16(L[i]) : 0;
            q->lut[n * 16 + i] = h;
            Lq[i] = (double)orc_bf16_to_f32(h);
        }
        for (int64_t k = 0; k < K; ++k)
            id[k] = (uint8_t)nearest(ws[k], Lq, q->Q);
    }
    free(ws);
    free(wt);
    return NULL;
}

/* Full any4 quantisation of W[N][K] (fp64) with per-input-channel importance
 * Ex[K] = E|x|: group scale, then per-row weighted k-means.  Rows are
 * independent; threads split them.  Returns 0 on success. */
int orc_kmeans_quantize_q(const double* W, const double* Ex, int64_t N, int64_t K, int64_t g,
                          int iters, int Q, uint8_t* idx, uint16_t* lut, uint16_t* alpha,
                          uint16_t* beta, int nthreads)
{
    if (Q < 2 || Q > 16)
        return 2;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > N)
        nthreads = N > 0 ? (int)N : 1;
    pthread_t th[256];
    quant_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (quant_job){W, Ex, N, K, g, N * t / nthreads, N * (t + 1) / nthreads,
                              iters, Q, idx, lut, alpha, beta, 0};
        if (nthreads == 1)
            quant_worker(&jobs[t]);
        else
            pthread_create(&th[t], NULL, quant_worker, &jobs[t]);
    }
    if (nthreads > 1)
        for (int t = 0; t < nthreads; ++t)
            pthread_join(th[t], NULL);
    for (int t = 0; t < nthreads; ++t)
        if (jobs[t].failed)
            return 1;
    return 0;
}

int orc_kmeans_quantize(const double* W, const double* Ex, int64_t N, int64_t K, int64_t g,
                        int iters, uint8_t* idx, uint16_t* lut, uint16_t* alpha,
                        uint16_t* beta, int nthreads)
{
    return orc_kmeans_quantize_q(W, Ex, N, K, g, iters, 16, idx, lut, alpha, beta, nthreads);
}
