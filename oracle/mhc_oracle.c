/*
 * mhc_oracle.c -- plain, slow, fp64 CPU reference of the mHC pre-mapping forward.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the checker, not the product: only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Sources (the web pages this method is described on):
 *   [V2]   "CANN ops-transformer 中 aclnnMhcPreV2 算子接口全解析" (kwkr.cn/news/422178),
 *          section 3 (math semantics): invRms, xGamma, hMix, w, split, hPre, hPost, hRes, hIn.
 *   [SK]   "CANN ops-transformer 算子详解：aclnnMhcPreSinkhorn 接口与 MhcPreSinkhorn 实现剖析"
 *          (m.mzlw.cn/news/197063), section 3.2 (Sinkhorn normalisation: normOut[k], sumOut[k],
 *          plus the description of the golden's stable softmax), section 5.1 (output shapes).
 *   [HC]   "CANN HcPre 融合算子解析：mHC 结构前处理 custom.npu_hc_pre 与 npu_hc_pre_v2 实战指南"
 *          (mhpn.cn/news/2282827), "function description" (rsqrt of the mean square, split
 *          order pre/post/comb, comb reshaped to n x n) and "parameters" (pre_mix).
 *   [BW]   "CANN ops-transformer 算子解析：MhcPreBackward 反向梯度算子实现与 aclnn 调用指南"
 *          (0539edu.com/news/4871844), section 3.7: the RMS mean runs over N*D elements.
 *
 * Arithmetic: every input is converted to double exactly (bf16 and f32 are subsets of
 * f64); every sum, product, exp and division is done in double; results are returned
 * in double. The only rounding to a narrower type is hIn -> bf16 (round to nearest,
 * ties to even, straight from double), because hIn is a bf16 output on every page.
 *
 * Readings taken where the pages are silent or garbled (each is also listed with the
 * design notes of the repository):
 *   R1  The RMS mean runs over all n*D elements of a token ([V2] mean(xFlat^2); [BW] 3.7).
 *   R2  invRms uses raw x; gamma only scales the projection input ([V2] first line uses xFlat).
 *   R3  hMix is the un-normalised product xGamma . phi^T; w = hMix * invRms ([V2]).
 *   R4  alpha holds one scalar per branch; bias holds one value per phi row, ordered
 *       pre (n), post (n), res (n*n) ([SK] 3.1; [HC] split order).
 *   R5  hPre gets +hcEps; hPost gets +hcEps only when alpha has 2 entries ([V2]).
 *   R6  The n*n res block is reshaped row-major: entry m -> (r = m / n, c = m % n) ([HC]).
 *   R7  Sinkhorn runs 2*numIters steps: step 0 is a softmax over each row plus hcEps,
 *       step 1 a column normalisation, then (row, column) pairs; every sum gets +hcEps;
 *       hRes is the last step's matrix ([SK] 3.2).
 *   R8  sumOut[0] (not defined by the formula) holds the softmax row denominators
 *       sum_c exp(L[r][c] - max_c' L[r][c']) (the stable softmax of the golden, [SK] 3.2).
 *       PARITY UNPINNED: no page fixes this plane.
 *   R9  hIn uses raw x: hIn[d] = sum_i wgt_i * x[i][d], wgt = pre_mix[t] when given,
 *       else hPre ([V2]; [HC] pre_mix). hPre is still computed and returned.
 *   R10 With alpha of 2 entries there is no res branch: hRes = 0, and no Sinkhorn
 *       intermediates exist ([V2]).
 *   R17 x may be bf16 or binary16 (fp16) ([SK] 5.1 and [V2] 5.1 list both); hIn takes
 *       x's format and is rounded to it once from double; the arithmetic is unchanged.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- bf16 <-> double */

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
double oracle_bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 (8 significant bits, binary32 exponent range),
 * ties to even, in one step (no detour through binary32, so no double rounding). */
uint16_t oracle_bf16_from_double(double v)
{
    if (isnan(v)) return (uint16_t)(signbit(v) ? 0xFFC0u : 0x7FC0u);
    if (isinf(v)) return (uint16_t)(signbit(v) ? 0xFF80u : 0x7F80u);
    if (v == 0.0) return (uint16_t)(signbit(v) ? 0x8000u : 0x0000u);

    int e2;                        /* |v| = f * 2^e2, f in [0.5, 1) */
    frexp(v, &e2);
    int e = e2 - 1;                /* |v| in [2^e, 2^(e+1)) */
    if (e < -126) e = -126;        /* below the normal range the spacing stays 2^-133 */
    double ulp = ldexp(1.0, e - 7);
    double q = v / ulp;            /* exact: scaling by a power of two */
    double qr = q;
    {   /* round half to even, written out instead of relying on the FP mode */
        double fl = floor(q);
        double diff = q - fl;
        if (diff > 0.5) qr = fl + 1.0;
        else if (diff < 0.5) qr = fl;
        else qr = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    }
    double r = qr * ulp;
    if (fabs(r) >= ldexp(1.0, 128))  /* beyond the largest finite bf16 */
        return (uint16_t)(signbit(v) ? 0xFF80u : 0x7F80u);
    float f = (float)r;            /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* ---------------------------------------------------------------- binary16 <-> double */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits; subnormals below 2^-14.
 * Widening is exact. */
double oracle_f16_to_double(uint16_t bits)
{
    const int sgn = bits >> 15, ex = (bits >> 10) & 0x1F, fr = bits & 0x3FF;
    double mag;
    if (ex == 0x1F) mag = fr ? NAN : INFINITY;
    else if (ex == 0) mag = ldexp((double)fr, -24);                 /* subnormal or zero */
    else mag = ldexp(1.0 + (double)fr / 1024.0, ex - 15);
    return sgn ? -mag : mag;
}

/* Round a double to the nearest binary16 (11 significant bits, exponent range 2^-14 to
 * 2^15, subnormal spacing 2^-24), ties to even, in one step. */
uint16_t oracle_f16_from_double(double v)
{
    const uint16_t sgn = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sgn | 0x7E00u);
    if (isinf(v)) return (uint16_t)(sgn | 0x7C00u);
    const double a = fabs(v);
    if (a == 0.0) return sgn;
    int e2;
    frexp(a, &e2);
    int e = e2 - 1;                /* a in [2^e, 2^(e+1)) */
    if (e < -14) e = -14;          /* below the normal range the spacing stays 2^-24 */
    const double ulp = ldexp(1.0, e - 10);
    const double q = a / ulp;      /* exact: scaling by a power of two */
    const double lo = floor(q), frac = q - lo;   /* round half to even, written out */
    const double qh = frac > 0.5 ? lo + 1.0 : (frac < 0.5 ? lo : (fmod(lo, 2.0) == 0.0 ? lo : lo + 1.0));
    const double r = qh * ulp;     /* the rounded magnitude, exact in binary16 or 2^16 */
    if (r >= 65536.0) return (uint16_t)(sgn | 0x7C00u);
    if (r < ldexp(1.0, -14)) return (uint16_t)(sgn | (uint16_t)(r / ldexp(1.0, -24)));
    int re2;
    const double f = frexp(r, &re2);   /* r = f 2^re2, f in [0.5, 1) */
    const int ex = re2 - 1 + 15;
    const uint16_t fr = (uint16_t)((2.0 * f - 1.0) * 1024.0);
    return (uint16_t)(sgn | (uint16_t)(ex << 10) | fr);
}

/* ---------------------------------------------------------------- problem description */

typedef struct oracle_cfg {
    int64_t T;        /* tokens */
    int32_t n;        /* hyper-streams (hcMult) */
    int32_t D;        /* hidden size per stream */
    int32_t n_alpha;  /* 3: pre/post/res branches; 2: pre/post only */
    int32_t num_iters;
    double norm_eps;
    double hc_eps;
    int32_t x_f16;    /* 0: x and hIn are bf16; 1: binary16 (R17) */
} oracle_cfg;

/* Outputs are optional (NULL = not wanted); all are double (h_in_bf16: the 16-bit
 * storage format of x, bf16 or binary16), laid out for the ntok
 * requested tokens in request order:
 *   inv_rms [ntok], h_mix [ntok][M], h_pre [ntok][n], h_post [ntok][n],
 *   h_res [ntok][n][n], sum_out [2*it][ntok][n], norm_out [2*it][ntok][n][n],
 *   h_in [ntok][D] (double, before rounding), h_in_bf16 [ntok][D] (bf16 bits). */
typedef struct oracle_out {
    double* inv_rms;
    double* h_mix;
    double* h_pre;
    double* h_post;
    double* h_res;
    double* sum_out;
    double* norm_out;
    double* h_in;
    uint16_t* h_in_bf16;
} oracle_out;

static double sigmoid(double z)
{
    if (z >= 0.0) return 1.0 / (1.0 + exp(-z));
    double e = exp(z);
    return e / (1.0 + e);
}

static int mix_rows(const oracle_cfg* c)
{
    return c->n_alpha == 3 ? c->n * c->n + 2 * c->n : 2 * c->n;
}

/* An element of x (or its 16-bit storage format, which hIn shares), widened exactly. */
static double x_val(const oracle_cfg* c, uint16_t bits)
{
    return c->x_f16 ? oracle_f16_to_double(bits) : oracle_bf16_to_double(bits);
}
static uint16_t x_round(const oracle_cfg* c, double v)
{
    return c->x_f16 ? oracle_f16_from_double(v) : oracle_bf16_from_double(v);
}

/* invRms = (mean(xFlat^2) + normEps)^(-1/2) of one token's K = n*D entries xt, the
 * mean taken over all of them (R1, R2). */
static double token_inv_rms(const oracle_cfg* c, const uint16_t* xt, int n, int D, double norm_eps)
{
    const int64_t K = (int64_t)n * D;
    double ss = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double v = x_val(c, xt[k]);
        ss += v * v;
    }
    return 1.0 / sqrt(ss / (double)K + norm_eps);
}

/* Everything of one token that follows from its mixes hmix [M] and its invRms: the
 * gates, the Sinkhorn and hIn. `slot` is the token's position in the output arrays,
 * `t` its index in x. scratch holds n*n + n doubles. */
static void finish_token(const oracle_cfg* c, int64_t ntok, int64_t slot, int64_t t,
                         const uint16_t* x, const double* hmix, double inv_rms,
                         const float* alpha, const float* bias, const float* pre_mix,
                         const oracle_out* o, double* scratch)
{
    const int n = c->n;
    const int D = c->D;
    const int64_t K = (int64_t)n * D;
    const int M = mix_rows(c);
    const double eps = c->hc_eps;
    const uint16_t* xt = x + t * K;

    double* A = scratch;                        /* [n*n] */
    double* s = A + n * n;                      /* [n]   */

    /* w = hMix * invRms, split into pPre = w[0:n], pPost = w[n:2n], pRes = w[2n:] (R4). */
    double hpre[8], hpost[8];
    for (int i = 0; i < n; ++i) {
        double p_pre = hmix[i] * inv_rms;
        double p_post = hmix[n + i] * inv_rms;
        hpre[i] = sigmoid((double)alpha[0] * p_pre + (double)bias[i]) + eps;            /* R5 */
        hpost[i] = 2.0 * sigmoid((double)alpha[1] * p_post + (double)bias[n + i]);
        if (c->n_alpha == 2) hpost[i] += eps;                                           /* R5 */
    }

    if (o->inv_rms) o->inv_rms[slot] = inv_rms;
    if (o->h_mix)
        for (int m = 0; m < M; ++m) o->h_mix[slot * M + m] = hmix[m];
    if (o->h_pre)
        for (int i = 0; i < n; ++i) o->h_pre[slot * n + i] = hpre[i];
    if (o->h_post)
        for (int i = 0; i < n; ++i) o->h_post[slot * n + i] = hpost[i];

    /* Residual logits and Sinkhorn (R6, R7, R8). */
    if (c->n_alpha == 3) {
        const int steps = 2 * c->num_iters;
        const int nn = n * n;
        for (int r = 0; r < n; ++r)
            for (int cc = 0; cc < n; ++cc) {
                int m = r * n + cc;
                A[m] = (double)alpha[2] * (hmix[2 * n + m] * inv_rms) + (double)bias[2 * n + m];
            }
        for (int k = 0; k < steps; ++k) {
            if (k == 0) {
                /* softmax over each row (the last dim), then + hcEps elementwise */
                for (int r = 0; r < n; ++r) {
                    double mx = A[r * n];
                    for (int cc = 1; cc < n; ++cc)
                        if (A[r * n + cc] > mx) mx = A[r * n + cc];
                    double sum = 0.0;
                    for (int cc = 0; cc < n; ++cc) {
                        A[r * n + cc] = exp(A[r * n + cc] - mx);
                        sum += A[r * n + cc];
                    }
                    for (int cc = 0; cc < n; ++cc) A[r * n + cc] = A[r * n + cc] / sum + eps;
                    s[r] = sum;
                }
            } else if (k % 2 == 1) {
                /* column step: divide every column by (its sum + hcEps) */
                for (int cc = 0; cc < n; ++cc) {
                    double sum = 0.0;
                    for (int r = 0; r < n; ++r) sum += A[r * n + cc];
                    sum += eps;
                    for (int r = 0; r < n; ++r) A[r * n + cc] = A[r * n + cc] / sum;
                    s[cc] = sum;
                }
            } else {
                /* row step: divide every row by (its sum + hcEps) */
                for (int r = 0; r < n; ++r) {
                    double sum = 0.0;
                    for (int cc = 0; cc < n; ++cc) sum += A[r * n + cc];
                    sum += eps;
                    for (int cc = 0; cc < n; ++cc) A[r * n + cc] = A[r * n + cc] / sum;
                    s[r] = sum;
                }
            }
            if (o->sum_out)
                for (int i = 0; i < n; ++i) o->sum_out[((int64_t)k * ntok + slot) * n + i] = s[i];
            if (o->norm_out)
                for (int m = 0; m < nn; ++m)
                    o->norm_out[((int64_t)k * ntok + slot) * nn + m] = A[m];
        }
        if (o->h_res)
            for (int m = 0; m < nn; ++m) o->h_res[slot * nn + m] = A[m];
    } else if (o->h_res) {
        for (int m = 0; m < n * n; ++m) o->h_res[slot * n * n + m] = 0.0;   /* R10 */
    }

    /* hIn[d] = sum_i wgt_i * x[i][d] over raw x (R9). */
    if (o->h_in || o->h_in_bf16) {
        double wgt[8];
        for (int i = 0; i < n; ++i)
            wgt[i] = pre_mix ? (double)pre_mix[t * n + i] : hpre[i];
        for (int d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int i = 0; i < n; ++i)
                acc += wgt[i] * x_val(c, xt[(int64_t)i * D + d]);
            if (o->h_in) o->h_in[slot * D + d] = acc;
            if (o->h_in_bf16) o->h_in_bf16[slot * D + d] = x_round(c, acc);
        }
    }
}

/* One token of the whole forward. scratch holds M + n*n + n doubles. */
static void one_token(const oracle_cfg* c, int64_t ntok, int64_t slot, int64_t t,
                      const uint16_t* x, const float* phi, const float* alpha,
                      const float* bias, const float* gamma, const float* pre_mix,
                      const oracle_out* o, double* scratch)
{
    const int64_t K = (int64_t)c->n * c->D;     /* length of xFlat */
    const int M = mix_rows(c);
    const uint16_t* xt = x + t * K;
    double* hmix = scratch;                     /* [M] */

    const double inv_rms = token_inv_rms(c, xt, c->n, c->D, c->norm_eps);

    /* hMix = xGamma . phi^T with xGamma = xFlat (.) gammaFlat (R3). */
    for (int m = 0; m < M; ++m) {
        const float* row = phi + (int64_t)m * K;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double xg = x_val(c, xt[k]);
            if (gamma) xg *= (double)gamma[k];
            acc += xg * (double)row[k];
        }
        hmix[m] = acc;
    }
    finish_token(c, ntok, slot, t, x, hmix, inv_rms, alpha, bias, pre_mix, o, scratch + M);
}

/* Forward for the listed tokens (tokens == NULL: all T tokens, in order).
 * Returns 0 on success, -1 on an invalid description. nthreads <= 0: OpenMP default. */
int oracle_pre_forward(const oracle_cfg* c, const uint16_t* x, const float* phi,
                       const float* alpha, const float* bias, const float* gamma,
                       const float* pre_mix, const int64_t* tokens, int64_t ntok,
                       const oracle_out* o, int nthreads)
{
    if (!c || !x || !phi || !alpha || !bias || !o) return -1;
    if (c->n < 1 || c->n > 8 || c->D < 1 || c->T < 0 || ntok < 0) return -1;
    if (c->n_alpha != 2 && c->n_alpha != 3) return -1;
    if (c->n_alpha == 3 && c->num_iters < 1) return -1;
    if (tokens == NULL && ntok != c->T) return -1;
    for (int64_t j = 0; tokens && j < ntok; ++j)
        if (tokens[j] < 0 || tokens[j] >= c->T) return -1;

    const int M = mix_rows(c);
    const size_t scratch_len = (size_t)M + (size_t)c->n * c->n + (size_t)c->n;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double* scratch = (double*)malloc(scratch_len * sizeof(double));
        if (!scratch) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t j = 0; j < ntok; ++j) {
                int64_t t = tokens ? tokens[j] : j;
                one_token(c, ntok, j, t, x, phi, alpha, bias, gamma, pre_mix, o, scratch);
            }
            free(scratch);
        }
    }
    return failed ? -1 : 0;
}

/* InvRms on its own, the standalone form of the normalisation step ([HC] "function
 * description": the reciprocal of the RMS over the token's n*D entries, plus normEps
 * under the root). inv_rms: [T] doubles. Returns 0, or -1 on an invalid description. */
int oracle_inv_rms(const oracle_cfg* c, const uint16_t* x, double* inv_rms, int nthreads)
{
    if (!c || !x || !inv_rms) return -1;
    if (c->n < 1 || c->n > 8 || c->D < 1 || c->T < 0) return -1;
    const int64_t K = (int64_t)c->n * c->D;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < c->T; ++t) inv_rms[t] = token_inv_rms(c, x + t * K, c->n, c->D, c->norm_eps);
    return 0;
}

/* The Sinkhorn stage on its own ([HC] "function description": the standalone operator
 * takes the mixes and the rsqrt instead of computing them): given hMix [T][M] and invRms
 * [T] (doubles), every output that follows from them -- hPre, hPost, hRes, the Sinkhorn
 * planes and hIn -- exactly as the whole forward derives them (R4 to R10). o->inv_rms
 * and o->h_mix must be NULL. Returns 0, or -1 on an invalid description. */
int oracle_pre_sinkhorn(const oracle_cfg* c, const uint16_t* x, const double* h_mix,
                        const double* inv_rms, const float* alpha, const float* bias,
                        const float* pre_mix, const oracle_out* o, int nthreads)
{
    if (!c || !x || !h_mix || !inv_rms || !alpha || !bias || !o) return -1;
    if (o->inv_rms || o->h_mix) return -1;
    if (c->n < 1 || c->n > 8 || c->D < 1 || c->T < 0) return -1;
    if (c->n_alpha != 2 && c->n_alpha != 3) return -1;
    if (c->n_alpha == 3 && c->num_iters < 1) return -1;
    const int M = mix_rows(c);
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double* scratch = (double*)malloc(((size_t)c->n * c->n + (size_t)c->n) * sizeof(double));
        if (!scratch) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < c->T; ++t)
                finish_token(c, c->T, t, t, x, h_mix + t * M, inv_rms[t], alpha, bias, pre_mix, o,
                             scratch);
            free(scratch);
        }
    }
    return failed ? -1 : 0;
}

/* Threads the OpenMP runtime would use for a parallel region. */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
