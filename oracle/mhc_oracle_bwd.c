/*
 * mhc_oracle_bwd.c -- plain, slow, fp64 CPU reference of the MhcPre backward, and of the
 * MhcPre forward on double inputs (the function whose gradient the backward is).
 *
 * TEST INFRASTRUCTURE ONLY, like mhc_oracle.c: only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it. It shares nothing with the HIP library.
 *
 * Sources:
 *   [BW]  "CANN ops-transformer 算子解析：MhcPreBackward 反向梯度算子实现与 aclnn 调用指南"
 *         (0539edu.com/news/4871844), section 3 (the eight backward stages 3.1-3.8),
 *         section 6.1 (inputs and outputs), section 8.2 (output shapes: gradAlpha has 3
 *         entries, gradX takes gradHIn's type, the rest are float32).
 *   [V2]  "CANN ops-transformer 中 aclnnMhcPreV2 算子接口全解析" (kwkr.cn/news/422178),
 *         section 3: the MhcPre forward (affine hRes = pRes * alpha2 + bias2, no Sinkhorn).
 *
 *   [SK]  "CANN ops-transformer 算子详解：aclnnMhcPreSinkhorn 接口与 MhcPreSinkhorn 实现剖析"
 *         (m.mzlw.cn/news/197063): section 1 names the MhcPreSinkhornBackward operator and
 *         says the forward's hPre, hMix, invRms, normOut and sumOut are its inputs;
 *         section 3.2 gives the Sinkhorn steps. The pages give no formula for that
 *         backward: with num_iters >= 1 the res branch below is the derivative of those
 *         steps, worked out by hand (reading B6).
 *
 * The backward takes the forward's saved values (invRms, hMix, hPre, hPost) as inputs, as
 * [BW] section 1 describes, and does not recompute them. Every input converts to double
 * exactly; every sum and product is in double; gradX is also returned rounded once
 * (round to nearest, ties to even) to gradHIn's type, bf16 or fp16 ([BW] 8.2: gradX
 * inherits grad_h_in's BF16/FP16 type; x, gradHIn and gradXPost then share that format).
 *
 * Readings (also listed with the design notes of the repository):
 *   B1 alpha_res's gradient sums gradHRes times pRes = w[2n:] (the input of the affine map;
 *      [BW] 3.4 names it H_res_2, which the page does not define further).
 *   B2 the RMS term of gradX uses raw x: invRms is computed from raw x ([V2] first line),
 *      so d invRms / d x_k = -invRms^3 x_k / (n D). [BW] 3.7 writes x_rs there; the two
 *      agree when gamma is absent. gradGamma = sum over tokens of x * (gHMix . phi) ([BW] 3.7).
 *   B3 the backward needs the res branch: alpha has 3 entries and phi n*n + 2n rows
 *      ([BW] 5 and 8.2: gradAlpha fixed at 3, fusion size n*n + 2n).
 *   B4 gradXPost, when given, is added to gradX before the single rounding ([BW] 3.8).
 *   B5 cross-token sums (gradPhi, gradGamma, gradAlpha, gradBias) run over all T tokens in
 *      token order. Alongside each, the sum of the absolute values of its terms is
 *      returned: the scale of the rounding error of any summation order, which the
 *      tests use to bound the error of a float32 evaluation.
 *   B6 MhcPreSinkhorn (num_iters >= 1): hRes = Sinkhorn(L), L = alpha2 pRes + biasRes, with
 *      the forward's steps ([SK] 3.2, as in mhc_oracle.c): A_0 = rowsoftmax(L) + eps, then
 *      for k = 1 .. 2 it - 1 A_k = A_{k-1} / s_k with s_k the column (k odd) or row (k
 *      even) sums of A_{k-1} plus eps. Given G = dLoss/dA_k, a column step passes back
 *      (G[r][c] - sum_r' G[r'][c] A_k[r'][c]) / s_k[c] (rows likewise), and the softmax
 *      step dL[r][c] = P[r][c] (G[r][c] - sum_c' G[r][c'] P[r][c']), P = A_0 - eps. The
 *      saved planes normOut[k] = A_k and sumOut[k] = s_k are the inputs it reads.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

double oracle_bf16_to_double(uint16_t bits);
uint16_t oracle_bf16_from_double(double v);
double oracle_f16_to_double(uint16_t bits);
uint16_t oracle_f16_from_double(double v);

static double sigm(double z)
{
    if (z >= 0.0) return 1.0 / (1.0 + exp(-z));
    double e = exp(z);
    return e / (1.0 + e);
}

/* ---------------------------------------------------------------- MhcPre forward, doubles */

/* [V2] section 3 on double inputs, all tokens: invRms [T], hMix [T][M], hPre [T][n],
 * hPost [T][n], hRes [T][n][n], hIn [T][D] (unrounded). gamma may be NULL. M = n*n + 2n
 * (alpha has 3 entries). num_iters == 0: hRes is the affine map of MhcPre; num_iters
 * >= 1: hRes is the Sinkhorn of that map ([SK] 3.2, 2 num_iters steps), with the planes
 * in sum_out [2it][T][n] and norm_out [2it][T][n][n] (step-major). Any output may be NULL. */
static void sinkhorn_f64(double* A, int n, double eps, int steps, int64_t T, int64_t t,
                         double* sum_out, double* norm_out)
{
    double s[8];
    for (int k = 0; k < steps; ++k) {
        if (k == 0) {
            for (int r = 0; r < n; ++r) {
                double mx = A[r * n];
                for (int c = 1; c < n; ++c) mx = A[r * n + c] > mx ? A[r * n + c] : mx;
                double sum = 0.0;
                for (int c = 0; c < n; ++c) { A[r * n + c] = exp(A[r * n + c] - mx); sum += A[r * n + c]; }
                for (int c = 0; c < n; ++c) A[r * n + c] = A[r * n + c] / sum + eps;
                s[r] = sum;
            }
        } else {
            for (int i = 0; i < n; ++i) {
                double sum = eps;
                for (int j = 0; j < n; ++j) sum += (k % 2) ? A[j * n + i] : A[i * n + j];
                for (int j = 0; j < n; ++j) {
                    if (k % 2) A[j * n + i] /= sum;
                    else A[i * n + j] /= sum;
                }
                s[i] = sum;
            }
        }
        for (int i = 0; i < n && sum_out; ++i) sum_out[((int64_t)k * T + t) * n + i] = s[i];
        for (int e = 0; e < n * n && norm_out; ++e) norm_out[((int64_t)k * T + t) * n * n + e] = A[e];
    }
}

int oracle_mhcpre_forward_f64(int64_t T, int n, int D, const double* x, const double* phi,
                              const double* alpha, const double* bias, const double* gamma,
                              double norm_eps, double hc_eps, int num_iters, double* inv_rms,
                              double* h_mix, double* h_pre, double* h_post, double* h_res,
                              double* h_in, double* sum_out, double* norm_out)
{
    if (T < 0 || n < 1 || n > 8 || D < 1 || num_iters < 0 || !x || !phi || !alpha || !bias) return -1;
    const int M = n * n + 2 * n;
    const int64_t K = (int64_t)n * D;
    for (int64_t t = 0; t < T; ++t) {
        const double* xt = x + t * K;
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) ss += xt[k] * xt[k];
        const double inv = 1.0 / sqrt(ss / (double)K + norm_eps);
        double hm[80], hp[8];
        for (int m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += (gamma ? xt[k] * gamma[k] : xt[k]) * phi[(int64_t)m * K + k];
            hm[m] = acc;
        }
        for (int i = 0; i < n; ++i) {
            hp[i] = sigm(alpha[0] * (hm[i] * inv) + bias[i]) + hc_eps;
            if (h_pre) h_pre[t * n + i] = hp[i];
            if (h_post) h_post[t * n + i] = 2.0 * sigm(alpha[1] * (hm[n + i] * inv) + bias[n + i]);
        }
        double L[64];
        for (int e = 0; e < n * n; ++e) L[e] = alpha[2] * (hm[2 * n + e] * inv) + bias[2 * n + e];
        if (num_iters > 0) sinkhorn_f64(L, n, hc_eps, 2 * num_iters, T, t, sum_out, norm_out);
        for (int e = 0; e < n * n && h_res; ++e) h_res[t * n * n + e] = L[e];
        if (inv_rms) inv_rms[t] = inv;
        for (int m = 0; m < M && h_mix; ++m) h_mix[t * M + m] = hm[m];
        for (int d = 0; d < D && h_in; ++d) {
            double acc = 0.0;
            for (int i = 0; i < n; ++i) acc += hp[i] * xt[(int64_t)i * D + d];
            h_in[t * D + d] = acc;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------- MhcPre backward */

typedef struct oracle_bwd_in {
    int64_t T;
    int32_t n;
    int32_t D;
    double hc_eps;
    const uint16_t* x;            /* bf16 or fp16 (x_f16) [T][n][D] */
    const float* phi;             /* [M][n*D] */
    const float* alpha;           /* [3] */
    const uint16_t* grad_h_in;    /* x's format [T][D] */
    const float* grad_h_post;     /* [T][n] */
    const float* grad_h_res;      /* [T][n][n] */
    const float* inv_rms;         /* [T] */
    const float* h_mix;           /* [T][M] */
    const float* h_pre;           /* [T][n] */
    const float* h_post;          /* [T][n] */
    const float* gamma;           /* [n][D] or NULL */
    const uint16_t* grad_x_post;  /* x's format [T][n][D] or NULL */
    int32_t num_iters;            /* 0: MhcPre; >= 1: MhcPreSinkhorn (planes below) */
    const float* sum_out;         /* [2 it][T][n] */
    const float* norm_out;        /* [2 it][T][n][n] */
    int32_t x_f16;                /* 0: x, gradHIn, gradXPost and gradX bf16; 1: fp16 */
} oracle_bwd_in;

/* A 16-bit value of x's format (exact), and the nearest one to a double. */
static double x16_value(const oracle_bwd_in* in, uint16_t bits)
{
    return in->x_f16 ? oracle_f16_to_double(bits) : oracle_bf16_to_double(bits);
}
static uint16_t x16_round(const oracle_bwd_in* in, double v)
{
    return in->x_f16 ? oracle_f16_from_double(v) : oracle_bf16_from_double(v);
}

/* gradX rows are produced for the listed tokens (ntok rows, request order); the other
 * outputs always cover all T tokens. Any output may be NULL. */
typedef struct oracle_bwd_out {
    double* grad_x;           /* [ntok][n][D] unrounded */
    uint16_t* grad_x_bits;    /* [ntok][n][D], rounded to x's format */
    double* grad_x_abs;       /* [ntok][n][D]: sum of |terms| of each gradX element */
    double* grad_phi;         /* [M][n*D] */
    double* grad_phi_abs;
    double* grad_alpha;       /* [3] */
    double* grad_alpha_abs;
    double* grad_bias;        /* [M] */
    double* grad_bias_abs;
    double* grad_gamma;       /* [n][D] (only with gamma) */
    double* grad_gamma_abs;
    double* g_mix;            /* [T][M]: the gradient with respect to hMix ([BW] 3.5), for tests */
} oracle_bwd_out;

/* Stages 3.1-3.5 of [BW] for token t: the gradient with respect to hMix (gmix [M]), the
 * invRms gradient (*ginv), and the token's terms of the alpha and bias gradients
 * (ta [3], tb [M]). */
static void token_head(const oracle_bwd_in* in, int64_t t, double* gmix, double* ginv,
                       double* ta, double* tb)
{
    const int n = in->n, D = in->D, M = n * n + 2 * n;
    const int64_t K = (int64_t)n * D;
    const double eps = in->hc_eps;
    const double inv = (double)in->inv_rms[t];
    const double a0 = in->alpha[0], a1 = in->alpha[1], a2 = in->alpha[2];
    double gw[80];
    /* 3.1 hIn branch: the gradient of hPre is gradHIn . x_i over d */
    ta[0] = 0.0;
    for (int i = 0; i < n; ++i) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d)
            acc += x16_value(in, in->grad_h_in[t * D + d]) *
                   x16_value(in, in->x[t * K + (int64_t)i * D + d]);
        /* 3.2 sigmoid of the pre branch: s = hPre - hcEps, derivative s (1 - s) */
        const double s = (double)in->h_pre[t * n + i] - eps;
        const double g2 = acc * s * (1.0 - s);
        gw[i] = g2 * a0;
        ta[0] += g2 * ((double)in->h_mix[t * M + i] * inv);
        tb[i] = g2;
    }
    /* 3.3 post branch: hPost = 2 sigmoid(z), derivative hPost (1 - hPost / 2) */
    ta[1] = 0.0;
    for (int i = 0; i < n; ++i) {
        const double hp = in->h_post[t * n + i];
        const double g2 = (double)in->grad_h_post[t * n + i] * hp * (1.0 - hp / 2.0);
        gw[n + i] = g2 * a1;
        ta[1] += g2 * ((double)in->h_mix[t * M + n + i] * inv);
        tb[n + i] = g2;
    }
    /* 3.4 res branch: hRes = alpha2 pRes + bias_res (reading B1), or its Sinkhorn (B6):
     * then the gradient of the logits comes back through the saved planes first */
    double gl[64];
    for (int e = 0; e < n * n; ++e) gl[e] = in->grad_h_res[t * n * n + e];
    if (in->num_iters > 0) {
        const int64_t T = in->T;
        for (int k = 2 * in->num_iters - 1; k >= 1; --k) {
            const float* A = in->norm_out + ((int64_t)k * T + t) * n * n;
            const float* sk = in->sum_out + ((int64_t)k * T + t) * n;
            for (int i = 0; i < n; ++i) {
                double u = 0.0;   /* column i (k odd) or row i (k even) of G . A_k */
                for (int j = 0; j < n; ++j) {
                    const int e = (k % 2) ? j * n + i : i * n + j;
                    u += gl[e] * (double)A[e];
                }
                for (int j = 0; j < n; ++j) {
                    const int e = (k % 2) ? j * n + i : i * n + j;
                    gl[e] = (gl[e] - u) / (double)sk[i];
                }
            }
        }
        const float* A0 = in->norm_out + t * n * n;    /* step 0: row softmax + eps */
        for (int r = 0; r < n; ++r) {
            double u = 0.0;
            for (int c = 0; c < n; ++c) u += gl[r * n + c] * ((double)A0[r * n + c] - eps);
            for (int c = 0; c < n; ++c) gl[r * n + c] = ((double)A0[r * n + c] - eps) * (gl[r * n + c] - u);
        }
    }
    ta[2] = 0.0;
    for (int e = 0; e < n * n; ++e) {
        const double g = gl[e];
        gw[2 * n + e] = g * a2;
        ta[2] += g * ((double)in->h_mix[t * M + 2 * n + e] * inv);
        tb[2 * n + e] = g;
    }
    /* 3.5 w = hMix * invRms: gradient of hMix and of invRms */
    double gi = 0.0;
    for (int m = 0; m < M; ++m) {
        gmix[m] = gw[m] * inv;
        gi += gw[m] * (double)in->h_mix[t * M + m];
    }
    *ginv = gi;
}

int oracle_pre_backward(const oracle_bwd_in* in, const int64_t* tokens, int64_t ntok,
                        const oracle_bwd_out* o, int nthreads)
{
    if (!in || !o || !in->x || !in->phi || !in->alpha || !in->grad_h_in || !in->grad_h_post ||
        !in->grad_h_res || !in->inv_rms || !in->h_mix || !in->h_pre || !in->h_post)
        return -1;
    if (in->n < 1 || in->n > 8 || in->D < 1 || in->T < 0 || ntok < 0 || in->num_iters < 0) return -1;
    if (in->num_iters > 0 && (!in->sum_out || !in->norm_out)) return -1;
    if (tokens == NULL && ntok != in->T) return -1;
    for (int64_t j = 0; tokens && j < ntok; ++j)
        if (tokens[j] < 0 || tokens[j] >= in->T) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const int n = in->n, D = in->D, M = n * n + 2 * n;
    const int64_t T = in->T, K = (int64_t)n * D;

    /* per-token head for every token (the cross-token sums need all of them) */
    double* gmix = (double*)malloc(sizeof(double) * (size_t)(T * M + 1));
    double* ginv = (double*)malloc(sizeof(double) * (size_t)(T + 1));
    double* ta = (double*)malloc(sizeof(double) * (size_t)(T * 3 + 1));
    double* tb = (double*)malloc(sizeof(double) * (size_t)(T * M + 1));
    if (!gmix || !ginv || !ta || !tb) {
        free(gmix); free(ginv); free(ta); free(tb);
        return -1;
    }
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) token_head(in, t, gmix + t * M, ginv + t, ta + t * 3, tb + t * M);
    if (o->g_mix) memcpy(o->g_mix, gmix, sizeof(double) * (size_t)(T * M));

    /* 3.2-3.4 cross-token sums of the gate parameters, in token order */
    for (int a = 0; a < 3; ++a) {
        double s = 0.0, sa = 0.0;
        for (int64_t t = 0; t < T; ++t) { s += ta[t * 3 + a]; sa += fabs(ta[t * 3 + a]); }
        if (o->grad_alpha) o->grad_alpha[a] = s;
        if (o->grad_alpha_abs) o->grad_alpha_abs[a] = sa;
    }
    for (int m = 0; m < M; ++m) {
        double s = 0.0, sa = 0.0;
        for (int64_t t = 0; t < T; ++t) { s += tb[t * M + m]; sa += fabs(tb[t * M + m]); }
        if (o->grad_bias) o->grad_bias[m] = s;
        if (o->grad_bias_abs) o->grad_bias_abs[m] = sa;
    }

    /* 3.6-3.7 column sums: gradPhi[m][k] = sum_t gmix[t][m] x_rs[t][k],
     * gradGamma[k] = sum_t x[t][k] (gmix[t] . phi[:, k]); parallel over columns k */
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k) {
        double pk[80];
        for (int m = 0; m < M; ++m) pk[m] = in->phi[(int64_t)m * K + k];
        const double gk = in->gamma ? (double)in->gamma[k] : 1.0;
        double sp[80], spa[80], sg = 0.0, sga = 0.0;
        for (int m = 0; m < M; ++m) { sp[m] = 0.0; spa[m] = 0.0; }
        for (int64_t t = 0; t < T; ++t) {
            const double xv = x16_value(in, in->x[t * K + k]);
            const double xrs = xv * gk;
            double xg = 0.0, xga = 0.0;
            for (int m = 0; m < M; ++m) {
                const double p = gmix[t * M + m] * xrs;
                sp[m] += p;
                spa[m] += fabs(p);
                xg += gmix[t * M + m] * pk[m];
                xga += fabs(gmix[t * M + m] * pk[m]);
            }
            sg += xv * xg;
            sga += fabs(xv) * xga;
        }
        for (int m = 0; m < M; ++m) {
            if (o->grad_phi) o->grad_phi[(int64_t)m * K + k] = sp[m];
            if (o->grad_phi_abs) o->grad_phi_abs[(int64_t)m * K + k] = spa[m];
        }
        if (in->gamma && o->grad_gamma) o->grad_gamma[k] = sg;
        if (in->gamma && o->grad_gamma_abs) o->grad_gamma_abs[k] = sga;
    }

    /* 3.1 + 3.6-3.8 gradX rows of the listed tokens */
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < ntok; ++j) {
        const int64_t t = tokens ? tokens[j] : j;
        const double inv = (double)in->inv_rms[t];
        const double c3 = ginv[t] * inv * inv * inv / (double)K;   /* reading B2 */
        for (int i = 0; i < n; ++i) {
            const double hp = in->h_pre[t * n + i];
            for (int d = 0; d < D; ++d) {
                const int64_t k = (int64_t)i * D + d;
                const double xv = x16_value(in, in->x[t * K + k]);
                double mm = 0.0, mma = 0.0;
                for (int m = 0; m < M; ++m) {
                    const double p = gmix[t * M + m] * (double)in->phi[(int64_t)m * K + k];
                    mm += p;
                    mma += fabs(p);
                }
                const double gk = in->gamma ? (double)in->gamma[k] : 1.0;
                const double v3 = x16_value(in, in->grad_h_in[t * D + d]) * hp;
                const double vr = -c3 * xv;
                double g = v3 + mm * gk + vr;
                double ga = fabs(v3) + mma * fabs(gk) + fabs(vr);
                if (in->grad_x_post) {
                    const double gp = x16_value(in, in->grad_x_post[t * K + k]);
                    g += gp;
                    ga += fabs(gp);
                }
                const int64_t at = j * K + k;
                if (o->grad_x) o->grad_x[at] = g;
                if (o->grad_x_bits) o->grad_x_bits[at] = x16_round(in, g);
                if (o->grad_x_abs) o->grad_x_abs[at] = ga;
            }
        }
    }
    free(gmix); free(ginv); free(ta); free(tb);
    return 0;
}
