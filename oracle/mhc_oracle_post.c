/* mhc_oracle_post.c -- fp64 oracle of hc_post, the mHC post-mapping (TEST INFRASTRUCTURE).
 *
 * Source: HcPre guide (mhpn.cn/news/2282827), section "mHC 架构与 HcPre 的定位": the
 * layer output is expanded back into the n streams by the post mapping and added to the
 * streams after the res mapping has fused them across streams. The page prints the
 * expression as torch broadcasting, and its section "返回值说明" gives comb_frag the
 * shape [b, s, hc_mult, hc_mult] (or [T, hc_mult, hc_mult]) and the streams [b, s,
 * hc_mult, d]. Evaluated on those 4-D shapes, comb.unsqueeze(-1) * residual.unsqueeze(-2)
 * pairs comb's first stream index with the residual's stream, and the sum over dim 2 runs
 * over that index, so output stream j takes column j of comb:
 *     out[t][j][d] = post[t][j] * x[t][d] + sum_i comb[t][i][j] * residual[t][i][d]
 * (a transposed product, comb^T residual; with Sinkhorn's last step normalising columns,
 * every output stream is then a convex combination of the residual streams).
 * x and residual are bf16 (exact in double), post and comb f32; the sum is exact in
 * double up to one rounding per addition, then rounded once to bf16 (nearest, ties to
 * even). out_abs is the sum of |terms| of each element (for the acceptance rule).
 * Parity pins: tests/test_oracle_post.py (the page's expression evaluated by numpy
 * broadcasting on 4-D arrays, permutation mixing, column sums, post-only, a library
 * einsum, planted mistakes).
 */
#include <stdint.h>
#include <math.h>

double oracle_bf16_to_double(uint16_t bits);
uint16_t oracle_bf16_from_double(double v);
double oracle_f16_to_double(uint16_t bits);
uint16_t oracle_f16_from_double(double v);

/* x_f16: x, residual and out in binary16 instead of bf16 (the 16-bit format of the
 * pre-mapping's x and hIn); the arithmetic is unchanged. */
int oracle_mhc_post_fmt(int64_t T, int n, int D, const uint16_t* x, const uint16_t* residual,
                        const float* post, const float* comb, uint16_t* out_bf16, double* out,
                        double* out_abs, int x_f16)
{
    if (T < 0 || n < 1 || D < 1) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int j = 0; j < n; ++j) {           /* output stream */
            const double p = (double)post[t * n + j];
            for (int d = 0; d < D; ++d) {
                const double xv = x_f16 ? oracle_f16_to_double(x[t * D + d]) : oracle_bf16_to_double(x[t * D + d]);
                double acc = p * xv;
                double mag = fabs(p * xv);
                for (int i = 0; i < n; ++i) {   /* summed index: comb's first, the residual's stream */
                    const double c = (double)comb[(t * n + i) * n + j];
                    const uint16_t rb = residual[(t * n + i) * (int64_t)D + d];
                    const double r = x_f16 ? oracle_f16_to_double(rb) : oracle_bf16_to_double(rb);
                    acc += c * r;
                    mag += fabs(c * r);
                }
                const int64_t o = (t * n + j) * (int64_t)D + d;
                if (out) out[o] = acc;
                if (out_abs) out_abs[o] = mag;
                if (out_bf16) out_bf16[o] = x_f16 ? oracle_f16_from_double(acc) : oracle_bf16_from_double(acc);
            }
        }
    }
    return 0;
}

int oracle_mhc_post(int64_t T, int n, int D, const uint16_t* x, const uint16_t* residual,
                    const float* post, const float* comb, uint16_t* out_bf16, double* out,
                    double* out_abs)
{
    return oracle_mhc_post_fmt(T, n, D, x, residual, post, comb, out_bf16, out, out_abs, 0);
}
