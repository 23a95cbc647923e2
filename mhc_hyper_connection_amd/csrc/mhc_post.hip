// mhc_post.hip -- gfx950 kernel of hc_post, the mHC post-mapping (HcPre guide,
// mhpn.cn/news/2282827, section "mHC 架构与 HcPre 的定位": the layer output expanded into
// the n streams by post, added to the streams fused across streams by comb). The guide's
// broadcast expression, on the [b, s, n, n] comb_frag its section "返回值说明" documents,
// sums over comb's first index, so output stream j takes column j of comb:
//     out[t][j][d] = post[t][j] x[t][d] + sum_i comb[t][i][j] residual[t][i][d]
//
// One thread per octet (8 positions) of one token: it reads the octet of x and of each of
// the n residual streams (16-byte loads, consecutive threads on consecutive octets), the
// token's post and comb (shared by the token's threads, cached), and writes the octet of
// each of the n output streams. fp32 fused multiply-adds in the order post term, then
// i = 0 .. n-1; one rounding to bf16 (fp16 when the tensors are fp16). Memory-bound: per
// token 2D + 2nD bytes read (+ 4n + 4n^2), 2nD written.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mhc_device.h"
#include "mhc_plan.h"

namespace mhc {
namespace {

template <int N, bool H>
__global__ void __launch_bounds__(256)
post_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ residual,
            const float* __restrict__ post, const float* __restrict__ comb,
            uint16_t* __restrict__ out, int64_t T, int D)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int D8 = D / 8;
    const int64_t t = idx / D8;
    const int d8 = (int)(idx % D8);
    if (t >= T) return;
    const u32x4 xv = *reinterpret_cast<const u32x4*>(x + t * (int64_t)D + d8 * 8);
    u32x4 rv[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
        rv[i] = *reinterpret_cast<const u32x4*>(residual + (t * N + i) * (int64_t)D + d8 * 8);
#pragma unroll
    for (int j = 0; j < N; ++j) {   // output stream
        const float p = post[t * N + j];
        float c[N];                 // column j of comb
#pragma unroll
        for (int i = 0; i < N; ++i) c[i] = comb[(t * N + i) * N + j];
        float acc[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] = p * x16_lo<H>(xv[e]);
            acc[2 * e + 1] = p * x16_hi<H>(xv[e]);
        }
#pragma unroll
        for (int i = 0; i < N; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] = fmaf(c[i], x16_lo<H>(rv[i][e]), acc[2 * e]);
                acc[2 * e + 1] = fmaf(c[i], x16_hi<H>(rv[i][e]), acc[2 * e + 1]);
            }
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = pack_x16<H>(acc[2 * e], acc[2 * e + 1]);
        // the output is not read again here: stream it past the caches
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out + (t * N + j) * (int64_t)D + d8 * 8));
    }
}

}  // namespace

int launch_post(int64_t T, int n, int D, const uint16_t* x, const uint16_t* residual, const float* post,
                const float* comb, uint16_t* out, int x_f16, void* stream)
{
    clear_pending_error();
    if (T <= 0) return 0;
    const int64_t items = T * (int64_t)(D / 8);
    const dim3 grid((unsigned)((items + 255) / 256));
    hipStream_t st = (hipStream_t)stream;
#define MHC_POST(NV, HV) hipLaunchKernelGGL((post_kernel<NV, HV>), grid, dim3(256), 0, st, x, residual, post, comb, out, T, D)
    if (n == 4 && !x_f16) MHC_POST(4, false);
    else if (n == 6 && !x_f16) MHC_POST(6, false);
    else if (n == 8 && !x_f16) MHC_POST(8, false);
    else if (n == 4) MHC_POST(4, true);
    else if (n == 6) MHC_POST(6, true);
    else if (n == 8) MHC_POST(8, true);
    else return (int)hipErrorInvalidValue;
#undef MHC_POST
    return (int)hipGetLastError();
}

}  // namespace mhc
