// mhc_kernels.hip -- gfx950 kernels of the fused mHC pre-mapping forward.
//
// Method (aclnnMhcPreV2 guide, kwkr.cn/news/422178, section 3; aclnnMhcPreSinkhorn guide,
// m.mzlw.cn/news/197063, section 3.2): per token, invRms over the n*D entries, the
// projection hMix = (x * gamma) . phi^T, sigmoid gates, a 2*numIters-step Sinkhorn of
// the n x n residual logits, and hIn = sum_i weight_i * x_i.
//
// Kernels
//   prepack_kernel  phi (f32) * gamma -> three bf16 terms (hi, mid, lo) in the chunked,
//                   octet-major order the projection consumes (layout in mhc_plan.h).
//   proj_kernel     one workgroup = 64 tokens x one d-slice of the reduction. x goes from
//                   HBM straight into MFMA A-registers (16-byte loads, no LDS); the packed
//                   weights of each 128-element chunk are staged in LDS and shared by the
//                   4 waves. v_mfma_f32_16x16x32_bf16 accumulates the 3*M columns; the
//                   "hi" columns are moved into fp64 every kFlush chunks so long fp32
//                   chains do not limit hMix accuracy. Squares are summed on the VALU
//                   from the same registers. Each workgroup writes fp32 partial sums; the
//                   last of the S workgroups of a tile (atomic ticket) reduces them in a
//                   fixed order (deterministic), then runs the gates and the Sinkhorn and
//                   writes every output except hIn, plus the hIn weights.
//   hin_kernel      hIn[t, d] = sum_i w[t, i] x[t, i, d], fp32 FMA, one rounding to bf16.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mhc_plan.h"

namespace mhc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kFlush = 2;   // chunks (8 MFMA K-steps) between fp64 flushes of the hi columns

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ double bf16_bits_to_double(uint32_t b)
{
    return (double)__uint_as_float(b << 16);
}

struct KArgs {
    ForwardArgs a;
    int64_t T;
    int64_t K;
    int D;
    int M;
    int S;
    int nch;
    int dc;
    int pstride;
    int n_alpha;
};

// ------------------------------------------------------------------ weight pre-pack

__global__ void __launch_bounds__(256)
prepack_kernel(const float* __restrict__ phi, const float* __restrict__ gamma,
               u32x4* __restrict__ packed, int n, int D, int M, int NC, int dc, int nch)
{
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)nch * kOctets * NC;
    if (u >= total) return;
    const int c = (int)(u % NC);
    const int64_t r = u / NC;
    const int q = (int)(r % kOctets);
    const int ch = (int)(r / kOctets);
    const int d0 = ch * dc + 8 * (q / n);
    u32x4 w = {0u, 0u, 0u, 0u};
    if (c < 3 * M && d0 < D) {
        const int term = c / M;
        const int m = c % M;
        const int64_t K = (int64_t)n * D;
        const int64_t k0 = (int64_t)(q % n) * D + d0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // exact product in double, then hi/mid/lo each the nearest bf16 of what is left
            double p = (double)phi[(int64_t)m * K + k0 + e];
            if (gamma) p *= (double)gamma[k0 + e];
            const uint32_t hb = f32_to_bf16_bits((float)p);
            const double r1 = p - bf16_bits_to_double(hb);
            const uint32_t mb = f32_to_bf16_bits((float)r1);
            const double r2 = r1 - bf16_bits_to_double(mb);
            const uint32_t lb = f32_to_bf16_bits((float)r2);
            const uint32_t bits = term == 0 ? hb : (term == 1 ? mb : lb);
            w[e >> 1] |= bits << (16 * (e & 1));
        }
    }
    packed[u] = w;
}

// ------------------------------------------------------------------ epilogue (one token)

__device__ __forceinline__ double sigmoid_d(double z)
{
    if (z >= 0.0) return 1.0 / (1.0 + exp(-z));
    const double e = exp(z);
    return e / (1.0 + e);
}

// Reduces the S partial records of token t in slice order, then the gates, Sinkhorn and
// every per-token output. Runs on one thread per token (the tile's last workgroup).
template <int N>
__device__ void epilogue_token(const KArgs& k, int64_t t)
{
    const ForwardArgs& a = k.a;
    const int M = k.M;
    const int64_t T = k.T;
    const float* part = a.part + t * k.pstride;
    const int64_t sstride = T * (int64_t)k.pstride;

    double ss = 0.0;
    for (int s = 0; s < k.S; ++s) ss += (double)part[s * sstride + M];
    const double inv_rms = 1.0 / sqrt(ss / (double)k.K + a.norm_eps);
    if (a.inv_rms) a.inv_rms[t] = (float)inv_rms;

    const double eps = a.hc_eps;
    const double a0 = a.alpha[0], a1 = a.alpha[1];
    const double a2 = k.n_alpha == 3 ? (double)a.alpha[2] : 0.0;
    float L[N * N];
#pragma unroll
    for (int i = 0; i < N * N; ++i) L[i] = 0.f;

    for (int m = 0; m < M; ++m) {
        double hm = 0.0;
        for (int s = 0; s < k.S; ++s) hm += (double)part[s * sstride + m];
        if (a.h_mix) a.h_mix[t * M + m] = (float)hm;
        const double w = hm * inv_rms;
        if (m < N) {
            const double hp = sigmoid_d(a0 * w + (double)a.bias[m]) + eps;
            if (a.h_pre) a.h_pre[t * N + m] = (float)hp;
            a.wts[t * N + m] = a.pre_mix ? a.pre_mix[t * N + m] : (float)hp;
        } else if (m < 2 * N) {
            double hq = 2.0 * sigmoid_d(a1 * w + (double)a.bias[m]);
            if (k.n_alpha == 2) hq += eps;
            a.h_post[t * N + (m - N)] = (float)hq;
        } else {
            const float z = (float)(a2 * w + (double)a.bias[m]);
#pragma unroll
            for (int i = 0; i < N * N; ++i)
                if (i == m - 2 * N) L[i] = z;
        }
    }

    if (k.n_alpha != 3) {
        if (a.h_res)
            for (int i = 0; i < N * N; ++i) a.h_res[t * N * N + i] = 0.f;
        return;
    }

    // Sinkhorn: step 0 softmax over each row + eps; odd steps normalise columns, even
    // steps rows; every sum gets + eps; 2*num_iters steps.
    const float epsf = (float)eps;
    const int steps = 2 * a.num_iters;
    float sums[N];
#pragma unroll
    for (int r = 0; r < N; ++r) {
        float mx = L[r * N];
#pragma unroll
        for (int c = 1; c < N; ++c) mx = fmaxf(mx, L[r * N + c]);
        float sum = 0.f;
#pragma unroll
        for (int c = 0; c < N; ++c) {
            L[r * N + c] = expf(L[r * N + c] - mx);
            sum += L[r * N + c];
        }
#pragma unroll
        for (int c = 0; c < N; ++c) L[r * N + c] = L[r * N + c] / sum + epsf;
        sums[r] = sum;
    }
    for (int step = 0; step < steps; ++step) {
        if (step > 0) {
            if (step & 1) {
#pragma unroll
                for (int c = 0; c < N; ++c) {
                    float sum = 0.f;
#pragma unroll
                    for (int r = 0; r < N; ++r) sum += L[r * N + c];
                    sum += epsf;
#pragma unroll
                    for (int r = 0; r < N; ++r) L[r * N + c] = L[r * N + c] / sum;
                    sums[c] = sum;
                }
            } else {
#pragma unroll
                for (int r = 0; r < N; ++r) {
                    float sum = 0.f;
#pragma unroll
                    for (int c = 0; c < N; ++c) sum += L[r * N + c];
                    sum += epsf;
#pragma unroll
                    for (int c = 0; c < N; ++c) L[r * N + c] = L[r * N + c] / sum;
                    sums[r] = sum;
                }
            }
        }
        if (a.sum_out) {
            float* so = a.sum_out + ((int64_t)step * T + t) * N;
#pragma unroll
            for (int i = 0; i < N; ++i) so[i] = sums[i];
        }
        if (a.norm_out) {
            float* no = a.norm_out + ((int64_t)step * T + t) * (N * N);
#pragma unroll
            for (int i = 0; i < N * N; ++i) no[i] = L[i];
        }
    }
#pragma unroll
    for (int i = 0; i < N * N; ++i) a.h_res[t * N * N + i] = L[i];
}

// ------------------------------------------------------------------ projection

template <int NT, int NTHI, int N>
__global__ void __launch_bounds__(kThreads)
proj_kernel(KArgs k)
{
    constexpr int NC = 16 * NT;
    __shared__ u32x4 lds[kOctets * NC];                 // one chunk of packed weights
    __shared__ float lds_ss[kTileTokens][4];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int j = lane & 15;      // A row (token) / B column / D column
    const int grp = lane >> 4;    // K-group of A and B; row block of D
    const int64_t tile = blockIdx.x / k.S;
    const int s = (int)(blockIdx.x % k.S);
    const int ch0 = slice_begin(k.nch, k.S, s);
    const int ch1 = slice_begin(k.nch, k.S, s + 1);

    // A-operand token of this lane; rows past T re-read the last token, results dropped.
    int64_t tok = tile * kTileTokens + wave * 16 + j;
    if (tok > k.T - 1) tok = k.T - 1;
    const uint16_t* xrow = k.a.x + tok * k.K;

    // Element offset inside a chunk, and d-offset, of the octet this lane feeds at K-step st.
    int off[4], dof[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const int q = 4 * st + grp;
        dof[st] = 8 * (q / N);
        off[st] = (q % N) * k.D + dof[st];
    }

    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    double hacc[NTHI][4];
#pragma unroll
    for (int nt = 0; nt < NTHI; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) hacc[nt][r] = 0.0;
    float ssq = 0.f;

    const u32x4* packed = static_cast<const u32x4*>(k.a.packed);
    int since_flush = 0;
    for (int ch = ch0; ch < ch1; ++ch) {
        __syncthreads();
        const u32x4* src = packed + (int64_t)ch * (kOctets * NC);
#pragma unroll
        for (int i = 0; i < NT; ++i) lds[tid + kThreads * i] = src[tid + kThreads * i];
        __syncthreads();
        const int dbase = ch * k.dc;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            u32x4 av = {0u, 0u, 0u, 0u};
            if (dbase + dof[st] < k.D) av = *reinterpret_cast<const u32x4*>(xrow + off[st] + dbase);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = bf16_lo(av[e]), hi = bf16_hi(av[e]);
                ssq = fmaf(lo, lo, ssq);
                ssq = fmaf(hi, hi, ssq);
            }
            const bf16x8 A = __builtin_bit_cast(bf16x8, av);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const u32x4 bv = lds[(4 * st + grp) * NC + nt * 16 + j];
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8, bv),
                                                                  acc[nt], 0, 0, 0);
            }
        }
        if (++since_flush == kFlush) {
            since_flush = 0;
#pragma unroll
            for (int nt = 0; nt < NTHI; ++nt) {
#pragma unroll
                for (int r = 0; r < 4; ++r) hacc[nt][r] += (double)acc[nt][r];
                acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }
#pragma unroll
    for (int nt = 0; nt < NTHI; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) hacc[nt][r] += (double)acc[nt][r];

    // Per-column totals of this slice into LDS ([64 tokens][NC], fp32), squares per group.
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = wave * 16 + 4 * grp + r;
            const float v = nt < NTHI ? (float)hacc[nt < NTHI ? nt : 0][r] : acc[nt][r];
            red[row * NC + nt * 16 + j] = v;
        }
    lds_ss[wave * 16 + j][grp] = ssq;
    __syncthreads();

    if (tid < kTileTokens) {
        const int64_t t = tile * kTileTokens + tid;
        if (t < k.T) {
            float* dst = k.a.part + ((int64_t)s * k.T + t) * k.pstride;
            const float* rr = red + tid * NC;
            for (int m = 0; m < k.M; ++m)
                dst[m] = (float)((double)rr[m] + (double)rr[k.M + m] + (double)rr[2 * k.M + m]);
            dst[k.M] = (lds_ss[tid][0] + lds_ss[tid][1]) + (lds_ss[tid][2] + lds_ss[tid][3]);
        }
    }

    // Last-arriver hand-off: the S workgroups of this tile take a ticket; the one that
    // completes the count owns the epilogue and resets the counter for the next call.
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        const int prev = atomicAdd(&k.a.tickets[tile], 1);
        s_last = (prev == k.S - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (tid == 0) k.a.tickets[tile] = 0;
    if (tid < kTileTokens) {
        const int64_t t = tile * kTileTokens + tid;
        if (t < k.T) epilogue_token<N>(k, t);
    }
}

// ------------------------------------------------------------------ hIn

template <int N>
__global__ void __launch_bounds__(256)
hin_kernel(const uint16_t* __restrict__ x, const float* __restrict__ wts,
           uint16_t* __restrict__ h_in, int64_t T, int D)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int D8 = D / 8;
    const int64_t t = idx / D8;
    const int d8 = (int)(idx % D8);
    if (t >= T) return;
    float w[N];
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = wts[t * N + i];
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(x + (t * N + i) * (int64_t)D + d8 * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] = fmaf(w[i], bf16_lo(v[e]), acc[2 * e]);
            acc[2 * e + 1] = fmaf(w[i], bf16_hi(v[e]), acc[2 * e + 1]);
        }
    }
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o[e] = f32_to_bf16_bits(acc[2 * e]) | (f32_to_bf16_bits(acc[2 * e + 1]) << 16);
    *reinterpret_cast<u32x4*>(h_in + t * (int64_t)D + d8 * 8) = o;
}

template <int NT, int NTHI, int N>
hipError_t launch_proj(const Plan& p, const KArgs& k, hipStream_t st)
{
    hipLaunchKernelGGL((proj_kernel<NT, NTHI, N>), dim3((unsigned)p.blocks), dim3(kThreads), 0, st, k);
    return hipGetLastError();
}

}  // namespace

int launch_prepack(const Geometry& g, const float* phi, const float* gamma, void* packed,
                   void* stream)
{
    const int64_t total = (int64_t)g.nch * kOctets * g.NC;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    hipLaunchKernelGGL(prepack_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, phi, gamma,
                       static_cast<u32x4*>(packed), g.n, g.D, g.M, g.NC, g.dc, g.nch);
    return (int)hipGetLastError();
}

int launch_forward(const Plan& p, const ForwardArgs& a, void* stream)
{
    if (p.T <= 0) return 0;
    hipStream_t st = (hipStream_t)stream;
    KArgs k;
    k.a = a;
    k.T = p.T;
    k.K = p.g.K;
    k.D = p.g.D;
    k.M = p.g.M;
    k.S = p.S;
    k.nch = p.g.nch;
    k.dc = p.g.dc;
    k.pstride = p.pstride;
    k.n_alpha = p.g.n_alpha;

    hipError_t e;
    if (p.g.n == 4 && p.g.n_alpha == 3) e = launch_proj<5, 2, 4>(p, k, st);
    else if (p.g.n == 4 && p.g.n_alpha == 2) e = launch_proj<2, 1, 4>(p, k, st);
    else if (p.g.n == 8 && p.g.n_alpha == 3) e = launch_proj<15, 5, 8>(p, k, st);
    else if (p.g.n == 8 && p.g.n_alpha == 2) e = launch_proj<3, 1, 8>(p, k, st);
    else return (int)hipErrorInvalidValue;
    if (e != hipSuccess) return (int)e;

    const int64_t items = p.T * (int64_t)(p.g.D / 8);
    const unsigned hb = (unsigned)((items + 255) / 256);
    if (p.g.n == 4)
        hipLaunchKernelGGL(hin_kernel<4>, dim3(hb), dim3(256), 0, st, a.x, a.wts, a.h_in, p.T, p.g.D);
    else
        hipLaunchKernelGGL(hin_kernel<8>, dim3(hb), dim3(256), 0, st, a.x, a.wts, a.h_in, p.T, p.g.D);
    return (int)hipGetLastError();
}

}  // namespace mhc
