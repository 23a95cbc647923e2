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
//   proj_kernel     one workgroup = 64 tokens x one K-slice of the reduction. x goes from
//                   HBM straight into MFMA A-registers (16-byte loads, no LDS); the packed
//                   weights of each 128-element chunk are staged in LDS (double-buffered,
//                   prefetched one chunk ahead) and shared by the 4 waves; x is prefetched
//                   two chunks ahead. v_mfma_f32_16x16x32_bf16 accumulates the 3*M columns; the
//                   "hi" columns are moved into fp64 every kFlush chunks so long fp32
//                   chains do not limit hMix accuracy. Squares come from the diagonal of
//                   x x^T on the matrix cores, from the same registers. Each workgroup writes fp32 partial sums; the
//                   last of the S workgroups of a tile (atomic ticket) reduces them in a
//                   fixed order (deterministic), then runs the gates and a lane-parallel
//                   Sinkhorn and writes every output except hIn, plus the hIn weights.
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
    int pstride;
    int n_alpha;
};

// ------------------------------------------------------------------ weight pre-pack

__global__ void __launch_bounds__(256)
prepack_kernel(const float* __restrict__ phi, const float* __restrict__ gamma,
               u32x4* __restrict__ packed, int64_t K, int M, int NC, int nch)
{
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)(nch + 1) * kOctets * NC;
    if (u >= total) return;
    const int c = (int)(u % NC);
    const int64_t r = u / NC;
    const int q = (int)(r % kOctets);
    const int64_t ch = r / kOctets;
    const int64_t k0 = ch * kChunk + 8 * q;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (c < 3 * M && k0 < K) {
        const int term = c / M;
        const int m = c % M;
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

// ------------------------------------------------------------------ tile epilogue

__device__ __forceinline__ float sigmoidf_stable(float z)
{
    if (z >= 0.f) return 1.f / (1.f + expf(-z));
    const float e = expf(z);
    return e / (1.f + e);
}

template <int N>
__device__ __forceinline__ float row_sum(float v)
{
#pragma unroll
    for (int m = 1; m < N; m <<= 1) v += __shfl_xor(v, m);
    return v;
}
template <int N>
__device__ __forceinline__ float row_max(float v)
{
#pragma unroll
    for (int m = 1; m < N; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}
template <int N>
__device__ __forceinline__ float col_sum(float v)
{
#pragma unroll
    for (int m = N; m < N * N; m <<= 1) v += __shfl_xor(v, m);
    return v;
}

// Runs on all threads of the tile's last workgroup. `scratch` is LDS of at least
// 64*(M+1)*8 + 64*8 + 64*N*N*4 bytes.
//   A  sum the S partial records of each (token, value) in slice order (fp64)
//   B  invRms per token
//   C  hMix, gates and residual logits, one (token, row) item per thread
//   D  Sinkhorn with one lane per matrix entry: 2*num_iters steps, row / column sums by
//      cross-lane shuffles, coalesced stores of every plane
template <int N>
__device__ void tile_epilogue(const KArgs& k, int64_t tile, char* scratch)
{
    constexpr int NN = N * N;
    const ForwardArgs& a = k.a;
    const int tid = threadIdx.x;
    const int M = k.M;
    const int R = M + 1;
    const int64_t T = k.T;
    const int64_t t0 = tile * kTileTokens;
    double* hm = reinterpret_cast<double*>(scratch);                  // [64][R]
    double* inv = hm + kTileTokens * R;                               // [64]
    float* Ls = reinterpret_cast<float*>(inv + kTileTokens);          // [64][NN]

    // A: partial sums, eight slices in flight at a time, added in slice order
    for (int idx = tid; idx < kTileTokens * R; idx += kThreads) {
        const int tl = idx / R, m = idx % R;
        const int64_t t = t0 + tl;
        double acc = 0.0;
        if (t < T) {
            const float* p = a.part + t * k.pstride + m;
            const int64_t ss = T * (int64_t)k.pstride;
            for (int s = 0; s < k.S; s += 8) {
                float v[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = (s + i < k.S) ? p[(s + i) * ss] : 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) acc += (double)v[i];
            }
        }
        hm[idx] = acc;
    }
    __syncthreads();

    // B: invRms = (mean of squares over n*D + normEps)^(-1/2)
    if (tid < kTileTokens) {
        const int64_t t = t0 + tid;
        const double r = 1.0 / sqrt(hm[tid * R + M] / (double)k.K + a.norm_eps);
        inv[tid] = r;
        if (t < T && a.inv_rms) a.inv_rms[t] = (float)r;
    }
    __syncthreads();

    // C: w = hMix * invRms; pre / post gates; residual logits
    const float eps = (float)a.hc_eps;
    for (int idx = tid; idx < kTileTokens * M; idx += kThreads) {
        const int tl = idx / M, m = idx % M;
        const int64_t t = t0 + tl;
        const double h = hm[tl * R + m];
        const double w = h * inv[tl];
        if (t < T && a.h_mix) a.h_mix[t * M + m] = (float)h;
        if (m < N) {
            const float hp = sigmoidf_stable((float)((double)a.alpha[0] * w + (double)a.bias[m])) + eps;
            if (t < T) {
                if (a.h_pre) a.h_pre[t * N + m] = hp;
                a.wts[t * N + m] = a.pre_mix ? a.pre_mix[t * N + m] : hp;
            }
        } else if (m < 2 * N) {
            float hq = 2.f * sigmoidf_stable((float)((double)a.alpha[1] * w + (double)a.bias[m]));
            if (k.n_alpha == 2) hq += eps;
            if (t < T) a.h_post[t * N + (m - N)] = hq;
        } else {
            Ls[tl * NN + (m - 2 * N)] = (float)((double)a.alpha[2] * w + (double)a.bias[m]);
        }
    }
    if (k.n_alpha != 3) {
        if (a.h_res)
            for (int idx = tid; idx < kTileTokens * NN; idx += kThreads)
                if (t0 + idx / NN < T) a.h_res[t0 * NN + idx] = 0.f;
        return;
    }
    __syncthreads();

    // D: Sinkhorn. Lane = (token slot, r, c) with c in the low bits: row sums are xor
    // shuffles over the c bits, column sums over the r bits.
    constexpr int TPW = 64 / NN;                        // tokens per wave per round
    const int lane = tid & 63, wave = tid >> 6;
    const int e = lane % NN, r = e / N, c = e % N;
    const int steps = 2 * a.num_iters;
    for (int base = 0; base < kTileTokens; base += kWaves * TPW) {
        const int tl = base + wave * TPW + lane / NN;
        const int64_t t = t0 + tl;
        const bool live = t < T;
        float v = Ls[tl * NN + e];
        const float mx = row_max<N>(v);
        const float ex = expf(v - mx);
        float sum = row_sum<N>(ex);
        v = ex / sum + eps;
        for (int step = 0; step < steps; ++step) {
            if (step > 0) {
                if (step & 1) sum = col_sum<N>(v) + eps;
                else sum = row_sum<N>(v) + eps;
                v = v / sum;
            }
            if (live) {
                if (a.sum_out) {
                    const bool writer = (step & 1) ? (r == 0) : (c == 0);
                    if (writer) a.sum_out[((int64_t)step * T + t) * N + ((step & 1) ? c : r)] = sum;
                }
                if (a.norm_out) a.norm_out[((int64_t)step * T + t) * NN + e] = v;
            }
        }
        if (live) a.h_res[t * NN + e] = v;
    }
}

// ------------------------------------------------------------------ projection

// x for one full chunk: lane (token row, group g) takes octets g, 4+g, 8+g, 12+g of
// the chunk, i.e. 16 bytes at element offset 8*(4*st + g) for K-step st. The four loads
// of a lane cover 64 of the row's 256 contiguous bytes; the 4 groups together cover
// both cache lines.
__device__ __forceinline__ void load_x_full(const uint16_t* xrow, int64_t base, int grp, u32x4 (&xr)[4])
{
#pragma unroll
    for (int st = 0; st < 4; ++st)
        xr[st] = *reinterpret_cast<const u32x4*>(xrow + base + 8 * (4 * st + grp));
}

// The same for the last chunk of a row when K is not a multiple of 128: octets at or
// beyond K read as zero.
__device__ __forceinline__ void load_x_tail(const uint16_t* xrow, int64_t base, int64_t K, int grp,
                                            u32x4 (&xr)[4])
{
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const int64_t k0 = base + 8 * (4 * st + grp);
        xr[st] = k0 < K ? *reinterpret_cast<const u32x4*>(xrow + k0) : u32x4{0u, 0u, 0u, 0u};
    }
}

// Matrix-core work of one chunk held in x registers `xr` and LDS weight buffer `w`:
// 4 K-steps x NT column tiles, plus the x tile times its own transpose, whose diagonal
// accumulates each token's sum of squares (exact bf16 products, fp32 sums), and the
// periodic fp64 flush of the hi columns.
template <int NT, int NTHI>
__device__ __forceinline__ void mma_chunk(const u32x4 (&xr)[4], const u32x4* w, int grp, int j,
                                          f32x4 (&acc)[NT], double (&hacc)[NTHI][4], f32x4& sq,
                                          int& since_flush)
{
    constexpr int NC = 16 * NT;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const u32x4 av = xr[st];
        const bf16x8 A = __builtin_bit_cast(bf16x8, av);
        sq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, A, sq, 0, 0, 0);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const u32x4 bv = w[(4 * st + grp) * NC + nt * 16 + j];
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

// One pipelined step over full chunk `ch`: first the weight loads of chunk ch+1 into
// registers and the x loads of chunk ch+2 into `xn` (whose last readers were the
// previous step's MFMAs, behind that step's barrier); then the chunk's MFMAs from `xc` and
// LDS buffer BUF; then the weights go to the other LDS buffer and one barrier closes
// the step. The packed weights end with a zero chunk, so the weight prefetch never
// needs a bounds test.
template <int NT, int NTHI>
__device__ __forceinline__ void proj_step(int BUF, int ch, int chf, int tid, int grp, int j, const KArgs& k,
                                          const uint16_t* xrow, const u32x4 (&xc)[4], u32x4 (&xn)[4],
                                          u32x4 (*lds)[kOctets * 16 * NT], f32x4 (&acc)[NT],
                                          double (&hacc)[NTHI][4], f32x4& sq, int& since_flush)
{
    constexpr int UNITS = kOctets * 16 * NT;
    // Weights first: the load counter retires in issue order, so the wait for them at
    // the end of the step must not also cover the x prefetch issued after them.
    const u32x4* src = static_cast<const u32x4*>(k.a.packed) + (int64_t)(ch + 1) * UNITS;
    u32x4 pre[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) pre[i] = src[tid + kThreads * i];
    if (ch + 2 < chf) load_x_full(xrow, (int64_t)(ch + 2) * kChunk, grp, xn);
    mma_chunk<NT, NTHI>(xc, lds[BUF], grp, j, acc, hacc, sq, since_flush);
#pragma unroll
    for (int i = 0; i < NT; ++i) lds[BUF ^ 1][tid + kThreads * i] = pre[i];
    __syncthreads();
}

template <int NT, int NTHI, int N>
__global__ void __launch_bounds__(kThreads)
proj_kernel(KArgs k)
{
    constexpr int NC = 16 * NT;
    constexpr int UNITS = kOctets * NC;
    __shared__ u32x4 lds[2][UNITS];                     // double-buffered weight chunks
    __shared__ float lds_ss[kTileTokens];
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

    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    double hacc[NTHI][4];
#pragma unroll
    for (int nt = 0; nt < NTHI; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) hacc[nt][r] = 0.0;
    f32x4 sq = {0.f, 0.f, 0.f, 0.f};   // x x^T of this wave's 16 tokens; diagonal = squares
    int since_flush = 0;

    // Full chunks [ch0, chf) run through a 3-buffer x pipeline (two chunks in flight
    // ahead of the one being multiplied) and a 2-buffer LDS weight pipeline; a partial
    // last chunk of the row (K not a multiple of 128) is done after it.
    const int nfull = (int)(k.K / kChunk);
    const int chf = ch1 < nfull ? ch1 : nfull;
    u32x4 x0[4], x1[4], x2[4];
    const u32x4* packed = static_cast<const u32x4*>(k.a.packed);
    if (ch0 < chf) load_x_full(xrow, (int64_t)ch0 * kChunk, grp, x0);
    if (ch0 + 1 < chf) load_x_full(xrow, (int64_t)(ch0 + 1) * kChunk, grp, x1);
    if (ch0 < ch1) {
#pragma unroll
        for (int i = 0; i < NT; ++i) lds[0][tid + kThreads * i] = packed[(int64_t)ch0 * UNITS + tid + kThreads * i];
    }
    __syncthreads();

    int ch = ch0;
    while (ch < chf) {
        proj_step<NT, NTHI>((ch - ch0) & 1, ch, chf, tid, grp, j, k, xrow, x0, x2, lds, acc, hacc, sq, since_flush);
        if (++ch >= chf) break;
        proj_step<NT, NTHI>((ch - ch0) & 1, ch, chf, tid, grp, j, k, xrow, x1, x0, lds, acc, hacc, sq, since_flush);
        if (++ch >= chf) break;
        proj_step<NT, NTHI>((ch - ch0) & 1, ch, chf, tid, grp, j, k, xrow, x2, x1, lds, acc, hacc, sq, since_flush);
        ++ch;
    }
    if (chf < ch1) {
        // partial last chunk; its weights are in LDS buffer (chf - ch0) & 1
        load_x_tail(xrow, (int64_t)chf * kChunk, k.K, grp, x0);
        mma_chunk<NT, NTHI>(x0, lds[(chf - ch0) & 1], grp, j, acc, hacc, sq, since_flush);
        __syncthreads();
    }
#pragma unroll
    for (int nt = 0; nt < NTHI; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) hacc[nt][r] += (double)acc[nt][r];

    // Per-column totals of this slice into LDS ([64 tokens][NC], fp32), squares per group.
    // (The last step ended with a barrier, so LDS buffer 0 is free.)
    float* red = reinterpret_cast<float*>(&lds[0][0]);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = wave * 16 + 4 * grp + r;
            const float v = nt < NTHI ? (float)hacc[nt < NTHI ? nt : 0][r] : acc[nt][r];
            red[row * NC + nt * 16 + j] = v;
        }
    // diagonal element (i, i) of x x^T sits in lane i + 12*(i/4) (i % 16 == lane % 16),
    // register i % 4
    {
        const int rr = j - 4 * grp;
        if (rr >= 0 && rr < 4) lds_ss[wave * 16 + j] = sq[rr];
    }
    __syncthreads();

    // Partial record of this slice: M projections (hi + mid + lo) and the square sum.
    const int R = k.M + 1;
    for (int idx = tid; idx < kTileTokens * R; idx += kThreads) {
        const int tl = idx / R, m = idx % R;
        const int64_t t = tile * kTileTokens + tl;
        if (t >= k.T) continue;
        float v;
        if (m < k.M) {
            const float* rr = red + tl * NC;
            v = (float)((double)rr[m] + (double)rr[k.M + m] + (double)rr[2 * k.M + m]);
        } else {
            v = lds_ss[tl];
        }
        k.a.part[((int64_t)s * k.T + t) * k.pstride + m] = v;
    }
}

// One workgroup per 64-token tile: reduce the tile's S partial records (written by the
// projection launch that precedes this one on the stream), then gates, Sinkhorn and
// all per-token outputs.
template <int N>
__global__ void __launch_bounds__(kThreads)
epilogue_kernel(KArgs k)
{
    constexpr int MMAX = N * N + 2 * N;
    __shared__ double scratch[kTileTokens * (MMAX + 1) + kTileTokens + kTileTokens * N * N / 2];
    tile_epilogue<N>(k, blockIdx.x, reinterpret_cast<char*>(scratch));
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
    const int64_t total = (int64_t)(g.nch + 1) * kOctets * g.NC;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    hipLaunchKernelGGL(prepack_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, phi, gamma,
                       static_cast<u32x4*>(packed), g.K, g.M, g.NC, g.nch);
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
    k.pstride = p.pstride;
    k.n_alpha = p.g.n_alpha;

    hipError_t e;
    if (p.g.n == 4 && p.g.n_alpha == 3) e = launch_proj<5, 2, 4>(p, k, st);
    else if (p.g.n == 4 && p.g.n_alpha == 2) e = launch_proj<2, 1, 4>(p, k, st);
    else if (p.g.n == 8 && p.g.n_alpha == 3) e = launch_proj<15, 5, 8>(p, k, st);
    else if (p.g.n == 8 && p.g.n_alpha == 2) e = launch_proj<3, 1, 8>(p, k, st);
    else return (int)hipErrorInvalidValue;
    if (e != hipSuccess) return (int)e;
    if (p.g.n == 4)
        hipLaunchKernelGGL(epilogue_kernel<4>, dim3((unsigned)p.tiles), dim3(kThreads), 0, st, k);
    else
        hipLaunchKernelGGL(epilogue_kernel<8>, dim3((unsigned)p.tiles), dim3(kThreads), 0, st, k);
    e = hipGetLastError();
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
