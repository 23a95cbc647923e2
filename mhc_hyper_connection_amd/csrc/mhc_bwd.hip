// mhc_bwd.hip -- gfx950 kernels of the MhcPre backward.
//
// Method (MhcPreBackward guide, 0539edu.com/news/4871844, section 3; forward in the
// aclnnMhcPreV2 guide, kwkr.cn/news/422178, section 3). Per token t, with the forward's
// saved invRms, hMix, hPre, hPost:
//   gHPre_i  = sum_d gradHIn[d] x[i, d]                                      (3.1)
//   gW       = [ gHPre s(1-s) alpha0 | gradHPost hPost(1-hPost/2) alpha1 |
//                gradHRes alpha2 ],  s = hPre - hcEps                        (3.2-3.4)
//   gMix     = gW invRms,  gInv = gW . hMix                                  (3.5)
//   xrsGrad  = gMix . phi                                                    (3.6)
//   gradX    = gradHIn hPre_i + xrsGrad gamma - gInv invRms^3 x / (n D)
//              (+ gradXPost)                                                 (3.7, 3.8)
// and over tokens: gradPhi = gamma (.) sum_t gMix^T x, gradGamma = sum_t x xrsGrad,
// gradAlpha / gradBias = sums of the gate terms.
//
// Kernels, in launch order on the caller's stream:
//   bwd_pack_kernel     phi -> three bf16 terms, ordered as the A operand of xrsGrad^T
//                       = phi^T . gMix^T per (d-block, stream, half, K-step, term)
//   bwd_token_kernel    one wave per token: the hPre gradient in fp64, the gate backward,
//                       gMix, c3 = gInv invRms^3 / (n D), and the token's alpha/bias terms
//   bwd_main_kernel     one workgroup per (token group, d-block, stream group): per tile
//                       of 64 tokens, xrsGrad on the matrix cores (phi terms x gMix terms,
//                       six products), gradX, the gradGamma sums, and gMix^T . x on the
//                       matrix cores with x transposed through LDS; group sums to partials
//   bwd_reduce_*        fixed-order fp64 sums of the partials (gradPhi, gradGamma) and
//                       of the per-token terms (gradAlpha, gradBias)
// x, gradHIn, gradXPost and gradX are bf16, or all fp16 (the guide's section 8.2: gradX
// takes gradHIn's type); template flag H selects fp16.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mhc_bwd_plan.h"
#include "mhc_device.h"

namespace mhc {
namespace bwd {
namespace {

// fp32 -> three bf16 terms whose sum is the value: hi = RNE(v), mid = RNE(v - hi),
// lo = RNE(v - hi - mid). Both differences are exact in fp32 (each removes the leading
// 8 significant bits), and lo holds the last 8.
struct Split3 {
    uint32_t t[3];
};
__device__ __forceinline__ Split3 split3(float v)
{
    Split3 s;
    s.t[0] = f32_to_bf16_bits(v);
    const float r1 = v - __uint_as_float(s.t[0] << 16);
    s.t[1] = f32_to_bf16_bits(r1);
    const float r2 = r1 - __uint_as_float(s.t[1] << 16);
    s.t[2] = f32_to_bf16_bits(r2);
    return s;
}

// Eight fp16 values -> two bf16 operands whose sum is each value exactly: hi = RNE(v)
// keeps 8 of its 11 significant bits; lo = v - hi is a multiple of v's fp16 ulp of at most
// 4 of them (3 significant bits), well inside bf16's exponent range.
__device__ __forceinline__ void split_f16x8(u32x4 w, bf16x8& hi, bf16x8& lo)
{
    u32x4 h, l;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
        const float v0 = f16_lo(w[e2]), v1 = f16_hi(w[e2]);
        h[e2] = pack_bf16x2(v0, v1);
        l[e2] = pack_bf16x2(v0 - bf16_lo(h[e2]), v1 - bf16_hi(h[e2]));
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}
// ------------------------------------------------------------------ weight pack

// Unit u = (((((b * n + i) * 2 + h) * KS + ks) * 3 + p) * 64 + lane holds, for lane
// (row = lane % 16, g = lane / 16), term p of phi[m][i D + d] for m = 32 ks + 8 g + e,
// e = 0..7, at d = 32 b + pack_col(h, row); zero past M or D. One thread writes the three
// terms of a (b, i, h, ks, lane), reading its eight weights once.
__global__ void __launch_bounds__(256)
bwd_pack_kernel(const float* __restrict__ phi, u32x4* __restrict__ pack, int n, int D, int M, int KS,
                int64_t triples)
{
    const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (v >= triples) return;
    const int lane = (int)(v % 64);
    int64_t r = v / 64;
    const int ks = (int)(r % KS);
    r /= KS;
    const int h = (int)(r % 2);
    r /= 2;
    const int i = (int)(r % n);
    const int b = (int)(r / n);
    const int row = lane % 16, g = lane / 16;
    const int d = kDBlock * b + pack_col(h, row);
    const int64_t K = (int64_t)n * D;
    u32x4 w[3] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    if (d < D) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int m = 32 * ks + 8 * g + e;
            if (m < M) {
                const Split3 sp = split3(phi[(int64_t)m * K + (int64_t)i * D + d]);
#pragma unroll
                for (int p = 0; p < 3; ++p) w[p][e >> 1] |= sp.t[p] << (16 * (e & 1));
            }
        }
    }
    const int64_t base = (((((int64_t)b * n + i) * 2 + h) * KS + ks) * 3) * 64 + lane;
#pragma unroll
    for (int p = 0; p < 3; ++p) pack[base + 64 * p] = w[p];
}

// ------------------------------------------------------------------ Sinkhorn backward

// MhcPreSinkhorn only: the residual logits' gradient through the forward's saved planes,
// fp64. 64 / (N*N) tokens per wave (one for n = 6, whose 36 entries do not tile a wave:
// lanes 36 to 63 then compute along from clamped addresses and store nothing), one lane
// per matrix entry e = r N + c. With G =
// gradHRes and, for k = 2 it - 1 down to 1, A_k = norm_out[k], s_k = sum_out[k]: a column
// step (k odd) passes G -> (G - sum_r G A_k) / s_k[c], a row step the same along the row;
// the first step (row softmax + eps) passes P (G - rowsum(G P)), P = A_0 - eps. The
// planes' loads and the reciprocals 1 / s_k go out ahead of the chain (all steps up to
// kSkAll, else kSkChunk at a time); row and column sums move values by DPP within a
// 16-lane row (across rows by __shfl_xor for the n = 8 columns); for n = 6 each lane
// gathers its row's (column's) entries by shuffles, in index order.
constexpr int kSkAll = 40;
constexpr int kSkChunk = 8;
template <int N>
__device__ __forceinline__ double sk_row_sum(double v, int r)
{
    if constexpr (N == 6) {
        double s = 0.0;
#pragma unroll
        for (int c = 0; c < N; ++c) s += __shfl(v, r * N + c);
        return s;
    }
    v += dpp<kQuadXor1>(v);
    v += dpp<kQuadXor2>(v);
    if constexpr (N == 8) v += dpp<kRowHalfMirror>(v);
    return v;
}
template <int N>
__device__ __forceinline__ double sk_col_sum(double v, int c)
{
    if constexpr (N == 6) {
        double s = 0.0;
#pragma unroll
        for (int r = 0; r < N; ++r) s += __shfl(v, r * N + c);
        return s;
    } else if constexpr (N == 4) {
        v += dpp<kRowRor4>(v);
        v += dpp<kRowRor8>(v);
    } else {
        v += dpp<kRowRor8>(v);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
    }
    return v;
}
template <int N>
__device__ __forceinline__ double sk_step(double G, float A, double rs, int k, int r, int c)
{
    const double u = (k & 1) ? sk_col_sum<N>(G * (double)A, c) : sk_row_sum<N>(G * (double)A, r);
    return (G - u) * rs;
}

template <int N>
__global__ void __launch_bounds__(256)
bwd_sinkhorn_kernel(Args a, int64_t T)
{
    constexpr int NN = N * N;
    constexpr int SW = 64 % NN == 0 ? NN : 64;      // lanes per matrix
    constexpr int TPW = 64 / SW;                    // tokens per wave
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e = lane < TPW * SW ? (lane % SW < NN ? lane % SW : NN - 1) : NN - 1;   // clamped entry
    const bool ent = lane % SW < NN;                // the lane holds an entry of its matrix
    const int er = e / N, ec = e % N;
    const int64_t t = ((int64_t)blockIdx.x * 4 + wave) * TPW + lane / SW;
    const bool live = t < T && ent;                 // groups of SW lanes: live or not as a whole
    const int64_t tt = live ? t : T - 1;            // loads stay in bounds and unpredicated
    const int steps = 2 * a.num_iters;
    // Loads under a branch make the compiler wait for each one before the next; every
    // load here is issued unconditionally from a clamped address and its value selected.
    auto A_at = [&](int k) {
        const float v = a.norm_out[((int64_t)(k >= 0 ? k : 0) * T + tt) * NN + e];
        return (live && k >= 0) ? v : 0.f;
    };
    auto s_at = [&](int k) {
        const float v = a.sum_out[((int64_t)(k >= 0 ? k : 0) * T + tt) * N + ((k & 1) ? ec : er)];
        return (live && k >= 0) ? v : 1.f;
    };
    const float g0 = a.grad_h_res[tt * NN + e];
    double G = live ? (double)g0 : 0.0;
    if (steps <= kSkAll) {
        float A[kSkAll];
        double R[kSkAll];
#pragma unroll
        for (int j = 0; j < kSkAll; ++j) {
            const int k = steps - 1 - j;
            A[j] = A_at(k);
            R[j] = 1.0 / (double)s_at(k);
        }
#pragma unroll
        for (int j = 0; j < kSkAll; ++j) {
            const int k = steps - 1 - j;
            if (k >= 1) G = sk_step<N>(G, A[j], R[j], k, er, ec);   // uniform across the wave
        }
    } else {
        for (int k0 = steps - 1; k0 >= 1; k0 -= kSkChunk) {
            float A[kSkChunk];
            double R[kSkChunk];
#pragma unroll
            for (int j = 0; j < kSkChunk; ++j) {
                const int k = k0 - j;
                A[j] = A_at(k);
                R[j] = 1.0 / (double)s_at(k);
            }
#pragma unroll
            for (int j = 0; j < kSkChunk; ++j) {
                const int k = k0 - j;
                if (k >= 1) G = sk_step<N>(G, A[j], R[j], k, er, ec);
            }
        }
    }
    const double P = (double)A_at(0) - a.hc_eps;
    const double u = sk_row_sum<N>(G * P, er);
    if (live) a.glog[t * NN + e] = P * (G - u);
}

// ------------------------------------------------------------------ token pass

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// One wave per token (4 per workgroup). Outputs: gMix [T][KS][3][32] (three bf16 terms
// of each f32 value, zero past M), c3 [T], terms [3 + M][T] (fp64: the token's alpha
// terms, then its bias terms).
template <int N, bool H>
__global__ void __launch_bounds__(256)
bwd_token_kernel(Args a, int64_t T, int D)
{
    constexpr int M = N * N + 2 * N;
    constexpr int MP = 32 * ((M + 31) / 32);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + wave;
    if (t >= T) return;
    const int64_t K = (int64_t)N * D;

    // 3.1: gHPre_i = sum_d gradHIn[d] x[i, d]; a product of two bf16 or two fp16 values is
    // exact in fp32 (at most 22 significant bits), the sums run in fp64 (per lane, then
    // across lanes)
    double acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = 0.0;
    const uint16_t* xt = a.x + t * K;
    const uint16_t* gt = a.grad_h_in + t * D;
    for (int o = lane; o < D / 8; o += 64) {
        const u32x4 gh = *reinterpret_cast<const u32x4*>(gt + 8 * o);
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const u32x4 xv = *reinterpret_cast<const u32x4*>(xt + (int64_t)i * D + 8 * o);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[i] += (double)(x16_lo<H>(gh[e]) * x16_lo<H>(xv[e]));
                acc[i] += (double)(x16_hi<H>(gh[e]) * x16_hi<H>(xv[e]));
            }
        }
    }
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = wave_sum(acc[i]);
    const double eps = a.hc_eps;

    // The residual logits' gradient, one lane per matrix entry: gradHRes itself (MhcPre),
    // or what bwd_sinkhorn_kernel passed back through the Sinkhorn planes.
    constexpr int NN = N * N;
    const bool ent = lane < NN;
    const double gres = !ent ? 0.0
                      : (a.num_iters > 0 ? a.glog[t * NN + lane] : (double)a.grad_h_res[t * NN + lane]);

    // 3.2-3.5, one lane per phi row m (two passes when MP > 64)
    const double inv = (double)a.inv_rms[t];
    const double a0 = a.alpha[0], a1 = a.alpha[1], a2 = a.alpha[2];
    double gi = 0.0, ta0 = 0.0, ta1 = 0.0, ta2 = 0.0;
    // the logit gradient of phi row m (m >= 2N) sits in lane m - 2N; fetched here, with
    // every lane active, for both passes of the loop below
    const double gl_pass[2] = {__shfl(gres, (lane - 2 * N) & 63), __shfl(gres, (lane + 64 - 2 * N) & 63)};
    for (int m = lane; m < MP; m += 64) {
        double gw = 0.0;
        const double gl = gl_pass[m >= 64];
        if (m < M) {
            const double w = (double)a.h_mix[t * M + m] * inv;   // the gate input
            double tb;
            if (m < N) {
                double ghp = 0.0;
#pragma unroll
                for (int i = 0; i < N; ++i) ghp = i == m ? acc[i] : ghp;
                const double s = (double)a.h_pre[t * N + m] - eps;
                tb = ghp * s * (1.0 - s);
                gw = tb * a0;
                ta0 += tb * w;
            } else if (m < 2 * N) {
                const double hq = a.h_post[t * N + (m - N)];
                tb = (double)a.grad_h_post[t * N + (m - N)] * hq * (1.0 - hq / 2.0);
                gw = tb * a1;
                ta1 += tb * w;
            } else {
                tb = gl;
                gw = tb * a2;
                ta2 += tb * w;
            }
            gi += gw * (double)a.h_mix[t * M + m];
            a.terms[(3 + m) * T + t] = tb;
        }
        const Split3 sp = split3((float)(gw * inv));
        uint16_t* dst = a.gmix + (t * (MP / 32) + m / 32) * 3 * 32 + m % 32;
#pragma unroll
        for (int p = 0; p < 3; ++p) dst[32 * p] = (uint16_t)sp.t[p];
    }
    gi = wave_sum(gi);
    ta0 = wave_sum(ta0);
    ta1 = wave_sum(ta1);
    ta2 = wave_sum(ta2);
    if (lane == 0) {
        a.c3[t] = (float)(gi * inv * inv * inv / (double)K);
        a.terms[0 * T + t] = ta0;
        a.terms[1 * T + t] = ta1;
        a.terms[2 * T + t] = ta2;
    }
}

// ------------------------------------------------------------------ main pass

// Products of A terms (phi) and B terms (gMix) kept for xrsGrad, smallest first: every
// pair (p, q) with p + q <= 2, i.e. down to 2^-16 of the leading product; the dropped
// pairs are below 2^-24 of it.
constexpr int kPairs = 6;
constexpr int pair_a(int q) { return q == 0 ? 2 : (q == 1 ? 0 : (q == 2 ? 1 : (q == 3 ? 1 : 0))); }
constexpr int pair_b(int q) { return q == 0 ? 0 : (q == 1 ? 2 : (q == 2 ? 1 : (q == 3 ? 0 : (q == 4 ? 1 : 0)))); }

// Transposed LDS rows ([column or m][64 tokens], 128 bytes) hold their eight 8-token
// chunks in a row-dependent order: chunk c of row r sits at c ^ swz(r). A 16-byte
// operand read (8 consecutive tokens of 16 rows r0..r0+15) then spreads over all banks,
// and so do the scattered 2-byte writes of one instruction (8 positions g*8 + e of a
// token, for the four lane groups g).
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ (((r >> 3) & 3) << 1); }
__device__ __forceinline__ int tslot(int r, int tok) { return r * kTile + (((tok >> 3) ^ swz(r)) << 3) + (tok & 7); }

template <int N, int SGN, int KS>
struct MainCfg {
    static constexpr int M = N * N + 2 * N;
    static constexpr int MP = 32 * KS;
    static constexpr int NCOL = kDBlock * SGN;           // local columns of a workgroup
    static constexpr int RB = MP / 16;                    // gradPhi row blocks
    static constexpr int CB = NCOL / 16;                  // gradPhi column blocks
    static constexpr int BPW = RB * CB / 4;               // gradPhi blocks per wave
    static constexpr int PACK_U = SGN * 2 * KS * 3 * 64;  // 16-byte units of packed phi
    static constexpr int XS = kTile;                      // bf16 per transposed-x row
    static constexpr int GXS = kTile;                     // bf16 per transposed-gMix row
    static constexpr int PACK_BYTES = PACK_U * 16;
    static constexpr int XT_BYTES = NCOL * XS * 2;
    static constexpr int GT_BYTES = 3 * MP * GXS * 2;     // three terms
    static constexpr int RED_BYTES = kTile * NCOL * 4;    // gradGamma reduction at the end
    static constexpr int MAIN_BYTES = PACK_BYTES + XT_BYTES + GT_BYTES;
    static constexpr int LDS_BYTES = MAIN_BYTES > RED_BYTES ? MAIN_BYTES : RED_BYTES;
    static_assert((RB * CB) % 4 == 0, "gradPhi blocks divide among the four waves");
    static_assert(CB % 4 == 0, "wave w's gradPhi blocks use column blocks w, w + 4, ..");
    static_assert(XT_BYTES % 16 == 0 && PACK_BYTES % 16 == 0, "LDS regions stay 16-byte aligned");
};

// GAMMA: gamma given (gradX scales xrsGrad, gradGamma is summed); XPOST: gradXPost given;
// H: x, gradHIn, gradXPost and gradX in fp16 (x then enters gMix^T . x as two exact bf16
// terms, six products instead of three).
template <int N, int SGN, int KS, bool GAMMA, bool XPOST, bool H>
__global__ void __launch_bounds__(kThreads, GAMMA ? 2 : 3)
bwd_main_kernel(Args a, int64_t T, int D, int nblk, int64_t tpg, int64_t tiles, int64_t tasks)
{
    using C = MainCfg<N, SGN, KS>;
    constexpr int M = C::M, MP = C::MP, NCOL = C::NCOL, CB = C::CB, BPW = C::BPW;
    constexpr int NSG = N / SGN;
    __shared__ __attribute__((aligned(16))) char lds[C::LDS_BYTES];
    u32x4* sp = reinterpret_cast<u32x4*>(lds);
    uint16_t* xT = reinterpret_cast<uint16_t*>(lds + C::PACK_BYTES);
    uint16_t* gT = reinterpret_cast<uint16_t*>(lds + C::PACK_BYTES + C::XT_BYTES);   // [term][m][token]

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int j = lane & 15, grp = lane >> 4;
    int64_t g;
    int b, sg;
    if (!main_task(blockIdx.x, nblk, NSG, tasks, &g, &b, &sg)) return;   // padding workgroup
    const int64_t K = (int64_t)N * D;
    const int d0 = kDBlock * b + 8 * grp;          // the lane's 8 positions d0 .. d0+7
    const bool dval = d0 < D;                        // D % 8 == 0: all 8 or none

    // the workgroup's packed phi (its d-block, its streams) into LDS
    {
        const u32x4* src = static_cast<const u32x4*>(a.pack) + pack_at(b, sg * SGN, N, KS);
        for (int u = tid; u < C::PACK_U; u += kThreads) sp[u] = src[u];
    }
    float gam[GAMMA ? SGN : 1][8];
    if constexpr (GAMMA) {
#pragma unroll
        for (int s = 0; s < SGN; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) gam[s][e] = dval ? a.gamma[(int64_t)(sg * SGN + s) * D + d0 + e] : 1.f;
    }

    float gg[GAMMA ? SGN : 1][8];
#pragma unroll
    for (int s = 0; s < (GAMMA ? SGN : 1); ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) gg[s][e] = 0.f;
    f32x4 pacc[BPW];
#pragma unroll
    for (int q = 0; q < BPW; ++q) pacc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();

    // A tile's per-lane inputs, loaded one tile ahead: the next tile's loads go out as
    // soon as the current tile's registers are consumed and stay in flight through the
    // gradPhi phase. Rows past the tile and positions past D read as zero.
    const int row = 16 * wave + j;                   // the lane's token in a tile
    // DB: x and gradHIn are loaded a whole tile ahead, into the other of two register sets
    // (where the registers allow it: no gamma, and not fp16 with gradXPost); the rest of a
    // tile's inputs after its predecessor's first phase, as with a single set
    constexpr bool DB = !GAMMA && !(XPOST && H);
    u32x4 xv[SGN], xv2[DB ? SGN : 1], xp[SGN], gh, gh2, gmt[KS][3];
    float hp[SGN], c3;
    auto load_xg = [&](int64_t tl, u32x4 (&xd)[SGN], u32x4& ghd) {
        const int64_t t0 = tl * kTile;
        const int ntile = (int)(T - t0 < kTile ? T - t0 : kTile);
        const rsrc_t rx = make_rsrc(a.x + t0 * K, (int64_t)ntile * K * 2);
        const rsrc_t rgh = make_rsrc(a.grad_h_in + t0 * D, (int64_t)ntile * D * 2);
#pragma unroll
        for (int s = 0; s < SGN; ++s) {
            const uint32_t off = dval ? (uint32_t)(((int64_t)row * K + (int64_t)(sg * SGN + s) * D + d0) * 2) : kOutOfRange;
            xd[s] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0);
        }
        ghd = __builtin_amdgcn_raw_buffer_load_b128(rgh, dval ? (int)(((int64_t)row * D + d0) * 2) : (int)kOutOfRange, 0, 0);
    };
    auto load_rest = [&](int64_t tl) {
        const int64_t t0 = tl * kTile;
        const int ntile = (int)(T - t0 < kTile ? T - t0 : kTile);
        const rsrc_t rgm = make_rsrc(a.gmix + t0 * (3 * MP), (int64_t)ntile * 3 * MP * 2);
        if constexpr (XPOST) {
            const rsrc_t rxp = make_rsrc(a.grad_x_post + t0 * K, (int64_t)ntile * K * 2);
#pragma unroll
            for (int s = 0; s < SGN; ++s) {
                const uint32_t off = dval ? (uint32_t)(((int64_t)row * K + (int64_t)(sg * SGN + s) * D + d0) * 2) : kOutOfRange;
                xp[s] = __builtin_amdgcn_raw_buffer_load_b128(rxp, (int)off, 0, 0);
            }
        }
        // gMix terms of the lane's token: B operand of xrsGrad (K-step ks, term p)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int p = 0; p < 3; ++p)
                gmt[ks][p] = __builtin_amdgcn_raw_buffer_load_b128(
                    rgm, (int)((((int64_t)row * KS + ks) * 3 * 32 + 32 * p + 8 * grp) * 2), 0, 0);
        // hPre and c3 through buffer loads too: rows past the tile read as zero with no
        // branch (a load under a branch leaves the compiler no exact wait count)
        const rsrc_t rhp = make_rsrc(a.h_pre + t0 * N, (int64_t)ntile * N * 4);
        const rsrc_t rc3 = make_rsrc(a.c3 + t0, (int64_t)ntile * 4);
#pragma unroll
        for (int s = 0; s < SGN; ++s)
            hp[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rhp, (row * N + sg * SGN + s) * 4, 0, 0));
        c3 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rc3, row * 4, 0, 0));
    };

    const int64_t tile_end = (g + 1) * tpg < tiles ? (g + 1) * tpg : tiles;
    load_xg(g * tpg, xv, gh);
    load_rest(g * tpg);
    auto step = [&](int64_t tile, u32x4 (&xc)[SGN], u32x4& ghc, u32x4 (&xn)[SGN], u32x4& ghn) __attribute__((always_inline)) {
        // the next tile's loads go out unconditionally (the last tile loads itself again), so
        // that every wait below has an exact count
        const int64_t nt = tile + 1 < tile_end ? tile + 1 : tile;
        if constexpr (DB) load_xg(nt, xn, ghn);
        const int64_t t0 = tile * kTile;
        const int ntile = (int)(T - t0 < kTile ? T - t0 : kTile);

        // xrsGrad^T = phi^T . gMix^T: A = packed phi (columns as rows), B = gMix (tokens)
        bf16x8 bt[KS][3];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int p = 0; p < 3; ++p) bt[ks][p] = __builtin_bit_cast(bf16x8, gmt[ks][p]);
        const rsrc_t rgx = make_rsrc(a.grad_x + t0 * K, (int64_t)ntile * K * 2);
#pragma unroll
        for (int s = 0; s < SGN; ++s) {
            float xg[8];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                    for (int q = 0; q < kPairs; ++q) {
                        const bf16x8 av = __builtin_bit_cast(
                            bf16x8, sp[(((s * 2 + h) * KS + ks) * 3 + pair_a(q)) * 64 + lane]);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bt[ks][pair_b(q)], acc, 0, 0, 0);
                    }
#pragma unroll
                for (int r = 0; r < 4; ++r) xg[4 * h + r] = acc[r];
            }
            // gradX = gradHIn hPre + xrsGrad gamma - c3 x (+ gradXPost), one RNE to x's format
            u32x4 o;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                float v[2];
#pragma unroll
                for (int hl = 0; hl < 2; ++hl) {
                    const int e = 2 * e2 + hl;
                    const float xe = hl ? x16_hi<H>(xc[s][e2]) : x16_lo<H>(xc[s][e2]);
                    const float ge = hl ? x16_hi<H>(ghc[e2]) : x16_lo<H>(ghc[e2]);
                    v[hl] = fmaf(ge, hp[s], GAMMA ? xg[e] * gam[GAMMA ? s : 0][e] : xg[e]);
                    v[hl] = fmaf(-c3, xe, v[hl]);
                    if constexpr (XPOST) v[hl] += hl ? x16_hi<H>(xp[s][e2]) : x16_lo<H>(xp[s][e2]);
                    if constexpr (GAMMA) gg[s][e] = fmaf(xe, xg[e], gg[s][e]);
                }
                o[e2] = pack_x16<H>(v[0], v[1]);
            }
            const uint32_t off = dval ? (uint32_t)(((int64_t)row * K + (int64_t)(sg * SGN + s) * D + d0) * 2) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b128(o, rgx, (int)off, 0, 0);
            // x of this tile, transposed: xT[local column][token]
#pragma unroll
            for (int e = 0; e < 8; ++e)
                xT[tslot(s * kDBlock + 8 * grp + e, row)] = (uint16_t)((xc[s][e >> 1] >> (16 * (e & 1))) & 0xffffu);
        }
        // gMix terms of this tile, transposed: gT[p][m][token]
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int p = 0; p < 3; ++p)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    gT[tslot(p * MP + 32 * ks + 8 * grp + e, row)] =
                        (uint16_t)((gmt[ks][p][e >> 1] >> (16 * (e & 1))) & 0xffffu);
        if constexpr (!DB) load_xg(nt, xn, ghn);
        load_rest(nt);
        __syncthreads();

        // gradPhi partial: C[m][col] += sum over the tile's tokens of gMix[t][m] x[t][col];
        // A = gMix^T (rows m, three terms), B = x (columns), 32 tokens per K-step. Block
        // bi = wave + 4 q has column block (wave + 4 q) % CB = wave + 4 (q % NCW): fp16 x
        // is split into its two bf16 terms once per column block and K-step.
        constexpr int NCW = CB / 4;
        bf16x8 bxh[H ? NCW : 1][2], bxl[H ? NCW : 1][2];
        if constexpr (H) {
#pragma unroll
            for (int c = 0; c < NCW; ++c)
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
                    split_f16x8(*reinterpret_cast<const u32x4*>(xT + tslot(16 * (wave + 4 * c) + j, 32 * kt + 8 * grp)),
                                bxh[c][kt], bxl[c][kt]);
        }
#pragma unroll
        for (int q = 0; q < BPW; ++q) {
            const int bi = wave + 4 * q;
            const int rb = bi / CB, cb = bi % CB;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                bf16x8 at[3];
#pragma unroll
                for (int p = 0; p < 3; ++p)
                    at[p] = *reinterpret_cast<const bf16x8*>(gT + tslot(p * MP + 16 * rb + j, 32 * kt + 8 * grp));
                if constexpr (H) {
                    const int c = q % NCW;
#pragma unroll
                    for (int p = 2; p >= 0; --p)
                        pacc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(at[p], bxl[c][kt], pacc[q], 0, 0, 0);
#pragma unroll
                    for (int p = 2; p >= 0; --p)
                        pacc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(at[p], bxh[c][kt], pacc[q], 0, 0, 0);
                } else {
                    const bf16x8 bv = *reinterpret_cast<const bf16x8*>(xT + tslot(16 * cb + j, 32 * kt + 8 * grp));
#pragma unroll
                    for (int p = 2; p >= 0; --p)
                        pacc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(at[p], bv, pacc[q], 0, 0, 0);
                }
            }
        }
        __syncthreads();   // xT and gT are rewritten by the next tile
    };
    if constexpr (DB) {
        for (int64_t tile = g * tpg; tile < tile_end; tile += 2) {
            step(tile, xv, gh, xv2, gh2);
            if (tile + 1 < tile_end) step(tile + 1, xv2, gh2, xv, gh);
        }
    } else {
        for (int64_t tile = g * tpg; tile < tile_end; ++tile) step(tile, xv, gh, xv, gh);
    }

    // gradPhi partial of the group: P[g][m][k], k = stream * D + d
    float* const P = a.pphi + g * (int64_t)M * K;
#pragma unroll
    for (int q = 0; q < BPW; ++q) {
        const int bi = wave + 4 * q;
        const int rb = bi / CB, cb = bi % CB;
        const int col = 16 * cb + j;                 // local column
        const int s = col / kDBlock, dd = kDBlock * b + col % kDBlock;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 16 * rb + 4 * grp + r;
            if (m < M && dd < D) P[(int64_t)m * K + (int64_t)(sg * SGN + s) * D + dd] = pacc[q][r];
        }
    }
    // gradGamma partial of the group: sum the 64 token lanes of each column in a fixed order
    if constexpr (GAMMA) {
        float* red = reinterpret_cast<float*>(lds);   // [64 token lanes][NCOL]
#pragma unroll
        for (int s = 0; s < SGN; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[(16 * wave + j) * NCOL + s * kDBlock + 8 * grp + e] = gg[s][e];
        __syncthreads();
        for (int col = tid; col < NCOL; col += kThreads) {
            float v = 0.f;
            for (int rr = 0; rr < kTile; ++rr) v += red[rr * NCOL + col];
            const int s = col / kDBlock, dd = kDBlock * b + col % kDBlock;
            if (dd < D) a.pgam[g * K + (int64_t)(sg * SGN + s) * D + dd] = v;
        }
    }
}

// ------------------------------------------------------------------ reductions

// gradPhi[m][k] = gamma[k] * sum_g P[g][m][k]; gradGamma[k] = sum_g Q[g][k] (fp64, g order)
__global__ void __launch_bounds__(256)
bwd_reduce_cols_kernel(Args a, int64_t MK, int64_t K, int64_t G)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx < MK) {
        // the group partials in group order, eight loads issued before their sums
        double s = 0.0;
        int64_t gg = 0;
        for (; gg + 8 <= G; gg += 8) {
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = a.pphi[(gg + q) * MK + idx];
#pragma unroll
            for (int q = 0; q < 8; ++q) s += (double)v[q];
        }
        for (; gg < G; ++gg) s += (double)a.pphi[gg * MK + idx];
        if (a.gamma) s *= (double)a.gamma[idx % K];
        a.grad_phi[idx] = (float)s;
    } else if (idx < MK + K && a.gamma) {
        const int64_t k = idx - MK;
        double s = 0.0;
        for (int64_t gg = 0; gg < G; ++gg) s += (double)a.pgam[gg * K + k];
        a.grad_gamma[k] = (float)s;
    }
}

// Workgroup c sums row c of terms [3 + M][T] over the tokens: 1024 threads, thread i
// summing tokens i, i + 1024, ... in that order (four loads in flight), then a fixed
// tree. c < 3: gradAlpha[c]; else gradBias[c - 3].
constexpr int kRedThreads = 1024;
__global__ void __launch_bounds__(kRedThreads)
bwd_reduce_terms_kernel(Args a, int64_t T, int M)
{
    __shared__ double part[kRedThreads];
    const int c = blockIdx.x, tid = threadIdx.x;
    const double* row = a.terms + c * T;
    double s = 0.0;
    int64_t t = tid;
    for (; t + 3 * kRedThreads < T; t += 4 * kRedThreads) {
        const double v0 = row[t], v1 = row[t + kRedThreads], v2 = row[t + 2 * kRedThreads],
                     v3 = row[t + 3 * kRedThreads];
        s += v0;
        s += v1;
        s += v2;
        s += v3;
    }
    for (; t < T; t += kRedThreads) s += row[t];
    part[tid] = s;
    __syncthreads();
    for (int w = kRedThreads / 2; w >= 1; w >>= 1) {
        if (tid < w) part[tid] += part[tid + w];
        __syncthreads();
    }
    if (tid == 0) {
        if (c < 3) a.grad_alpha[c] = (float)part[0];
        else a.grad_bias[c - 3] = (float)part[0];
    }
}

// T == 0: every cross-token gradient is an empty sum.
__global__ void __launch_bounds__(256)
bwd_zero_kernel(Args a, int64_t MK, int64_t K, int M)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx < MK) a.grad_phi[idx] = 0.f;
    if (idx < K && a.gamma) a.grad_gamma[idx] = 0.f;
    if (idx < 3) a.grad_alpha[idx] = 0.f;
    if (idx < M) a.grad_bias[idx] = 0.f;
}

template <int N, int SGN, int KS, bool GAMMA, bool XPOST, bool H>
void launch_main(const Plan& p, const Args& a, hipStream_t st)
{
    hipLaunchKernelGGL((bwd_main_kernel<N, SGN, KS, GAMMA, XPOST, H>), dim3((unsigned)p.main_blocks),
                       dim3(kThreads), 0, st, a, p.T, p.g.D, p.g.nblk, p.tpg, p.tiles, p.main_tasks);
}

template <int N, int SGN, int KS, bool H>
hipError_t launch_all(const Plan& p, const Args& a, hipStream_t st)
{
    const Geometry& g = p.g;
    const int64_t triples = (int64_t)g.nblk * g.n * pack_units_per_stream(g.KS) / 3;   // one thread each
    hipLaunchKernelGGL(bwd_pack_kernel, dim3((unsigned)((triples + 255) / 256)), dim3(256), 0, st, a.phi,
                       static_cast<u32x4*>(a.pack), g.n, g.D, g.M, g.KS, triples);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.num_iters > 0) {
        constexpr int tok_per_block = 4 * (64 / (N * N));
        hipLaunchKernelGGL(bwd_sinkhorn_kernel<N>, dim3((unsigned)((p.T + tok_per_block - 1) / tok_per_block)),
                           dim3(256), 0, st, a, p.T);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_token_kernel<N, H>), dim3((unsigned)p.token_blocks), dim3(256), 0, st, a, p.T, g.D);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.gamma) {
        if (a.grad_x_post) launch_main<N, SGN, KS, true, true, H>(p, a, st);
        else launch_main<N, SGN, KS, true, false, H>(p, a, st);
    } else {
        if (a.grad_x_post) launch_main<N, SGN, KS, false, true, H>(p, a, st);
        else launch_main<N, SGN, KS, false, false, H>(p, a, st);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t MK = (int64_t)g.M * g.K;
    hipLaunchKernelGGL(bwd_reduce_cols_kernel, dim3((unsigned)((MK + g.K + 255) / 256)), dim3(256), 0, st, a,
                       MK, g.K, p.G);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_reduce_terms_kernel, dim3((unsigned)(3 + g.M)), dim3(kRedThreads), 0, st, a, p.T, g.M);
    return hipGetLastError();
}

}  // namespace

int launch_backward(const Plan& p, const Args& a, void* stream)
{
    clear_pending_error();
    hipStream_t st = (hipStream_t)stream;
    const Geometry& g = p.g;
    if (p.T == 0) {
        const int64_t MK = (int64_t)g.M * g.K;
        hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)((MK + 255) / 256)), dim3(256), 0, st, a, MK, g.K, g.M);
        return (int)hipGetLastError();
    }
    if (g.n == 4 && g.SGN == 4 && g.KS == 1)
        return (int)(g.x_f16 ? launch_all<4, 4, 1, true>(p, a, st) : launch_all<4, 4, 1, false>(p, a, st));
    if (g.n == 6 && g.SGN == 2 && g.KS == 2)
        return (int)(g.x_f16 ? launch_all<6, 2, 2, true>(p, a, st) : launch_all<6, 2, 2, false>(p, a, st));
    if (g.n == 8 && g.SGN == 2 && g.KS == 3)
        return (int)(g.x_f16 ? launch_all<8, 2, 3, true>(p, a, st) : launch_all<8, 2, 3, false>(p, a, st));
    return (int)hipErrorInvalidValue;
}

}  // namespace bwd
}  // namespace mhc
