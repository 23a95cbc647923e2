// mhc_kernels.hip -- gfx950 kernels of the mHC pre-mapping forward.
//
// Method (aclnnMhcPreV2 guide, kwkr.cn/news/422178, section 3; aclnnMhcPreSinkhorn guide,
// m.mzlw.cn/news/197063, section 3.2): per token, invRms over the n*D entries, the
// projection hMix = (x * gamma) . phi^T, sigmoid gates, a 2*numIters-step Sinkhorn of
// the n x n residual logits, and hIn = sum_i weight_i * x_i.
//
// Kernels (one launch each, in this order on the caller's stream)
//   prepack_kernel   phi (f32) * gamma -> three bf16 terms (hi, mid, lo) in the K-step
//                    order the projection consumes (layout in mhc_plan.h); only when the
//                    caller passes no packed weights.
//   proj_kernel      one workgroup per task = 64 tokens x one d-slice (the same positions
//                    of all n streams). The task's x goes from HBM into registers once,
//                    already in matrix-core operand order; the packed weights of the slice
//                    stream into an LDS ring by direct-to-LDS loads issued ahead of the x
//                    loads, and are shared by the 4 waves. v_mfma_f32_16x16x32_bf16
//                    accumulates the 3M columns; the squares come from the diagonal of
//                    x x^T. The task writes one partial record per token. With pre_mix the
//                    hIn weights are inputs, and the task also writes its slice of hIn
//                    from the registers it already holds (x is read once).
//   epilogue_kernel  one workgroup per 16 (n = 4, T >= 8192) or 8 tokens: sums the S partial records of each token
//                    in a fixed order (fp64), then invRms, hMix, the gates, the Sinkhorn
//                    planes (one lane per matrix entry, sums across lanes by DPP) and,
//                    without pre_mix, hIn[t, d] = sum_i hPre[t, i] x[t, i, d] of its
//                    tokens (after the streaming or classic projection), or the hIn
//                    weights (after the single-read kernel, which has written hIn).
//   proj_stream_kernel  the projection of the streaming path: persistent workgroups,
//                    one slice of packed weights resident in LDS each, x read in
//                    contiguous 1 KB runs of each token's row (see the kernel).
//   hin_kernel       hIn of the standalone Sinkhorn stage.
//   fused_kernel     the single-read path (n = 4, alpha[3], no pre_mix, large T), in place
//                    of proj_kernel and hin_kernel: one launch whose workgroups (a group of
//                    32 per XCD) keep their weights in LDS and each tile's x in registers
//                    until its hPre (summed by a designated workgroup, exchanged through
//                    tagged words in the XCD's L2) is known, so x is read once; the epilogue
//                    follows.
// Standalone stages (the HcPre guide, mhpn.cn/news/2282827, "function description", names
// invRms and the Sinkhorn stage as operators of their own):
//   inv_rms_kernel   invRms alone: one wave per token, squares and sums in fp64.
//   mix_gates_kernel the Sinkhorn stage from given mixes and invRms: the epilogue's gates and
//                    Sinkhorn for 8 or 16 tokens per workgroup; hin_kernel follows.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "mhc_device.h"
#include "mhc_plan.h"

namespace mhc {
namespace {

// ------------------------------------------------------------------ configuration

template <int N, int A>
struct Cfg {
    static constexpr int M = A == 3 ? N * N + 2 * N : 2 * N;
    static constexpr int NT = (3 * M + 15) / 16;
    static constexpr int NC = 16 * NT;
    static constexpr int SK = (A == 3) ? 1 : (N == 4 ? 4 : 2);   // K-steps per stage
    static constexpr int RING = (N == 8 && A == 3) ? 3 : (N == 6 && A == 3) ? 5 : (A == 3 ? 7 : 5);   // LDS weight slots: stages in flight + 1
    static constexpr int NN = N * N;
    static constexpr int PPS = (N + 4) / 4 * 4;   // pre-branch record: n sums, square, padding
    static constexpr int V = (PPS + (M - N) + 3) / 4 * 4;   // floats per partial record (16-byte multiple)
    static constexpr int CH = V / 4;              // 16-byte chunks per record
    static constexpr int KU = 4 * NC;             // 16-byte units per K-step of packed weights
    static constexpr int STAGE_U = SK * KU;
    static_assert(STAGE_U % 64 == 0, "a stage is whole 64-lane load instructions");
    static constexpr int PROJ_LDS = RING * STAGE_U * 16 > kTileTokens * NC * 4 ? RING * STAGE_U * 16 : kTileTokens * NC * 4;
};

struct KArgs {
    ForwardArgs a;
    int64_t T;
    int64_t K;
    int64_t tiles;
    int D;
    int S;
    int GS;
    int NG;
};

__device__ __forceinline__ int tile_tokens(const KArgs& k, int64_t t0)
{
    return (int)(k.T - t0 < kTileTokens ? k.T - t0 : kTileTokens);
}

// ------------------------------------------------------------------ weight pre-pack

// double -> float, round to nearest even, kept as a float: the empty asm statement stops
// the compiler from merging this rounding with a following float -> bf16 (or fp16) one
// into a single rounding, which it does in some code shapes and not in others. Every
// pack of the weights (the pack kernel, the single-read and the one-launch kernels) then
// rounds the same way, whatever code surrounds it, and the packed terms agree bit for bit.
__device__ __forceinline__ float f64_to_f32(double d)
{
    float f = (float)d;
    asm volatile("" : "+v"(f));
    return f;
}

// phi * gamma (the exact product in double) as three bf16 terms, each the nearest bf16 of
// the nearest float of what the previous ones leave: hi + mid + lo equals the product to
// ~2^-26 relative.
__device__ __forceinline__ void split3(double p, uint32_t (&tb)[3])
{
    tb[0] = f32_to_bf16_bits(f64_to_f32(p));
    const double r1 = p - bf16_bits_to_double(tb[0]);
    tb[1] = f32_to_bf16_bits(f64_to_f32(r1));
    const double r2 = r1 - bf16_bits_to_double(tb[1]);
    tb[2] = f32_to_bf16_bits(f64_to_f32(r2));
}

// The fp16 form: the terms would fall below fp16's normal range, so each remainder is
// scaled by 2^11 before it is rounded: p = hi + 2^-11 mid + 2^-22 lo, and the projection
// scales the mid and lo column sums back (exact powers of two). Exact to ~2^-33 relative
// for |p| in [2^-14, 65504]; larger weights overflow fp16.
__device__ __forceinline__ void split3_f16(double p, uint32_t (&tb)[3])
{
    const _Float16 h0 = (_Float16)f64_to_f32(p);
    const double r1 = (p - (double)(float)h0) * 2048.0;
    const _Float16 h1 = (_Float16)f64_to_f32(r1);
    const double r2 = (r1 - (double)(float)h1) * 2048.0;
    const _Float16 h2 = (_Float16)f64_to_f32(r2);
    tb[0] = __builtin_bit_cast(uint16_t, h0);
    tb[1] = __builtin_bit_cast(uint16_t, h1);
    tb[2] = __builtin_bit_cast(uint16_t, h2);
}

// The three-term split for x's format: bf16 terms, or scaled fp16 terms.
template <bool H>
__device__ __forceinline__ void split3_x(double p, uint32_t (&tb)[3])
{
    if constexpr (H) split3_f16(p, tb);
    else split3(p, tb);
}
// The same splits of a float weight (no gamma), in fp32: the same bits as split3_x of
// (double)p (its double -> float roundings are then exact). Every remainder is exact in fp32 too: p - hi is a multiple of p's fp32 ulp
// and at most half a bf16 (fp16) ulp of p, so it needs at most 16 (13) significant bits,
// and the next remainder fewer still; the scalings by 2^11 are exact.
__device__ __forceinline__ void split3_f32(float p, uint32_t (&tb)[3])
{
    tb[0] = f32_to_bf16_bits(p);
    const float r1 = p - __uint_as_float(tb[0] << 16);
    tb[1] = f32_to_bf16_bits(r1);
    const float r2 = r1 - __uint_as_float(tb[1] << 16);
    tb[2] = f32_to_bf16_bits(r2);
}
__device__ __forceinline__ void split3_f16_f32(float p, uint32_t (&tb)[3])
{
    const _Float16 h0 = (_Float16)p;
    const float r1 = (p - (float)h0) * 2048.f;
    const _Float16 h1 = (_Float16)r1;
    const float r2 = (r1 - (float)h1) * 2048.f;
    const _Float16 h2 = (_Float16)r2;
    tb[0] = __builtin_bit_cast(uint16_t, h0);
    tb[1] = __builtin_bit_cast(uint16_t, h1);
    tb[2] = __builtin_bit_cast(uint16_t, h2);
}
template <bool H>
__device__ __forceinline__ void split3_x32(float p, uint32_t (&tb)[3])
{
    if constexpr (H) split3_f16_f32(p, tb);
    else split3_f32(p, tb);
}
// Scales of the mid and lo term sums (split3_f16 scales the remainders by 2^11 each).
template <bool H> constexpr float kMidScale = H ? 0x1p-11f : 1.f;
template <bool H> constexpr float kLoScale = H ? 0x1p-22f : 1.f;

// One 16 x 16 x 32 matrix-core step on x's format (fp16 or bf16 operands, fp32 sums).
template <bool H>
__device__ __forceinline__ f32x4 mfma_x16(u32x4 a, u32x4 b, f32x4 c)
{
    if constexpr (H)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// One thread per (K-step k, K-group g, phi row m): reads the row's 8 weights of that
// octet once, splits each into its three terms and writes the three 16-byte units of
// columns m, M + m and 2M + m; threads m < NC - 3M also zero padding column 3M + m.
// K-steps past the data and octets past D are written as zeros.
template <bool H>
__global__ void __launch_bounds__(256)
prepack_kernel(const float* __restrict__ phi, const float* __restrict__ gamma,
               u32x4* __restrict__ packed, int n, int D, int M, int NC, int nks, int64_t total)
{
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= total) return;
    const int m = (int)(u % M);
    const int64_t r = u / M;
    const int g = (int)(r % 4);
    const int64_t k = r / 4;
    const int64_t K = (int64_t)n * D;
    u32x4 w[3] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    const int d = kBlock * (int)(k / n) + 8 * g;
    if (k < nks && d < D) {
        const int64_t k0 = (k % n) * (int64_t)D + d;
        // the octet's 8 weights (and gammas) are consecutive and start at a multiple of 8
        // elements: two 16-byte loads each where the arrays are 16-byte aligned
        float pv[8], gv[8];
        const bool vec = ((reinterpret_cast<uintptr_t>(phi) | reinterpret_cast<uintptr_t>(gamma)) & 15) == 0;
        if (vec) {
            const float4* pp4 = reinterpret_cast<const float4*>(phi + (int64_t)m * K + k0);
            const float4 p0 = pp4[0], p1 = pp4[1];
            pv[0] = p0.x; pv[1] = p0.y; pv[2] = p0.z; pv[3] = p0.w;
            pv[4] = p1.x; pv[5] = p1.y; pv[6] = p1.z; pv[7] = p1.w;
            if (gamma) {
                const float4* gp4 = reinterpret_cast<const float4*>(gamma + k0);
                const float4 g0 = gp4[0], g1 = gp4[1];
                gv[0] = g0.x; gv[1] = g0.y; gv[2] = g0.z; gv[3] = g0.w;
                gv[4] = g1.x; gv[5] = g1.y; gv[6] = g1.z; gv[7] = g1.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pv[e] = phi[(int64_t)m * K + k0 + e];
                gv[e] = gamma ? gamma[k0 + e] : 1.f;
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t tb[3];   // in fp32 without gamma (the same bits), else of the product in fp64
            if (gamma) split3_x<H>((double)pv[e] * (double)gv[e], tb);
            else split3_x32<H>(pv[e], tb);
#pragma unroll
            for (int t = 0; t < 3; ++t) w[t][e >> 1] |= tb[t] << (16 * (e & 1));
        }
    }
    u32x4* row = packed + r * NC;
#pragma unroll
    for (int t = 0; t < 3; ++t) row[t * M + m] = w[t];
    if (m < NC - 3 * M) row[3 * M + m] = u32x4{0u, 0u, 0u, 0u};
}

// ------------------------------------------------------------------ hIn from registers

// hIn[t, d] = sum_i w_i x[t, i, d] for the lane's token and its octet of each d-block of
// the slice: the n K-steps of a d-block hold the n streams of the same 8 positions, so
// the sum is local to the lane. fp32 FMA in stream order, one rounding to bf16. `hres`
// covers the tile's rows of hIn (rows past T are dropped by its range); `lim` excludes
// octets past D.
template <int N, int NKS, bool H>
__device__ __forceinline__ void hin_store(rsrc_t hres, uint32_t off, const u32x4 (&xr)[NKS],
                                          const float (&w)[N], int lim)
{
#pragma unroll
    for (int blk = 0; blk < NKS / N; ++blk) {
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const u32x4 v = xr[blk * N + i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] = fmaf(w[i], x16_lo<H>(v[e]), acc[2 * e]);
                acc[2 * e + 1] = fmaf(w[i], x16_hi<H>(v[e]), acc[2 * e + 1]);
            }
        }
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = pack_x16<H>(acc[2 * e], acc[2 * e + 1]);
        if (kBlock * blk < lim)
            __builtin_amdgcn_raw_buffer_store_b128(o, hres, (int)(off + 2 * kBlock * blk), 0, 0);
    }
}

// ------------------------------------------------------------------ projection

// One weight stage (STAGE_U 16-byte units) moves from global memory straight into LDS:
// wave w's i-th instruction moves units [256 i + 64 w, +64), one per lane, to the same
// place in the destination slot (the LDS address is M0 plus 16 bytes per lane). The
// instruction is issued from inline assembly so that the compiler neither tracks it nor
// inserts waits of its own before LDS reads; the kernel waits for it explicitly with the
// in-order vector memory counter.
__device__ __forceinline__ void dma16(const u32x4* g, uint32_t lds_wave_base)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(lds_wave_base) : "memory");
}
template <int STAGE_U>
__device__ __forceinline__ void dma_stage(const u32x4* src, const u32x4* dst, int wave, int lane)
{
#pragma unroll
    for (int i = 0; i < (STAGE_U + kThreads - 1) / kThreads; ++i) {
        const int base = kThreads * i + 64 * wave;
        if (STAGE_U % kThreads == 0 || base < STAGE_U)
            dma16(src + base + lane,
                  __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(dst + base)));
    }
}
// Direct-to-LDS instructions every wave issues per stage (the fewest over the waves).
template <int STAGE_U>
constexpr int dma_ops_min() { return STAGE_U / kThreads; }

// Vector memory operations a wave has issued after the DMA of stage c when it waits for
// stage c at iteration c: stages 0 .. DEPTH-1 go out before the NKS x loads, stage c + DEPTH
// after the barrier of iteration c. Counting the fewest DMA instructions per stage can
// only undercount, which makes the wait stronger than needed, never weaker.
template <int NKS, int NSTAGE, int DEPTH, int OPS>
constexpr int younger_than_stage(int c)
{
    int n = 0;
    if (c < DEPTH) {
        n += (DEPTH - 1 - c) * OPS + NKS;
        for (int it = 0; it < c; ++it)
            if (it + DEPTH < NSTAGE) n += OPS;
    } else {
        for (int it = c - DEPTH + 1; it < c; ++it)
            if (it + DEPTH < NSTAGE) n += OPS;
    }
    return n;
}

template <int N, int A, int NKS, bool H>
__global__ void __launch_bounds__(kThreads, NKS > 16 ? 2 : 3)
proj_kernel(KArgs k)
{
    using C = Cfg<N, A>;
    constexpr int NT = C::NT, NC = C::NC, SK = C::SK, M = C::M, CH = C::CH, PPS = C::PPS;
    constexpr int STAGE_U = C::STAGE_U;
    constexpr int NSTAGE = NKS / SK;
    constexpr int DEPTH = C::RING - 1 < NSTAGE ? C::RING - 1 : NSTAGE;   // stages in flight
    constexpr int R = DEPTH + 1;                                           // LDS slots
    constexpr int OPS = dma_ops_min<STAGE_U>();
    static_assert(NKS % SK == 0 && NKS % N == 0, "a slice is whole stages and whole d-blocks");
    static_assert(NKS <= kPadSteps, "the zero tail of the packed weights covers one slice");
    static_assert(OPS >= 1, "every wave moves part of each stage");
    __shared__ __attribute__((aligned(16))) char lds[C::PROJ_LDS];   // R weight slots; then column totals
    __shared__ float lds_ss[kTileTokens];
    const u32x4* ring = reinterpret_cast<const u32x4*>(lds);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int j = lane & 15;      // A row (token) / B column / D column
    const int grp = lane >> 4;    // K-group of A and B; row block of D
    const int row = wave * 16 + j;   // the lane's token within the tile
    int64_t tile;
    int s;
    if (!task_of_block(blockIdx.x, k.tiles, k.S, &tile, &s)) return;   // padding workgroup
    const int64_t t0 = tile * kTileTokens;
    const int ntile = tile_tokens(k, t0);
    const int b0 = s * (NKS / N);
    // octets of d-block b0 + blk exist for this lane iff kBlock * blk < lim
    const int lim = k.D - kBlock * b0 - 8 * grp;
    const u32x4* pk = static_cast<const u32x4*>(k.a.packed) + packed_slice(s, NKS, NC);

    // Weight stages 0 .. DEPTH-1 first, then all of the task's x: the load counter retires
    // in issue order, so waiting for a weight stage never waits for x. Rows past T lie
    // outside the tile's x range and read as zero.
#pragma unroll
    for (int st = 0; st < DEPTH; ++st) dma_stage<STAGE_U>(pk + st * STAGE_U, ring + st * STAGE_U, wave, lane);
    const rsrc_t xres = make_rsrc(k.a.x + t0 * k.K, (int64_t)ntile * k.K * 2);
    u32x4 xr[NKS];
    uint32_t xo[N];
#pragma unroll
    for (int i = 0; i < N; ++i) xo[i] = x_lane_off(k.K, k.D, row, grp, b0, i);
#pragma unroll
    for (int st = 0; st < NKS; ++st)   // in K-step order: the loop below consumes them in order
        xr[st] = __builtin_amdgcn_raw_buffer_load_b128(xres, (int)(xo[st % N] + 2 * kBlock * (st / N)), 0, 0);

    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 sq = {0.f, 0.f, 0.f, 0.f};   // x x^T of this wave's 16 tokens; diagonal = squares
#pragma unroll
    for (int c = 0; c < NSTAGE; ++c) {
        wait_vm(younger_than_stage<NKS, NSTAGE, DEPTH, OPS>(c));   // this wave's part of stage c
        // every wave's part of stage c is in LDS; every wave is done with stage c - 1,
        // whose slot the next DMA overwrites
        __syncthreads();
        if (c + DEPTH < NSTAGE)
            dma_stage<STAGE_U>(pk + (c + DEPTH) * STAGE_U, ring + ((c + DEPTH) % R) * STAGE_U, wave, lane);
        const u32x4* w = ring + (c % R) * STAGE_U + grp * NC + j;
#pragma unroll
        for (int kk = 0; kk < SK; ++kk) {
            const int st = c * SK + kk;
            if constexpr (NT > 8) __builtin_amdgcn_sched_barrier(0);
            const u32x4 z = {0u, 0u, 0u, 0u};
            const u32x4 xa = kBlock * (st / N) < lim ? xr[st] : z;
            if constexpr (H) {
                const f16x8 Av = __builtin_bit_cast(f16x8, xa);
                sq = __builtin_amdgcn_mfma_f32_16x16x32_f16(Av, Av, sq, 0, 0, 0);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const u32x4 bv = w[kk * 4 * NC + nt * 16];
                    acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Av, __builtin_bit_cast(f16x8, bv),
                                                                     acc[nt], 0, 0, 0);
                }
            } else {
                const bf16x8 Av = __builtin_bit_cast(bf16x8, xa);
                sq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Av, Av, sq, 0, 0, 0);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const u32x4 bv = w[kk * 4 * NC + nt * 16];
                    acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Av, __builtin_bit_cast(bf16x8, bv),
                                                                      acc[nt], 0, 0, 0);
                }
            }
        }
    }
    __syncthreads();   // the ring is free

    // Column totals of this slice into LDS ([64 tokens][NC]); the square of token i is
    // element (i, i) of x x^T: lane i + 16 * (i / 4), register i % 4.
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(wave * 16 + 4 * grp + r) * NC + nt * 16 + j] = acc[nt][r];
    {
        const int rr = j - 4 * grp;
        if (rr >= 0 && rr < 4) lds_ss[wave * 16 + j] = sq[rr];
    }

    // With pre_mix the hIn weights are known: the slice's hIn from the x registers.
    if (k.a.pre_mix) {
        const int64_t tok = t0 + row < k.T ? t0 + row : k.T - 1;
        float wv[N];
#pragma unroll
        for (int i = 0; i < N; ++i) wv[i] = k.a.pre_mix[tok * N + i];
        const rsrc_t hres = make_rsrc(k.a.h_in + t0 * k.D, (int64_t)ntile * k.D * 2);
        hin_store<N, NKS, H>(hres, (uint32_t)(((int64_t)row * k.D + kBlock * b0 + 8 * grp) * 2), xr, wv, lim);
    }
    __syncthreads();

    // Partial records (hi + mid + lo of each phi row, added in fp64, rounded once),
    // 16 bytes per store.
    const rsrc_t rec = make_rsrc(k.a.rec + rec_tile(tile, k.S, N, M), (int64_t)k.S * kTileTokens * C::V * 4);
    for (int idx = tid; idx < kTileTokens * CH; idx += kThreads) {
        const int tl = idx / CH, ch = idx % CH;
        const float* rr = red + tl * NC;
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int v = 4 * ch + e;
            const int m = v < N ? v : N + (v - PPS);
            float val;
            if (v == N) val = lds_ss[tl];
            else if ((v > N && v < PPS) || v >= PPS + (M - N)) val = 0.f;   // padding
            else if (H)   // the fp16 terms carry scales 1, 2^11, 2^22 (split3_f16)
                val = (float)((double)rr[m] + 0x1p-11 * (double)rr[M + m] + 0x1p-22 * (double)rr[2 * M + m]);
            else val = (float)((double)rr[m] + (double)rr[M + m] + (double)rr[2 * M + m]);
            o[e] = __float_as_uint(val);
        }
        const uint32_t off = tl < ntile ? (uint32_t)(rec_loc(s, tl, N, M) + 4 * ch) * 4 : kOutOfRange;
        __builtin_amdgcn_raw_buffer_store_b128(o, rec, (int)off, 0, 0);
    }
}

// ------------------------------------------------------------------ projection on the VALU

// The projection with plain fp32 FMAs instead of the matrix cores, for the classic path:
// the same tasks (64-token tile, slice of NKS K-steps) and the same partial records, so the
// epilogue and hIn kernels are unchanged. Weights: phiT[k][m] = phi[m][k] gamma[k] in fp32
// (the product rounded once), K rows of M, read by whole rows with scalar loads: every lane
// of a wave uses the same weight row at once. A lane is a token of the tile; wave w takes
// the d positions [DW w, DW (w + 1)) of the slice (all n streams of each), so with pre_mix
// its hIn is local; the four waves' sums meet in LDS and are added in wave order.
__global__ void __launch_bounds__(256) pack_valu_kernel(const float* __restrict__ phi, const float* __restrict__ gamma,
                                                        float* __restrict__ phiT, int64_t K, int M)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // element (k, m) of phiT, m fastest
    if (i >= K * M) return;
    const int64_t kk = i / M;
    const int m = (int)(i % M);
    double w = (double)phi[(int64_t)m * K + kk];
    if (gamma) w *= (double)gamma[kk];
    phiT[i] = (float)w;
}

template <int N, int A, int NKS, bool H>
__global__ void __launch_bounds__(kThreads, 2)
proj_valu_kernel(KArgs k, const float* __restrict__ phiT)
{
    using C = Cfg<N, A>;
    constexpr int M = C::M, CH = C::CH, PPS = C::PPS;
    constexpr int NBS = NKS / N;                 // d-blocks of a slice
    constexpr int DW = NBS * kBlock / 4;         // d positions per wave
    constexpr int NL = DW / 8;                   // 16-byte x loads per stream and lane
    static_assert(NKS % N == 0 && DW % 8 == 0 && M <= 32, "slice and weight shapes of the VALU projection");
    __shared__ float red[4][kTileTokens][M + 1];   // each wave's sums of the M rows, then the square
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: the weight rows are scalar loads
    const int lane = tid & 63;
    int64_t tile;
    int s;
    if (!task_of_block(blockIdx.x, k.tiles, k.S, &tile, &s)) return;   // padding workgroup
    const int64_t t0 = tile * kTileTokens;
    const int ntile = tile_tokens(k, t0);
    const int d_lo = kBlock * s * NBS + wave * DW;   // this wave's first d position

    // x of token t0 + lane: stream i, positions [d_lo, d_lo + DW); past D or T: zero
    const rsrc_t xres = make_rsrc(k.a.x + t0 * k.K, (int64_t)ntile * k.K * 2);
    u32x4 xr[N][NL];
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            const int d = d_lo + 8 * l;
            const uint32_t off = d < k.D ? (uint32_t)(((int64_t)lane * k.K + (int64_t)i * k.D + d) * 2) : kOutOfRange;
            xr[i][l] = __builtin_amdgcn_raw_buffer_load_b128(xres, (int)off, 0, 0);
        }
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.f;
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            const int d0 = d_lo + 8 * l;
            if (d0 >= k.D) continue;   // (the same for every lane) positions past D have no weights
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xe = (e & 1) ? x16_hi<H>(xr[i][l][e >> 1]) : x16_lo<H>(xr[i][l][e >> 1]);
                // one weight row, the same for every lane: read from the constant address
                // space, so that the loads are scalar (the weights are not written meanwhile)
                const __attribute__((address_space(4))) float* w =
                    (const __attribute__((address_space(4))) float*)(phiT + ((int64_t)i * k.D + d0 + e) * M);
                sq = fmaf(xe, xe, sq);
#pragma unroll
                for (int m = 0; m < M; ++m) acc[m] = fmaf(xe, w[m], acc[m]);
            }
        }
#pragma unroll
    for (int m = 0; m < M; ++m) red[wave][lane][m] = acc[m];
    red[wave][lane][M] = sq;

    // With pre_mix the hIn weights are known: this wave's positions of hIn from the x registers.
    if (k.a.pre_mix) {
        const int64_t tok = t0 + lane < k.T ? t0 + lane : k.T - 1;
        float wv[N];
#pragma unroll
        for (int i = 0; i < N; ++i) wv[i] = k.a.pre_mix[tok * N + i];
        const rsrc_t hres = make_rsrc(k.a.h_in + t0 * k.D, (int64_t)ntile * k.D * 2);
#pragma unroll
        for (int l = 0; l < NL; ++l) {
            float h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = 0.f;
#pragma unroll
            for (int i = 0; i < N; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[2 * e] = fmaf(wv[i], x16_lo<H>(xr[i][l][e]), h[2 * e]);
                    h[2 * e + 1] = fmaf(wv[i], x16_hi<H>(xr[i][l][e]), h[2 * e + 1]);
                }
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = pack_x16<H>(h[2 * e], h[2 * e + 1]);
            const int d = d_lo + 8 * l;
            const uint32_t off = d < k.D ? (uint32_t)(((int64_t)lane * k.D + d) * 2) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b128(o, hres, (int)off, 0, 0);
        }
    }
    __syncthreads();

    // partial records of the slice, 16 bytes per store: the waves' sums in wave order (fp32)
    const rsrc_t rec = make_rsrc(k.a.rec + rec_tile(tile, k.S, N, M), (int64_t)k.S * kTileTokens * C::V * 4);
    for (int idx = tid; idx < kTileTokens * CH; idx += kThreads) {
        const int tl = idx / CH, ch = idx % CH;
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int v = 4 * ch + e;
            const int m = v < N ? v : (v == N ? M : N + (v - PPS));   // row, or M for the square
            float val = 0.f;
            if (!((v > N && v < PPS) || v >= PPS + (M - N))) {   // not padding
#pragma unroll
                for (int w = 0; w < 4; ++w) val += red[w][tl][m];
            }
            o[e] = __float_as_uint(val);
        }
        const uint32_t off = tl < ntile ? (uint32_t)(rec_loc(s, tl, N, M) + 4 * ch) * 4 : kOutOfRange;
        __builtin_amdgcn_raw_buffer_store_b128(o, rec, (int)off, 0, 0);
    }
}

// ------------------------------------------------------------------ per-token math

__device__ __forceinline__ float sigmoidf_stable(float z)
{
    if (z >= 0.f) return 1.f / (1.f + expf(-z));
    const float e = expf(z);
    return e / (1.f + e);
}

__device__ __forceinline__ double inv_rms_of(double sq, double K, double eps)
{
    return 1.0 / sqrt(sq / K + eps);
}
__device__ __forceinline__ float gate_pre(double h, double inv, float alpha, float bias, float eps)
{
    return sigmoidf_stable((float)fma((double)alpha, h * inv, (double)bias)) + eps;
}
__device__ __forceinline__ float gate_post(double h, double inv, float alpha, float bias, float eps,
                                           bool plus_eps)
{
    const float g = 2.f * sigmoidf_stable((float)fma((double)alpha, h * inv, (double)bias));
    return plus_eps ? g + eps : g;
}
__device__ __forceinline__ float res_logit(double h, double inv, float alpha, float bias)
{
    return (float)fma((double)alpha, h * inv, (double)bias);
}

// Cross-lane sums and maxima over the rows / columns of an n x n matrix held one entry
// per lane, entry (r, c) in lane n*r + c of an n*n-lane group (16 lanes for n = 4, the
// whole wave for n = 8). DPP moves within 16-lane rows; the column sums of n = 8 cross
// rows with lane shuffles. Every lane of a row (column) ends with the same total.

template <int N>
__device__ __forceinline__ float row_sum(float v)
{
    v += dpp<kQuadXor1>(v);
    v += dpp<kQuadXor2>(v);
    if constexpr (N == 8) v += dpp<kRowHalfMirror>(v);
    return v;
}
template <int N>
__device__ __forceinline__ float row_max(float v)
{
    v = fmaxf(v, dpp<kQuadXor1>(v));
    v = fmaxf(v, dpp<kQuadXor2>(v));
    if constexpr (N == 8) v = fmaxf(v, dpp<kRowHalfMirror>(v));
    return v;
}
template <int N>
__device__ __forceinline__ float col_sum(float v)
{
    if constexpr (N == 4) {
        v += dpp<kRowRor4>(v);
        v += dpp<kRowRor8>(v);
    } else {
        v += dpp<kRowRor8>(v);
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
    }
    return v;
}

// n = 6: 36 entries do not tile a wave, so each matrix takes a wave of its own (lanes 36
// to 63 idle) and the sums gather the row's (column's) lanes by shuffles, in index order.
template <int N>
__device__ __forceinline__ float sk_row_sum(float v, int r)
{
    if constexpr (N == 6) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < N; ++c) s += __shfl(v, r * N + c);
        return s;
    } else {
        return row_sum<N>(v);
    }
}
template <int N>
__device__ __forceinline__ float sk_row_max(float v, int r)
{
    if constexpr (N == 6) {
        float m = __shfl(v, r * N);
#pragma unroll
        for (int c = 1; c < N; ++c) m = fmaxf(m, __shfl(v, r * N + c));
        return m;
    } else {
        return row_max<N>(v);
    }
}
template <int N>
__device__ __forceinline__ float sk_col_sum(float v, int c)
{
    if constexpr (N == 6) {
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < N; ++r) s += __shfl(v, r * N + c);
        return s;
    } else {
        return col_sum<N>(v);
    }
}

// Sinkhorn of nb tokens (the first is token tfirst) whose logits are in Ls ([nb][N*N]):
// one lane per matrix entry, 2*num_iters steps, every plane stored. A matrix takes SW
// consecutive lanes (N*N, or a whole wave for n = 6); a lane past the N*N entries of
// its matrix computes along and stores nothing.
// THREADS consecutive threads (tid = 0 .. THREADS - 1) take part; T sizes the plane arrays.
template <int N, int THREADS>
__device__ void sinkhorn_by(const ForwardArgs& a, int64_t T, const float* Ls, int64_t tfirst, int nb, int tid)
{
    constexpr int NN = N * N;
    constexpr int SW = 64 % NN == 0 ? NN : 64;
    static_assert(THREADS % SW == 0, "a pass is whole matrices");
    const int e = tid % SW;
    const bool used = SW == NN || e < NN;
    const int r = used ? e / N : 0, c = used ? e % N : 0;
    const float eps = (float)a.hc_eps;
    const int steps = 2 * a.num_iters;
    for (int base = 0; base < nb * SW; base += THREADS) {
        const int q = (base + tid) / SW;
        const bool live = used && q < nb;
        const int64_t t1 = tfirst + base / SW;   // first token of this pass
        const int nlive = nb - base / SW;          // tokens of this pass that exist
        const int qq = q - base / SW;              // token within the pass
        float v = live ? Ls[q * NN + e] : 0.f;
        const float mx = sk_row_max<N>(v, r);
        const float ex = expf(v - mx);
        float sum = sk_row_sum<N>(ex, r);
        v = ex / sum + eps;
        for (int step = 0; step < steps; ++step) {
            if (step > 0) {
                if (step & 1) sum = sk_col_sum<N>(v, c) + eps;
                else sum = sk_row_sum<N>(v, r) + eps;
                v = v / sum;
            }
            // this pass's tokens of plane `step`; lanes past them fall outside the range
            if (a.sum_out) {
                const rsrc_t rs = make_rsrc(a.sum_out + ((int64_t)step * T + t1) * N, (int64_t)nlive * N * 4);
                const bool writer = used && ((step & 1) ? (r == 0) : (c == 0));
                if (writer) st_buf(rs, (uint32_t)(qq * N + ((step & 1) ? c : r)) * 4, sum);
            }
            if (a.norm_out) {
                const rsrc_t rn = make_rsrc(a.norm_out + ((int64_t)step * T + t1) * NN, (int64_t)nlive * NN * 4);
                if (used) st_buf(rn, (uint32_t)(qq * NN + e) * 4, v);
            }
        }
        const rsrc_t rh = make_rsrc(a.h_res + t1 * NN, (int64_t)nlive * NN * 4);
        if (used) st_buf(rh, (uint32_t)(qq * NN + e) * 4, v);
    }
}
template <int N>
__device__ void sinkhorn(const KArgs& k, const float* Ls, int64_t tfirst, int nb)
{
    sinkhorn_by<N, kThreads>(k.a, k.T, Ls, tfirst, nb, (int)threadIdx.x);
}

// ------------------------------------------------------------------ epilogue

// Tokens [OB b, OB b + OB) of workgroup b, OB = out_tokens(N, T) (all in one tile). A load item is (token, group,
// chunk): one 16-byte chunk of the token's record from the slices of one summation group
// (slices [g GS, (g+1) GS)), summed in slice order in fp64; the group sums are then added
// in group order. Every output of the tokens follows from the totals. HIN: the workgroup
// then also writes its tokens' hIn from hPre and x (each token's n x D values are one
// contiguous run of x), as hin_kernel would, so no hIn launch follows; H: x in fp16.
template <int N, int A, int OB, bool HIN = false, bool H = false>
__global__ void __launch_bounds__(kThreads)
epilogue_kernel(KArgs k)
{
    using C = Cfg<N, A>;
    constexpr int NN = C::NN, V = C::V, CH = C::CH, M = C::M, PPS = C::PPS;
    static_assert(kTileTokens % OB == 0, "a workgroup's tokens lie in one tile");
    __shared__ double gs[OB * V * 8];    // [token][value][group]; group 0 then holds the total
    __shared__ float Ls[OB * NN];
    __shared__ float gpar[3 + M];        // alpha, bias
    __shared__ float hps[HIN ? OB * N : 1];   // the tokens' hPre (HIN)
    const ForwardArgs& a = k.a;
    const int tid = threadIdx.x;
    const int64_t tf = (int64_t)blockIdx.x * OB;
    const int nb = k.T - tf < OB ? (int)(k.T - tf) : OB;
    const int64_t tile = tf / kTileTokens;
    const int tl0 = (int)(tf % kTileTokens);
    if (tid < A) gpar[tid] = a.alpha[tid];
    for (int i = tid; i < M; i += kThreads) gpar[3 + i] = a.bias[i];
    // the epilogue is the call's last reader of the counter's value: the next call's tag;
    // the single-read kernel's per-XCD arrival counters start from zero again
    if (blockIdx.x == 0 && tid == 0) a.sync[0] = a.sync[0] + 1u;
    if (blockIdx.x == 0 && tid < kXcds) a.sync[kTicket0 + tid] = 0u;

    const rsrc_t rec = make_rsrc(a.rec + rec_tile(tile, k.S, N, M), (int64_t)k.S * kTileTokens * V * 4);
    // two items per thread and pass, their loads issued together (eight in flight)
    const int items = nb * k.NG * CH;
    for (int it0 = tid; it0 < items; it0 += 2 * kThreads) {
        int ch[2], g[2], q[2], sb[2], se[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int it = it0 + h * kThreads;
            ch[h] = it % CH;
            g[h] = (it / CH) % k.NG;
            q[h] = it / (CH * k.NG);
            sb[h] = group_begin(k.GS, g[h]);
            se[h] = it < items ? group_end(k.S, k.GS, g[h]) : sb[h];   // no slices: nothing loaded
        }
        double acc[2][4] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
        for (int c0 = 0; c0 < k.GS; c0 += 4) {
            u32x4 ov[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int sl = sb[h] + c0 + c;
                    const uint32_t off = sl < se[h] ? (uint32_t)(rec_loc(sl, tl0 + q[h], N, M) + 4 * ch[h]) * 4
                                                    : kOutOfRange;
                    ov[h][c] = __builtin_amdgcn_raw_buffer_load_b128(rec, (int)off, 0, 0);
                }
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (sb[h] + c0 + c < se[h]) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[h][e] += (double)__uint_as_float(ov[h][c][e]);
                    }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
            if (it0 + h * kThreads < items) {
#pragma unroll
                for (int e = 0; e < 4; ++e) gs[(q[h] * V + 4 * ch[h] + e) * 8 + g[h]] = acc[h][e];
            }
    }
    __syncthreads();
    for (int it = tid; it < nb * V; it += kThreads) {
        double t = 0.0;
        for (int g = 0; g < k.NG; ++g) t += gs[it * 8 + g];
        gs[it * 8] = t;
    }
    __syncthreads();
    // HIN: the first batch of x for hIn goes out now, to arrive while the gates and the
    // Sinkhorn (LDS and stores only) run; rows past the call's tokens lie outside the ranges
    constexpr int IB = HIN ? 16 / N : 1;   // octets of a thread per batch (16 or 12 loads)
    const int D8 = k.D / 8;
    const int hin_items = HIN ? nb * D8 : 0;
    const rsrc_t xr = make_rsrc(a.x + tf * k.K, HIN ? (int64_t)nb * k.K * 2 : 0);
    const rsrc_t hr = make_rsrc(a.h_in + tf * k.D, HIN ? (int64_t)nb * k.D * 2 : 0);
    u32x4 xv[IB][N];
    auto hin_batch = [&](int it0) {
#pragma unroll
        for (int u = 0; u < IB; ++u) {
            const int it = it0 + u * kThreads;
            const int q = it / D8, o = it % D8;
#pragma unroll
            for (int i = 0; i < N; ++i)
                xv[u][i] = __builtin_amdgcn_raw_buffer_load_b128(
                    xr, (int)(it < hin_items ? (uint32_t)((q * N + i) * k.D + 8 * o) * 2 : kOutOfRange), 0, 0);
        }
    };
    if constexpr (HIN) {
        if (tid < hin_items) hin_batch(tid);
    }

    const float eps = (float)a.hc_eps;
    const rsrc_t r_mix = make_rsrc(a.h_mix + tf * M, a.h_mix ? (int64_t)nb * M * 4 : 0);
    const rsrc_t r_inv = make_rsrc(a.inv_rms + tf, a.inv_rms ? (int64_t)nb * 4 : 0);
    const rsrc_t r_pre = make_rsrc(a.h_pre + tf * N, a.h_pre ? (int64_t)nb * N * 4 : 0);
    const rsrc_t r_wts = make_rsrc(a.wts + tf * N, a.pre_mix ? 0 : (int64_t)nb * N * 4);
    const rsrc_t r_post = make_rsrc(a.h_post + tf * N, (int64_t)nb * N * 4);
    for (int it = tid; it < nb * M; it += kThreads) {
        const int q = it / M, m = it % M;
        const double inv = inv_rms_of(gs[(q * V + N) * 8], (double)k.K, a.norm_eps);
        const double h = gs[(q * V + (m < N ? m : PPS + (m - N))) * 8];
        st_buf(r_mix, (uint32_t)it * 4, (float)h);
        if (m == 0) st_buf(r_inv, (uint32_t)q * 4, (float)inv);
        if (m < N) {
            const float hp = gate_pre(h, inv, gpar[0], gpar[3 + m], eps);
            st_buf(r_pre, (uint32_t)(q * N + m) * 4, hp);
            if constexpr (HIN) hps[q * N + m] = hp;
            else st_buf(r_wts, (uint32_t)(q * N + m) * 4, hp);
        } else if (m < 2 * N) {
            st_buf(r_post, (uint32_t)(q * N + m - N) * 4, gate_post(h, inv, gpar[1], gpar[3 + m], eps, A == 2));
        } else {
            Ls[q * NN + (m - 2 * N)] = res_logit(h, inv, gpar[2], gpar[3 + m]);
        }
    }
    if constexpr (A == 3 || HIN) __syncthreads();
    if constexpr (A == 3) {
        sinkhorn<N>(k, Ls, tf, nb);
    } else {
        const rsrc_t r_res = make_rsrc(a.h_res + tf * NN, a.h_res ? (int64_t)nb * NN * 4 : 0);
        for (int it = tid; it < nb * NN; it += kThreads) st_buf(r_res, (uint32_t)it * 4, 0.f);
    }
    if constexpr (HIN) {
        // hIn[t, d] = sum_i hPre[t, i] x[t, i, d], octet by octet (the arithmetic of
        // hin_kernel: the same bits), IB octets of a thread per batch; the first batch was
        // loaded before the gates and the Sinkhorn
#pragma unroll 1
        for (int it0 = tid; it0 < hin_items; it0 += IB * kThreads) {
#pragma unroll
            for (int u = 0; u < IB; ++u) {
                const int it = it0 + u * kThreads;
                if (it >= hin_items) continue;
                const int q = it / D8, o = it % D8;
                float acc[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
                for (int i = 0; i < N; ++i) {
                    const float w = hps[q * N + i];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[2 * e] = fmaf(w, x16_lo<H>(xv[u][i][e]), acc[2 * e]);
                        acc[2 * e + 1] = fmaf(w, x16_hi<H>(xv[u][i][e]), acc[2 * e + 1]);
                    }
                }
                u32x4 ov;
#pragma unroll
                for (int e = 0; e < 4; ++e) ov[e] = pack_x16<H>(acc[2 * e], acc[2 * e + 1]);
                __builtin_amdgcn_raw_buffer_store_b128(ov, hr, (int)((uint32_t)(q * k.D + 8 * o) * 2), 0, 0);
            }
            if (it0 + IB * kThreads < hin_items) hin_batch(it0 + IB * kThreads);
        }
    }
}

// ------------------------------------------------------------------ hIn

template <int N, bool H>
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
            acc[2 * e] = fmaf(w[i], x16_lo<H>(v[e]), acc[2 * e]);
            acc[2 * e + 1] = fmaf(w[i], x16_hi<H>(v[e]), acc[2 * e + 1]);
        }
    }
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o[e] = pack_x16<H>(acc[2 * e], acc[2 * e + 1]);
    // hIn is not read again by this forward: stream it past the caches
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(h_in + t * (int64_t)D + d8 * 8));
}

// ------------------------------------------------------------------ standalone stages

// invRms alone: one wave per token, kThreads / 64 tokens per workgroup. A lane widens its
// bf16 values to fp64 and adds their squares in fp64 (a bf16 square is exact there); the
// 64 lane sums are added in fp64 across the wave.
template <int N, bool H>
__global__ void __launch_bounds__(kThreads)
inv_rms_kernel(const uint16_t* __restrict__ x, float* __restrict__ inv_rms, int64_t T, int D,
               double norm_eps)
{
    const int lane = threadIdx.x % 64;
    const int64_t t = (int64_t)blockIdx.x * (kThreads / 64) + threadIdx.x / 64;
    if (t >= T) return;
    const int units = N * D / 8;   // 16-byte units of the token
    const u32x4* xt = reinterpret_cast<const u32x4*>(x + t * (int64_t)N * D);
    double acc = 0.0;
    int u = lane;
    for (; u + 192 < units; u += 256) {   // four loads in flight per lane
        u32x4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = __builtin_nontemporal_load(xt + u + 64 * j);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double lo = x16_lo<H>(v[j][e]), hi = x16_hi<H>(v[j][e]);
                acc = fma(lo, lo, acc);
                acc = fma(hi, hi, acc);
            }
    }
    for (; u < units; u += 64) {
        const u32x4 v = __builtin_nontemporal_load(xt + u);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double lo = x16_lo<H>(v[e]), hi = x16_hi<H>(v[e]);
            acc = fma(lo, lo, acc);
            acc = fma(hi, hi, acc);
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o /= 2) acc += __shfl_xor(acc, o);
    if (lane == 0) inv_rms[t] = (float)inv_rms_of(acc, (double)N * D, norm_eps);
}

// The Sinkhorn stage alone: OB = out_tokens(N, T) tokens per workgroup, from given mixes and invRms
// to hPre, hPost and the Sinkhorn (hIn follows in hin_kernel). The gates are those of
// epilogue_kernel, fed with the f32 inputs widened to fp64.
template <int N, int A, int OB>
__global__ void __launch_bounds__(kThreads)
mix_gates_kernel(KArgs k, const float* __restrict__ h_mix, const float* __restrict__ inv_in)
{
    using C = Cfg<N, A>;
    constexpr int NN = C::NN, M = C::M;
    __shared__ float Ls[OB * NN];
    const ForwardArgs& a = k.a;
    const int tid = threadIdx.x;
    const int64_t tf = (int64_t)blockIdx.x * OB;
    const int nb = k.T - tf < OB ? (int)(k.T - tf) : OB;
    const float eps = (float)a.hc_eps;
    for (int it = tid; it < nb * M; it += kThreads) {
        const int q = it / M, m = it % M;
        const int64_t t = tf + q;
        const double h = (double)h_mix[t * M + m];
        const double inv = (double)inv_in[t];
        if (m < N) a.h_pre[t * N + m] = gate_pre(h, inv, a.alpha[0], a.bias[m], eps);
        else if (m < 2 * N) a.h_post[t * N + m - N] = gate_post(h, inv, a.alpha[1], a.bias[m], eps, A == 2);
        else Ls[q * NN + (m - 2 * N)] = res_logit(h, inv, a.alpha[2], a.bias[m]);
    }
    if constexpr (A == 3) {
        __syncthreads();
        sinkhorn<N>(k, Ls, tf, nb);
    } else if (a.h_res) {
        for (int it = tid; it < nb * NN; it += kThreads) a.h_res[tf * NN + it] = 0.f;
    }
}

template <int N, int A, bool H>
hipError_t launch_stage(int64_t T, int D, const ForwardArgs& a, const float* h_mix, const float* inv_rms,
                        hipStream_t st)
{
    KArgs k;
    std::memset(&k, 0, sizeof k);
    k.a = a;
    k.T = T;
    k.D = D;
    if (N == 4 && out_tokens(N, T) == 16)
        hipLaunchKernelGGL((mix_gates_kernel<N, A, 16>), dim3((unsigned)((T + 15) / 16)), dim3(kThreads), 0, st, k,
                           h_mix, inv_rms);
    else
        hipLaunchKernelGGL((mix_gates_kernel<N, A, 8>), dim3((unsigned)((T + 7) / 8)), dim3(kThreads), 0, st, k,
                           h_mix, inv_rms);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t items = T * (int64_t)(D / 8);
    hipLaunchKernelGGL((hin_kernel<N, H>), dim3((unsigned)((items + 255) / 256)), dim3(256), 0, st, a.x,
                       a.pre_mix ? a.pre_mix : a.h_pre, a.h_in, T, D);
    return hipGetLastError();
}

// ------------------------------------------------------------------ single-read forward

// A 64-bit word carrying a value and the tag of the call that wrote it; written and read
// as one relaxed device-scope atomic, so a reader sees either an older word or the whole
// new one, on whatever XCD it runs.
__device__ __forceinline__ void put_tagged(uint64_t* p, uint32_t tag, float v)
{
    __hip_atomic_store(p, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get_tagged(const uint64_t* p)
{
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_is(uint64_t w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }
// The same 64-bit word read through the XCD's L2 (sc0: past the CU's L1 only) and waited
// for in the same statement. Cheaper than get_tagged when writer and reader share an XCD;
// from another XCD the L2 may hold an older copy, whose tag then does not match, so
// callers fall back to get_tagged. A naturally aligned 64-bit load is single-copy atomic
// (it is how get_tagged itself compiles, with the device-coherence bit).
__device__ __forceinline__ uint64_t get_tagged_l2(const uint64_t* p)
{
    uint64_t w;
    asm volatile("global_load_dwordx2 %0, %1, off sc0\n\ts_waitcnt vmcnt(0)" : "=v"(w) : "v"(p) : "memory");
    return w;
}
__device__ __forceinline__ float tagged_value(uint64_t w) { return __uint_as_float((uint32_t)w); }

constexpr int kSpinLimit = 1 << 18;   // polls of global memory before a wait gives up (about 0.3 s)
constexpr int kLdsSpinLimit = 1 << 24;   // polls of an LDS word (a guard: these waits end by construction)

// x loads for the register ring, issued from inline assembly: the compiler's own wait
// insertion cannot follow loads whose registers are consumed several iterations of a
// loop later (it drains them every iteration), so these loads are invisible to it and
// the kernel waits for them explicitly (wait_vm_only, ring_ready). A ring register is read
// only after its wait; every load issued is consumed, so none lands in a register the compiler
// has given to something else.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 raw_desc(const void* base, uint32_t bytes)
{
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return i32x4{(int32_t)(uint32_t)p, (int32_t)((uint32_t)(p >> 32) & 0xffffu), (int32_t)bytes, kRsrcWord3};
}
__device__ __forceinline__ u32x4 load_ring(i32x4 desc, uint32_t off)
{
    u32x4 v;
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(off), "s"(desc) : "memory");
    return v;
}
// s_waitcnt vmcnt(K) alone (no register operands: the count may depend on a branch, and
// a register operand inside a branch makes the compiler copy the register, unloaded, to
// merge the branches); then ring_ready, an empty statement tied to the four registers, so
// that no read of them moves above the wait.
template <int K>
__device__ __forceinline__ void wait_vm_only()
{
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(K) : "memory");
}
// s_waitcnt vmcnt(n) for a wave-uniform n (a scalar branch to the instruction with that
// count); n at most the deepest prefetch's count
__device__ __forceinline__ void wait_vm_upto(int n)
{
    switch (n) {
    case 0: wait_vm_only<0>(); break;
    case 1: wait_vm_only<1>(); break;
    case 2: wait_vm_only<2>(); break;
    case 3: wait_vm_only<3>(); break;
    case 4: wait_vm_only<4>(); break;
    case 5: wait_vm_only<5>(); break;
    case 6: wait_vm_only<6>(); break;
    case 7: wait_vm_only<7>(); break;
    case 8: wait_vm_only<8>(); break;
    case 9: wait_vm_only<9>(); break;
    case 10: wait_vm_only<10>(); break;
    case 11: wait_vm_only<11>(); break;
    case 12: wait_vm_only<12>(); break;
    case 13: wait_vm_only<13>(); break;
    case 14: wait_vm_only<14>(); break;
    default: wait_vm_only<0>(); break;   // (never: a wait for everything is always safe)
    static_assert(kFMaxYounger <= 14, "a case per count");
    }
}
__device__ __forceinline__ void ring_ready(u32x4 (&v)[4])
{
    asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]) : : "memory");
}

struct FArgs {
    ForwardArgs a;
    int64_t T;
    int64_t K;
    int64_t tiles16;
    int D;
    int nblk;
    int G;               // groups (of kFMembers members): XCDs taking part
};

// One workgroup = member s of group g: g is its XCD (hardware XCC id), s its arrival order
// on that XCD (a workgroup that arrives after the group is full, or on an XCD beyond the
// G groups needed, leaves), so the tagged words a group exchanges stay in one L2. Waves
// 0 .. 6 compute: wave w
// owns d-block member_begin + w and, for a tile of 16 tokens, its n K-steps (the n streams
// of the block), so a lane holds the n streams of one octet and hIn is local to it. Wave 7
// is the control wave: it alone waits on other workgroups. Round r of the group is tile
// r G + g. Per round (one workgroup barrier, at its middle):
//   compute waves: project the round's tile (x loaded kFAhead rounds ago), fold each phi
//     row's hi, mid and lo sums and put them in LDS; barrier of the compute waves; one
//     value each of the tile's partial record (totals over the waves), stored for the
//     epilogue and, for the pre sums and the square, tagged for the designated member;
//     hIn of the tile of round r - kFLag from the registers still holding its x and the
//     hPre the control wave placed in LDS; then the x loads of round r + kFAhead into the
//     registers just freed (stores first, loads last: the wait for a round's x counts the
//     stores issued after its loads).
//   control wave (outside the barrier): iteration k, once the compute waves have passed
//     their barrier of round k + 1 (so their records of round k are stored): if this
//     member is designated for round k (designated = round mod P), sums the members'
//     tagged pre-branch records of that tile in the epilogue's order and publishes its
//     hPre; then polls the hPre of round k - 2 and hands it to the compute waves through
//     LDS slot (k - 2) mod 4 and its flag.
// Every wait at round r is for work other members finish by their round r - 1, so with
// all workgroups of a group resident at once (one per compute unit of the XCD, which an
// otherwise idle device gives) the waits end; a wait that does not end within
// kSpinLimit polls sets sync[1] and yields NaN hPre for that tile. NeverReady: the
// instance for the test of that path, whose waits accept no tag and give up after 8 polls.
template <int N, int A, bool NeverReady, bool H>
__global__ void __launch_bounds__(kFThreads, 1)
fused_kernel(FArgs f)
{
    using C = Cfg<N, A>;
    constexpr int M = C::M, NT = C::NT, NC = C::NC, PPS = C::PPS, V = C::V, CH = C::CH;
    constexpr int NCL = 3 * M;                 // packed columns kept in LDS
    constexpr int NW = kFMaxBlocks;            // compute waves
    constexpr int CTRL = kFWaves - 1;
    static_assert(N == 4 && A == 3, "single-read kernel: n = 4 with alpha[3]");
    static_assert(NW == CTRL, "one compute wave per d-block, then the control wave");
    constexpr int P = kFMembers;               // members per group
    constexpr int GS = (P + 7) / 8;            // the epilogue's summation groups over members
    static_assert(P % GS == 0, "whole summation groups");
    static_assert(NT == 5 && NCL == 72 && M == 24, "column pairing of hi, mid and lo below");
    __shared__ u32x4 wl[NW * N * 4 * NCL];        // the member's packed weights
    constexpr int MP = 32;                       // row stride: lanes 8..15 write into the padding
    __shared__ float part[2][NW][kFTok][MP];     // each compute wave's row sums, by round parity
    __shared__ float part_sq[2][NW][kFTok];      // and its squares
    constexpr int NS = 4;                        // hPre slots handed from the control wave
    __shared__ float hp_lds[NS][kFTok * N];
    __shared__ uint32_t hp_flag[NS];             // 1 + the round whose hPre the slot holds
    __shared__ uint32_t cbar;                    // compute-wave arrivals (NW per round)
    const ForwardArgs& a = f.a;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int j = lane & 15, grp = lane >> 4;
    __shared__ int sh_member;
    if (tid == 0) {
        uint32_t xcc;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
        const int x = (int)(xcc & 0xFu) % kXcds;
        const uint32_t t = __hip_atomic_fetch_add(a.sync + kTicket0 + x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh_member = t < (uint32_t)P && x < f.G ? x * P + (int)t : -1;
    }
    __syncthreads();
    const int gm = __builtin_amdgcn_readfirstlane(sh_member);
    if (gm < 0) return;   // the group of this XCD is full, or not needed
    const int g = gm / P, s = gm % P;
    const int b_lo = member_begin(s, f.nblk, P);
    const int nb = member_begin(s + 1, f.nblk, P) - b_lo;
    const int64_t R = g < f.tiles16 ? (f.tiles16 - g + f.G - 1) / f.G : 0;   // rounds of group g
    const uint32_t tag = (f.a.sync[0] << 1) | 1u;
    const uint32_t want = NeverReady ? tag ^ 0x40000000u : tag;   // the tag a wait accepts
    constexpr int spin_limit = kSpinLimit;

    if (a.packed) {   // the member's K-steps of the packed weights, without the zero columns past 3M
        const u32x4* src = static_cast<const u32x4*>(a.packed) + (int64_t)b_lo * N * 4 * NC;
        const int units = nb * N * 4 * NCL;
        for (int u = tid; u < units; u += kFThreads) wl[u] = src[(int64_t)(u / NCL) * NC + u % NCL];
    } else {          // packed here from phi (and gamma), as prepack_kernel packs them
        // (K-step, octet row, phi row) items, three LDS units each: every item's phi (and
        // gamma) loads go out first, two 16-byte loads each where the arrays are 16-byte
        // aligned (an item's 8 weights are consecutive and start at a multiple of 8
        // elements), then the splits: in fp32 without gamma (the same bits), else of the
        // product in fp64
        const int items = nb * N * 4 * M;
        constexpr int PER = (NW * N * 4 * M + kFThreads - 1) / kFThreads;
        float pv[PER][8], gv[PER][8];
        const bool vec = ((reinterpret_cast<uintptr_t>(a.phi) | reinterpret_cast<uintptr_t>(a.gamma)) & 15) == 0;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int it = tid + q * kFThreads;
            const int m = it % M, row = it / M;        // row = K-step * 4 + octet
            const int kk = row / 4, og = row % 4;
            const int k = b_lo * N + kk;               // K-step: d-block k / N, stream k % N
            const int d = kBlock * (k / N) + 8 * og;
            const bool live = it < items && d < f.D;
            const int64_t k0 = (int64_t)(k % N) * f.D + d;
            if (vec) {
                const float4 z = {0.f, 0.f, 0.f, 0.f}, o = {1.f, 1.f, 1.f, 1.f};
                const float4* pp4 = reinterpret_cast<const float4*>(a.phi + (int64_t)m * f.K + k0);
                const float4* gp4 = reinterpret_cast<const float4*>(a.gamma + k0);
                const float4 p0 = live ? pp4[0] : z, p1 = live ? pp4[1] : z;
                const float4 g0 = live && a.gamma ? gp4[0] : o, g1 = live && a.gamma ? gp4[1] : o;
                pv[q][0] = p0.x; pv[q][1] = p0.y; pv[q][2] = p0.z; pv[q][3] = p0.w;
                pv[q][4] = p1.x; pv[q][5] = p1.y; pv[q][6] = p1.z; pv[q][7] = p1.w;
                gv[q][0] = g0.x; gv[q][1] = g0.y; gv[q][2] = g0.z; gv[q][3] = g0.w;
                gv[q][4] = g1.x; gv[q][5] = g1.y; gv[q][6] = g1.z; gv[q][7] = g1.w;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pv[q][e] = live ? a.phi[(int64_t)m * f.K + k0 + e] : 0.f;
                    gv[q][e] = live && a.gamma ? a.gamma[k0 + e] : 1.f;
                }
            }
        }
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int it = tid + q * kFThreads;
            if (it >= items) continue;
            const int m = it % M, row = it / M;
            u32x4 w3[3] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint32_t tb[3];
                if (a.gamma) split3_x<H>((double)pv[q][e] * (double)gv[q][e], tb);
                else split3_x32<H>(pv[q][e], tb);
#pragma unroll
                for (int term = 0; term < 3; ++term) w3[term][e >> 1] |= tb[term] << (16 * (e & 1));
            }
#pragma unroll
            for (int term = 0; term < 3; ++term) wl[row * NCL + term * M + m] = w3[term];
        }
    }
    if (tid < NS) hp_flag[tid] = 0u;
    if (tid == 0) cbar = 0u;
    __syncthreads();   // the only barrier of all eight waves
    // LDS words the waves poll: relaxed atomics; asm statements with a memory clobber keep
    // the compiler from moving other LDS accesses across them (a wave's LDS operations
    // execute in order)
    auto lds_get = [](uint32_t* w) { return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); };
    auto wait_lds_at_least = [&](uint32_t* w, uint32_t target) {
        for (int it = 0; lds_get(w) < target && it < kLdsSpinLimit; ++it) __builtin_amdgcn_s_sleep(1);
        asm volatile("" : : : "memory");
    };

    if (wave != CTRL) {
        const bool has_blk = wave < nb;
        const int b = b_lo + wave;
        const bool oct_ok = has_blk && kBlock * b + 8 * grp < f.D;
        const uint32_t xo = (uint32_t)(((int64_t)j * f.K + kBlock * b + 8 * grp) * 2);
        const uint32_t ho = (uint32_t)(((int64_t)j * f.D + kBlock * b + 8 * grp) * 2);
        const u32x4* wb = wl + wave * N * 4 * NCL + grp * NCL;
        u32x4 xr[kFRing][N];
        // x of round q (tile q G + g) into dst; only rounds < R and waves with a block
        // load, so the untracked loads in flight are exactly those of the next rounds
        auto load_round = [&](int64_t q, u32x4 (&dst)[N]) {
            const int64_t t0 = (q * f.G + g) * kFTok;
            const int64_t nt = f.T - t0 < kFTok ? f.T - t0 : kFTok;
            const i32x4 desc = raw_desc(a.x + t0 * f.K, (uint32_t)(nt * f.K * 2));
#pragma unroll
            for (int i = 0; i < N; ++i) dst[i] = load_ring(desc, xo + 2 * (uint32_t)f.D * i);
        };
        static_assert(N == kFLoads, "wait counts: one x load per stream and round");
        if (has_blk) {
#pragma unroll
            for (int q = 0; q < kFAhead; ++q)
                if (q < R) load_round(q, xr[q]);
        }

        // One barrier per round (B). Partial sums alternate between two LDS buffers by
        // round parity: a wave writes buffer r & 1 in round r only after every wave has
        // passed barrier r - 1, so after every read of round r - 2's sums; the hPre slot
        // the compute waves read in round r was written before barrier r - 1 and is
        // rewritten only after barrier r.
        for (int64_t r0 = 0; r0 < R + kFLag; r0 += kFRing) {
#pragma unroll
            for (int u = 0; u < kFRing; ++u) {
                const int64_t r = r0 + u;
                if (r >= R + kFLag) break;
                const int pb = (int)(r & 1);
                if (r < R && has_blk) {
                    // this round's x
                    wait_vm_upto(fused_younger_than_x(r, R));
                    ring_ready(xr[u]);
                    f32x4 acc[NT];
                    f32x4 sq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
                    // the weight operands from LDS two K-steps at a time, all issued before
                    // their first product (columns past 3M feed only output columns nobody
                    // reads: any in-bounds LDS column serves)
#pragma unroll
                    for (int i0 = 0; i0 < N; i0 += 2) {
                        u32x4 bw[2][NT];
#pragma unroll
                        for (int di = 0; di < 2; ++di)
#pragma unroll
                            for (int nt = 0; nt < NT; ++nt) {
                                const int col = 16 * nt + j < NCL ? 16 * nt + j : 16 * nt + j - 16;
                                bw[di][nt] = wb[(i0 + di) * 4 * NCL + col];
                            }
                        __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the products
#pragma unroll
                        for (int di = 0; di < 2; ++di) {
                            const u32x4 z = {0u, 0u, 0u, 0u};
                            const u32x4 Av = oct_ok ? xr[u][i0 + di] : z;
                            sq = mfma_x16<H>(Av, Av, sq);
#pragma unroll
                            for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma_x16<H>(Av, bw[di][nt], acc[nt]);
                        }
                    }
                    // phi row m's hi, mid and lo are columns m, M + m, 2M + m: lane j of a
                    // 16-lane row holds row m = j (and m = 16 + j when j < 8), its mid term
                    // in lane (j + 8) mod 16; added in fp32 (hi, then mid, then lo: two
                    // roundings of the wave's sum, well inside the accuracy kept)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int t = 4 * grp + q;
                        const float m1 = dpp<kRowRor8>(acc[1][q]), m2 = dpp<kRowRor8>(acc[2][q]);
                        part[pb][wave][t][j] = (acc[0][q] + kMidScale<H> * (j < 8 ? m1 : m2)) + kLoScale<H> * acc[3][q];
                        part[pb][wave][t][16 + j] = (acc[1][q] + kMidScale<H> * m2) + kLoScale<H> * acc[4][q];   // j >= 8: padding
                    }
                    const int rr = j - 4 * grp;
                    if (rr >= 0 && rr < 4) part_sq[pb][wave][j] = sq[rr];
                }
                // barrier of the compute waves: every wave's sums of this round are in LDS
                asm volatile("" : : : "memory");
                if (lane == 0) __hip_atomic_fetch_add(&cbar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                wait_lds_at_least(&cbar, (uint32_t)(NW * (r + 1)));

                if (r < R) {
                    // the tile's partial record, one value per compute lane: token t, record
                    // value v (the n pre sums, the square, padding, the other M - n sums),
                    // summed over the compute waves in wave order. Two stores per wave (the
                    // record value, the tagged word: some lane of every wave has v <= n).
                    const int64_t jt = r * f.G + g;
                    const int64_t t0 = jt * kFTok;
                    const int ntile = (int)(f.T - t0 < kFTok ? f.T - t0 : kFTok);
                    // the epilogue's record layout: slice = member, 64-token tiles
                    const rsrc_t rec = make_rsrc(a.rec + rec_tile(jt / 4, P, N, M), (int64_t)P * kTileTokens * V * 4);
                    const int tl0 = kFTok * (int)(jt % 4);
                    uint64_t* prx_tile = a.prx + prx_at(jt, P, s, 0, 0, N);
                    auto reduce_item = [&](int L) {
                        const int t = L / V, v = L % V;
                        const int m = v < N ? v : (v < PPS ? 0 : N + (v - PPS));   // square / padding: row 0, unused
                        float qv[NW], qs[NW];
#pragma unroll
                        for (int w = 0; w < NW; ++w) {   // all reads first, then the sums
                            qv[w] = part[pb][w][t][m];
                            qs[w] = part_sq[pb][w][t];
                        }
                        float hsum = 0.f, ssum = 0.f;   // fp32, in wave order
                        if (nb == NW) {
#pragma unroll
                            for (int w = 0; w < NW; ++w) {
                                hsum += qv[w];
                                ssum += qs[w];
                            }
                        } else {
#pragma unroll
                            for (int w = 0; w < NW; ++w) {
                                hsum += w < nb ? qv[w] : 0.f;
                                ssum += w < nb ? qs[w] : 0.f;
                            }
                        }
                        const float val = v == N ? ssum : (v > N && v < PPS) ? 0.f : hsum;
                        st_buf(rec, t < ntile ? (uint32_t)(rec_loc(s, tl0 + t, N, M) + v) * 4 : kOutOfRange, val);
                        // the tagged pre-branch sums and square for the designated member
                        if (v <= N) put_tagged(prx_tile + t * (N + 1) + v, tag, val);
                    };
                    static_assert(kFTok * V == 64 * NW, "one record value per compute lane");
                    reduce_item(wave * 64 + lane);
                }
                // hIn of round r - kFLag from the registers that still hold its x (one store)
                const int us = (u + kFAhead) % kFRing;
                const int64_t rh = r - kFLag;
                if (rh >= 0 && has_blk) {
                    const int64_t t0 = (rh * f.G + g) * kFTok;
                    const int64_t nt = f.T - t0 < kFTok ? f.T - t0 : kFTok;
                    wait_lds_at_least(&hp_flag[rh % NS], (uint32_t)rh + 1u);   // the control wave's hand-over
                    float w[N];
#pragma unroll
                    for (int i = 0; i < N; ++i) w[i] = hp_lds[rh % NS][j * N + i];
                    float hacc[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) hacc[e] = 0.f;
#pragma unroll
                    for (int i = 0; i < N; ++i) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            hacc[2 * e] = fmaf(w[i], x16_lo<H>(xr[us][i][e]), hacc[2 * e]);
                            hacc[2 * e + 1] = fmaf(w[i], x16_hi<H>(xr[us][i][e]), hacc[2 * e + 1]);
                        }
                    }
                    u32x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = pack_x16<H>(hacc[2 * e], hacc[2 * e + 1]);
                    const rsrc_t hres = make_rsrc(a.h_in + t0 * f.D, nt * f.D * 2);
                    __builtin_amdgcn_raw_buffer_store_b128(o, hres, (int)(oct_ok ? ho : kOutOfRange), 0, 0);
                }
                if (has_blk && r + kFAhead < R) load_round(r + kFAhead, xr[us]);
            }
        }
    } else {
        // control wave
        const int tq = lane / N, iq = lane % N;   // (token, stream) of this lane's hPre word
        bool failed = false;
        auto fail = [&]() {
            if (!failed && lane == 0)
                __hip_atomic_store(a.sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            failed = true;
        };
        // the tagged pre-branch records of tile jt, half of the members at a time (members
        // q0 .. q0 + P/2 - 1: whole summation groups; fewer registers than all at once)
        constexpr int PH = P / 2;
        static_assert(PH % GS == 0, "whole summation groups per half");
        uint64_t pre[PH], pss[PH];
        auto load_records = [&](int64_t jt, int q0) {
#pragma unroll
            for (int q = 0; q < PH; ++q) {
                pre[q] = get_tagged(a.prx + prx_at(jt, P, q0 + q, tq, iq, N));
                pss[q] = get_tagged(a.prx + prx_at(jt, P, q0 + q, tq, N, N));
            }
        };
        auto records_ready = [&]() {
            bool ok = true;
#pragma unroll
            for (int q = 0; q < PH; ++q) ok = ok && tag_is(pre[q], want) && tag_is(pss[q], want);
            return __all(ok);
        };
        const float alpha0 = a.alpha[0];
        const float bias_i = a.bias[iq];
        const float eps = (float)a.hc_eps;
        // Iteration k: the designated duty for tile round k, then the hand-over of round
        // k - 2's hPre. Both wait first for the compute waves to pass their barrier of
        // round k + 1, i.e. to have stored their records of round k (the other members'
        // are then nearly always visible too); the hand-over slot's previous round
        // (k - 2 - NS) was consumed in compute round k - 2 - NS + kFLag <= k + 1. The
        // compute waves need round k - 2's hPre only in their round k - 2 + kFLag.
        static_assert(kFLag >= 5 && NS >= 4, "the hand-over comes at least one round before its use");
        for (int64_t k = 0; k < R + 2; ++k) {
            wait_lds_at_least(&cbar, (uint32_t)(NW * (k + 2 < R + kFLag ? k + 2 : R + kFLag)));
            if (k < R && k % P == s) {
                const int64_t jt = k * f.G + g;
                // the epilogue's order: members in groups of GS, each group in member
                // order from 0.0, then the group totals in order from 0.0
                double hs = 0.0, ss = 0.0;
                bool ok = true;
                for (int h0 = 0; h0 < P; h0 += PH) {
                    load_records(jt, h0);
                    bool ready = records_ready();
                    for (int it = 0; !ready && !failed; ++it) {
                        if (it == spin_limit) { fail(); break; }
                        __builtin_amdgcn_s_sleep(2);
                        load_records(jt, h0);
                        ready = records_ready();
                    }
                    ok = ok && ready;
#pragma unroll
                    for (int q0 = 0; q0 < PH; q0 += GS) {
                        double ga = 0.0, gb = 0.0;
#pragma unroll
                        for (int q = q0; q < q0 + GS; ++q) {
                            ga += (double)tagged_value(pre[q]);
                            gb += (double)tagged_value(pss[q]);
                        }
                        hs += ga;
                        ss += gb;
                    }
                }
                const double inv = inv_rms_of(ss, (double)f.K, a.norm_eps);
                const float hp = ok ? gate_pre(hs, inv, alpha0, bias_i, eps) : __builtin_nanf("");
                put_tagged(a.hpx + hpx_at(jt, tq, iq, N), tag, hp);
            }
            const int64_t rp = k - 2;
            if (rp >= 0 && rp < R) {
                const uint64_t* src = a.hpx + hpx_at(rp * f.G + g, tq, iq, N);
                uint64_t w = get_tagged_l2(src);
                bool ok = tag_is(w, want);
                for (int it = 0; !__all(ok) && !failed; ++it) {
                    if (it == spin_limit) { fail(); break; }
                    __builtin_amdgcn_s_sleep(1);
                    w = (it & 1) ? get_tagged(src) : get_tagged_l2(src);   // every other poll device-coherent
                    ok = tag_is(w, want);
                }
                hp_lds[rp % NS][lane] = ok ? tagged_value(w) : __builtin_nanf("");
                asm volatile("" : : : "memory");
                if (lane == 0) __hip_atomic_store(&hp_flag[rp % NS], (uint32_t)rp + 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    }
}

// ------------------------------------------------------------------ one-launch small-T forward

struct DArgs {
    ForwardArgs a;
    int64_t T;
    int64_t K;
    int D;
    int nblk;    // d-blocks
    int nwg;     // workgroups: ceil(nblk / BPW)
};

// v / s for the Sinkhorn's positive operands (v in [0, 2], s in [eps, 5]: no scaling
// needed): the hardware reciprocal (1 ulp), the quotient, and one Newton correction of it
// from its exact fma residual; within an ulp of the correctly rounded quotient, and equal
// to it in almost every case, in four dependent operations instead of the ten of a full
// IEEE division.
__device__ __forceinline__ float div_pos(float v, float s)
{
    const float r = __builtin_amdgcn_rcpf(s);
    const float q = v * r;
    return fmaf(fmaf(-q, s, v), r, q);
}

// The Sinkhorn of one token's 4 x 4 residual logits Ls[0 .. 15] (the steps of sinkhorn_by,
// its sums in the same order, its divisions by div_pos), entry (r, c) in lane 4 r + c of a
// 16-lane group; `live` false: the group computes along and stores nothing. PLANES: sum_out
// and norm_out of every step are stored too.
template <bool PLANES>
__device__ __forceinline__ void sinkhorn4(const ForwardArgs& a, int64_t T, const float* Ls, int64_t tk, bool live, int e)
{
    constexpr int N = 4, NN = 16;
    const int r = e >> 2, c = e & 3;
    const float eps = (float)a.hc_eps;
    const int iters = a.num_iters;
    auto planes = [&](int step, float sum, float v, bool col) {
        if (!PLANES || !live) return;
        if (a.sum_out && (col ? r == 0 : c == 0)) a.sum_out[((int64_t)step * T + tk) * N + (col ? c : r)] = sum;
        if (a.norm_out) a.norm_out[((int64_t)step * T + tk) * NN + e] = v;
    };
    float v = live ? Ls[e] : 0.f;
    const float mx = row_max<N>(v);
    const float ex = expf(v - mx);
    float sum = row_sum<N>(ex);
    v = div_pos(ex, sum) + eps;
    if (iters > 0) planes(0, sum, v, false);
    for (int k = 0; k < iters; ++k) {
        sum = col_sum<N>(v) + eps;             // step 2k + 1: columns
        v = div_pos(v, sum);
        planes(2 * k + 1, sum, v, true);
        if (k + 1 < iters) {
            sum = row_sum<N>(v) + eps;         // step 2k + 2: rows
            v = div_pos(v, sum);
            planes(2 * k + 2, sum, v, false);
        }
    }
    if (live) a.h_res[tk * NN + e] = v;
}

// ------------------------------------------------------------------ streaming projection

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 47] (a scalar branch to the instruction
// with that count); a larger n waits for everything, which is always safe.
template <int K>
__device__ __forceinline__ void wait_vm_case()
{
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(K) : "memory");
}
template <int B>
__device__ __forceinline__ bool wait_vm_range(int n)
{
    if constexpr (B < kStreamMaxWait + 1) {
        if (n == B) {
            wait_vm_case<B>();
            return true;
        }
        return wait_vm_range<B + 1>(n);
    } else {
        return false;
    }
}
__device__ __forceinline__ void wait_vm_n(int n)
{
    if (!wait_vm_range<0>(n)) wait_vm_case<0>();
}
// A ring load into a register whose previous value is still read: the register is the
// asm statement's input and output, so the compiler keeps the value in place (the reads of
// the old value it orders before the load) and never copies the register while the load is
// in flight.
__device__ __forceinline__ void reload_ring(u32x4& v, i32x4 desc, uint32_t off)
{
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "+v"(v) : "v"(off), "s"(desc) : "memory");
}
// s_barrier after this wave's LDS operations have completed, without the vector memory
// wait a workgroup fence would add (x loads of the next task stay in flight across it).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// The classic path's projection (same 64-token tiles and partial-record layout, so the
// epilogue and hIn kernels follow unchanged) for calls without pre_mix and with D a
// multiple of 32, by persistent workgroups with a different split of K: slice s is the NKS
// K-steps [NKS s, NKS s + NKS) of the flattened row (K-step g holds elements [32 g, 32 g + 32)
// of x[t] as n*D values, i.e. stream g / nblk, d-block g mod nblk), so a task reads one
// contiguous run of 64 NKS bytes of each token row. On MI355X such 1 KB runs stream at about
// 6.2 TB/s, against about 4.5 TB/s for the 128 to 256-byte runs per stream of the
// projection kernel's slices (all n streams of a few d-blocks, which hIn from registers
// needs). Workgroup b keeps the packed weights of slice s = b mod S in LDS for the whole
// launch (gathered from phi_packed, whose K-steps are d-block-major, or split from phi and
// gamma by the workgroup itself as the pack kernel splits them: no pack launch), and its two
// halves (waves 0-3 and 4-7) each walk the tiles h, h + 2W, h + 4W, .. with h = 2 (b / S) +
// half and W workgroups per slice; each half holds two tasks' x in registers, the next
// task's x streaming in while the current one runs on the matrix cores. With S a multiple
// of 8 every workgroup of a slice runs on the same XCD (workgroups are dealt to the XCDs in
// turn), whose L2 then serves the slice's weights to all of them.
// Per task and half: wait for the task's x; 16 x 16 x 32 products of each wave's 16 tokens
// (and x x^T for the squares) in K-step order, two K-steps at a time, each pair's registers
// reloaded with the x of the task after next as soon as its products are issued (so about
// two tasks' x stay in flight all along); column totals to LDS; barrier; the records;
// barrier. The x loads are issued from inline assembly, invisible to the compiler, and
// waited for with explicit counts (stream_younger_than_x); every thread issues the same
// number of record stores per task (out-of-range offsets for the ones with nothing to
// write), so the counts hold for every wave.
template <int N, int A, int NKS, bool H>
__global__ void __launch_bounds__(kSThreads, 1)
proj_stream_kernel(KArgs k, int W, int NI)
{
    using C = Cfg<N, A>;
    constexpr int NT = C::NT, NC = C::NC, M = C::M, CH = C::CH, PPS = C::PPS;
    constexpr int WU = NKS * 4 * NC;               // 16-byte weight units of a slice
    constexpr int NREC = stream_rec_stores(CH);    // record stores per thread and task
    static_assert(stream_fits(N, A, NKS), "weights and column totals in LDS, x in registers");
    __shared__ u32x4 wl[WU];
    __shared__ float red[2][kTileTokens * NC];     // each half's column totals
    __shared__ float lds_ss[2][kTileTokens];       // and squares

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = wave >> 2, hw = wave & 3;
    const int htid = tid & (kThreads - 1);         // thread within the half
    const int lane = tid & 63;
    const int j = lane & 15, grp = lane >> 4;
    const int row = hw * 16 + j;                   // the lane's token within its tile
    const int s = (int)(blockIdx.x % (unsigned)k.S);
    const int64_t h0 = 2 * (int64_t)(blockIdx.x / (unsigned)k.S) + half;   // first tile of this half
    const int64_t hstep = 2 * (int64_t)W;
    const int nblk = k.D / kBlock;
    const int nks = N * nblk;                      // K-steps holding data
    const int g0 = s * NKS;                        // the slice's first K-step
    // the lane's octet of K-step g0 in its token's row; K-steps past the data read zero
    const uint32_t xo = (uint32_t)(((int64_t)row * k.K + (int64_t)kBlock * g0 + 8 * grp) * 2);

    u32x4 xr[2][NKS];
    auto live = [&](int it) { return h0 + hstep * it < k.tiles; };
    auto xoff = [&](int st) { return g0 + st < nks ? xo + 2 * kBlock * st : kOutOfRange; };
    auto xdesc = [&](int it) {
        const int64_t t0 = (h0 + hstep * it) * kTileTokens;
        const int64_t nt = k.T - t0 < kTileTokens ? k.T - t0 : kTileTokens;
        return raw_desc(k.a.x + t0 * k.K, (uint32_t)(nt * k.K * 2));
    };
    auto issue = [&](int it, u32x4 (&dst)[NKS]) {
        const i32x4 desc = xdesc(it);
#pragma unroll
        for (int st = 0; st < NKS; ++st) dst[st] = load_ring(desc, xoff(st));
    };
    // x loads in flight once both first tasks' loads are out
    const int x_out = (live(0) ? NKS : 0) + (live(1) ? NKS : 0);

    // Prologue: the slice's weights first, then the x of tasks 0 and 1, all in flight at once;
    // the weights are waited for by count (x keeps streaming meanwhile), then copied or split
    // into LDS. (With phi not 16-byte aligned, the compiler's own loads split it, and the x
    // loads go out after them.)
    constexpr int PU = (WU + kSThreads - 1) / kSThreads;   // packed units a thread copies
    constexpr int ITEMS = NKS * 4 * M;                     // (K-step, octet row, phi row) items
    constexpr int PER = (ITEMS + kSThreads - 1) / kSThreads;
    const bool vec = ((reinterpret_cast<uintptr_t>(k.a.phi) | reinterpret_cast<uintptr_t>(k.a.gamma)) & 15) == 0;
    // split an item's 8 weights (times gamma) into its three LDS units, as prepack_kernel
    // does: in fp32 without gamma (the same bits), else of the product in fp64
    auto split_item = [&](int it, const float (&pv)[8], const float (&gv)[8]) {
        const int m = it % M, rw = it / M;             // rw = K-step * 4 + octet
        u32x4 w3[3] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t tb[3];
            if (k.a.gamma) split3_x<H>((double)pv[e] * (double)gv[e], tb);
            else split3_x32<H>(pv[e], tb);
#pragma unroll
            for (int term = 0; term < 3; ++term) w3[term][e >> 1] |= tb[term] << (16 * (e & 1));
        }
#pragma unroll
        for (int term = 0; term < 3; ++term) wl[rw * NC + term * M + m] = w3[term];
    };
    if (k.a.packed) {
        // K-step g is packed K-step (g mod nblk) N + g / nblk; past the data: the packed
        // buffer's zero K-steps
        const i32x4 pd = raw_desc(k.a.packed, (uint32_t)((int64_t)(nks + kPadSteps) * 4 * NC * 16));
        u32x4 pw[PU];
#pragma unroll
        for (int q = 0; q < PU; ++q) {
            const int u = tid + q * kSThreads;
            const int g = g0 + u / (4 * NC);
            const int64_t pst = g < nks ? (int64_t)(g % nblk) * N + g / nblk : (int64_t)nks;
            pw[q] = load_ring(pd, u < WU ? (uint32_t)((pst * 4 * NC + u % (4 * NC)) * 16) : kOutOfRange);
        }
        if (live(0)) issue(0, xr[0]);
        if (live(1)) issue(1, xr[1]);
        wait_vm_n(x_out);
#pragma unroll
        for (int q = 0; q < PU; ++q) {
            asm volatile("" : "+v"(pw[q]) : : "memory");
            const int u = tid + q * kSThreads;
            if (u < WU) wl[u] = pw[q];
        }
    } else if (vec) {
        // an item's 8 weights (and gammas) are consecutive and start at a multiple of 8
        // elements: two 16-byte loads each; items past the data read zeros
        const i32x4 phd = raw_desc(k.a.phi, (uint32_t)((int64_t)M * k.K * 4));
        const i32x4 gmd = raw_desc(k.a.gamma, (uint32_t)(k.K * 4));
        u32x4 pl[PER][2], gl[PER][2];
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int it = tid + q * kSThreads;
            const int m = it % M, rw = it / M;
            const int g = g0 + rw / 4;
            const bool ok = it < ITEMS && g < nks;
            const int64_t k0 = (int64_t)kBlock * g + 8 * (rw % 4);   // flattened K index
            const uint32_t po = ok ? (uint32_t)(((int64_t)m * k.K + k0) * 4) : kOutOfRange;
            pl[q][0] = load_ring(phd, po);
            pl[q][1] = load_ring(phd, ok ? po + 16 : kOutOfRange);
            if (k.a.gamma) {
                const uint32_t go = ok ? (uint32_t)(k0 * 4) : kOutOfRange;
                gl[q][0] = load_ring(gmd, go);
                gl[q][1] = load_ring(gmd, ok ? go + 16 : kOutOfRange);
            }
        }
        if (live(0)) issue(0, xr[0]);
        if (live(1)) issue(1, xr[1]);
        wait_vm_n(x_out);
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            asm volatile("" : "+v"(pl[q][0]), "+v"(pl[q][1]) : : "memory");
            if (k.a.gamma) asm volatile("" : "+v"(gl[q][0]), "+v"(gl[q][1]) : : "memory");
            const int it = tid + q * kSThreads;
            if (it >= ITEMS) continue;
            float pv[8], gv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pv[e] = __uint_as_float(pl[q][e >> 2][e & 3]);
                gv[e] = k.a.gamma ? __uint_as_float(gl[q][e >> 2][e & 3]) : 1.f;
            }
            split_item(it, pv, gv);
        }
    } else {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int it = tid + q * kSThreads;
            if (it >= ITEMS) continue;
            const int m = it % M, rw = it / M;
            const int g = g0 + rw / 4;
            const bool ok = g < nks;
            const int64_t k0 = (int64_t)kBlock * g + 8 * (rw % 4);
            float pv[8], gv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pv[e] = ok ? k.a.phi[(int64_t)m * k.K + k0 + e] : 0.f;
                gv[e] = ok && k.a.gamma ? k.a.gamma[k0 + e] : 1.f;
            }
            split_item(it, pv, gv);
        }
        if (live(0)) issue(0, xr[0]);
        if (live(1)) issue(1, xr[1]);
    }
    if (!k.a.packed) {
        // the padding columns 3M .. NC - 1 (their products land in columns no record reads)
        if constexpr (NC > 3 * M) {
            for (int u = tid; u < NKS * 4 * (NC - 3 * M); u += kSThreads)
                wl[(u / (NC - 3 * M)) * NC + 3 * M + u % (NC - 3 * M)] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    lds_barrier();   // the weights are in LDS (the x loads stay in flight)

    const u32x4* wb = wl + grp * NC + j;
    for (int it0 = 0; it0 < NI; it0 += 2) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int it = it0 + u;
            if (it >= NI) break;                       // (the same for the whole workgroup)
            const bool on = live(it);
            const int64_t tile = h0 + hstep * it;
            const int ntile = on ? tile_tokens(k, tile * kTileTokens) : 0;
            if (on) {
                wait_vm_n(stream_younger_than_x(it, live(it + 1), NKS, NREC));
#pragma unroll
                for (int st = 0; st < NKS; ++st) asm volatile("" : "+v"(xr[u][st]) : : "memory");
                // the x of task it + 2 goes into each register pair once its products are issued
                const bool next2 = live(it + 2);
                const i32x4 desc2 = xdesc(next2 ? it + 2 : it);
                f32x4 acc[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
                f32x4 sq = {0.f, 0.f, 0.f, 0.f};
                // the weight operands of two K-steps read from LDS before their products
#pragma unroll
                for (int st0 = 0; st0 < NKS; st0 += 2) {
                    u32x4 bw[2][NT];
#pragma unroll
                    for (int di = 0; di < 2; ++di)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) bw[di][nt] = wb[(st0 + di) * 4 * NC + nt * 16];
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int di = 0; di < 2; ++di) {
                        const u32x4 xa = xr[u][st0 + di];
                        sq = mfma_x16<H>(xa, xa, sq);
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma_x16<H>(xa, bw[di][nt], acc[nt]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    if (next2) {
#pragma unroll
                        for (int di = 0; di < 2; ++di) reload_ring(xr[u][st0 + di], desc2, xoff(st0 + di));
                    }
                }
                float* rd = red[half];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) rd[(hw * 16 + 4 * grp + r) * NC + nt * 16 + j] = acc[nt][r];
                const int rr = j - 4 * grp;
                if (rr >= 0 && rr < 4) lds_ss[half][hw * 16 + j] = sq[rr];
            }
            lds_barrier();   // A: the column totals of both halves are in LDS
            if (on) {
                // the records (hi + mid + lo of each phi row added in fp64, rounded once)
                const float* rd = red[half];
                const rsrc_t rec = make_rsrc(k.a.rec + rec_tile(tile, k.S, N, M), (int64_t)k.S * kTileTokens * C::V * 4);
#pragma unroll
                for (int q = 0; q < NREC; ++q) {
                    const int idx0 = htid + q * kThreads;
                    const bool ok = idx0 < kTileTokens * CH;
                    const int idx = ok ? idx0 : 0;
                    const int tl = idx / CH, ch = idx % CH;
                    const float* rp = rd + tl * NC;
                    u32x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int v = 4 * ch + e;
                        const int m = v < N ? v : N + (v - PPS);
                        float val;
                        if (v == N) val = lds_ss[half][tl];
                        else if ((v > N && v < PPS) || v >= PPS + (M - N)) val = 0.f;   // padding
                        else if (H)   // the fp16 terms carry scales 1, 2^11, 2^22 (split3_f16)
                            val = (float)((double)rp[m] + 0x1p-11 * (double)rp[M + m] + 0x1p-22 * (double)rp[2 * M + m]);
                        else val = (float)((double)rp[m] + (double)rp[M + m] + (double)rp[2 * M + m]);
                        o[e] = __float_as_uint(val);
                    }
                    const uint32_t off = ok && tl < ntile ? (uint32_t)(rec_loc(s, tl, N, M) + 4 * ch) * 4 : kOutOfRange;
                    __builtin_amdgcn_raw_buffer_store_b128(o, rec, (int)off, 0, 0);
                }
            }
            lds_barrier();   // B: both halves are done reading the column totals
        }
    }
}

// The whole forward of up to kDecodeTokens tokens in one launch (n = 4, alpha[3]): workgroup
// b owns BPW d-blocks, BPW b .. BPW b + BPW - 1 (32 positions of each stream each; two
// blocks a workgroup halve the records every token's owner reads, where there are still
// at least as many workgroups as tokens).
//   Phase 1: its weights into LDS (copied from phi_packed, or split from phi and gamma as
//   the pack kernel splits them), x of every token for its blocks into registers (wave w:
//   tokens 16 w .. 16 w + 15), the projection and the squares on the matrix cores, and the
//   workgroup's partial record of every token to the workspace.
//   Phase 2, workgroups b < T, for tokens b, b + nwg, ..: the token's records summed over
//   the workgroups (fp64: in workgroup order within each of 10 partitions, then the partitions in
//   order), then the per-token math of the epilogue kernel (hMix, invRms, hPre, hPost), hPre
//   to the workspace, and the Sinkhorn planes and hRes (on one wave while the others go on).
//   Phase 3: hIn of the blocks from the x registers, once every token's hPre is there.
// The records and hPre cross workgroups (and XCDs, whose L2 caches are not coherent with
// each other) as tagged words: value and the call's tag in one 64-bit word, stored and
// loaded as device-scope atomics, and a reader polls a word until it carries this call's
// tag. No barrier and no fence at device scope (on this GPU such a fence writes back or
// invalidates a whole L2). The tag comes from flag word b, which only workgroup b reads
// and writes, adding 1 per call to flags b, b + nwg, .. (all kDecodeMaxBlocks of them):
// every flag holds the same count at the start of a call, whatever the grids of earlier
// calls, so every workgroup derives the same tag, and a word of an earlier call never
// carries it. The polls are bounded: a time-out sets sync[1] and the outputs that depend
// on it are NaN (all of the token's at a record, hIn at an hPre). Workgroups wait on each
// other, so all nwg of them must be resident at once: the path is taken only where the
// device holds them.
template <int N, int A, bool NeverReady, bool H, int BPW>
__global__ void __launch_bounds__(kThreads)
decode_kernel(DArgs f)
{
    using C = Cfg<N, A>;
    constexpr int M = C::M, NT = C::NT, NC = C::NC, NN = C::NN, NCL = 3 * M;
    constexpr int R = M + 1;                        // record values: n pre sums, the square, M - n sums
    constexpr int RS = kDecodeRecWords;             // record stride in words (R and a pad word)
    static_assert(RS == R + 1 && RS % 2 == 0, "record layout: whole 16-byte chunks");
    static_assert(N == 4 && A == 3 && NT == 5 && NCL == 72, "the single-read kernel's column pairing");
    static_assert(kDecodeTokens == 4 * 16, "one matrix row per token, 16 per wave");
    constexpr int MP = 32;
    constexpr int NPART = 10;                       // partitions of the block sum
    constexpr int BATCH = 32;                       // record words in flight per thread
    static_assert(NPART * R <= kThreads, "one thread per (partition, value)");
    static_assert(BPW == 1 || BPW == 2, "one or two d-blocks a workgroup");
    __shared__ u32x4 wl[BPW * N * 4 * NCL];         // the blocks' packed weights
    __shared__ float part[4][16][MP];               // each wave's row sums
    __shared__ float part_sq[4][16];
    __shared__ double red[NPART][R];
    __shared__ float Ls[kDecodeTokens * NN];        // residual logits of this workgroup's tokens
    __shared__ float gpar[3 + M];                   // alpha, bias
    __shared__ u32x4 xs[64][BPW][N];                // wave 3's x while it runs the Sinkhorn
    __shared__ uint32_t sh_epoch;
    __shared__ int sh_bad;
    const ForwardArgs& a = f.a;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int j = lane & 15, grp = lane >> 4;
    const int b = blockIdx.x;                        // workgroup
    const int nwg = f.nwg;
    uint32_t* const flags = a.sync + kDecodeFlag0;
    uint64_t* const rec = reinterpret_cast<uint64_t*>(a.dpart);
    uint64_t* const hpw = reinterpret_cast<uint64_t*>(a.dhp);

    if (tid == 0) sh_epoch = __hip_atomic_load(flags + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) sh_bad = 0;
    if (tid < A) gpar[tid] = a.alpha[tid];
    if (tid < M) gpar[3 + tid] = a.bias[tid];

    // phase 1: x (first: the longest wait), weights, projection
    const int t = 16 * wave + j;                     // the lane's token
    const bool wave_live = 16 * wave < f.T;          // the wave has tokens
    // bit e: the lane's octet of block e lies before D
    const uint32_t oct_ok = (kBlock * (BPW * b) + 8 * grp < f.D ? 1u : 0u) |
                            (BPW > 1 && kBlock * (BPW * b + 1) + 8 * grp < f.D ? 2u : 0u);
    const rsrc_t xres = make_rsrc(a.x, f.T * f.K * 2);
    u32x4 xr[BPW][N];
#pragma unroll
    for (int e = 0; e < BPW; ++e)
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const uint32_t off = ((oct_ok >> e) & 1u) && t < f.T
                                     ? (uint32_t)(((int64_t)t * f.K + (int64_t)i * f.D + kBlock * (BPW * b + e) + 8 * grp) * 2)
                                     : kOutOfRange;
            xr[e][i] = __builtin_amdgcn_raw_buffer_load_b128(xres, (int)off, 0, 0);
        }
    constexpr int WU = BPW * N * 4 * NCL;            // 16-byte weight units of the blocks
    if (a.packed) {
        // every load issued before the first LDS store (a second block past the data reads
        // the packed buffer's zero K-steps)
        constexpr int PER = (WU + kThreads - 1) / kThreads;
        const u32x4* src = static_cast<const u32x4*>(a.packed) + (int64_t)(BPW * b) * N * 4 * NC;
        u32x4 wv[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int u = tid + k * kThreads;
            if (u < WU) wv[k] = src[(int64_t)(u / NCL) * NC + u % NCL];
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int u = tid + k * kThreads;
            if (u < WU) wl[u] = wv[k];
        }
    } else {
        // (phi row m, K-step kk, octet og) items: their phi and gamma loads first, then the splits
        constexpr int ITEMS = BPW * N * 4 * M;
        constexpr int PER = (ITEMS + kThreads - 1) / kThreads;
        float pv[PER][8], gv[PER][8];
        // an item's 8 weights (and gammas) are consecutive and start at a multiple of 8
        // elements: two 16-byte loads each where the arrays are 16-byte aligned
        const bool vec = ((reinterpret_cast<uintptr_t>(a.phi) | reinterpret_cast<uintptr_t>(a.gamma)) & 15) == 0;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int it = tid + k * kThreads;
            const int m = it % M, row = it / M, kl = row / 4, og = row % 4;   // K-step kl of the workgroup's
            const int d = kBlock * (BPW * b + kl / N) + 8 * og;                 // blocks: stream kl % N
            const bool live = it < ITEMS && d < f.D;
            const int64_t k0 = (int64_t)(kl % N) * f.D + d;
            if (vec) {
                const float4 z = {0.f, 0.f, 0.f, 0.f}, o = {1.f, 1.f, 1.f, 1.f};
                const float4* pp4 = reinterpret_cast<const float4*>(a.phi + (int64_t)m * f.K + k0);
                const float4* gp4 = reinterpret_cast<const float4*>(a.gamma + k0);
                const float4 p0 = live ? pp4[0] : z, p1 = live ? pp4[1] : z;
                const float4 g0 = live && a.gamma ? gp4[0] : o, g1 = live && a.gamma ? gp4[1] : o;
                pv[k][0] = p0.x; pv[k][1] = p0.y; pv[k][2] = p0.z; pv[k][3] = p0.w;
                pv[k][4] = p1.x; pv[k][5] = p1.y; pv[k][6] = p1.z; pv[k][7] = p1.w;
                gv[k][0] = g0.x; gv[k][1] = g0.y; gv[k][2] = g0.z; gv[k][3] = g0.w;
                gv[k][4] = g1.x; gv[k][5] = g1.y; gv[k][6] = g1.z; gv[k][7] = g1.w;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pv[k][e] = live ? a.phi[(int64_t)m * f.K + k0 + e] : 0.f;
                    gv[k][e] = live && a.gamma ? a.gamma[k0 + e] : 1.f;
                }
            }
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int it = tid + k * kThreads;
            if (it >= ITEMS) continue;
            const int m = it % M, row = it / M;      // row = K-step * 4 + octet
            u32x4 w3[3] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint32_t tb[3];   // in fp32 without gamma (the same bits), else of the product in fp64
                if (a.gamma) split3_x<H>((double)pv[k][e] * (double)gv[k][e], tb);
                else split3_x32<H>(pv[k][e], tb);
#pragma unroll
                for (int term = 0; term < 3; ++term) w3[term][e >> 1] |= tb[term] << (16 * (e & 1));
            }
#pragma unroll
            for (int term = 0; term < 3; ++term) wl[row * NCL + term * M + m] = w3[term];
        }
    }
    __syncthreads();   // the weights, parameters and epoch are in LDS
    const uint32_t epoch = sh_epoch;
    const uint32_t tag = 2u * epoch + 1u;            // odd: never the zero of a fresh workspace
    const uint32_t want = NeverReady ? tag ^ 0x40000000u : tag;
    if (wave_live) {
        f32x4 acc[NT];
        f32x4 sq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < BPW; ++e)
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const u32x4* wb = wl + (e * N + i) * 4 * NCL + grp * NCL;
                sq = mfma_x16<H>(xr[e][i], xr[e][i], sq);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const int col = 16 * nt + j < NCL ? 16 * nt + j : 16 * nt + j - 16;
                    acc[nt] = mfma_x16<H>(xr[e][i], wb[col], acc[nt]);
                }
            }
        // phi row m's hi, mid and lo are columns m, M + m, 2M + m (as in the single-read kernel)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int tt = 4 * grp + q;
            const float m1 = dpp<kRowRor8>(acc[1][q]), m2 = dpp<kRowRor8>(acc[2][q]);
            part[wave][tt][j] = (acc[0][q] + kMidScale<H> * (j < 8 ? m1 : m2)) + kLoScale<H> * acc[3][q];
            part[wave][tt][16 + j] = (acc[1][q] + kMidScale<H> * m2) + kLoScale<H> * acc[4][q];   // j >= 8: padding
        }
        const int rr = j - 4 * grp;
        if (rr >= 0 && rr < 4) part_sq[wave][j] = sq[rr];
    }
    __syncthreads();
    // the workgroup's partial record of every token ([token][workgroup][word]: a token's records
    // are one run): word w < n the pre sums, n the square, n + 1 + i the sum of phi row n + i,
    // then a pad word (zero). All LDS reads first, then the stores.
    const int T32 = (int)f.T;
    {
        constexpr int PER = (int)((kDecodeTokens * RS + kThreads - 1) / kThreads);
        float val[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int idx = tid + k * kThreads;
            const int tk = idx / RS, w = idx - tk * RS;
            const int tq = tk < T32 ? tk : 0;
            val[k] = w < N ? part[tq >> 4][tq & 15][w] : w == N ? part_sq[tq >> 4][tq & 15]
                   : w < R ? part[tq >> 4][tq & 15][w - 1] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int idx = tid + k * kThreads;
            const int tk = idx / RS, w = idx - tk * RS;
            if (tk < T32) put_tagged(rec + (tk * nwg + b) * RS + w, tag, val[k]);
        }
    }

    // phase 2: the tokens of this workgroup
    const int ntok = b < T32 ? (T32 - b + nwg - 1) / nwg : 0;
    const float eps = (float)a.hc_eps;
    for (int q = 0; q < ntok; ++q) {
        const int tk = b + q * nwg;
        // first word 0 of every block's record (one poll word per block: light traffic while
        // the records land), then every word, each checked again
        {
            bool bad = false;
            for (int i = tid; i < nwg; i += kThreads) {
                const uint64_t* p = rec + (tk * nwg + i) * RS;
                int it = 0;
                for (; it < kSpinLimit && !tag_is(get_tagged(p), want); ++it) __builtin_amdgcn_s_sleep(1);
                bad = bad || it == kSpinLimit;
            }
            if (bad) sh_bad = 1;
        }
        __syncthreads();
        // thread (pp, v): the words v of the blocks of partition pp, in block order, fp64
        const int pp = tid / R, v = tid % R;
        if (pp < NPART && !sh_bad) {
            const int lo = pp * nwg / NPART, hi = (pp + 1) * nwg / NPART;
            const uint64_t* src = rec + tk * nwg * RS + v;
            double sacc = 0.0;
            bool bad = false;
            for (int b0 = lo; b0 < hi; b0 += BATCH) {
                const int nb = hi - b0 < BATCH ? hi - b0 : BATCH;
                uint64_t w[BATCH];
#pragma unroll
                for (int e = 0; e < BATCH; ++e) w[e] = e < nb ? get_tagged(src + (b0 + e) * RS) : 0;
                int it = 0;
                for (; it < kSpinLimit; ++it) {
                    bool all = true;
#pragma unroll
                    for (int e = 0; e < BATCH; ++e) all = all && (e >= nb || tag_is(w[e], want));
                    if (all) break;
                    __builtin_amdgcn_s_sleep(1);
#pragma unroll
                    for (int e = 0; e < BATCH; ++e)
                        if (e < nb && !tag_is(w[e], want)) w[e] = get_tagged(src + (b0 + e) * RS);
                }
                bad = bad || it == kSpinLimit;
#pragma unroll
                for (int e = 0; e < BATCH; ++e) sacc += e < nb ? (double)tagged_value(w[e]) : 0.0;   // + 0: exact
            }
            red[pp][v] = sacc;
            if (bad) sh_bad = 1;
        }
        __syncthreads();
        if (tid == 0 && sh_bad) __hip_atomic_store(a.sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tid < R) {
            double tot = 0.0;
#pragma unroll
            for (int k = 0; k < NPART; ++k) tot += red[k][tid];
            red[0][tid] = sh_bad ? __builtin_nan("") : tot;
        }
        __syncthreads();
        // the epilogue kernel's per-token math
        if (tid < M) {
            const int m = tid;
            const double inv = inv_rms_of(red[0][N], (double)f.K, a.norm_eps);
            const double h = red[0][m < N ? m : m + 1];
            if (a.h_mix) a.h_mix[tk * M + m] = (float)h;
            if (m == 0 && a.inv_rms) a.inv_rms[tk] = (float)inv;
            if (m < N) {
                const float hv = gate_pre(h, inv, gpar[0], gpar[3 + m], eps);
                if (a.h_pre) a.h_pre[tk * N + m] = hv;
                put_tagged(hpw + tk * N + m, tag, hv);
            } else if (m < 2 * N) {
                a.h_post[tk * N + m - N] = gate_post(h, inv, gpar[1], gpar[3 + m], eps, false);
            } else {
                Ls[q * NN + (m - 2 * N)] = res_logit(h, inv, gpar[2], gpar[3 + m]);
            }
        }
    }
    // the Sinkhorn planes and hRes, one token per 16-lane group: up to 4 tokens all on wave
    // 3, which hands its x to wave 0 for hIn first; more tokens on every wave
    const bool one_wave = ntok > 0 && ntok <= 4;
    if (one_wave && wave == 3) {
#pragma unroll
        for (int e = 0; e < BPW; ++e)
#pragma unroll
            for (int i = 0; i < N; ++i) xs[lane][e][i] = xr[e][i];
    }
    if (ntok > 0) {
        __syncthreads();   // Ls, xs
        const bool planes = a.sum_out || a.norm_out;
        if (!one_wave || wave == 3) {
            for (int q0 = one_wave ? 0 : 4 * wave; q0 < ntok; q0 += one_wave ? 4 : 16) {
                const int q = q0 + grp;
                const bool live = q < ntok;
                const float* L = Ls + (live ? q : 0) * NN;
                if (planes) sinkhorn4<true>(a, f.T, L, b + q * nwg, live, j);
                else sinkhorn4<false>(a, f.T, L, b + q * nwg, live, j);
            }
        }
    }

    // phase 3: hIn of the block, from the registers that hold its x (wave 0 also does wave
    // 3's tokens from LDS when wave 3 runs the Sinkhorn)
    auto hin_token = [&](int tt, const u32x4 (&xw)[BPW][N]) __attribute__((always_inline)) {
        uint64_t w[N];
#pragma unroll
        for (int i = 0; i < N; ++i) w[i] = get_tagged(hpw + tt * N + i);
        int it = 0;
        for (; it < kSpinLimit; ++it) {
            bool all = true;
#pragma unroll
            for (int i = 0; i < N; ++i) all = all && tag_is(w[i], want);
            if (all) break;
            __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int i = 0; i < N; ++i)
                if (!tag_is(w[i], want)) w[i] = get_tagged(hpw + tt * N + i);
        }
        const bool ok = it < kSpinLimit;
        if (!ok) __hip_atomic_store(a.sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        float wv[N];
#pragma unroll
        for (int i = 0; i < N; ++i) wv[i] = ok ? tagged_value(w[i]) : __builtin_nanf("");
        const rsrc_t hres = make_rsrc(a.h_in, f.T * f.D * 2);
#pragma unroll
        for (int bl = 0; bl < BPW; ++bl) {
            float hacc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) hacc[e] = 0.f;
#pragma unroll
            for (int i = 0; i < N; ++i) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hacc[2 * e] = fmaf(wv[i], x16_lo<H>(xw[bl][i][e]), hacc[2 * e]);
                    hacc[2 * e + 1] = fmaf(wv[i], x16_hi<H>(xw[bl][i][e]), hacc[2 * e + 1]);
                }
            }
            u32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = pack_x16<H>(hacc[2 * e], hacc[2 * e + 1]);
            __builtin_amdgcn_raw_buffer_store_b128(
                o, hres, (int)(((oct_ok >> bl) & 1u) ? (uint32_t)((tt * f.D + kBlock * (BPW * b + bl) + 8 * grp) * 2) : kOutOfRange), 0, 0);
        }
    };
    if (!(one_wave && wave == 3) && t < T32) hin_token(t, xr);
    if (one_wave && wave == 0 && 48 + j < T32) {
        u32x4 xv[BPW][N];
#pragma unroll
        for (int e = 0; e < BPW; ++e)
#pragma unroll
            for (int i = 0; i < N; ++i) xv[e][i] = xs[lane][e][i];
        hin_token(48 + j, xv);
    }
    // this call's count into flags b, b + nwg, ..: the next call's epoch
    if (wave == 0)
        for (int v = b + nwg * lane; v < kDecodeMaxBlocks; v += nwg * 64)
            __hip_atomic_store(flags + v, epoch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Records events[i] (a caller-created hipEvent_t) on the stream when events is given and
// its entry is not NULL.
hipError_t mark(void* const* events, int i, hipStream_t st)
{
    return events && events[i] ? hipEventRecord((hipEvent_t)events[i], st) : hipSuccess;
}

template <int N, int A, int NKS, bool H>
hipError_t launch_group(const Plan& p, const KArgs& k, hipStream_t st, void* const* events, const float* phiT,
                        int stream_W)
{
    // Workgroups map to tasks so that each XCD's L2 holds the weights of a few slices
    // only (task_of_block). phiT: the VALU projection's weights, or NULL for the matrix cores.
    // stream_W > 0: the streaming projection with that many workgroups per slice.
    if (stream_W > 0) {
        if constexpr (stream_fits(N, A, NKS)) {
            const int64_t NI = (p.tiles + 2 * (int64_t)stream_W - 1) / (2 * (int64_t)stream_W);
            hipLaunchKernelGGL((proj_stream_kernel<N, A, NKS, H>), dim3((unsigned)(p.S * stream_W)), dim3(kSThreads),
                               0, st, k, stream_W, (int)NI);
        } else {
            return hipErrorInvalidValue;
        }
    } else if constexpr (Cfg<N, A>::M <= 32) {
        if (phiT)
            hipLaunchKernelGGL((proj_valu_kernel<N, A, NKS, H>), dim3((unsigned)p.proj_blocks), dim3(kThreads), 0, st, k,
                               phiT);
        else
            hipLaunchKernelGGL((proj_kernel<N, A, NKS, H>), dim3((unsigned)p.proj_blocks), dim3(kThreads), 0, st, k);
    } else {
        if (phiT) return hipErrorInvalidValue;
        hipLaunchKernelGGL((proj_kernel<N, A, NKS, H>), dim3((unsigned)p.proj_blocks), dim3(kThreads), 0, st, k);
    }
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = mark(events, kStageProj + 1, st);
    if (e != hipSuccess) return e;
    // without pre_mix the epilogue also writes hIn (no hIn launch)
    if (k.a.pre_mix) {
        if (N == 4 && p.OB == 16)
            hipLaunchKernelGGL((epilogue_kernel<N, A, 16>), dim3((unsigned)p.out_blocks), dim3(kThreads), 0, st, k);
        else
            hipLaunchKernelGGL((epilogue_kernel<N, A, 8>), dim3((unsigned)p.out_blocks), dim3(kThreads), 0, st, k);
    } else {
        if (N == 4 && p.OB == 16)
            hipLaunchKernelGGL((epilogue_kernel<N, A, 16, true, H>), dim3((unsigned)p.out_blocks), dim3(kThreads), 0,
                               st, k);
        else
            hipLaunchKernelGGL((epilogue_kernel<N, A, 8, true, H>), dim3((unsigned)p.out_blocks), dim3(kThreads), 0, st,
                               k);
    }
    e = hipGetLastError();
    if (e == hipSuccess) e = mark(events, kStageEpi + 1, st);
    if (e == hipSuccess) e = mark(events, kStageHin + 1, st);
    return e;
}

// Whether a kernel's code keeps everything in registers. The single-read kernel's x loads
// are invisible to the compiler (inline assembly, waited for by hand): were it to spill
// registers to scratch memory, it could spill or reuse a register such a load has yet to
// write. The kernel is refused then (the classic path serves), never run.
bool no_scratch(const void* fn)
{
    hipFuncAttributes at;
    return hipFuncGetAttributes(&at, fn) == hipSuccess && at.localSizeBytes == 0;
}

// What the path choice needs to know of a device, found once per device (these queries
// cost about a microsecond per call otherwise): its compute units, whether the single-read
// kernel's code keeps everything in registers, and how many workgroups of the single-read
// and one-launch kernels a compute unit holds.
struct DeviceFacts {
    int cus = 0;
    bool fused_ok[2] = {false, false};       // [fp16 x]: no scratch, at least one workgroup per compute unit
    int decode_per_cu[2][2] = {{0, 0}, {0, 0}};   // [fp16 x][blocks a workgroup - 1]: 0, cannot run here
    bool stream_ok[2][4] = {{false, false, false, false}, {false, false, false, false}};   // [fp16 x][stream_variant]
};

// The variants the streaming projection is compiled for (index into stream_ok), -1 others.
int stream_variant(int n, int n_alpha, int nks)
{
    if (n == 4 && n_alpha == 3 && nks == 16) return 0;
    if (n == 4 && n_alpha == 2 && nks == 16) return 1;
    if (n == 8 && n_alpha == 2 && nks == 16) return 2;
    if (n == 6 && n_alpha == 2 && nks == 12) return 3;
    return -1;
}

// The streaming projection's x loads are invisible to the compiler, like the single-read
// kernel's: it runs only from code without scratch memory, one workgroup per compute unit.
template <int N, int A, int NKS, bool H>
bool stream_kernel_ok()
{
    int per_cu = 0;
    return no_scratch(reinterpret_cast<const void*>(proj_stream_kernel<N, A, NKS, H>)) &&
           hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, proj_stream_kernel<N, A, NKS, H>, kSThreads, 0) ==
               hipSuccess &&
           per_cu >= 1;
}
constexpr int kMaxDevices = 64;

// Workgroups of the one-launch kernel a compute unit holds at once. (Its loads are all the
// compiler's own, so unlike the single-read kernel it needs no scratch-free guarantee.)
template <bool H, int BPW>
int decode_per_cu()
{
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<4, 3, false, H, BPW>, kThreads, 0) == hipSuccess)
        return per_cu;
    return 0;
}

template <bool H>
void fill_facts(DeviceFacts& f)
{
    int per_cu = 0;
    f.fused_ok[H] = no_scratch(reinterpret_cast<const void*>(fused_kernel<4, 3, false, H>)) &&
                    no_scratch(reinterpret_cast<const void*>(fused_kernel<4, 3, true, H>)) &&
                    hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fused_kernel<4, 3, false, H>, kFThreads, 0) == hipSuccess &&
                    per_cu >= 1;
    f.decode_per_cu[H][0] = decode_per_cu<H, 1>();
    f.decode_per_cu[H][1] = decode_per_cu<H, 2>();
    f.stream_ok[H][0] = stream_kernel_ok<4, 3, 16, H>();
    f.stream_ok[H][1] = stream_kernel_ok<4, 2, 16, H>();
    f.stream_ok[H][2] = stream_kernel_ok<8, 2, 16, H>();
    f.stream_ok[H][3] = stream_kernel_ok<6, 2, 12, H>();
}

const DeviceFacts* device_facts()
{
    static DeviceFacts facts[kMaxDevices];
    static std::once_flag once[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(once[dev], [dev]() {
        DeviceFacts f;
        if (hipDeviceGetAttribute(&f.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) f.cus = 0;
        fill_facts<false>(f);
        fill_facts<true>(f);
        facts[dev] = f;
    });
    return &facts[dev];
}

// Groups of the single-read kernel on the current device (one per XCD, at most one per
// tile), 0 when it cannot run here: the kernel needs kXcds XCDs of kFMembers compute units,
// one workgroup on each, and code without scratch memory.
int fused_groups(const Plan& p)
{
    const DeviceFacts* d = device_facts();
    if (!d || d->cus != kXcds * kFMembers || !d->fused_ok[p.g.x_f16 ? 1 : 0]) return 0;
    int64_t G = kXcds;
    if (G > p.tiles16) G = p.tiles16;
    return (int)G;
}

bool fused_wanted(const Plan& p, bool has_pre_mix)
{
    if (!p.fused_geom || has_pre_mix || p.T <= 0) return false;
    const char* env = std::getenv("MHC_FORWARD_PATH");
    if (env && std::strcmp(env, "classic") == 0) return false;
    const bool forced = env && std::strcmp(env, "fused") == 0;
    return forced || p.T >= kFMinTokens;
}

// Blocks a workgroup of the one-launch kernel takes on the current device. With packed
// weights passed in, two where that still leaves a workgroup per token (half the records
// for every token's owner to read); with weights split inside the kernel, one, so that the
// split (the larger cost there) stays spread over every d-block's workgroup. 0 when the
// device cannot hold all its workgroups at once.
int decode_blocks_per_wg(const Plan& p, bool packed)
{
    const DeviceFacts* d = device_facts();
    if (!d) return 0;
    const int h = p.g.x_f16 ? 1 : 0;
    const int64_t nwg2 = (p.g.nblk + 1) / 2;
    if (packed && nwg2 >= p.T && (int64_t)d->decode_per_cu[h][1] * d->cus >= nwg2) return 2;
    if ((int64_t)d->decode_per_cu[h][0] * d->cus >= p.g.nblk) return 1;
    return 0;
}

// Whether the one-launch kernel serves this call on the current device: the geometry
// admits it, no pre_mix, MHC_FORWARD_PATH does not ask for another path, and the device
// holds all its workgroups at once.
bool decode_wanted(const Plan& p, bool has_pre_mix)
{
    if (!p.decode_geom || has_pre_mix || p.T <= 0) return false;
    const char* env = std::getenv("MHC_FORWARD_PATH");
    if (env && (std::strcmp(env, "classic") == 0 || std::strcmp(env, "fused") == 0)) return false;
    return decode_blocks_per_wg(p, false) > 0;
}

hipError_t launch_decode(const Plan& p, const ForwardArgs& a, hipStream_t st, void* const* events)
{
    DArgs f;
    f.a = a;
    f.T = p.T;
    f.K = p.g.K;
    f.D = p.g.D;
    f.nblk = p.g.nblk;
    const int bpw = decode_blocks_per_wg(p, a.packed != nullptr);
    if (bpw == 0) return hipErrorInvalidValue;
    f.nwg = (p.g.nblk + bpw - 1) / bpw;
    hipError_t e = mark(events, kStagePack + 1, st);
    if (e != hipSuccess) return e;
    // test hook, as for the single-read kernel: every wait gives up at its limit
    const char* never = std::getenv("MHC_TEST_EXCHANGE_NEVER_READY");
    const bool nr = never && std::strcmp(never, "1") == 0;
    const dim3 grid((unsigned)f.nwg), block(kThreads);
#define MHC_DECODE(NR, HV, BV) hipLaunchKernelGGL((decode_kernel<4, 3, NR, HV, BV>), grid, block, 0, st, f)
    if (bpw == 2) {
        if (p.g.x_f16) { if (nr) MHC_DECODE(true, true, 2); else MHC_DECODE(false, true, 2); }
        else { if (nr) MHC_DECODE(true, false, 2); else MHC_DECODE(false, false, 2); }
    } else {
        if (p.g.x_f16) { if (nr) MHC_DECODE(true, true, 1); else MHC_DECODE(false, true, 1); }
        else { if (nr) MHC_DECODE(true, false, 1); else MHC_DECODE(false, false, 1); }
    }
#undef MHC_DECODE
    e = hipGetLastError();
    if (e == hipSuccess) e = mark(events, kStageProj + 1, st);
    if (e == hipSuccess) e = mark(events, kStageEpi + 1, st);
    if (e == hipSuccess) e = mark(events, kStageHin + 1, st);
    return e;
}

hipError_t launch_fused(const Plan& p, const ForwardArgs& a, int G, hipStream_t st, void* const* events)
{
    FArgs f;
    f.a = a;
    f.T = p.T;
    f.K = p.g.K;
    f.tiles16 = p.tiles16;
    f.D = p.g.D;
    f.nblk = p.g.nblk;
    f.G = G;
    // test hook: every exchange wait gives up after a few polls (all kernels still exit
    // normally); the time-out then shows in the workspace's flag
    const char* never = std::getenv("MHC_TEST_EXCHANGE_NEVER_READY");
    const bool test_never_ready = never && std::strcmp(never, "1") == 0;
    // one workgroup per compute unit: the hardware deals workgroups to the XCDs in turn,
    // kFMembers to each; a workgroup whose XCD's group is full (or not needed) leaves
    const dim3 grid((unsigned)(kXcds * p.FP)), block(kFThreads);
    if (p.g.x_f16) {
        if (test_never_ready) hipLaunchKernelGGL((fused_kernel<4, 3, true, true>), grid, block, 0, st, f);
        else hipLaunchKernelGGL((fused_kernel<4, 3, false, true>), grid, block, 0, st, f);
    } else {
        if (test_never_ready) hipLaunchKernelGGL((fused_kernel<4, 3, true, false>), grid, block, 0, st, f);
        else hipLaunchKernelGGL((fused_kernel<4, 3, false, false>), grid, block, 0, st, f);
    }
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = mark(events, kStageProj + 1, st);
    if (e != hipSuccess) return e;
    KArgs k;
    k.a = a;
    k.T = p.T;
    k.K = p.g.K;
    k.tiles = p.tiles;
    k.D = p.g.D;
    k.S = p.FP;
    k.GS = p.FGS;
    k.NG = p.FNG;
    if (p.OB == 16)
        hipLaunchKernelGGL((epilogue_kernel<4, 3, 16>), dim3((unsigned)p.out_blocks), dim3(kThreads), 0, st, k);
    else
        hipLaunchKernelGGL((epilogue_kernel<4, 3, 8>), dim3((unsigned)p.out_blocks), dim3(kThreads), 0, st, k);
    e = hipGetLastError();
    if (e == hipSuccess) e = mark(events, kStageEpi + 1, st);
    if (e == hipSuccess) e = mark(events, kStageHin + 1, st);
    return e;
}

}  // namespace

// Whether the classic path projects on the VALU (fp32 FMA) rather than the matrix
// cores: MHC_PROJECTION = "valu" or "mfma" decides; otherwise the measured choice, the
// matrix cores (on MI355X the VALU projection kernel took 1.9 to 3.8 times as long on every
// workload of the benchmark, fp32 FMA at about a third of the VALU's fp32 peak against a
// matrix-core projection bound by memory). The VALU path needs phi itself (it packs its own
// fp32 weights) and M <= 32.
static bool projection_on_valu(const Plan& p, const ForwardArgs& a)
{
    if (!a.phi || p.g.M > 32) return false;
    const char* env = std::getenv("MHC_PROJECTION");
    if (env && std::strcmp(env, "valu") == 0) return true;
    if (env && std::strcmp(env, "mfma") == 0) return false;
    return false;
}

// Workgroups per slice of the streaming projection on the current device (one workgroup
// per compute unit at most, no more than the tile pairs), 0 when it does not serve: with
// pre_mix (whose hIn the projection kernel writes from registers, which needs all n streams
// of a position in a lane), D not a multiple of 32, a variant it is not compiled for, code
// that cannot run here, or MHC_FORWARD_PATH = "classic" / MHC_PROJECTION = "valu" asking
// for the classic path.
int stream_workgroups_per_slice(const Plan& p, bool has_pre_mix)
{
    if (has_pre_mix || p.g.D % kBlock != 0) return 0;
    const char* env = std::getenv("MHC_FORWARD_PATH");
    if (env && std::strcmp(env, "classic") == 0) return 0;
    const char* pe = std::getenv("MHC_PROJECTION");
    if (pe && std::strcmp(pe, "valu") == 0) return 0;
    const int v = stream_variant(p.g.n, p.g.n_alpha, p.NKS);
    const DeviceFacts* d = device_facts();
    if (v < 0 || !d || d->cus <= 0 || p.S <= 0 || p.tiles <= 0 || !d->stream_ok[p.g.x_f16 ? 1 : 0][v]) return 0;
    int64_t W = d->cus / p.S;
    if (W > (p.tiles + 1) / 2) W = (p.tiles + 1) / 2;
    return W < 1 ? 1 : (int)W;
}

int forward_path(const Plan& p, bool has_pre_mix)
{
    if (decode_wanted(p, has_pre_mix)) return 2;
    if (fused_wanted(p, has_pre_mix) && fused_groups(p) > 0) return 1;
    return stream_workgroups_per_slice(p, has_pre_mix) > 0 ? 3 : 0;
}

int launch_prepack(const Geometry& g, const float* phi, const float* gamma, void* packed,
                   void* stream)
{
    clear_pending_error();
    // one thread per (K-step, K-group, phi row); the padding columns fit the row threads
    if (g.NC - 3 * g.M > g.M) return (int)hipErrorInvalidValue;
    const int64_t total = (int64_t)(g.nks + kPadSteps) * 4 * g.M;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    if (g.x_f16)
        hipLaunchKernelGGL(prepack_kernel<true>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, phi, gamma,
                           static_cast<u32x4*>(packed), g.n, g.D, g.M, g.NC, g.nks, total);
    else
        hipLaunchKernelGGL(prepack_kernel<false>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, phi, gamma,
                           static_cast<u32x4*>(packed), g.n, g.D, g.M, g.NC, g.nks, total);
    return (int)hipGetLastError();
}

int launch_inv_rms(int64_t T, int n, int D, double norm_eps, const uint16_t* x, float* inv_rms,
                   int x_f16, void* stream)
{
    clear_pending_error();
    if (T <= 0) return 0;
    constexpr int per_block = kThreads / 64;
    const dim3 grid((unsigned)((T + per_block - 1) / per_block));
    hipStream_t st = (hipStream_t)stream;
#define MHC_INV_RMS(NV, HV) hipLaunchKernelGGL((inv_rms_kernel<NV, HV>), grid, dim3(kThreads), 0, st, x, inv_rms, T, D, norm_eps)
    if (n == 4 && !x_f16) MHC_INV_RMS(4, false);
    else if (n == 6 && !x_f16) MHC_INV_RMS(6, false);
    else if (n == 8 && !x_f16) MHC_INV_RMS(8, false);
    else if (n == 4) MHC_INV_RMS(4, true);
    else if (n == 6) MHC_INV_RMS(6, true);
    else if (n == 8) MHC_INV_RMS(8, true);
#undef MHC_INV_RMS
    else return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

int launch_pre_sinkhorn(int64_t T, int n, int D, int n_alpha, int x_f16, const ForwardArgs& a,
                        const float* h_mix, const float* inv_rms, void* stream)
{
    clear_pending_error();
    if (T <= 0) return 0;
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipErrorInvalidValue;
    const bool h = x_f16 != 0;
#define MHC_STAGE(NV, AV) (h ? launch_stage<NV, AV, true>(T, D, a, h_mix, inv_rms, st) \
                             : launch_stage<NV, AV, false>(T, D, a, h_mix, inv_rms, st))
    if (n == 4 && n_alpha == 3) e = MHC_STAGE(4, 3);
    else if (n == 4 && n_alpha == 2) e = MHC_STAGE(4, 2);
    else if (n == 8 && n_alpha == 3) e = MHC_STAGE(8, 3);
    else if (n == 8 && n_alpha == 2) e = MHC_STAGE(8, 2);
    else if (n == 6 && n_alpha == 3) e = MHC_STAGE(6, 3);
    else if (n == 6 && n_alpha == 2) e = MHC_STAGE(6, 2);
#undef MHC_STAGE
    return (int)e;
}

int record_event(void* event, void* stream)
{
    return (int)hipEventRecord((hipEvent_t)event, (hipStream_t)stream);
}

int read_and_clear_wait_flag(uint32_t* sync, int32_t* timed_out, void* stream)
{
    hipStream_t st = (hipStream_t)stream;
    uint32_t v = 0;
    hipError_t e = hipMemcpyAsync(&v, sync + 1, sizeof v, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e == hipSuccess && v != 0) {
        e = hipMemsetAsync(sync + 1, 0, sizeof v, st);
        if (e == hipSuccess) e = hipStreamSynchronize(st);
    }
    if (e != hipSuccess) return (int)e;
    *timed_out = v != 0 ? 1 : 0;
    return 0;
}

int launch_forward(const Plan& p, const ForwardArgs& a_in, void* stream, void* const* events)
{
    clear_pending_error();
    if (p.T <= 0) return 0;
    hipStream_t st = (hipStream_t)stream;
    ForwardArgs a = a_in;
    if (mark(events, kStagePack, st) != hipSuccess) return (int)hipErrorUnknown;
    if (decode_wanted(p, a.pre_mix != nullptr)) return (int)launch_decode(p, a, st, events);   // packs in the kernel
    if (fused_wanted(p, a.pre_mix != nullptr)) {
        // unpacked weights are packed inside the kernel
        const int G = fused_groups(p);
        if (G > 0) {
            hipError_t e = mark(events, kStagePack + 1, st);
            if (e != hipSuccess) return (int)e;
            return (int)launch_fused(p, a, G, st, events);
        }
    }
    // the streaming projection (weights packed inside the kernel), else the projection on
    // the VALU (fp32 weights packed here, from phi) or the matrix cores
    const int stream_W = stream_workgroups_per_slice(p, a.pre_mix != nullptr);
    const bool valu = stream_W == 0 && projection_on_valu(p, a);
    const float* phiT = nullptr;
    if (valu) {
        const int64_t items = p.g.K * (int64_t)p.g.M;
        hipLaunchKernelGGL(pack_valu_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, st, a.phi, a.gamma,
                           static_cast<float*>(a.packed_ws), p.g.K, p.g.M);
        if (hipGetLastError() != hipSuccess) return (int)hipErrorUnknown;
        phiT = static_cast<const float*>(a.packed_ws);
    } else if (!a.packed && stream_W == 0) {
        if (launch_prepack(p.g, a.phi, a.gamma, a.packed_ws, stream) != 0) return (int)hipErrorUnknown;
        a.packed = a.packed_ws;
    }
    {
        const hipError_t e = mark(events, kStagePack + 1, st);
        if (e != hipSuccess) return (int)e;
    }
    KArgs k;
    k.a = a;
    k.T = p.T;
    k.K = p.g.K;
    k.tiles = p.tiles;
    k.D = p.g.D;
    k.S = p.S;
    k.GS = p.GS;
    k.NG = p.NG;
    const int n = p.g.n, na = p.g.n_alpha, nks = p.NKS;
    const Variant v = variant_of(n, na);
    if (n == 4 && na == 3 && (v.nt != Cfg<4, 3>::NT || v.sk != Cfg<4, 3>::SK)) return (int)hipErrorInvalidValue;
    if (n == 4 && na == 2 && (v.nt != Cfg<4, 2>::NT || v.sk != Cfg<4, 2>::SK)) return (int)hipErrorInvalidValue;
    if (n == 8 && na == 3 && (v.nt != Cfg<8, 3>::NT || v.sk != Cfg<8, 3>::SK)) return (int)hipErrorInvalidValue;
    if (n == 8 && na == 2 && (v.nt != Cfg<8, 2>::NT || v.sk != Cfg<8, 2>::SK)) return (int)hipErrorInvalidValue;
    if (n == 6 && na == 3 && (v.nt != Cfg<6, 3>::NT || v.sk != Cfg<6, 3>::SK)) return (int)hipErrorInvalidValue;
    if (n == 6 && na == 2 && (v.nt != Cfg<6, 2>::NT || v.sk != Cfg<6, 2>::SK)) return (int)hipErrorInvalidValue;
    hipError_t e = hipErrorInvalidValue;
    const bool h = p.g.x_f16 != 0;
#define MHC_GROUP(NV, AV, KV) (h ? launch_group<NV, AV, KV, true>(p, k, st, events, phiT, stream_W) \
                                 : launch_group<NV, AV, KV, false>(p, k, st, events, phiT, stream_W))
    if (n == 4 && na == 3 && nks == 16) e = MHC_GROUP(4, 3, 16);
    else if (n == 4 && na == 2 && nks == 16) e = MHC_GROUP(4, 2, 16);
    else if (n == 8 && na == 3 && nks == 8) e = MHC_GROUP(8, 3, 8);
    else if (n == 8 && na == 2 && nks == 16) e = MHC_GROUP(8, 2, 16);
    else if (n == 8 && na == 2 && nks == 32) e = MHC_GROUP(8, 2, 32);
    else if (n == 6 && na == 3 && nks == 12) e = MHC_GROUP(6, 3, 12);
    else if (n == 6 && na == 2 && nks == 12) e = MHC_GROUP(6, 2, 12);
#undef MHC_GROUP
    return (int)e;
}

}  // namespace mhc
