// mhc_bwd_plan.h -- geometry, packed-weight order and workspace layout of the MhcPre
// backward (MhcPreBackward guide, 0539edu.com/news/4871844, section 3).
//
// Host-side and plain C++ (no HIP headers), like mhc_plan.h: validation, planning and
// the index checks of the tests build without a GPU; the offset helpers below are the
// ones the kernels use.
//
// Work decomposition
//   token pass   one wave per token: the hPre gradient (gradHIn . x_i over d, fp64), the
//                gate and residual backward, the gradient with respect to hMix as three
//                bf16 terms (gMix [T][KS][3][32], zero past M: the matrix-core operand
//                layout), c3 = dL/dinvRms * invRms^3 / (n D), and the token's terms of the
//                alpha and bias gradients (fp64, [3 + M][T]).
//   main pass    one workgroup per (token group, d-block of 32 positions, stream group of
//                SGN streams): for each tile of 64 tokens, xrsGrad = gMix . phi on the
//                matrix cores (phi^T as the A operand, packed per d-block; gMix as B),
//                gradX, and the tile's share of gradGamma (x * xrsGrad) and gradPhi
//                (gMix^T . x on the matrix cores, x transposed through LDS); the group's
//                sums go to partial buffers.
//   reduction    gradPhi = gamma (.) sum over groups, gradGamma = sum over groups, gradAlpha
//                and gradBias = sums over tokens; every sum in a fixed order in fp64.
//   Sinkhorn     (MhcPreSinkhorn backward only, before the token pass) the residual
//                logits' gradient through the saved planes, 64 / (n*n) tokens per wave,
//                into glog [T][n*n] (fp64).
#pragma once

#include <cstddef>
#include <cstdint>

#ifdef __HIP__
#define MHC_BWD_HOST_DEVICE __host__ __device__
#else
#define MHC_BWD_HOST_DEVICE
#endif

namespace mhc {
namespace bwd {

constexpr int kThreads = 256;        // 4 waves
constexpr int kTile = 64;            // tokens per tile (4 waves x 16)
constexpr int kDBlock = 32;          // positions per d-block
constexpr int kMaxD = 16384;
constexpr int kTargetBlocks = 2048;  // main-pass workgroups aimed for (token groups x blocks)

struct Geometry {
    int n = 0;
    int D = 0;
    int M = 0;           // n*n + 2n phi rows
    int KS = 0;          // 32-wide K-steps covering M
    int MP = 0;          // 32 * KS: padded rows
    int64_t K = 0;       // n * D
    int nblk = 0;        // d-blocks: ceil(D / 32)
    int SGN = 0;         // streams per main-pass workgroup
    int NSG = 0;         // stream groups: n / SGN
    int x_f16 = 0;       // x, gradHIn, gradXPost and gradX in fp16 (else bf16)
    size_t pack_bytes = 0;
};

// 16-byte units of the packed A operand for one (d-block, stream): 2 halves x KS
// K-steps x 3 terms x 64 lanes.
MHC_BWD_HOST_DEVICE inline int64_t pack_units_per_stream(int KS) { return (int64_t)2 * KS * 3 * 64; }
// First unit of (d-block b, stream i).
MHC_BWD_HOST_DEVICE inline int64_t pack_at(int b, int i, int n, int KS)
{
    return ((int64_t)b * n + i) * pack_units_per_stream(KS);
}
// Column (within stream, 0 .. 31 from the d-block start) that matrix row `row` (0..15)
// of half h stands for: a lane (group g) then holds the 8 consecutive positions
// 8g .. 8g+7 across the two halves (rows 4g .. 4g+3 of each).
MHC_BWD_HOST_DEVICE inline int pack_col(int h, int row) { return 8 * (row / 4) + 4 * h + (row % 4); }

inline bool make_geometry(int n, int D, Geometry* g, bool x_f16 = false)
{
    if (n != 4 && n != 6 && n != 8) return false;   // the guide's section 5: N = 4, 6, 8
    if (D < 8 || D % 8 != 0 || D > kMaxD) return false;
    Geometry r;
    r.n = n;
    r.D = D;
    r.M = n * n + 2 * n;
    r.KS = (r.M + 31) / 32;
    r.MP = 32 * r.KS;
    r.K = (int64_t)n * D;
    r.nblk = (D + kDBlock - 1) / kDBlock;
    r.SGN = n == 4 ? 4 : 2;
    r.NSG = n / r.SGN;
    r.pack_bytes = (size_t)r.nblk * n * pack_units_per_stream(r.KS) * 16;
    r.x_f16 = x_f16 ? 1 : 0;
    *g = r;
    return true;
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Main-pass workgroup -> task (token group, stream group, d-block), tasks numbered with
// the d-block fastest. Workgroups b and b + 8 run on the same XCD (the hardware deals
// workgroups to the 8 XCDs in turn), and they take tasks 2u and 2u + 1: adjacent
// d-blocks, whose 64-byte pieces of a token row share 128-byte lines, so each line of
// x, gradHIn and gradX goes through one XCD's L2 only. Workgroups in flight still cover
// nearby columns of the same rows. Returns false for the padding workgroups.
MHC_BWD_HOST_DEVICE inline int64_t main_blocks_for(int64_t tasks) { return (tasks + 15) / 16 * 16; }
MHC_BWD_HOST_DEVICE inline bool main_task(int64_t blk, int nblk, int NSG, int64_t tasks, int64_t* grp,
                                          int* b, int* sg)
{
    const int64_t q = blk % 8, r = blk / 8;
    const int64_t t = ((r / 2) * 8 + q) * 2 + (r % 2);
    if (t >= tasks) return false;
    *b = (int)(t % nblk);
    const int64_t gs = t / nblk;
    *sg = (int)(gs % NSG);
    *grp = gs / NSG;
    return true;
}

struct Plan {
    Geometry g;
    int64_t T = 0;
    int64_t tiles = 0;        // ceil(T / 64)
    int64_t G = 0;            // token groups
    int64_t tpg = 0;          // tiles per group (the last group may have fewer)
    int64_t main_tasks = 0;   // G * nblk * NSG
    int64_t main_blocks = 0;  // main_tasks rounded up to 16 (see main_task)
    int64_t token_blocks = 0; // ceil(T / 4): one wave per token
    size_t off_pack = 0, off_gmix = 0, off_c3 = 0, off_terms = 0, off_pphi = 0, off_pgam = 0, off_glog = 0;
    size_t ws_bytes = 0;
};

inline Plan make_plan(const Geometry& g, int64_t T)
{
    Plan p;
    p.g = g;
    p.T = T;
    p.tiles = (T + kTile - 1) / kTile;
    const int64_t per_group = (int64_t)g.nblk * g.NSG;
    int64_t G = (kTargetBlocks + per_group - 1) / per_group;
    if (G > p.tiles) G = p.tiles;
    if (G < 1) G = 1;
    p.tpg = (p.tiles + G - 1) / G;
    p.G = p.tiles > 0 ? (p.tiles + p.tpg - 1) / p.tpg : 1;   // no empty group
    p.main_tasks = p.G * per_group;
    p.main_blocks = main_blocks_for(p.main_tasks);
    p.token_blocks = (T + 3) / 4;
    size_t off = 0;
    p.off_pack = off;
    off = align_up(off + g.pack_bytes, 256);
    p.off_gmix = off;
    off = align_up(off + (size_t)T * g.KS * 3 * 32 * 2, 256);
    p.off_c3 = off;
    off = align_up(off + (size_t)T * 4, 256);
    p.off_terms = off;
    off = align_up(off + (size_t)T * (3 + g.M) * 8, 256);
    p.off_pphi = off;
    off = align_up(off + (size_t)p.G * g.M * g.K * 4, 256);
    p.off_pgam = off;
    off = align_up(off + (size_t)p.G * g.K * 4, 256);
    p.off_glog = off;
    off = align_up(off + (size_t)T * g.n * g.n * 8, 256);
    p.ws_bytes = off;
    return p;
}

// Device pointers of one backward call.
struct Args {
    const uint16_t* x;
    const float* phi;
    const float* alpha;
    const uint16_t* grad_h_in;
    const float* grad_h_post;
    const float* grad_h_res;
    const float* inv_rms;
    const float* h_mix;
    const float* h_pre;
    const float* h_post;
    const float* gamma;
    const uint16_t* grad_x_post;
    uint16_t* grad_x;
    float* grad_phi;
    float* grad_alpha;
    float* grad_bias;
    float* grad_gamma;
    double hc_eps;
    int num_iters;             // 0: MhcPre; >= 1: MhcPreSinkhorn (the planes below)
    const float* sum_out;      // [2 it][T][n]
    const float* norm_out;     // [2 it][T][n][n]
    // workspace
    void* pack;
    uint16_t* gmix;    // [T][KS][3][32] bf16 terms of the hMix gradient
    float* c3;
    double* terms;     // [3 + M][T]
    float* pphi;
    float* pgam;
    double* glog;      // [T][n*n] residual logits' gradient (Sinkhorn backward)
};

// Implemented in mhc_bwd.hip. Returns 0 or the HIP error code.
int launch_backward(const Plan& p, const Args& a, void* stream);

}  // namespace bwd
}  // namespace mhc
