// mhc_plan.h -- launch geometry, packed-weight order and workspace layout of the mHC pre
// forward.
//
// Host-side and plain C++ (no HIP headers): the validation / planning code that uses it,
// and the index checks of the tests, build and run on a machine without a GPU. The
// offset helpers below are the ones the kernels use.
//
// Work decomposition
//   The projection runs as tasks of one tile of 64 tokens x one d-slice: the same range
//   of hidden positions d in every one of the n streams, so that with pre_mix (hIn weights
//   given) the task's x, loaded once, also yields the slice's part of hIn = sum_i w_i x_i.
//   Each task writes a partial record per token; a per-token epilogue sums the S records
//   of a token and computes every other output; without pre_mix a last pass computes hIn
//   from the epilogue's hPre.
//   Single-read variant (n = 4, alpha[3], no pre_mix, 32 to 224 d-blocks): the
//   workgroups form G groups of P members; member s of a group keeps the packed weights
//   of its run of d-blocks in LDS for the whole call, and the group walks its tiles of 16
//   tokens in rounds. Each round a member projects one tile (one d-block per compute
//   wave), writes its partial record and, tagged for this call, the record's pre-branch
//   sums and square; the tile's designated member (round mod P) sums those, publishes
//   hPre, and every member computes its share of hIn from the x it still holds in
//   registers kFLag rounds later. x is read from HBM once.
//
// Reduction order ("K-steps")
//   Positions are grouped in d-blocks of 32 (four octets of 8 bf16). K-step k = (block
//   b = k / n, stream i = k % n) covers xFlat elements i*D + 32b + [0, 32); matrix-core
//   lane group g (= lane / 16) takes octet g of it. A slice is a run of NKS consecutive
//   K-steps (NKS a multiple of n: whole d-blocks). Any order of the reduction gives the
//   same dot product; the packed weights use this same order.
//   Packed weights: for each K-step, 4 octet rows (g) x NC columns of 8 bf16 (16 bytes),
//   row-major. Column c < 3M is term (c / M) of phi row (c % M) with gamma folded in:
//   term 0 = hi, 1 = mid, 2 = lo, hi + mid + lo = phi * gamma to ~2^-26 relative. Columns
//   >= 3M, octets at or beyond D, and kPadSteps trailing K-steps hold zeros (the last
//   slice may run past the data).
#pragma once

#include <cstddef>
#include <cstdint>

// Functions the kernels call too carry the device qualifier when a HIP compiler reads
// this header; a plain C++ compiler sees ordinary inline functions.
#ifdef __HIP__
#define MHC_HOST_DEVICE __host__ __device__
#else
#define MHC_HOST_DEVICE
#endif

namespace mhc {

constexpr int kThreads = 256;          // workgroup: 4 waves of 64
constexpr int kWaves = 4;
constexpr int kTileTokens = 64;        // tokens per task: 4 waves x 16 matrix rows
constexpr int kBlock = 32;             // positions per d-block
constexpr int kPadSteps = 32;          // zero K-steps after the data (>= the largest NKS)
constexpr int kMaxD = 16384;
constexpr int kMaxN = 8;
constexpr int64_t kBigTasks = 1024;    // prefer the large slice when it still gives this many tasks
constexpr int kMaxSlices = 256;        // slices per tile
// Tokens per epilogue workgroup: 16 for n = 4 with many tokens (16 Sinkhorn matrices of 16
// lanes fill the 256 threads), else 8 (more workgroups share the work of a small T).
constexpr int64_t kWideEpilogueTokens = 8192;
MHC_HOST_DEVICE constexpr int out_tokens(int n, int64_t T) { return n == 4 && T >= kWideEpilogueTokens ? 16 : 8; }

// Single-read kernel (see above).
constexpr int kFTok = 16;              // tokens per tile
constexpr int kFMembers = 32;          // members per group
constexpr int kFMaxBlocks = 7;         // d-blocks per member: one per compute wave
constexpr int kFWaves = 8;             // 7 compute waves + 1 control wave
constexpr int kFThreads = 64 * kFWaves;
constexpr int kFRing = 8;              // x register slots, one per round
constexpr int kFAhead = 2;             // rounds between a tile's x loads and its projection
constexpr int kFLag = kFRing - kFAhead;   // rounds between a tile's projection and its hIn
constexpr int kFLoads = 4;             // x loads of a compute wave per round (one per stream, n = 4)
constexpr int64_t kFMinTokens = 8192;  // below this the classic path is used (ramp and drain dominate)

// Streaming projection (proj_stream_kernel): persistent workgroups of two halves of
// kThreads, each half on its own 64-token tile of the workgroup's slice.
constexpr int kSThreads = 2 * kThreads;
constexpr int kLdsBytes = 160 * 1024;  // LDS of a compute unit (gfx950)
// Record stores a thread issues per task (64 tokens x CH 16-byte chunks over kThreads).
MHC_HOST_DEVICE constexpr int stream_rec_stores(int CH) { return (kTileTokens * CH + kThreads - 1) / kThreads; }
// Whether a variant's slice fits the streaming projection: its packed weights (NKS K-steps
// of 4 x NC 16-byte units) and both halves' column totals in LDS, and two tasks' x (NKS
// 16-byte registers each) per lane.
MHC_HOST_DEVICE constexpr bool stream_fits(int n, int n_alpha, int nks)
{
    return nks <= 16 && nks % n == 0 &&
           nks * 4 * (16 * ((3 * (n_alpha == 3 ? n * n + 2 * n : 2 * n) + 15) / 16)) * 16 +
                   2 * kTileTokens * (16 * ((3 * (n_alpha == 3 ? n * n + 2 * n : 2 * n) + 15) / 16)) * 4 +
                   2 * kTileTokens * 4 <=
               kLdsBytes - 8 * 1024;
}
// Vector memory operations a half's wave has issued after the x loads of its task `it`
// when it waits for them. Task 0's and 1's loads go out in the prologue; task it + 2's
// during task it's products, before task it's record stores (nstore). So after task it's
// loads come: task it + 1's loads (lg, if that task exists) and the record stores of tasks
// it - 1 (for it >= 1) and it - 2 (for it >= 2).
MHC_HOST_DEVICE constexpr int stream_younger_than_x(int it, bool next_live, int lg, int nstore)
{
    return (it >= 2 ? nstore : 0) + (it >= 1 ? nstore : 0) + (next_live ? lg : 0);
}
constexpr int kStreamMaxWait = 47;     // the largest vmcnt the streaming kernel waits down to

// Groups of the single-read kernel: one per XCD (the hardware's XCC id), so the values
// its members exchange stay in that XCD's L2; member = arrival order on the XCD.
constexpr int kXcds = 8;               // XCDs (groups at most)
constexpr int kTicket0 = 8;            // sync word of XCD 0's arrival counter (kXcds words)

// One-launch forward of a few tokens (n = 4, alpha[3], no pre_mix): one workgroup per
// d-block projects every token's x of its block, two grid-wide barriers separate the
// blocks' partial records, the per-token math and hIn.
constexpr int64_t kDecodeTokens = 64;  // tokens at most (4 waves x 16 matrix rows)
constexpr int kDecodeMaxBlocks = kMaxD / kBlock;   // barrier flag words (one per possible d-block)
constexpr int kDecodeFlag0 = 256;      // sync word of the first flag
constexpr int kDecodeRecWords = 26;    // tagged words per partial record (n = 4, alpha[3]): M + 1 and a pad

// The workspace's sync section: the call counter, the time-out flag, the per-XCD arrival
// counters and the one-launch kernel's barrier flags, at the same offsets for every size.
constexpr size_t kSyncBytes = 4096;

struct Geometry {
    int n = 0;
    int D = 0;
    int n_alpha = 0;
    int M = 0;           // phi rows: n*n + 2n or 2n
    int64_t K = 0;       // n * D
    int NT = 0;          // 16-wide column tiles covering the 3*M packed columns
    int NC = 0;          // 16 * NT
    int nblk = 0;        // d-blocks: ceil(D / 32)
    int nks = 0;         // K-steps holding data: nblk * n
    int x_f16 = 0;       // x and hIn in binary16 (else bf16); weights packed as fp16 terms
    size_t packed_bytes = 0;
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }


// Kernel variant of an (n, n_alpha) pair: column tiles, K-steps per LDS weight stage,
// and the two slice lengths (K-steps) compiled for it.
struct Variant {
    int nt = 0;
    int sk = 0;
    int nks_big = 0;
    int nks_small = 0;
    int nks_premix = 0;   // the large slice of a call with pre_mix
};

inline Variant variant_of(int n, int n_alpha)
{
    Variant v;
    if (n == 4 && n_alpha == 3) { v.nt = 5; v.sk = 1; v.nks_big = 16; v.nks_small = 16; }
    else if (n == 4 && n_alpha == 2) { v.nt = 2; v.sk = 4; v.nks_big = 16; v.nks_small = 16; }
    else if (n == 8 && n_alpha == 3) { v.nt = 15; v.sk = 1; v.nks_big = 8; v.nks_small = 8; }
    else if (n == 8 && n_alpha == 2) { v.nt = 3; v.sk = 2; v.nks_big = 16; v.nks_small = 16; v.nks_premix = 32; }
    else if (n == 6 && n_alpha == 3) { v.nt = 9; v.sk = 1; v.nks_big = 12; v.nks_small = 12; }
    else if (n == 6 && n_alpha == 2) { v.nt = 3; v.sk = 2; v.nks_big = 12; v.nks_small = 12; }
    if (v.nks_premix == 0) v.nks_premix = v.nks_big;
    return v;
}

// Returns false for a combination the kernels do not support.
inline bool make_geometry(int n, int D, int n_alpha, Geometry* g)
{
    if (n != 4 && n != 6 && n != 8) return false;
    if (D <= 0 || D % 8 != 0 || D > kMaxD) return false;
    if (n_alpha != 2 && n_alpha != 3) return false;
    Geometry r;
    r.n = n;
    r.D = D;
    r.n_alpha = n_alpha;
    r.M = n_alpha == 3 ? n * n + 2 * n : 2 * n;
    r.K = (int64_t)n * D;
    r.NT = (3 * r.M + 15) / 16;
    r.NC = 16 * r.NT;
    r.nblk = (D + kBlock - 1) / kBlock;
    r.nks = r.nblk * n;
    r.packed_bytes = (size_t)(r.nks + kPadSteps) * 4 * r.NC * 16;
    // bounded number of partial records per token
    const Variant v = variant_of(n, n_alpha);
    if ((r.nks + v.nks_small - 1) / v.nks_small > kMaxSlices) return false;
    *g = r;
    return true;
}

// Projection workgroup -> task. Workgroup b runs on XCD b % 8 (the hardware deals
// workgroups to the 8 XCDs in turn). The XCDs are split into G groups of 8 / G, G the
// largest of 8, 4, 2, 1 dividing S: an XCD of group g works only on the slices
// s = g + G j, so its L2 holds S / G slices of the weights, and the XCDs of one group
// share out the tiles. Returns false for the padding workgroups of the last round.
MHC_HOST_DEVICE inline int xcd_groups(int S) { return S % 8 == 0 ? 8 : (S % 4 == 0 ? 4 : (S % 2 == 0 ? 2 : 1)); }
MHC_HOST_DEVICE inline int64_t proj_blocks(int64_t tiles, int S)
{
    const int G = xcd_groups(S), per = 8 / G;                 // XCDs per group
    const int64_t rounds = (tiles + per - 1) / per;           // tiles per XCD (rounded up)
    return rounds * (int64_t)(S / G) * 8;
}
MHC_HOST_DEVICE inline bool task_of_block(int64_t b, int64_t tiles, int S, int64_t* tile, int* s)
{
    const int G = xcd_groups(S), per = 8 / G, spg = S / G;
    const int q = (int)(b % 8);
    const int64_t r = b / 8;
    *s = q % G + G * (int)(r % spg);
    *tile = (r / spg) * per + q / G;
    return *tile < tiles;
}

struct Plan {
    Geometry g;
    int64_t T = 0;
    int64_t tiles = 0;        // ceil(T / 64)
    int NKS = 0;              // K-steps per slice
    int S = 0;                // slices per tile
    int GS = 0;               // slices per summation group: ceil(S / 8)
    int NG = 0;               // summation groups: ceil(S / GS) <= 8
    int64_t tasks = 0;        // tiles * S
    int64_t proj_blocks = 0;  // projection workgroups (tasks plus padding, see task_of_block)
    int OB = 8;               // tokens per epilogue workgroup: out_tokens(n, T)
    int64_t out_blocks = 0;   // epilogue workgroups: ceil(T / OB)
    // single-read variant
    bool fused_geom = false;  // the geometry admits it (n = 4, alpha[3], <= 7 blocks per member; bf16 or fp16 x)
    int FP = 0;               // members per group
    int FGS = 0, FNG = 0;     // summation groups over the FP member records (as GS, NG)
    int64_t tiles16 = 0;      // ceil(T / 16)
    // single-read kernel with XCD groups
    size_t off_prx = 0, off_hpx = 0, off_sync = 0;
    // one-launch kernel of a few tokens: the geometry admits it; its partial records
    // ([T][nblk][kDecodeRecWords] tagged 64-bit words) and hPre ([T][n] tagged words)
    bool decode_geom = false;
    size_t off_dpart = 0, off_dhp = 0;
    size_t off_packed = 0, off_wts = 0, off_rec = 0, ws_bytes = 0;
};

MHC_HOST_DEVICE inline int pp_stride(int n);
MHC_HOST_DEVICE inline int rec_stride(int n, int M);

// pre_mix: the plan of a call with pre_mix, whose projection writes hIn from the x it holds
// and so reads all n streams of a few d-blocks per slice: at n = 8 with alpha[2] and many
// tokens its slices are twice as long (32 K-steps: 256-byte runs of each stream's row, half
// the partial records). Its workspace sections are never larger than those of the same call
// without pre_mix (mhc_pre_workspace_size's plan).
inline Plan make_plan(const Geometry& g, int64_t T, bool pre_mix = false)
{
    Plan p;
    p.g = g;
    p.T = T;
    p.tiles = (T + kTileTokens - 1) / kTileTokens;
    const Variant v = variant_of(g.n, g.n_alpha);
    const int big = pre_mix ? v.nks_premix : v.nks_big;
    const int s_big = (g.nks + big - 1) / big;
    p.NKS = p.tiles * s_big >= kBigTasks ? big : v.nks_small;
    p.S = (g.nks + p.NKS - 1) / p.NKS;
    p.GS = (p.S + 7) / 8;
    p.NG = (p.S + p.GS - 1) / p.GS;
    p.tasks = p.tiles * p.S;
    p.proj_blocks = proj_blocks(p.tiles, p.S);
    p.OB = out_tokens(g.n, T);
    p.out_blocks = (T + p.OB - 1) / p.OB;
    p.FP = kFMembers;
    p.fused_geom = g.n == 4 && g.n_alpha == 3 && g.nblk >= kFMembers && (g.nblk + p.FP - 1) / p.FP <= kFMaxBlocks;
    p.FGS = (p.FP + 7) / 8;
    p.FNG = (p.FP + p.FGS - 1) / p.FGS;
    p.tiles16 = (T + kFTok - 1) / kFTok;
    const int rec_slices = p.fused_geom && p.FP > p.S ? p.FP : p.S;
    // the call counter first, at the same offset for every problem size
    size_t off = 0;
    p.off_sync = off;
    off += kSyncBytes;
    p.off_packed = off;
    off = align_up(off + g.packed_bytes, 256);
    p.off_wts = off;
    off = align_up(off + (size_t)T * g.n * sizeof(float), 256);
    p.off_rec = off;
    off = align_up(off + (size_t)p.tiles * rec_slices * kTileTokens * rec_stride(g.n, g.M) * sizeof(float), 256);
    if (p.fused_geom) {
        p.off_prx = off;
        off = align_up(off + (size_t)p.tiles16 * p.FP * kFTok * (g.n + 1) * 8, 256);
        p.off_hpx = off;
        off = align_up(off + (size_t)p.tiles16 * kFTok * g.n * 8, 256);
    }
    p.decode_geom = g.n == 4 && g.n_alpha == 3 && T <= kDecodeTokens;
    if (p.decode_geom) {
        p.off_dpart = off;
        off = align_up(off + (size_t)T * g.nblk * kDecodeRecWords * 8, 256);
        p.off_dhp = off;
        off = align_up(off + (size_t)T * g.n * 8, 256);
    }
    p.ws_bytes = off;
    return p;
}

// ---- offsets shared by the kernels and the host-side index checks (in elements) ----

// First slice-local summation group member: slices [g*GS, min(S, (g+1)*GS)).
MHC_HOST_DEVICE inline int group_begin(int GS, int g) { return g * GS; }
MHC_HOST_DEVICE inline int group_end(int S, int GS, int g)
{
    const int e = (g + 1) * GS;
    return e < S ? e : S;
}

// Tokens [tok_begin, tok_end) of a tile whose per-token outputs task (tile, s) writes.
MHC_HOST_DEVICE inline int out_tok_begin(int S, int s) { return (kTileTokens * s) / S; }
MHC_HOST_DEVICE inline int out_tok_end(int S, int s) { return (kTileTokens * (s + 1)) / S; }

// Byte offset, within the 64-token tile, of lane (row, grp)'s octet of stream i in the
// first d-block of the slice starting at d-block b0; d-block a of the slice adds 64 * a.
MHC_HOST_DEVICE inline uint32_t x_lane_off(int64_t K, int D, int row, int grp, int b0, int i)
{
    return (uint32_t)(((int64_t)row * K + (int64_t)i * D + kBlock * b0 + 8 * grp) * 2);
}

// 16-byte unit offset of the first packed unit of slice s.
MHC_HOST_DEVICE inline int64_t packed_slice(int s, int NKS, int NC) { return (int64_t)s * NKS * 4 * NC; }

// Partial record of a task for one token: the pre-branch sums and the square sum,
// padded to pp_stride(n) floats ([pre_0 .. pre_{n-1}, sq, 0...], a 16-byte multiple),
// then the remaining M - n projections, padded to a 16-byte multiple (only n = 6 needs
// it); rec_stride floats in all. A tile's records
// form one block of S * 64 records, slice-major. Offsets in floats.
MHC_HOST_DEVICE inline int pp_stride(int n) { return (n + 1 + 3) / 4 * 4; }
MHC_HOST_DEVICE inline int rec_stride(int n, int M) { return (pp_stride(n) + (M - n) + 3) / 4 * 4; }
MHC_HOST_DEVICE inline int64_t rec_tile(int64_t tile, int S, int n, int M)
{
    return tile * S * kTileTokens * rec_stride(n, M);
}
MHC_HOST_DEVICE inline int rec_loc(int s, int tl, int n, int M) { return (s * kTileTokens + tl) * rec_stride(n, M); }

// Single-read kernel: first d-block of member s (members take consecutive runs of the
// nblk d-blocks, sizes differing by at most one); word of the tagged pre-branch record of
// (tile jt, member s, token t, value v: the n pre sums, then the square); word of the
// published hPre of (tile jt, token t, stream i).
MHC_HOST_DEVICE inline int member_begin(int s, int nblk, int P) { return (int)((int64_t)s * nblk / P); }
MHC_HOST_DEVICE inline int64_t prx_at(int64_t jt, int P, int s, int t, int v, int n)
{
    return ((jt * P + s) * kFTok + t) * (n + 1) + v;
}
MHC_HOST_DEVICE inline int64_t hpx_at(int64_t jt, int t, int i, int n) { return (jt * kFTok + t) * n + i; }

// Single-read kernel, a compute wave with a d-block (R rounds): the memory operations it
// issues in round j after its x wait (the two record stores in rounds < R, the hIn store
// from round kFLag on, the kFLoads x loads of round j + kFAhead where that round exists),
// and how many of its operations are issued after round r's x loads and before round r's
// x wait (the later prologue loads when r < kFAhead, else every operation of the rounds in
// between). Operations complete in issue order, so waiting until no more than that many
// are outstanding waits for round r's x.
MHC_HOST_DEVICE inline int fused_round_ops(int64_t j, int64_t R)
{
    return (j < R ? 2 : 0) + (j >= kFLag ? 1 : 0) + (j + kFAhead < R ? kFLoads : 0);
}
MHC_HOST_DEVICE inline int fused_younger_than_x(int64_t r, int64_t R)
{
    int c = 0;
    if (r < kFAhead) {
        for (int64_t q = r + 1; q < kFAhead; ++q) c += q < R ? kFLoads : 0;
        for (int64_t j = 0; j < r; ++j) c += fused_round_ops(j, R);
    } else {
        for (int64_t j = r - kFAhead + 1; j < r; ++j) c += fused_round_ops(j, R);
    }
    return c;
}
constexpr int kFMaxYounger = (kFAhead - 1) * (2 + 1 + kFLoads);   // the largest such count

// Everything a forward launch needs (device pointers are raw).
struct ForwardArgs {
    const uint16_t* x;
    const void* packed;    // packed weights, or NULL: packed from phi / gamma into packed_ws
    const float* phi;
    const float* gamma;
    void* packed_ws;       // workspace section for the packed weights
    const float* alpha;
    const float* bias;
    const float* pre_mix;
    uint16_t* h_in;
    float* h_post;
    float* h_res;
    float* inv_rms;
    float* h_mix;
    float* h_pre;
    float* sum_out;
    float* norm_out;
    float* wts;        // [T][n] hIn weights (hPre) from the epilogue
    float* rec;        // partial records, one block per tile
    uint64_t* prx;     // single-read kernel: tagged pre-branch records
    uint64_t* hpx;     // single-read kernel: tagged hPre per tile
    uint64_t* dpart;   // one-launch kernel: tagged partial records of the d-blocks
    uint64_t* dhp;     // one-launch kernel: tagged hPre
    uint32_t* sync;    // [0] call counter (the epilogue adds 1; the single-read kernel's tag),
                       // [1] set when a single-read wait timed out,
                       // [8 .. 15] arrivals per XCD (the epilogue clears them),
                       // [256 .. 256 + kDecodeMaxBlocks) the one-launch kernel's barrier flags
    int num_iters;
    double norm_eps;
    double hc_eps;
};

// Kernels of one forward, in launch order, for per-kernel event timing: events[i] is
// recorded before stage i's kernel and events[i + 1] after it; a stage that launches
// nothing (pack with packed weights given, hIn with pre_mix) records its two events
// back to back.
constexpr int kStagePack = 0, kStageProj = 1, kStageEpi = 2, kStageHin = 3, kStages = 4;

// Implemented in mhc_kernels.hip. Return 0 on success, else the HIP error code.
int launch_prepack(const Geometry& g, const float* phi, const float* gamma, void* packed,
                   void* stream);
// events: NULL, or kStages + 1 caller-created events (hipEvent_t) recorded around the
// weight pack, projection, epilogue and hIn kernels.
int launch_forward(const Plan& p, const ForwardArgs& a, void* stream, void* const* events);
// Which kernels launch_forward runs for this plan and these arguments on the current
// device: 2 the one-launch kernel, 1 the single-read kernel, 0 the classic path.
int forward_path(const Plan& p, bool has_pre_mix);
int record_event(void* event, void* stream);
// Reads the workspace's time-out flag (sync word 1) after synchronising the stream, then
// clears it. 0 or the HIP error code.
int read_and_clear_wait_flag(uint32_t* sync, int32_t* timed_out, void* stream);
// Standalone stages (mhc_kernels.hip). launch_pre_sinkhorn reads h_mix / inv_rms from the
// given inputs, and from a: x, alpha, bias, pre_mix, the outputs h_in, h_pre, h_post, h_res,
// sum_out, norm_out, num_iters and hc_eps. 0 or the HIP error code.
int launch_inv_rms(int64_t T, int n, int D, double norm_eps, const uint16_t* x, float* inv_rms,
                   int x_f16, void* stream);
int launch_pre_sinkhorn(int64_t T, int n, int D, int n_alpha, int x_f16, const ForwardArgs& a,
                        const float* h_mix, const float* inv_rms, void* stream);
// mhc_scratch.hip: the device array that mhc_pre_forward_noalloc uses as its workspace
// (kScratchBytes per GPU), and its address on the current device, looked up once per device.
// 0 or the HIP error code.
constexpr size_t kScratchBytes = (size_t)64 << 20;
int scratch_for_current_device(void** ptr);

// hc_post (mhc_post.hip): out = post x + comb residual per token; 0 or the HIP error code.
int launch_post(int64_t T, int n, int D, const uint16_t* x, const uint16_t* residual, const float* post,
                const float* comb, uint16_t* out, int x_f16, void* stream);

}  // namespace mhc
