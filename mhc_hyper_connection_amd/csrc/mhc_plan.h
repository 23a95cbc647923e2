// mhc_plan.h -- launch geometry and workspace layout of the fused mHC pre forward.
//
// Host-side and plain C++ (no HIP headers): the validation / planning code that uses it
// can be built and tested on a machine without a GPU.
//
// Data layout the kernels rely on
//   xFlat of token t is x[t*K .. t*K + K) with K = n*D (TND, row-major; stream i occupies
//   [i*D, (i+1)*D)). The reduction dimension K is walked in chunks of 128 consecutive
//   xFlat elements (256 bytes of a token row: two whole cache lines), as 16 "octets" of
//   8 bf16. The matrix-core K-step s of a chunk consumes octets 4s .. 4s+3, lane group g
//   (= lane / 16) holding octet 4s + g. Any order of K gives the same dot product, so
//   the packed weights only need to use this same order. D % 8 == 0 keeps every octet
//   inside one stream.
//   Packed weights: for each chunk, 16 octet rows x NC columns of 8 bf16 (16 bytes),
//   octet-major. Column c < 3M is term (c / M) of phi row (c % M) with gamma folded in:
//   term 0 = hi, 1 = mid, 2 = lo, hi + mid + lo = phi * gamma to ~2^-26 relative.
//   Columns >= 3M, octets at or beyond K, and one extra all-zero chunk at the end (so the
//   one-chunk-ahead weight prefetch never needs a bounds test) hold zeros.
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
constexpr int kTileTokens = 64;        // tokens per projection tile: 4 waves x 16 rows
constexpr int kOctets = 16;            // octets per chunk
constexpr int kChunk = 8 * kOctets;    // xFlat elements per chunk
constexpr int kMaxN = 8;
constexpr int kTargetBlocks = 2048;    // projection workgroups to aim for (256 CUs)

struct Geometry {
    int n = 0;
    int D = 0;
    int n_alpha = 0;
    int M = 0;           // phi rows: n*n + 2n or 2n
    int64_t K = 0;       // n * D
    int NT = 0;          // 16-wide column tiles covering the 3*M packed columns
    int NC = 0;          // 16 * NT
    int NTHI = 0;        // column tiles holding the "hi" term (accumulated in fp64)
    int nch = 0;         // chunks of 128 xFlat elements: ceil(K / 128)
    size_t packed_bytes = 0;
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Returns false for a combination the kernels do not support.
inline bool make_geometry(int n, int D, int n_alpha, Geometry* g)
{
    if (n != 4 && n != 8) return false;
    if (D <= 0 || D % 8 != 0) return false;
    if (n_alpha != 2 && n_alpha != 3) return false;
    Geometry r;
    r.n = n;
    r.D = D;
    r.n_alpha = n_alpha;
    r.M = n_alpha == 3 ? n * n + 2 * n : 2 * n;
    r.K = (int64_t)n * D;
    r.NT = (3 * r.M + 15) / 16;
    r.NC = 16 * r.NT;
    r.NTHI = (r.M + 15) / 16;
    r.nch = (int)((r.K + kChunk - 1) / kChunk);
    r.packed_bytes = (size_t)(r.nch + 1) * kOctets * r.NC * 16;
    *g = r;
    return true;
}

struct Plan {
    Geometry g;
    int64_t T = 0;
    int64_t tiles = 0;        // ceil(T / kTileTokens)
    int S = 0;                // K-slices (split of the reduction across workgroups)
    int64_t blocks = 0;       // projection workgroups = tiles * S
    int pstride = 0;          // floats per token in a partial record: M sums + 1 square sum
    size_t off_packed = 0, off_wts = 0, off_part = 0, ws_bytes = 0;
};

// First chunk of slice s when nch chunks are split into S nearly equal ranges.
MHC_HOST_DEVICE inline int slice_begin(int nch, int S, int s)
{
    const int base = nch / S, rem = nch % S;
    return s * base + (s < rem ? s : rem);
}

inline Plan make_plan(const Geometry& g, int64_t T)
{
    Plan p;
    p.g = g;
    p.T = T;
    p.tiles = (T + kTileTokens - 1) / kTileTokens;
    int64_t want = p.tiles > 0 ? (kTargetBlocks + p.tiles - 1) / p.tiles : 1;
    if (want > g.nch) want = g.nch;
    if (want < 1) want = 1;
    int S = (int)want;
    if (S >= 8) S -= S % 8;   // a multiple of 8 maps each slice onto one XCD
    p.S = S;
    p.blocks = p.tiles * S;
    p.pstride = g.M + 1;
    size_t off = 0;
    p.off_packed = off;
    off = align_up(off + g.packed_bytes, 256);
    p.off_wts = off;
    off = align_up(off + (size_t)T * g.n * sizeof(float), 256);
    p.off_part = off;
    off = align_up(off + (size_t)S * (size_t)T * p.pstride * sizeof(float), 256);
    p.ws_bytes = off;
    return p;
}

// Everything a forward launch needs (device pointers are raw).
struct ForwardArgs {
    const uint16_t* x;
    const void* packed;
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
    float* wts;
    float* part;
    int num_iters;
    double norm_eps;
    double hc_eps;
};

// Implemented in mhc_kernels.hip. Return 0 on success, else the HIP error code.
int launch_prepack(const Geometry& g, const float* phi, const float* gamma, void* packed,
                   void* stream);
int launch_forward(const Plan& p, const ForwardArgs& a, void* stream);

}  // namespace mhc
