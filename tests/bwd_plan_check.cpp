// bwd_plan_check.cpp -- host-side bounds checks of the MhcPre backward's launch plan.
//
// Built with g++ by tests/test_plan_bounds.py (no GPU, no HIP headers). For a sweep of
// sizes it replays, with the offset helpers the kernels use (mhc_bwd_plan.h), the
// indices the backward kernels form -- packed-phi units and the columns they stand for,
// main-pass workgroup -> (token group, d-block, stream group), x / gradX byte offsets,
// partial-sum and per-token-term indices, workspace sections -- and checks each against
// the extent of what it addresses. Prints "ok <cases>" or the first violation.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "mhc_bwd_plan.h"

using namespace mhc::bwd;

static int fail(const char* what, int n, int D, long long T, long long a, long long b)
{
    std::printf("FAIL %s n=%d D=%d T=%lld (%lld vs %lld)\n", what, n, D, T, a, b);
    return 1;
}

static int check(int n, int D, long long T)
{
    Geometry g;
    if (!make_geometry(n, D, &g)) return fail("geometry", n, D, T, 0, 0);
    const Plan p = make_plan(g, T);
    if (g.MP < g.M || g.MP % 32 || g.MP - g.M >= 32) return fail("padded rows", n, D, T, g.MP, g.M);
    if (g.n % g.SGN || g.NSG * g.SGN != g.n) return fail("stream groups", n, D, T, g.SGN, g.NSG);
    if ((long long)g.nblk * kDBlock < D || (long long)(g.nblk - 1) * kDBlock >= D)
        return fail("d-blocks", n, D, T, g.nblk, D);
    const long long units = (long long)g.nblk * n * pack_units_per_stream(g.KS);
    if ((long long)g.pack_bytes != units * 16) return fail("pack bytes", n, D, T, g.pack_bytes, units * 16);
    // pack: within one (d-block, stream), each lane group holds 8 consecutive positions
    // across the two halves, each position once
    for (int grp = 0; grp < 4; ++grp) {
        int seen = 0;
        for (int h = 0; h < 2; ++h)
            for (int r = 0; r < 4; ++r) {
                const int c = pack_col(h, 4 * grp + r);
                if (c < 8 * grp || c >= 8 * grp + 8) return fail("pack column", n, D, T, c, grp);
                seen |= 1 << (c - 8 * grp);
            }
        if (seen != 0xff) return fail("pack columns cover", n, D, T, seen, grp);
    }
    // a main-pass workgroup stages units [pack_at(b, sg SGN), + SGN units_per_stream)
    for (int b = 0; b < g.nblk; ++b)
        for (int sg = 0; sg < g.NSG; ++sg) {
            const long long e = pack_at(b, sg * g.SGN, n, g.KS) + g.SGN * pack_units_per_stream(g.KS);
            if (e > units) return fail("pack staging past end", n, D, T, e, units);
        }
    if (T == 0) return 0;
    // token groups: non-empty, covering [0, tiles)
    if (p.G < 1 || p.G * p.tpg < p.tiles || (p.G - 1) * p.tpg >= p.tiles)
        return fail("token groups", n, D, T, p.G, p.tpg);
    if (p.main_tasks != p.G * g.nblk * g.NSG) return fail("main tasks", n, D, T, p.main_tasks, p.G);
    if (p.main_blocks < p.main_tasks || p.main_blocks % 16) return fail("main blocks", n, D, T, p.main_blocks, p.main_tasks);
    if (p.token_blocks * 4 < T) return fail("token blocks", n, D, T, p.token_blocks, T);
    if (p.main_blocks <= 4000000) {
        // every task exactly once; the two d-blocks of a pair (2u, 2u + 1, same token
        // group and stream group) go to workgroups 8 apart, i.e. the same XCD
        std::vector<long long> at((size_t)p.main_tasks, -1);
        for (long long blk = 0; blk < p.main_blocks; ++blk) {
            int64_t gr;
            int b, sg;
            if (!main_task(blk, g.nblk, g.NSG, p.main_tasks, &gr, &b, &sg)) continue;
            if (gr < 0 || gr >= p.G || b < 0 || b >= g.nblk || sg < 0 || sg >= g.NSG)
                return fail("main task range", n, D, T, gr, b);
            const size_t id = ((size_t)gr * g.NSG + sg) * g.nblk + b;
            if (at[id] >= 0) return fail("main task twice", n, D, T, blk, (long long)id);
            at[id] = blk;
        }
        for (size_t id = 0; id < at.size(); ++id) {
            if (at[id] < 0) return fail("main task missing", n, D, T, (long long)id, 0);
            if (id % 2 == 1 && at[id] - at[id - 1] != 8) return fail("pair not on one XCD", n, D, T, at[id - 1], at[id]);
        }
    }
    // byte offsets the main pass forms inside one tile stay below 2^31 (buffer offsets)
    const long long K = g.K;
    const long long xoff = (long long)(kTile - 1) * K * 2 + (long long)(n - 1) * D * 2 + (long long)(D - 8) * 2 + 16;
    if (xoff >= (1LL << 31)) return fail("x offset", n, D, T, xoff, 1LL << 31);
    const long long goff = ((long long)(kTile - 1) * g.KS * 3 * 32 + (long long)g.KS * 3 * 32) * 2;
    if (goff >= (1LL << 31)) return fail("gMix offset", n, D, T, goff, 1LL << 31);
    // partial sums: P[g][m][k] and Q[g][k]; per-token terms [T][3 + M]
    const long long pmax = (p.G - 1) * (long long)g.M * K + (long long)(g.M - 1) * K + (K - 1);
    if (pmax >= p.G * (long long)g.M * K) return fail("gradPhi partial index", n, D, T, pmax, 0);
    // workspace sections in order, each large enough, inside ws_bytes
    const size_t need[] = {g.pack_bytes, (size_t)T * g.KS * 3 * 32 * 2, (size_t)T * 4, (size_t)T * (3 + g.M) * 8,
                           (size_t)p.G * g.M * K * 4, (size_t)p.G * K * 4, (size_t)T * n * n * 8};
    const size_t off[] = {p.off_pack, p.off_gmix, p.off_c3, p.off_terms, p.off_pphi, p.off_pgam, p.off_glog,
                          p.ws_bytes};
    for (int s = 0; s < 7; ++s) {
        if (off[s] % 256) return fail("section alignment", n, D, T, s, off[s]);
        if (off[s] + need[s] > off[s + 1]) return fail("section overlap", n, D, T, s, off[s + 1]);
    }
    return 0;
}

int main()
{
    const int Ds[] = {8, 16, 24, 32, 40, 256, 1000, 2048, 2056, 4096, 7168, 16384};
    const long long Ts[] = {0, 1, 3, 63, 64, 65, 130, 4096, 16384, 100003};
    long long cases = 0;
    for (int n : {4, 6, 8})
        for (int D : Ds)
            for (long long T : Ts) {
                if (check(n, D, T)) return 1;
                ++cases;
            }
    std::printf("ok %lld\n", cases);
    return 0;
}
