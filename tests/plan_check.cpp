// plan_check.cpp -- host-side bounds checks of the fused forward's launch plan.
//
// Built with g++ by tests/test_plan_bounds.py (no GPU, no HIP headers). For a sweep of
// problem sizes it replays, with the offset helpers the kernels use (mhc_plan.h), every
// index the fused kernel forms from the plan -- packed-weight stage loads, x / hIn byte
// offsets, partial-record blocks, summation groups, output token shares, workspace
// sections -- and checks each against the extent of the buffer it addresses, for plans of
// calls without and with pre_mix. Prints
// "ok <cases>" or the first violation and exits non-zero.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "mhc_plan.h"

using namespace mhc;

static int fail(const char* what, int n, int D, int na, long long T, long long a, long long b)
{
    std::printf("FAIL %s n=%d D=%d n_alpha=%d T=%lld (%lld vs %lld)\n", what, n, D, na, T, a, b);
    return 1;
}

static int check(int n, int D, int na, long long T, bool pm)
{
    Geometry g;
    if (!make_geometry(n, D, na, &g)) {
        // refused only when a token would need more than kMaxSlices partial records
        const Variant v0 = variant_of(n, na);
        const int nks = (D + kBlock - 1) / kBlock * n;
        if ((nks + v0.nks_small - 1) / v0.nks_small > kMaxSlices) return 0;
        return fail("geometry", n, D, na, T, 0, 0);
    }
    const Plan p = make_plan(g, T, pm);
    // a call with pre_mix fits the workspace that mhc_pre_workspace_size reports (the plan
    // without pre_mix)
    if (pm && p.ws_bytes > make_plan(g, T).ws_bytes)
        return fail("pre_mix workspace", n, D, na, T, (long long)p.ws_bytes, (long long)make_plan(g, T).ws_bytes);
    const Variant v = variant_of(n, na);
    if (v.nt != g.NT) return fail("variant nt", n, D, na, T, v.nt, g.NT);
    // the pack kernel's row threads also zero the padding columns [3M, NC)
    if (g.NC - 3 * g.M > g.M || g.NC < 3 * g.M) return fail("pack padding columns", n, D, na, T, g.NC, g.M);
    if (p.NKS % n || p.NKS % v.sk) return fail("slice not whole blocks/stages", n, D, na, T, p.NKS, v.sk);
    if (p.NKS > kPadSteps) return fail("slice longer than the zero tail", n, D, na, T, p.NKS, kPadSteps);
    // every K-step with data is in some slice; the last slice's loads stay in the packed buffer
    if ((long long)p.S * p.NKS < g.nks) return fail("slices miss K-steps", n, D, na, T, p.S * p.NKS, g.nks);
    const long long units = (long long)(g.nks + kPadSteps) * 4 * g.NC;
    if ((long long)g.packed_bytes != units * 16) return fail("packed bytes", n, D, na, T, g.packed_bytes, units * 16);
    const long long last_unit = packed_slice(p.S - 1, p.NKS, g.NC) + (long long)p.NKS * 4 * g.NC;
    if (last_unit > units) return fail("packed stage load past end", n, D, na, T, last_unit, units);
    // bounded records per token
    if (p.S > kMaxSlices) return fail("too many slices", n, D, na, T, p.S, kMaxSlices);
    // summation groups: at most 8, contiguous, covering [0, S)
    if (p.NG < 1 || p.NG > 8) return fail("groups", n, D, na, T, p.NG, 8);
    int next = 0;
    for (int gi = 0; gi < p.NG; ++gi) {
        const int b = group_begin(p.GS, gi), e = group_end(p.S, p.GS, gi);
        if (b != next || e <= b) return fail("group partition", n, D, na, T, b, next);
        next = e;
    }
    if (next != p.S) return fail("group cover", n, D, na, T, next, p.S);
    // projection workgroups cover every (tile, slice) exactly once, each XCD (b % 8) works
    // on at most ceil(S / 8) distinct slices when S is even... (S / xcd_groups(S) slices)
    if (p.tiles > 0 && p.tiles * (long long)p.S <= 4000000) {
        std::vector<unsigned char> seen((size_t)(p.tiles * p.S), 0);
        std::vector<std::vector<unsigned char>> xs(8, std::vector<unsigned char>(p.S, 0));
        for (long long b = 0; b < p.proj_blocks; ++b) {
            int64_t tile; int s;
            if (!task_of_block(b, p.tiles, p.S, &tile, &s)) continue;
            if (tile < 0 || tile >= p.tiles || s < 0 || s >= p.S) return fail("task range", n, D, na, T, tile, s);
            if (seen[(size_t)(tile * p.S + s)]++) return fail("task twice", n, D, na, T, tile, s);
            xs[b % 8][s] = 1;
        }
        for (size_t i = 0; i < seen.size(); ++i)
            if (!seen[i]) return fail("task missed", n, D, na, T, (long long)i, 0);
        for (int q = 0; q < 8; ++q) {
            int cnt = 0;
            for (int s = 0; s < p.S; ++s) cnt += xs[q][s];
            if (cnt > p.S / xcd_groups(p.S)) return fail("slices per XCD", n, D, na, T, cnt, p.S / xcd_groups(p.S));
        }
    }
    // output token shares partition [0, 64)
    next = 0;
    for (int s = 0; s < p.S; ++s) {
        const int b = out_tok_begin(p.S, s), e = out_tok_end(p.S, s);
        if (b != next || e < b) return fail("token shares", n, D, na, T, b, next);
        next = e;
    }
    if (next != kTileTokens) return fail("token cover", n, D, na, T, next, kTileTokens);
    // x byte offsets within a tile fit the 32-bit buffer offset; the largest one any lane
    // forms (row 63, last stream, last block of the last slice, group 3, 16 bytes)
    const int bps = p.NKS / n;
    const long long xmax = (long long)x_lane_off(g.K, D, 63, 3, (p.S - 1) * bps, n - 1) +
                           2LL * kBlock * (bps - 1) + 16;
    const long long xexact = ((63LL * g.K) + (long long)(n - 1) * D + kBlock * ((long long)(p.S - 1) * bps + bps - 1) + 24 + 8) * 2;
    if (xmax != xexact) return fail("x offset helper", n, D, na, T, xmax, xexact);
    if (xmax >= (1LL << 31)) return fail("x offset overflow", n, D, na, T, xmax, 1LL << 31);
    if (64LL * g.K * 2 >= (1LL << 31)) return fail("x tile range overflow", n, D, na, T, 64LL * g.K * 2, 1LL << 31);
    // hIn offsets: row 63, last block of the last slice
    const long long hmax = ((63LL * D) + kBlock * ((long long)(p.S - 1) * bps + bps - 1) + 24 + 8) * 2;
    if (hmax >= (1LL << 31)) return fail("hIn offset overflow", n, D, na, T, hmax, 1LL << 31);
    // partial-record blocks: per-tile byte ranges fit the buffer offsets; records of
    // different (slice, token) pairs do not overlap; 16-byte chunks stay 16-byte aligned
    const long long pps = pp_stride(n), rs = rec_stride(n, g.M);
    if (pps % 4 || rs % 4 || pps < n + 1 || rs < pps + g.M - n || rs > pps + g.M - n + 3)
        return fail("record strides", n, D, na, T, pps, rs);
    const long long recb = (long long)p.S * kTileTokens * rs * 4;
    if (recb >= (1LL << 31)) return fail("record block overflow", n, D, na, T, recb, 1LL << 31);
    if (rec_tile(1, p.S, n, g.M) * 4 != recb) return fail("record tile stride", n, D, na, T, rec_tile(1, p.S, n, g.M) * 4, recb);
    if (((long long)rec_loc(p.S - 1, 63, n, g.M) + rs) * 4 != recb)
        return fail("record local", n, D, na, T, rec_loc(p.S - 1, 63, n, g.M), recb / 4);
    if ((rec_loc(0, 1, n, g.M) * 4) % 16) return fail("record alignment", n, D, na, T, 0, 0);
    // streaming projection (no pre_mix, D a multiple of 32, the variants it is compiled for):
    // slice s holds K-steps [s NKS, s NKS + NKS) of the flattened row; every K-step with data
    // lies in exactly one slice; each lane's x octet stays inside its token's row; the gather
    // from the d-block-major packed layout reads inside the packed buffer (K-steps past the
    // data: its first zero K-step); the in-kernel split reads inside phi and gamma; a slice's
    // weights and both halves' column totals fit LDS; the grid's halves cover every tile once
    const bool stream_variant = (n == 4 && p.NKS == 16) || (n == 8 && na == 2 && p.NKS == 16) ||
                                (n == 6 && na == 2 && p.NKS == 12);
    if (!pm && D % kBlock == 0 && stream_variant) {
        if (!stream_fits(n, na, p.NKS)) return fail("stream LDS", n, D, na, T, p.NKS, 0);
        const int nblk = D / kBlock, nks = n * nblk;
        if (nks != g.nks || (long long)nks * kBlock != g.K) return fail("stream K-steps", n, D, na, T, nks, g.nks);
        const long long units = (long long)(g.nks + kPadSteps) * 4 * g.NC;
        for (int sl = 0; sl < p.S; ++sl)
            for (int st = 0; st < p.NKS; ++st) {
                const int gk = sl * p.NKS + st;
                if (gk >= nks) continue;   // past the data: x reads out of range, weights the zero step
                const long long xlast = 63LL * g.K + (long long)kBlock * gk + 8 * 3 + 8;   // elements, exclusive
                if (xlast > 64LL * g.K || (long long)kBlock * gk + 32 > g.K) return fail("stream x", n, D, na, T, gk, xlast);
                const long long pst = (long long)(gk % nblk) * n + gk / nblk;
                if (pst < 0 || pst >= nks || (pst + 1) * 4 * g.NC > units) return fail("stream gather", n, D, na, T, gk, pst);
                // the packed K-step holds stream gk / nblk, d-block gk % nblk: the same 32 elements
                if ((pst % n) * (long long)D + kBlock * (pst / n) != (long long)kBlock * gk)
                    return fail("stream K order", n, D, na, T, gk, pst);
            }
        if ((long long)(nks + 1) * 4 * g.NC > units) return fail("stream zero step", n, D, na, T, nks, units);
        for (int cus : {256, 304, 80}) {
            long long W = cus / p.S;
            if (W > (p.tiles + 1) / 2) W = (p.tiles + 1) / 2;
            if (W < 1) W = 1;
            const long long NI = (p.tiles + 2 * W - 1) / (2 * W);
            std::vector<unsigned char> seen((size_t)p.tiles + 1, 0);
            for (long long h = 0; h < 2 * W; ++h)
                for (long long it = 0; it < NI; ++it) {
                    const long long tile = h + 2 * W * it;
                    if (tile < p.tiles && seen[(size_t)tile]++) return fail("stream tile twice", n, D, na, T, tile, W);
                }
            for (long long t = 0; t < p.tiles; ++t)
                if (!seen[(size_t)t]) return fail("stream tile missed", n, D, na, T, t, W);
        }
    }
    // epilogue workgroups: 8 tokens each, inside one tile
    const int ob = p.OB;
    if (ob != out_tokens(n, T) || (ob != 8 && ob != 16)) return fail("epilogue token count", n, D, na, T, ob, 0);
    if (kTileTokens % ob) return fail("epilogue tokens", n, D, na, T, ob, 0);
    if (p.out_blocks * ob < T || (p.out_blocks - 1) * ob >= T) return fail("epilogue grid", n, D, na, T, p.out_blocks, 0);
    // workspace sections: ordered, 256-aligned, large enough
    const size_t secs[] = {p.off_packed, p.off_wts, p.off_rec, p.ws_bytes};
    for (int i = 0; i < 4; ++i)
        if (secs[i] % 256) return fail("section alignment", n, D, na, T, i, secs[i]);
    if (p.off_wts < p.off_packed + g.packed_bytes) return fail("packed size", n, D, na, T, p.off_wts, 0);
    if (p.off_rec < p.off_wts + (size_t)T * n * 4) return fail("wts size", n, D, na, T, p.off_rec, 0);
    if (p.ws_bytes < p.off_rec + (size_t)p.tiles * recb) return fail("record size", n, D, na, T, p.ws_bytes, 0);
    // the call counter sits first, at the same offset for every size
    if (p.off_sync != 0 || p.off_packed < kSyncBytes) return fail("sync section", n, D, na, T, p.off_sync, p.off_packed);
    // single-read variant
    const bool want = n == 4 && na == 3 && g.nblk >= kFMembers && (g.nblk + kFMembers - 1) / kFMembers <= kFMaxBlocks;
    if (p.fused_geom != want) return fail("single-read admission", n, D, na, T, p.fused_geom, want);
    if (p.fused_geom) {
        if (p.FP != kFMembers || p.FGS * 8 < p.FP || p.FP % p.FGS || p.FNG > 8)
            return fail("member groups", n, D, na, T, p.FP, p.FGS);
        int prev = 0;
        for (int s = 0; s < p.FP; ++s) {
            const int b0 = member_begin(s, g.nblk, p.FP), b1 = member_begin(s + 1, g.nblk, p.FP);
            if (b0 != prev || b1 - b0 < 1 || b1 - b0 > kFMaxBlocks) return fail("member blocks", n, D, na, T, b0, b1);
            // the member's weights: whole K-steps inside the packed buffer
            if ((long long)b1 * n * 4 * g.NC > (long long)(g.nks + kPadSteps) * 4 * g.NC)
                return fail("member weights", n, D, na, T, b1, g.nks);
            prev = b1;
        }
        if (prev != g.nblk) return fail("member cover", n, D, na, T, prev, g.nblk);
        // LDS: weights (3M columns), two buffers of every compute wave's row sums (rows
        // padded to 32) and squares, four hPre slots and their flags, the barrier count
        const long long lds = (long long)kFMaxBlocks * n * 4 * 3 * g.M * 16 +
                              2LL * kFMaxBlocks * kFTok * (32 + 1) * 4 + 4 * kFTok * n * 4 + 5 * 4;
        if (lds > 160 * 1024) return fail("single-read LDS", n, D, na, T, lds, 160 * 1024);
        if (T > 0 && (p.tiles16 * kFTok < T || (p.tiles16 - 1) * kFTok >= T)) return fail("tiles16", n, D, na, T, p.tiles16, 0);
        // 16-token x tile: the largest lane offset (row 15, last stream, last block, octet 3)
        const long long xo = ((15LL * g.K) + (long long)(n - 1) * D + kBlock * (g.nblk - 1LL) + 24) * 2 + 16;
        if (xo >= (1LL << 31) || 16LL * g.K * 2 >= (1LL << 31)) return fail("single-read x offsets", n, D, na, T, xo, 0);
        // records with slice = member fill the record area
        const long long frec = (long long)p.FP * kTileTokens * rs * 4;
        if (rec_tile(p.tiles, p.FP, n, g.M) * 4 != p.tiles * frec) return fail("member record tiles", n, D, na, T, 0, 0);
        if ((size_t)(p.tiles * frec) > p.off_prx - p.off_rec) return fail("member record area", n, D, na, T, p.tiles * frec, 0);
        // tagged exchange areas
        if (p.tiles16 > 0) {
            const long long pw = p.tiles16 * p.FP * kFTok * (n + 1);
            if (prx_at(p.tiles16 - 1, p.FP, p.FP - 1, kFTok - 1, n, n) + 1 != pw) return fail("prx index", n, D, na, T, pw, 0);
            if (p.off_hpx < p.off_prx + (size_t)pw * 8 || p.off_hpx % 256) return fail("prx area", n, D, na, T, p.off_hpx, 0);
            const long long hw = p.tiles16 * kFTok * n;
            if (hpx_at(p.tiles16 - 1, kFTok - 1, n - 1, n) + 1 != hw) return fail("hpx index", n, D, na, T, hw, 0);
            if (p.ws_bytes < p.off_hpx + (size_t)hw * 8) return fail("hpx area", n, D, na, T, p.ws_bytes, 0);
        }
    }
    // one-launch kernel of a few tokens: its sync words inside the 256-byte sync section,
    // after the per-XCD counters; partial records [T][nblk][rs] and hPre [T][n] in order
    if (kDecodeFlag0 < kTicket0 + kXcds || (size_t)(kDecodeFlag0 + kDecodeMaxBlocks) * 4 > kSyncBytes ||
        kDecodeMaxBlocks * kBlock < kMaxD)
        return fail("decode flag words", n, D, na, T, kDecodeFlag0, kDecodeMaxBlocks);
    const bool dwant = n == 4 && na == 3 && T <= kDecodeTokens;
    if (p.decode_geom != dwant) return fail("decode admission", n, D, na, T, p.decode_geom, dwant);
    if (p.decode_geom) {
        const size_t end_before = p.fused_geom ? p.off_hpx + (size_t)p.tiles16 * kFTok * n * 8 : p.off_rec + (size_t)p.tiles * recb;
        if (p.off_dpart % 256 || p.off_dhp % 256 || p.off_dpart < end_before) return fail("decode sections", n, D, na, T, p.off_dpart, end_before);
        if (kDecodeRecWords != g.M + 2 || kDecodeRecWords % 2) return fail("decode record words", n, D, na, T, kDecodeRecWords, g.M);
        const long long last = ((T - 1) * g.nblk + (g.nblk - 1LL)) * kDecodeRecWords + kDecodeRecWords;   // one past the last word
        if (p.off_dhp < p.off_dpart + (size_t)last * 8) return fail("decode records", n, D, na, T, p.off_dhp, last);
        if (p.ws_bytes < p.off_dhp + (size_t)T * n * 8) return fail("decode hPre", n, D, na, T, p.ws_bytes, 0);
        // x and hIn byte offsets of the last lane (token T-1, stream n-1, last block, octet 3)
        const long long xo = (((T - 1) * g.K) + (long long)(n - 1) * D + kBlock * (g.nblk - 1LL) + 24) * 2 + 16;
        if (xo >= (1LL << 31)) return fail("decode x offsets", n, D, na, T, xo, 0);
    }
    return 0;
}

int main()
{
    long long cases = 0;
    const long long Ts[] = {1, 2, 15, 63, 64, 65, 127, 128, 200, 1000, 4096, 16384, 32768, 100000};
    std::vector<int> Ds;
    for (int d = 8; d <= 1024; d += 8) Ds.push_back(d);
    for (int d = 1032; d <= kMaxD; d += 8 * 37) Ds.push_back(d);
    const int fixed[] = {2048, 2560, 4096, 5120, 7168, 8192, 16384};
    for (int d : fixed) Ds.push_back(d);
    for (int n : {4, 6, 8})
        for (int na : {2, 3})
            for (int D : Ds)
                for (long long T : Ts)
                    for (bool pm : {false, true}) {
                        if (check(n, D, na, T, pm)) return 1;
                        ++cases;
                    }
    std::printf("ok %lld\n", cases);
    return 0;
}
