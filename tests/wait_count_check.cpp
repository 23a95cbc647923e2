// Replays, as an explicit list of issued memory operations, what a compute wave with a
// d-block of the single-read kernel issues (the prologue's x loads, then per round: the x
// wait, two record stores in rounds < R, the hIn store from round kFLag on, the x loads of
// round r + kFAhead where that round exists), and checks for every round r < R and a sweep
// of R that the number of operations issued between round r's last x load and round r's x
// wait equals fused_younger_than_x(r, R), the count the kernel waits down to (operations
// complete in issue order), and that it stays within the counts the kernel can wait for.
// Then the same for a wave of the streaming projection (proj_stream_kernel): per half, the
// weights' loads, the x loads of tasks 0 and 1, a wait down to those x loads, then per task
// it: the wait for task it's loads, the loads of task it + 2 (issued among its products)
// and its record stores, for every count of tasks a half has and every variant's load and
// store counts; each wait must equal
// stream_younger_than_x and lie within the counts the kernel can wait for (0 to kStreamMaxWait).
#include <cstdio>
#include <vector>

#include "mhc_plan.h"

using namespace mhc;

int main()
{
    long long checks = 0;
    for (long long R = 1; R <= 80; ++R) {
        // event list: load of round q (kind 0, round q) or another operation (kind 1)
        struct Ev { int kind; long long round; };
        std::vector<Ev> ev;
        std::vector<long long> wait_pos(R, -1);   // position in ev of round r's x wait
        for (long long q = 0; q < kFAhead; ++q)
            if (q < R)
                for (int l = 0; l < kFLoads; ++l) ev.push_back({0, q});
        for (long long r = 0; r < R + kFLag; ++r) {
            if (r < R) wait_pos[r] = (long long)ev.size();
            if (r < R) { ev.push_back({1, -1}); ev.push_back({1, -1}); }   // record value, tagged word
            if (r >= kFLag) ev.push_back({1, -1});                          // hIn of round r - kFLag
            if (r + kFAhead < R)
                for (int l = 0; l < kFLoads; ++l) ev.push_back({0, r + kFAhead});
        }
        for (long long r = 0; r < R; ++r) {
            long long last = -1;
            for (long long i = 0; i < wait_pos[r]; ++i)
                if (ev[i].kind == 0 && ev[i].round == r) last = i;
            if (last < 0) { std::printf("round %lld of R=%lld: no load before its wait\n", r, R); return 1; }
            const long long younger = wait_pos[r] - 1 - last;
            const int want = fused_younger_than_x(r, R);
            if (younger != want) {
                std::printf("R=%lld round %lld: %lld operations after its x loads, kernel waits to %d\n",
                            R, r, younger, want);
                return 1;
            }
            if (want < 0 || want > kFMaxYounger || want > 14) {
                std::printf("R=%lld round %lld: count %d outside the waits the kernel has\n", R, r, want);
                return 1;
            }
            ++checks;
        }
    }
    std::printf("ok %lld rounds checked (kFAhead %d, kFLag %d)\n", checks, kFAhead, kFLag);

    // streaming projection: (n, NKS, CH) of the compiled variants
    struct SV { int n, nks, ch; };
    const SV svs[] = {{4, 16, 7}, {4, 16, 3}, {8, 16, 5}, {6, 12, 4}};
    long long schecks = 0;
    for (const SV& v : svs)
        for (int pm = 0; pm < 1; ++pm) {
            const int lg = v.nks;
            const int nstore = stream_rec_stores(v.ch);
            for (int NI = 1; NI <= 40; ++NI)
                for (int L = 0; L <= NI; ++L) {   // tasks 0 .. L - 1 of this half exist
                    struct Ev { int kind; int task; };   // 0 load of a task, 1 other, 2 wait for all
                    std::vector<Ev> ev;
                    std::vector<long long> wait_pos(NI, -1);
                    auto loads = [&](int t) { if (t < L) for (int l = 0; l < lg; ++l) ev.push_back({0, t}); };
                    for (int w = 0; w < 12; ++w) ev.push_back({1, -1});   // the weights
                    loads(0);
                    loads(1);
                    for (int it = 0; it < NI; ++it) {
                        if (it < L) {
                            wait_pos[it] = (long long)ev.size();
                            loads(it + 2);
                            for (int q = 0; q < nstore; ++q) ev.push_back({1, -1});
                        }
                    }
                    for (int it = 0; it < L; ++it) {
                        long long last = -1;
                        bool drained = false;
                        for (long long i = 0; i < wait_pos[it]; ++i)
                            if (ev[i].kind == 0 && ev[i].task == it) last = i;
                        for (long long i = last + 1; i < wait_pos[it]; ++i)
                            if (ev[i].kind == 2) drained = true;
                        if (last < 0) { std::printf("stream: task %d has no loads before its wait\n", it); return 1; }
                        long long younger = 0;
                        for (long long i = last + 1; i < wait_pos[it]; ++i) younger += ev[i].kind != 2;
                        const int want = stream_younger_than_x(it, it + 1 < L, lg, nstore);
                        if (!drained && younger != want) {
                            std::printf("stream n=%d pm=%d NI=%d L=%d task %d: %lld after its loads, kernel waits to %d\n",
                                        v.n, pm, NI, L, it, younger, want);
                            return 1;
                        }
                        if (want < 0 || want > kStreamMaxWait) {
                            std::printf("stream n=%d pm=%d: count %d outside 0..%d\n", v.n, pm, want, kStreamMaxWait);
                            return 1;
                        }
                        ++schecks;
                    }
                }
        }
    std::printf("ok %lld streaming waits checked\n", schecks);
    return 0;
}
