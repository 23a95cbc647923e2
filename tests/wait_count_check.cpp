// Replays, as an explicit list of issued memory operations, what a compute wave with a
// d-block of the single-read kernel issues (the prologue's x loads, then per round: the x
// wait, two record stores in rounds < R, the hIn store from round kFLag on, the x loads of
// round r + kFAhead where that round exists), and checks for every round r < R and a sweep
// of R that the number of operations issued between round r's last x load and round r's x
// wait equals fused_younger_than_x(r, R), the count the kernel waits down to (operations
// complete in issue order), and that it stays within the counts the kernel can wait for.
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
    return 0;
}
