// Host-side model of the attention kernel's LDS ring schedule (the functions the kernel
// calls, from ring_schedule.hpp): eight waves issue their copies, wait, meet at barriers
// and read ring groups as the kernel does, with random copy latencies and compute times.
// Checks that a group is read only after every wave's copies of its round have landed, and
// that no round is issued into a group while a wave may still read the group's previous
// round.  Prints "ok" or the first violation.
#include <cstdio>
#include <vector>
#include "ring_schedule.hpp"

namespace {
struct Copy { int round; double land; };

unsigned long long rng = 88172645463325252ull;
double urand() {
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (rng >> 11) * (1.0 / 9007199254740992.0);
}

bool run(int NR, int nrounds, int waves) {
    // per wave: copies in issue order (landing times never decrease: in-order completion)
    std::vector<std::vector<Copy>> issued(waves);
    std::vector<double> now(waves, 0.0);
    auto issue = [&](int w, int round) {
        double land = now[w] + 0.5 + 5.0 * urand();
        if (!issued[w].empty() && issued[w].back().land > land) land = issued[w].back().land;
        issued[w].push_back({round, land});
    };
    for (int w = 0; w < waves; ++w)
        for (int x = 0; x < NR; ++x) issue(w, x);
    std::vector<double> read_end(nrounds, 0.0);   // when the last wave finished reading round r
    for (int r = 0; r < nrounds; ++r) {
        const int n = tmv_ring::inflight(r, NR);
        // the wait: all but the n most recent rounds of this wave's copies have landed
        for (int w = 0; w < waves; ++w) {
            const int done = static_cast<int>(issued[w].size()) - n;
            for (int i = 0; i < done; ++i) if (issued[w][i].land > now[w]) now[w] = issued[w][i].land;
        }
        double bar = 0.0;                            // the barrier
        for (int w = 0; w < waves; ++w) if (now[w] > bar) bar = now[w];
        for (int w = 0; w < waves; ++w) now[w] = bar;
        for (int w = 0; w < waves; ++w)
            for (const Copy &c : issued[w])
                if (c.round == r && c.land > bar) {
                    std::printf("round %d read before it landed (NR %d, rounds %d)\n", r, NR, nrounds);
                    return false;
                }
        const int x = tmv_ring::issue_at(r, NR);
        if (x >= 0) {
            const int prev = x - NR;                 // the group's previous round
            if (prev >= 0 && (prev >= r || read_end[prev] > bar)) {
                std::printf("round %d issued over round %d still in use\n", x, prev);
                return false;
            }
            for (int w = 0; w < waves; ++w) issue(w, x);
        }
        double end = 0.0;
        for (int w = 0; w < waves; ++w) { now[w] += 0.2 + 2.0 * urand(); if (now[w] > end) end = now[w]; }
        read_end[r] = end;
    }
    for (int r = 0; r < nrounds; ++r) {
        int cnt = 0;
        for (const Copy &c : issued[0]) cnt += c.round == r;   // (rounds past the last are empty copies)
        if (cnt != 1) { std::printf("round %d issued %d times\n", r, cnt); return false; }
    }
    return true;
}
}  // namespace

int main() {
    for (int NR : {2, 4})
        for (int n = 0; n <= 64; ++n)
            for (int trial = 0; trial < 20; ++trial)
                if (!run(NR, n, 8)) return 1;
    std::printf("ok\n");
    return 0;
}
