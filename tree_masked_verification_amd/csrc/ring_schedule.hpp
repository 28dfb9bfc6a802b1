// Copy/wait schedule of the bf16 attention kernel's LDS ring (verify_attention.hip).
//
// The ring holds its chunk slots as NR groups of R chunks.  A split's local chunks are
// copied in rounds of R chunks; round x goes to group x % NR.
//   * Before the chunk loop every wave issues its copies of rounds 0 .. NR-1.
//   * Iteration r of the loop: the wave waits until at most inflight(r) rounds of its
//     copies are outstanding; vector-memory operations complete in issue order and every
//     wave issues the same number of copies per round, so its copies of round r have then
//     landed.  All waves meet at a barrier: after it round r is complete in LDS and every
//     wave has finished reading round r - 1 (its LDS reads were waited for before the
//     barrier).  From iteration 1 on the wave then issues round issue_at(r) = r + NR - 1
//     into group (r - 1) % NR, the one round r - 1 used, and computes round r.
//   * Rounds past the split's last one are issued all the same, as empty copies (they
//     write zeros into a free group and still count), so every iteration past the first
//     issues exactly one round and the wait count is the same in all of them.
// The functions are constexpr so that the kernel and the checks below (and a host-side
// model in the tests) use the same definitions.
#pragma once

namespace tmv_ring {

// round whose copies a wave issues after the barrier of iteration r (-1: none)
constexpr int issue_at(int r, int NR) { return r >= 1 ? r + NR - 1 : -1; }

// rounds of copies a wave has issued before its wait in iteration r
constexpr int issued_before(int r, int NR) { return r == 0 ? NR : NR + r - 1; }

// rounds of copies that may remain outstanding once round r has landed
constexpr int inflight(int r, int NR) { return issued_before(r, NR) - (r + 1); }

// Replays the schedule event by event for one geometry and checks that
//   (a) the closed forms above agree with the replay,
//   (b) each wait leaves round r landed and asks for an encodable count (0 .. NR-1 rounds),
//   (c) a round is issued into a group only once every wave has finished reading the
//       group's previous round (it is issued at the iteration after that round was
//       computed, past the barrier), and never into the group being computed,
//   (d) every round 0 .. nrounds-1 is issued exactly once, before it is computed.
constexpr bool replay(int NR, int nrounds) {
    int issued = 0;                 // rounds issued so far, in order
    int issue_iter[96] = {};        // iteration after whose barrier round x was issued (-1: prologue)
    for (int x = 0; x < NR; ++x) issue_iter[issued++] = -1;
    for (int r = 0; r < nrounds; ++r) {
        if (issued != issued_before(r, NR)) return false;                                // (a)
        const int n = inflight(r, NR);
        if (n < 0 || n > NR - 1 || issued - n < r + 1) return false;                     // (b)
        const int x = issue_at(r, NR);
        if (x >= 0) {
            if (x != issued) return false;                                                // in order
            if (x % NR != (r - 1 + NR) % NR || x % NR == r % NR) return false;           // (c)
            if (x - NR != r - 1) return false;                                            // (c)
            issue_iter[issued++] = r;
        }
    }
    for (int x = 0; x < nrounds; ++x)                                                     // (d)
        if (x >= issued || issue_iter[x] >= x) return false;
    return true;
}

constexpr bool replay_all(int NR) {
    for (int n = 0; n <= 72; ++n)
        if (!replay(NR, n)) return false;
    return true;
}

static_assert(replay_all(2) && replay_all(4), "ring schedule");

}  // namespace tmv_ring
