"""Pins of the oracle's sampling acceptance (modified rejection sampling on a tree).

Independent evidence:
  * Philox4x64-10 stream equals numpy.random.Philox (numpy's own implementation);
  * the integer accept test keeps exactly min(2^24, ceil(b/a)) of the 2^24 uniform codes,
    i.e. min(1, p/q) quantised to 2^-24 (modified rejection sampling section of the
    hierarchical speculative decoding blog), without wrapping at its full widths;
  * the inverse-CDF draw gives token x to exactly the codes in [ceil(C_{x-1} 2^32 / T),
    ceil(C_x 2^32 / T));
  * iterated refusals against one draft row stay in the threshold form (p - c q)+ that
    the oracle's integer state follows (exact rationals);
  * outcome frequencies over many streams match the exact rational outcome distribution
    (oracle/exact.py) -- chi-square;
  * the tree reading itself is lossless: with children drawn i.i.d. from q, the first
    emitted token follows p exactly (identity min(q,p) + max(0,p-q) = p)."""
import math
import zlib
from collections import Counter
from fractions import Fraction

import numpy as np
import pytest
from scipy import stats

import tmv_inputs as ti
from oracle import exact


def test_philox_matches_numpy(ref):
    for seed, stream in [(5, 0), (5, 3), (2**63 + 11, (7 << 32) | 31), (0, 0)]:
        ours = ref.philox_words(seed, stream, 37)
        theirs = np.random.Philox(key=np.array([seed, stream], np.uint64)).random_raw(37)
        assert np.array_equal(ours, theirs.astype(np.uint64))


def test_accept_threshold_closed_form(ref):
    """The integer test U * WQ(x) * T < R(x) * SQ * 2^24 keeps the codes U below
    min(2^24, ceil(b / a)), a = WQ(x) T, b = R(x) SQ 2^24, at the full widths it is used
    with (T < 2^111, R < 2^87, SQ < 2^55): no product may wrap."""
    rng = np.random.default_rng(31)
    cases = [(0, 2**31, 5, 2**31), (0, 2**31, 0, 2**31), (2**31, 2**62, 2**62, 2**31),
             (2**31, 2**110 - 1, 2**86, 2**55 - 1), (1, 2**110 - 1, 2**86, 1), (2**31, 1, 2**86, 2**55 - 1)]
    for _ in range(300):
        SQ = int(rng.integers(1, 2**55))
        T = int(rng.integers(1, 2**55)) * SQ + int(rng.integers(0, SQ))
        wq = int(rng.integers(0, 2**31 + 1))
        r = int(rng.integers(0, 2**62)) << int(rng.integers(0, 25))
        cases.append((wq, T, r, SQ))
    for wq, T, r, SQ in cases:
        a, b = wq * T, r * SQ * 2**24
        thr = (2**24 if b > 0 else 0) if a == 0 else min(2**24, -(-b // a))
        lo, hi = 0, 2**24                     # smallest U that is refused, by bisection
        while lo < hi:
            mid = (lo + hi) // 2
            if ref.sample_accept_test(mid, wq, T, r, SQ):
                lo = mid + 1
            else:
                hi = mid
        assert lo == thr, (wq, T, r, SQ)
        if thr > 0:
            assert ref.sample_accept_test(thr - 1, wq, T, r, SQ)
        if thr < 2**24:
            assert not ref.sample_accept_test(thr, wq, T, r, SQ)


def test_draw_boundaries_closed_form(ref):
    """Word w (high half h) draws the least x with C_x > floor(h T / 2^32): token x owns
    exactly the h in [ceil(C_{x-1} 2^32 / T), ceil(C_x 2^32 / T)), weights up to 2^100."""
    rng = np.random.default_rng(32)
    for _ in range(100):
        V = int(rng.integers(1, 7))
        scale = int(rng.integers(0, 61))
        w = [int(rng.integers(0, 2**40)) << scale for _ in range(V)]
        for i in range(V):
            if rng.random() < 0.3:
                w[i] = 0
        if sum(w) == 0:
            w[0] = 1
        T = sum(w)
        cum = np.cumsum(np.array(w, dtype=object))
        for x in range(V):
            start = -(-(int(cum[x - 1]) if x else 0) * 2**32 // T)
            end = -(-int(cum[x]) * 2**32 // T)
            if start == end:
                continue
            low = int(rng.integers(0, 2**32))
            assert ref.sample_draw(w, (start << 32) | low) == x
            assert ref.sample_draw(w, ((end - 1) << 32) | low) == x


def test_refusals_keep_the_threshold_form():
    """Refusing again and again against one draft row q: the residual after j refusals,
    iterated as max(0, r - q) normalised (exact rationals), equals (p - c_j q)+ normalised
    with c_0 = 0, c_{j+1} = c_j + sum (p - c_j q)+ -- the form the oracle's integer state
    (M, T) follows."""
    checked = 0
    for seed in range(40):
        rng = np.random.default_rng(seed)
        V = int(rng.integers(2, 8))
        p = [Fraction(int(x)) for x in rng.integers(0, 9, size=V)]
        q = [Fraction(int(x)) for x in rng.integers(0, 9, size=V)]
        if sum(p) == 0 or sum(q) == 0:
            continue
        p = [x / sum(p) for x in p]
        q = [x / sum(q) for x in q]
        cur, c = p, Fraction(0)
        for _ in range(6):
            nxt = exact._residual(cur, q)
            z = sum(max(Fraction(0), a - c * b) for a, b in zip(p, q))
            form = [max(Fraction(0), a - (c + z) * b) for a, b in zip(p, q)]
            if sum(form) == 0:                 # empty residual: the distribution is kept
                assert nxt == cur
                break
            assert nxt == [f / sum(form) for f in form]
            cur, c = nxt, c + z
            checked += 1
    assert checked > 60


def _tiny_tree_case(rng, V, overlap):
    # root 0 -> {1, 2, 3}; 1 -> {4, 5}; 2 -> {6}
    parents = np.array([0, 0, 0, 0, 1, 1, 2], np.int32)
    M = 6
    zp = rng.standard_normal((M + 1, V))
    zq = overlap * zp + math.sqrt(1 - overlap**2) * rng.standard_normal((M + 1, V))
    p = np.exp(zp) / np.exp(zp).sum(1, keepdims=True)
    q = np.exp(zq) / np.exp(zq).sum(1, keepdims=True)
    tokens = rng.integers(0, V, size=M + 1).astype(np.int32)
    return parents, M, p.astype(np.float32), q.astype(np.float32), tokens


@pytest.mark.parametrize("overlap,seed", [(0.9, 41), (0.3, 42), (0.97, 43)])
def test_outcome_frequencies_match_exact_model(ref, overlap, seed):
    rng = np.random.default_rng(seed)
    V = 4
    parents, M, p, q, tokens = _tiny_tree_case(rng, V, overlap)
    kids = ti.children_lists(parents, M)
    want = exact.outcome_distribution({u: p[u] for u in range(M + 1)}, {u: q[u] for u in range(M + 1)},
                                      kids, [int(t) for t in tokens])
    assert sum(want.values()) == 1
    B, steps = 50_000, 4
    P = np.repeat(parents[None], B, 0)
    n = np.full(B, M, np.int32)
    anc, depth, st = ref.build_ancestors(P, n, M, 3)
    counts = Counter()
    for step in range(steps):
        A, path, nxt, st2 = ref.accept_sample(np.repeat(tokens[None], B, 0), np.repeat(p[None], B, 0),
                                              np.repeat(q[None], B, 0), 1234, step, n, anc, depth, st)
        assert np.all(st2 == 0)
        for b in range(B):
            counts[(tuple(path[b, : A[b]].tolist()), int(nxt[b]))] += 1
    total = B * steps
    assert set(counts) <= set(want), set(counts) - set(want)
    keys = sorted(want, key=lambda k: -want[k])
    obs, exp_ = [], []
    rest_o, rest_e = 0, 0.0
    for kk in keys:
        e = float(want[kk]) * total
        if e >= 20:
            obs.append(counts[kk])
            exp_.append(e)
        else:
            rest_o += counts[kk]
            rest_e += e
    if rest_e > 0:
        obs.append(rest_o)
        exp_.append(rest_e)
    chi2 = sum((o - e) ** 2 / e for o, e in zip(obs, exp_))
    pval = stats.chi2.sf(chi2, len(obs) - 1)
    assert pval > 1e-4, (chi2, len(obs), pval)


@pytest.mark.parametrize("seed", [51, 52])
def test_repeated_refusals_match_exact_model(ref, seed):
    """A root with six children under a draft row far from the teacher's: most walks
    refuse several children in a row, so every outcome after the second refusal depends
    on how the residual state is carried from one refusal to the next."""
    rng = np.random.default_rng(seed)
    V, M = 4, 6
    parents = np.zeros(M + 1, np.int32)
    p = np.zeros((M + 1, V), np.float32)
    q = np.zeros((M + 1, V), np.float32)
    p[:] = rng.dirichlet(np.ones(V))
    p[0] = [0.05, 0.15, 0.3, 0.5]
    q[:] = 1.0 / V
    q[0] = [0.55, 0.3, 0.1, 0.05]
    tokens = np.array([0, 0, 1, 0, 1, 2, 0], np.int32)      # drafts mostly where q > p
    kids = ti.children_lists(parents, M)
    want = exact.outcome_distribution({u: p[u] for u in range(M + 1)}, {u: q[u] for u in range(M + 1)},
                                      kids, [int(t) for t in tokens])
    after_two = sum(v for (path, _), v in want.items() if not path or path[0] >= 3)
    assert after_two > 0.3                     # mass of walks that get past two refusals
    B, steps = 50_000, 4
    P = np.repeat(parents[None], B, 0)
    n = np.full(B, M, np.int32)
    anc, depth, st = ref.build_ancestors(P, n, M, 2)
    counts = Counter()
    for step in range(steps):
        A, path, nxt, st2 = ref.accept_sample(np.repeat(tokens[None], B, 0), np.repeat(p[None], B, 0),
                                              np.repeat(q[None], B, 0), 4321 + seed, step, n, anc, depth, st)
        assert np.all(st2 == 0)
        for b in range(B):
            counts[(tuple(path[b, : A[b]].tolist()), int(nxt[b]))] += 1
    total = B * steps
    assert set(counts) <= set(want), set(counts) - set(want)
    obs, exp_ = [], []
    rest_o, rest_e = 0, 0.0
    for kk in sorted(want, key=lambda k: -want[k]):
        e = float(want[kk]) * total
        if e >= 20:
            obs.append(counts[kk])
            exp_.append(e)
        else:
            rest_o += counts[kk]
            rest_e += e
    if rest_e > 0:
        obs.append(rest_o)
        exp_.append(rest_e)
    chi2 = sum((o - e) ** 2 / e for o, e in zip(obs, exp_))
    pval = stats.chi2.sf(chi2, len(obs) - 1)
    assert pval > 1e-4, (chi2, len(obs), pval)


def test_chain_acceptance_rate_and_residual(ref):
    """Single draft token: accepted with probability sum_x q(x) min(1, p(x)/q(x)) =
    sum min(p, q); after a refusal the correction follows max(0, p - q) normalised."""
    rng = np.random.default_rng(44)
    V = 5
    p = np.array([0.4, 0.3, 0.2, 0.1, 0.0], np.float32)
    qv = np.array([0.1, 0.1, 0.3, 0.3, 0.2], np.float32)
    B = 200_000
    parents = np.repeat(np.array([[0, 0]], np.int32), B, 0)
    tokens = np.zeros((B, 2), np.int32)
    tokens[:, 1] = rng.choice(V, size=B, p=qv / qv.sum())
    P = np.zeros((B, 2, V), np.float32)
    Q = np.zeros((B, 2, V), np.float32)
    P[:, 0] = p
    P[:, 1] = np.array([0, 0, 0, 0, 1], np.float32)       # bonus after an accept is token 4
    Q[:, 0] = qv
    Q[:, 1] = 1.0 / V
    n = np.ones(B, np.int32)
    anc, depth, st = ref.build_ancestors(parents, n, 1, 1)
    A, path, nxt, st2 = ref.accept_sample(tokens, P, Q, 9, 0, n, anc, depth, st)
    acc = A == 1
    expect_acc = float(np.minimum(p, qv).sum())
    assert abs(acc.mean() - expect_acc) < 5 * math.sqrt(expect_acc * (1 - expect_acc) / B)
    assert np.all(nxt[acc] == 4)
    emitted = np.where(acc, tokens[:, 1], nxt)
    freq = np.bincount(emitted, minlength=V) / B
    assert np.all(np.abs(freq - p) < 5 * np.sqrt(p * (1 - p) / B) + 1e-9)    # lossless
    res = np.maximum(p - qv, 0)
    res /= res.sum()
    cfreq = np.bincount(nxt[~acc], minlength=V) / max(1, (~acc).sum())
    assert np.all(np.abs(cfreq - res) < 0.01)


def test_tree_reading_is_lossless_exactly():
    V = 3

    def dist(ctx, salt):
        r = np.random.default_rng(zlib.crc32(repr((ctx, salt)).encode()))
        w = r.integers(0, 5, size=V)
        w[r.integers(0, V)] += 1
        return [Fraction(int(x)) for x in w]

    p_of = lambda ctx: dist(ctx, "p")
    q_of = lambda ctx: dist(ctx, "q")
    for shape in ([3, [2, 1, 0]], 2, [1, [[2, [1, 0]]]], [4, [0, 0, 0, 0]]):
        first, cond = exact.emitted_first_tokens(p_of, q_of, shape, V)
        p0 = p_of(())
        assert first == {x: p0[x] / sum(p0) for x in range(V) if p0[x]}
        for x, d in cond.items():
            px = p_of((x,))
            assert d == {y: px[y] / sum(px) for y in range(V) if px[y]}


def test_input_errors(ref):
    rng = np.random.default_rng(45)
    parents, n, tokens, p, q = ti.small_sampling_case(rng, 6, 5, 8, 3, overlap=0.8)
    anc, depth, st = ref.build_ancestors(parents, n, 5, 3)
    p = p.copy()
    q = q.copy()
    p[0, 0, 3] = -0.1                              # negative entry in the root row
    p[1, 0, 2] = np.nan
    kids = ti.children_lists(parents[2], 5)
    q[2, 0, :] = 0.0                               # root of sequence 2 has children
    tokens = tokens.copy()
    tokens[3, 1] = 8                               # out of range token
    st[4] = ref.ERR_CLOSURE
    A, path, nxt, st2 = ref.accept_sample(tokens, p, q, 3, 0, n, anc, depth, st)
    assert kids[0]
    assert st2.tolist()[:5] == [ref.ERR_INPUT] * 4 + [ref.ERR_CLOSURE]
    assert st2[5] == 0
    assert np.all(A[:5] == 0) and np.all(nxt[:5] == 0) and np.all(path[:5] == 0)


def test_unvisited_rows_are_not_checked(ref):
    parents = np.array([[0, 0, 1]], np.int32)
    V = 4
    p = np.zeros((1, 3, V), np.float32)
    q = np.zeros((1, 3, V), np.float32)
    p[0, 0] = [0, 0, 0, 1]           # teacher puts all mass on token 3
    q[0, 0] = [1, 0, 0, 0]           # draft proposes token 0 -> always refused
    p[0, 1] = np.nan                 # never visited
    tokens = np.array([[0, 0, 2]], np.int32)
    anc, depth, st = ref.build_ancestors(parents, np.array([2]), 2, 2)
    A, path, nxt, st2 = ref.accept_sample(tokens, p, q, 1, 0, np.array([2]), anc, depth, st)
    assert st2[0] == 0 and A[0] == 0 and nxt[0] == 3
