"""Pins of the oracle's best-first tree construction (BASTION summary, sections 1-3).

Independent evidence:
  * brute force on tiny vocabularies: every token tuple up to depth D is enumerated, its
    path score computed as the product of the positions' marginals, and the tuples
    sorted by (score descending, depth, rank tuple).  The first N of that order are
    exactly the N nodes best-first expansion adds, in the same order -- a parent always
    precedes its children in that order, so the top-N set is a prefix-closed tree and the
    greedy choice never misses it (the optimality claim of section 2);
  * scores in id order never increase, so the surrogate A(n) is concave (section 2);
  * the budget controller on hand-computed cases (section 3)."""
import itertools

import numpy as np
import pytest

import oracle as ref


def _ranks(row):
    """rank of each token: by value descending, then token ascending"""
    order = sorted(range(len(row)), key=lambda x: (-float(row[x]), x))
    rk = [0] * len(row)
    for r, x in enumerate(order):
        rk[x] = r
    return rk


def _brute_force(q, N):
    """the first N token tuples in (score desc, depth, rank tuple) order"""
    D, V = q.shape
    rks = [_ranks(q[k]) for k in range(D)]
    nodes = []
    for d in range(1, D + 1):
        for tup in itertools.product(range(V), repeat=d):
            s = 1.0
            for k, x in enumerate(tup):
                s = s * float(q[k][x])                 # fp64, in depth order
            nodes.append((-s, d, tuple(rks[k][x] for k, x in enumerate(tup)), tup, s))
    nodes.sort(key=lambda t: t[:3])
    return [(t[3], t[4]) for t in nodes[:N]]


def _paths(parents, tokens, n):
    """token tuple of every node 1..n from the parent pointers"""
    out = []
    for i in range(1, n + 1):
        tup, j = [], i
        while j != 0:
            tup.append(int(tokens[j]))
            j = int(parents[j])
        out.append(tuple(reversed(tup)))
    return out


@pytest.mark.parametrize("V,D,levels", [(1, 3, 4), (2, 3, 4), (3, 2, 3), (5, 2, 8), (4, 3, 2), (7, 1, 5)])
def test_matches_brute_force_order(V, D, levels):
    rng = np.random.default_rng(900 + 10 * V + D)
    total = sum(V ** d for d in range(1, D + 1))
    for trial in range(6):
        # values on a coarse grid, so equal scores (and the tie rule) come up often
        q = (rng.integers(0, levels + 1, size=(1, D, V)) / levels).astype(np.float32)
        for N in sorted({1, 2, min(total, 5), min(total, 12), min(total, 128)}):
            parents, tokens, n, rho, st = ref.tree_best_first(q, N)
            assert st[0] == 0 and n[0] == min(N, total)
            want = _brute_force(q[0], int(n[0]))
            got = _paths(parents[0], tokens[0], int(n[0]))
            assert got == [t for t, _ in want], (V, D, N, trial)
            assert [float(x) for x in rho[0, 1:n[0] + 1]] == [s for _, s in want]
            assert all(parents[0, i] < i for i in range(1, n[0] + 1))          # ids in pop order


def test_scores_never_increase_and_tree_is_prefix_closed():
    rng = np.random.default_rng(910)
    D, V, N = 5, 300, 128
    z = rng.standard_normal((3, D, V)) * 2.0
    q = (np.exp(z) / np.exp(z).sum(-1, keepdims=True)).astype(np.float32)
    parents, tokens, n, rho, st = ref.tree_best_first(q, N)
    assert np.all(st == 0) and np.all(n == N)
    for b in range(3):
        r = rho[b, 1:N + 1]
        assert np.all(np.diff(r) <= 0)                        # concave surrogate
        for i in range(1, N + 1):
            p = parents[b, i]
            assert 0 <= p < i and (p == 0 or rho[b, p] >= rho[b, i])


def test_budget_controller_hand_cases():
    # one position, q = (1/2, 1/4, 1/8, 1/8): scores 1/2, 1/4, 1/8, 1/8 (token 2 before 3),
    # A(n) = 1/2, 3/4, 7/8, 1
    q = np.array([[[0.5, 0.25, 0.125, 0.125]]], np.float32)
    # L_AR = 2, C = (1, 1.2, 1.5, 1.6): S = 1, 1.25, 1.1667, 1.25 -> stops at the first fall, n* = 2
    _, tokens, n, rho, _ = ref.tree_best_first(q, 4, cost=np.array([1.0, 1.2, 1.5, 1.6]), l_ar=2.0)
    assert n[0] == 2 and tokens[0].tolist() == [0, 0, 1, 0, 0] and rho[0, 3] == 0.0
    # flat cost: S rises all the way, every node is kept
    _, tokens, n, _, _ = ref.tree_best_first(q, 4, cost=np.ones(4), l_ar=2.0)
    assert n[0] == 4 and tokens[0].tolist() == [0, 0, 1, 2, 3]
    # steep cost: S(2) = 0.75 * 2 / 3 = 0.5 < S(1) = 1: only the best node
    _, _, n, _, _ = ref.tree_best_first(q, 4, cost=np.array([1.0, 3.0, 3.0, 3.0]), l_ar=2.0)
    assert n[0] == 1
    # without a cost table the budget is fixed
    _, _, n, _, _ = ref.tree_best_first(q, 3)
    assert n[0] == 3


def test_input_errors_and_failed_sequences():
    q = np.full((4, 2, 6), 1.0 / 6, np.float32)
    q[0, 1, 3] = -0.5
    q[1, 0, 0] = np.nan
    q[2, 1, 5] = 1.5
    st = np.array([0, 0, 0, 3], np.int32)
    parents, tokens, n, rho, st2 = ref.tree_best_first(q, 8, status=st)
    assert st2.tolist() == [ref.ERR_INPUT] * 3 + [3]
    assert np.all(n == 0) and np.all(parents == 0) and np.all(tokens == 0) and np.all(rho[:, 1:] == 0)
