"""Pins of the oracle's greedy acceptance (deepest matching path).

Independent evidence: enumeration of every root->node path with numpy's argmax (first
maximum = smallest index) on small random trees with forced ties; the expected-tokens
closed form E[N] = (1 - a^(g+1)) / (1 - a) of the hierarchical speculative decoding
blog (section on acceptance rate and cost ratio), by Monte Carlo on planted chains."""
import numpy as np

import tmv_inputs as ti
from tests.test_oracle_build import random_labelled_tree


def brute_force(par, M, tokens, logits, D_max):
    t = {u: int(np.argmax(logits[u])) for u in range(M + 1)}
    best, best_depth = 0, 0
    for i in range(1, M + 1):
        path, h = [], i
        while h:
            path.append(h)
            h = int(par[h])
        path = path[::-1]
        ok = all(tokens[c] == t[int(par[c])] for c in path)
        if ok and (len(path) > best_depth or (len(path) == best_depth and i < best)):
            best, best_depth = i, len(path)
    path, h = [], best
    while h:
        path.append(h)
        h = int(par[h])
    path = path[::-1] + [0] * (D_max - len(path))
    return best_depth, path, t[best]


def test_enumeration_small_trees_with_ties(ref):
    rng = np.random.default_rng(21)
    B, M_max, D_max, V = 64, 9, 9, 5
    parents = np.zeros((B, M_max + 1), np.int32)
    n = rng.integers(0, M_max + 1, size=B).astype(np.int32)
    for b in range(B):
        parents[b, : n[b] + 1] = random_labelled_tree(rng, int(n[b]), max_depth=6)
    logits = rng.integers(0, 3, size=(B, M_max + 1, V)).astype(np.float32)   # many ties
    tokens = rng.integers(0, V, size=(B, M_max + 1)).astype(np.int32)
    anc, depth, st = ref.build_ancestors(parents, n, M_max, D_max)
    A, path, nxt, st2 = ref.accept_greedy(tokens, logits, n, anc, depth, st)
    assert np.all(st2 == 0)
    hits = 0
    for b in range(B):
        a, pth, x = brute_force(parents[b], int(n[b]), tokens[b], logits[b], D_max)
        assert (A[b], path[b].tolist(), nxt[b]) == (a, pth, x), b
        hits += a > 0
    assert hits > 10


def test_distinct_siblings_equal_root_walk(ref):
    """With distinct sibling tokens at most one child can match, so the deepest matching
    node is the end of the walk that follows the unique matching child."""
    rng = np.random.default_rng(22)
    w = ti.workload(1)
    for trial in range(30):
        w = ti.workload(1, seed=5000 + trial)
        anc, depth, st = ref.build_ancestors(w.parents, w.n_nodes, w.M_max, w.D_max)
        A, path, nxt, _ = ref.accept_greedy(w.tokens, w.logits, w.n_nodes, anc, depth, st)
        kids = ti.children_lists(w.parents[0], 7)
        u, walk = 0, []
        while True:
            t = int(np.argmax(w.logits[0, u]))
            nxt_u = [c for c in kids[u] if w.tokens[0, c] == t]
            if not nxt_u:
                break
            u = nxt_u[0]
            walk.append(u)
        assert A[0] == len(walk) and path[0, : A[0]].tolist() == walk
        assert nxt[0] == int(np.argmax(w.logits[0, u]))


def test_expected_tokens_closed_form(ref):
    """Planted chains of gamma nodes, each matching independently with probability
    alpha: mean emitted tokens A + 1 must follow (1 - alpha^(gamma+1)) / (1 - alpha)."""
    rng = np.random.default_rng(23)
    B, gamma, V = 100_000, 6, 16
    for alpha in (0.3, 0.7, 0.9):
        parents = np.repeat(ti.tree_chain(gamma)[None, :], B, axis=0)
        logits = np.zeros((B, gamma + 1, V), np.float32)
        choice = rng.integers(0, V, size=(B, gamma + 1))
        logits[np.arange(B)[:, None], np.arange(gamma + 1)[None, :], choice] = 1.0
        other = (choice + 1 + rng.integers(0, V - 1, size=choice.shape)) % V     # != choice
        hit = rng.random((B, gamma + 1)) < alpha
        tokens = np.zeros((B, gamma + 1), np.int32)
        tokens[:, 1:] = np.where(hit[:, :-1], choice[:, :-1], other[:, :-1])      # node i vs row i-1
        n = np.full(B, gamma, np.int32)
        anc, depth, st = ref.build_ancestors(parents, n, gamma, gamma)
        A, path, nxt, st2 = ref.accept_greedy(tokens, logits, n, anc, depth, st)
        mean = float(np.mean(A + 1))
        expect = (1 - alpha ** (gamma + 1)) / (1 - alpha)
        sem = float(np.std(A + 1)) / np.sqrt(B)
        assert abs(mean - expect) < 5 * sem + 1e-9, (alpha, mean, expect)
        assert np.array_equal(nxt, choice[np.arange(B), A])


def test_input_errors_and_inert(ref):
    w = ti.workload(1)
    B = 4
    parents = np.repeat(w.parents, B, axis=0)
    logits = np.repeat(w.logits, B, axis=0)
    tokens = np.repeat(w.tokens, B, axis=0)
    logits[1, 3, 7] = np.nan                     # NaN in a scanned row
    tokens[2, 5] = 32                            # token outside [0, V)
    n = np.full(B, 7, np.int32)
    anc, depth, st = ref.build_ancestors(parents, n, 7, 3)
    st[3] = ref.ERR_DEPTH                        # upstream failure
    A, path, nxt, st2 = ref.accept_greedy(tokens, logits, n, anc, depth, st)
    assert st2.tolist() == [0, ref.ERR_INPUT, ref.ERR_INPUT, ref.ERR_DEPTH]
    assert np.all(A[1:] == 0) and np.all(path[1:] == 0) and np.all(nxt[1:] == 0)


def test_bf16_rows_widen_exactly(ref):
    w = ti.workload(1)
    lb = ti.bf16_bits(w.logits)
    anc, depth, st = ref.build_ancestors(w.parents, w.n_nodes, 7, 3)
    r1 = ref.accept_greedy(w.tokens, lb, w.n_nodes, anc, depth, st, row_dtype=ref.BF16)
    r2 = ref.accept_greedy(w.tokens, ti.bf16_to_f32(lb), w.n_nodes, anc, depth, st)
    for a, b in zip(r1, r2):
        assert np.array_equal(a, b)


def test_empty_tree_emits_root_choice(ref):
    logits = np.array([[[0.0, 3.0, 3.0, 1.0]]], np.float32)
    anc, depth, st = ref.build_ancestors(np.zeros((1, 1), np.int32), np.array([0]), 0, 0)
    A, path, nxt, st2 = ref.accept_greedy(np.zeros((1, 1), np.int32), logits, np.array([0]), anc, depth, st)
    assert A[0] == 0 and nxt[0] == 1 and st2[0] == 0 and path.shape == (1, 0)


def signed_zero_rows(rng, B, M_max, V):
    """Chains whose rows are all negative except a -0.0 and a +0.0 at random places (either
    order): the row maximum is zero twice, and -0 == +0 makes the first of the two the
    argmax.  Each child carries that first position with probability 0.8."""
    logits = -rng.uniform(0.5, 2.0, size=(B, M_max + 1, V)).astype(np.float32)
    parents = np.zeros((B, M_max + 1), np.int32)
    parents[:, 1:] = np.arange(M_max)[None, :]
    tokens = np.zeros((B, M_max + 1), np.int32)
    first = np.zeros((B, M_max + 1), np.int64)
    for b in range(B):
        for u in range(M_max + 1):
            p1, p2 = rng.choice(V, size=2, replace=False)
            logits[b, u, p1], logits[b, u, p2] = (-0.0, 0.0) if rng.random() < 0.5 else (0.0, -0.0)
            first[b, u] = min(p1, p2)
        for c in range(1, M_max + 1):
            tokens[b, c] = first[b, c - 1] if rng.random() < 0.8 else (first[b, c - 1] + 1) % V
    return parents, tokens, logits, first


def test_signed_zeros_tie_to_first_index(ref):
    rng = np.random.default_rng(23)
    B, M_max, V = 12, 8, 300
    parents, tokens, logits, first = signed_zero_rows(rng, B, M_max, V)
    assert np.array_equal(np.argmax(logits, axis=2), first)          # numpy: -0 == +0
    n = np.full(B, M_max, np.int32)
    anc, depth, st = ref.build_ancestors(parents, n, M_max, M_max)
    A, path, nxt, st2 = ref.accept_greedy(tokens, logits, n, anc, depth, st)
    assert np.all(st2 == 0)
    for b in range(B):
        assert (A[b], path[b].tolist(), nxt[b]) == brute_force(parents[b], M_max, tokens[b], logits[b], M_max)
    assert np.any(A > 1)
