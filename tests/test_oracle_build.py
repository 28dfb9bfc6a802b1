"""Pins of the oracle's tree tensors (virtual root, ancestor table, invariant checks).

Independent evidence: transitive closure by boolean matrix powers and BFS depths on
brute-forced small trees (random node labels, so ids need not be topological), the
hand-derived table of the tiny workload, and the malformed-table fixtures."""
import itertools
import os

import numpy as np
import pytest

import tmv_inputs as ti

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def closure_and_depth(par, M):
    """Ancestor-or-self relation by repeated boolean products; depth by BFS from 0."""
    E = np.zeros((M + 1, M + 1), bool)          # E[i][j]: j is the parent of i
    for i in range(1, M + 1):
        E[i, par[i]] = True
    reach = np.eye(M + 1, dtype=bool)
    power = np.eye(M + 1, dtype=bool)
    for _ in range(M + 1):
        power = (power.astype(int) @ E.astype(int)) > 0
        reach |= power
    depth = {0: 0}
    frontier = [0]
    while frontier:
        nxt = []
        for u in frontier:
            for i in range(1, M + 1):
                if par[i] == u and i not in depth:
                    depth[i] = depth[u] + 1
                    nxt.append(i)
        frontier = nxt
    return reach, depth


def random_labelled_tree(rng, M, max_depth):
    base = ti.tree_random(rng, M, max_depth)
    perm = np.concatenate([[0], rng.permutation(M) + 1])     # relabel node i -> perm[i]
    par = np.zeros(M + 1, np.int32)
    for i in range(1, M + 1):
        par[perm[i]] = perm[base[i]]
    return par


def test_closure_and_depth_bruteforce(ref):
    rng = np.random.default_rng(7)
    for M in range(0, 9):
        for trial in range(25):
            par = random_labelled_tree(rng, M, max_depth=M if M else 1)
            D_max = 8
            padded = np.zeros((1, 9), np.int32)
            padded[0, : M + 1] = par
            anc, depth, st = ref.build_ancestors(padded, np.array([M]), 8, D_max)
            assert st[0] == ref.OK
            reach, bfs = closure_and_depth(par, M)
            for i in range(1, M + 1):
                assert depth[0, i] == bfs[i]
                row = anc[0, i]
                # entries: self, ancestors in order, then the root 0 repeated
                assert set(row[: depth[0, i]].tolist()) == {j for j in range(1, M + 1) if reach[i, j]}
                assert row[depth[0, i]] == 0 and np.all(row[depth[0, i]:] == 0)
                assert row[0] == i
                for kk in range(depth[0, i] - 1):
                    assert par[row[kk]] == row[kk + 1]
                assert np.all((row >= 0) & (row <= M))
            assert depth[0, 0] == 0 and np.all(anc[0, 0] == 0)
            assert np.all(anc[0, M + 1:] == 0) and np.all(depth[0, M + 1:] == 0)


def test_all_trees_up_to_five_nodes(ref):
    """Every parent table over {0..M} with M <= 5 (trees and non-trees): status OK iff the
    table is a tree, CYCLE otherwise (RANGE cannot occur: all values are in range)."""
    for M in range(1, 6):
        for choice in itertools.product(range(M + 1), repeat=M):
            par = np.array((0,) + choice, np.int32)
            ok = True
            for i in range(1, M + 1):
                seen, h = set(), i
                while h != 0 and h not in seen:
                    seen.add(h)
                    h = par[h]
                ok &= h == 0
            anc, depth, st = ref.build_ancestors(par[None, :], np.array([M]), M, M)
            assert st[0] == (ref.OK if ok else ref.ERR_CYCLE), (par, st)


def test_tiny_workload_golden(ref):
    rows = [l.split() for l in open(os.path.join(GOLD, "c1_tree_tensors.txt")) if l.strip() and l[0] != "#"]
    w = ti.workload(1)
    anc, depth, st = ref.build_ancestors(w.parents, w.n_nodes, w.M_max, w.D_max)
    assert st[0] == ref.OK
    for r in rows:
        node, parent, dep = int(r[0]), int(r[1]), int(r[2])
        assert w.parents[0, node] == parent or node == 0
        assert depth[0, node] == dep
        assert anc[0, node].tolist() == [int(x) for x in r[3:7]]
        mask = 0
        for kk in range(depth[0, node]):
            mask |= 1 << (int(anc[0, node, kk]) - 1)
        assert mask == int(r[7], 16)


def test_malformed_fixtures(ref):
    for line in open(os.path.join(GOLD, "malformed_trees.txt")):
        if not line.strip() or line[0] == "#":
            continue
        name, M, D, pars, valid, want = [f.strip() for f in line.split("|")]
        M, D, want = int(M), int(D), int(want)
        par = np.zeros((1, max(M, 1) + 1), np.int32)
        if M:
            par[0, 1:M + 1] = [int(x) for x in pars.split()]
        vmask = None
        if valid != "-":
            vmask = np.ones((1, max(M, 1) + 1), np.uint8)
            vmask[0, 1:M + 1] = [int(x) for x in valid.split()]
        anc, depth, st = ref.build_ancestors(par, np.array([M]), max(M, 1), D, valid=vmask)
        assert st[0] == want, name
        if want != ref.OK:
            assert np.all(anc == 0) and np.all(depth == 0), name
        assert np.all((anc >= 0) & (anc <= max(M, 0))), name


def test_neg1_format_equals_vroot(ref):
    rng = np.random.default_rng(3)
    B, M_max, D_max = 6, 12, 6
    vroot = np.zeros((B, M_max + 1), np.int32)
    neg1 = np.full((B, M_max), 0, np.int32)
    n = rng.integers(0, M_max + 1, size=B).astype(np.int32)
    for b in range(B):
        par = ti.tree_random(rng, int(n[b]), 6)
        vroot[b, : n[b] + 1] = par
        neg1[b, : n[b]] = par[1:] - 1           # 0-based ids, root sentinel -1
    a1, d1, s1 = ref.build_ancestors(vroot, n, M_max, D_max)
    a2, d2, s2 = ref.build_ancestors(neg1, n, M_max, D_max, parent_format=ref.PARENTS_NEG1)
    assert np.array_equal(a1, a2) and np.array_equal(d1, d2) and np.array_equal(s1, s2)
    bad = neg1.copy()
    bad[0, 0] = -2
    _, _, s3 = ref.build_ancestors(bad, np.maximum(n, 1), M_max, D_max, parent_format=ref.PARENTS_NEG1)
    assert s3[0] == ref.ERR_RANGE


def test_node_count_out_of_range(ref):
    par = np.zeros((2, 5), np.int32)
    par[1, 1:5] = [0, 1, 1, 2]
    anc, depth, st = ref.build_ancestors(par, np.array([5, -1]), 4, 4)
    assert st.tolist() == [ref.ERR_RANGE, ref.ERR_RANGE]
    assert np.all(anc == 0)


def test_per_sequence_isolation(ref):
    """A malformed sequence is inert and does not disturb its neighbours."""
    w = ti.workload(1)
    par = np.repeat(w.parents, 3, axis=0)
    par[1, 3] = 3                                       # self loop in sequence 1
    anc, depth, st = ref.build_ancestors(par, np.array([7, 7, 7]), 7, 3)
    assert st.tolist() == [ref.OK, ref.ERR_CYCLE, ref.OK]
    assert np.array_equal(anc[0], anc[2]) and np.all(anc[1] == 0)
