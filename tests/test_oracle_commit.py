"""Pins of the oracle's prefix-sharing path-index commit.

Independent evidence: the committed layout is checked row by row against a copy of the
pre-commit cache (prefix rows identical, new rows are the accepted path's rows in depth
order, everything else unchanged); a chain that is fully accepted moves nothing (the
length-based commit of section 2.1 of the Chinese EAGLE-Pangu summary); a query attending
over the committed length equals causal attention over prefix + path (torch SDPA)."""
import numpy as np
import torch

import oracle
import tmv_inputs as ti
from tests.test_oracle_build import random_labelled_tree


def _path_nodes(par, leaf):
    out = []
    while leaf:
        out.append(leaf)
        leaf = int(par[leaf])
    return out[::-1]


def test_layout_after_commit(ref):
    rng = np.random.default_rng(51)
    nl, B, Hkv, d, M_max, D_max = 3, 5, 2, 8, 10, 10
    P = rng.integers(0, 12, size=B).astype(np.int32)
    n = rng.integers(0, M_max + 1, size=B).astype(np.int32)
    L_cap = int((P + n).max()) + 2
    parents = np.zeros((B, M_max + 1), np.int32)
    leaves = []
    for b in range(B):
        parents[b, : n[b] + 1] = random_labelled_tree(rng, int(n[b]), 8)     # ids not topological
        leaves.append(int(rng.integers(0, n[b] + 1)))
    anc, depth, st = ref.build_ancestors(parents, n, M_max, D_max)
    A = np.zeros(B, np.int32)
    path = np.zeros((B, D_max), np.int32)
    for b in range(B):
        pn = _path_nodes(parents[b], leaves[b])
        A[b] = len(pn)
        path[b, : len(pn)] = pn
    for dt in (np.float32, np.uint16):
        k = (rng.standard_normal((nl, B, Hkv, L_cap, d)) * 100).astype(dt)
        v = (rng.standard_normal((nl, B, Hkv, L_cap, d)) * 100).astype(dt)
        k0, v0 = k.copy(), v.copy()
        new_len, st2 = ref.commit(k, v, P, n, A, path, st, M_max)
        assert np.all(st2 == 0) and np.array_equal(new_len, P + A)
        for b in range(B):
            for cache, before in ((k, k0), (v, v0)):
                assert np.array_equal(cache[:, b, :, : P[b]], before[:, b, :, : P[b]])
                for j in range(A[b]):
                    assert np.array_equal(cache[:, b, :, P[b] + j], before[:, b, :, P[b] + path[b, j] - 1])
                assert np.array_equal(cache[:, b, :, P[b] + A[b]:], before[:, b, :, P[b] + A[b]:])


def test_overlapping_sources_use_snapshot(ref):
    # node 3 at depth 1, node 1 at depth 2: dst P+0 <- src P+2, dst P+1 <- src P+0
    k = np.arange(1 * 1 * 1 * 6 * 2, dtype=np.float32).reshape(1, 1, 1, 6, 2)
    v = -k
    k0 = k.copy()
    new_len, st = ref.commit(k, v, np.array([2]), np.array([3]), np.array([2]), np.array([[3, 1, 0]]),
                             np.zeros(1, np.int32), 3)
    assert new_len[0] == 4 and st[0] == 0
    assert np.array_equal(k[0, 0, 0, 2], k0[0, 0, 0, 4]) and np.array_equal(k[0, 0, 0, 3], k0[0, 0, 0, 2])
    assert np.array_equal(v[0, 0, 0, 3], -k0[0, 0, 0, 2])


def test_full_chain_accept_moves_nothing(ref):
    rng = np.random.default_rng(52)
    M = 7
    k = rng.standard_normal((2, 1, 3, 20, 4)).astype(np.float32)
    v = rng.standard_normal((2, 1, 3, 20, 4)).astype(np.float32)
    k0, v0 = k.copy(), v.copy()
    path = np.arange(1, M + 1, dtype=np.int32)[None]
    new_len, st = ref.commit(k, v, np.array([9]), np.array([M]), np.array([M]), path, np.zeros(1, np.int32), M)
    assert new_len[0] == 16 and np.array_equal(k, k0) and np.array_equal(v, v0)


def test_failed_or_misfit_sequences_move_nothing(ref):
    rng = np.random.default_rng(53)
    k = rng.standard_normal((1, 4, 1, 12, 4)).astype(np.float32)
    v = k * 2
    k0 = k.copy()
    path = np.array([[2, 0], [2, 0], [5, 0], [1, 2]], np.int32)
    st_in = np.array([ref.ERR_CYCLE, 0, 0, 0], np.int32)
    # seq 1: prefix 9 + 4 nodes > L_cap 12; seq 2: path entry 5 > M 3; seq 3 fine
    new_len, st = ref.commit(k, v, np.array([3, 9, 3, 3]), np.array([3, 4, 3, 3]), np.array([1, 1, 1, 2]),
                             path, st_in, 3)
    assert st.tolist() == [ref.ERR_CYCLE, ref.ERR_INPUT, ref.ERR_INPUT, 0]
    assert new_len.tolist() == [3, 9, 3, 5]
    assert np.array_equal(k[:, :3], k0[:, :3])


def test_attention_over_committed_length(ref):
    """After the commit, a fresh query over the first new_len rows sees exactly the
    prefix followed by the accepted path in depth order."""
    rng = np.random.default_rng(54)
    M, P, d = 9, 5, 8
    par = random_labelled_tree(rng, M, 5)
    leaf = max(range(1, M + 1), key=lambda i: len(_path_nodes(par, i)))
    pn = _path_nodes(par, leaf)
    k = rng.standard_normal((1, 1, 1, P + M, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, 1, P + M, d)).astype(np.float32)
    k0, v0 = k.copy(), v.copy()
    path = np.zeros((1, M), np.int32)
    path[0, : len(pn)] = pn
    new_len, _ = ref.commit(k, v, np.array([P]), np.array([M]), np.array([len(pn)]), path, np.zeros(1, np.int32), M)
    qv = torch.tensor(rng.standard_normal((1, 1, 1, d)))
    L = int(new_len[0])
    t64 = lambda a: torch.tensor(a, dtype=torch.float64)[None, None]
    after = torch.nn.functional.scaled_dot_product_attention(qv, t64(k[0, 0, 0, :L]), t64(v[0, 0, 0, :L]))
    slots = list(range(P)) + [P + j - 1 for j in pn]
    before = torch.nn.functional.scaled_dot_product_attention(qv, t64(k0[0, 0, 0][slots]), t64(v0[0, 0, 0][slots]))
    assert torch.equal(after, before)


def test_block_eviction_hand_cases():
    """Block eviction after a paged commit (runtime-memory question of the hierarchical
    speculative decoding blog): blocks of the tree wholly past the new length are freed."""
    table = np.array([[10, 11, 12, 13, 14]], np.int32)
    # page 4, prefix 6, 7 tree slots (6..12), 2 accepted -> new length 8: blocks 2 and 3 go
    t2, freed = oracle.commit_paged_table(table, 4, 100, [6], [7], [8], [0])
    assert t2.tolist() == [[10, 11, -1, -1, 14]] and freed == [12, 13]
    # one accepted: block 1 (slots 4..7) still holds slot 6, so it stays
    t2, freed = oracle.commit_paged_table(table, 4, 100, [6], [7], [7], [0])
    assert t2.tolist() == [[10, 11, -1, -1, 14]] and freed == [12, 13]
    # none accepted: block 1 also holds prefix slots 4 and 5, so it stays
    t2, freed = oracle.commit_paged_table(table, 4, 100, [6], [7], [6], [0])
    assert t2.tolist() == [[10, 11, -1, -1, 14]] and freed == [12, 13]
    # a fully accepted chain keeps everything; a failed sequence is left alone
    t2, freed = oracle.commit_paged_table(table, 4, 100, [6], [7], [13], [0])
    assert t2.tolist() == table.tolist() and freed == []
    t2, freed = oracle.commit_paged_table(table, 4, 100, [6], [7], [6], [oracle.ERR_INPUT])
    assert t2.tolist() == table.tolist() and freed == []
    # invalid entries are skipped, page-aligned new length frees the following block
    t2, freed = oracle.commit_paged_table(np.array([[1, 2, -1, 300, 5]], np.int32), 4, 100, [4], [16], [8], [0])
    assert t2.tolist() == [[1, 2, -1, 300, -1]] and freed == [5]


def test_block_eviction_invariants():
    rng = np.random.default_rng(91)
    for _ in range(300):
        ps = int(rng.choice([1, 2, 4, 8, 16]))
        P = int(rng.integers(0, 40))
        M = int(rng.integers(0, 30))
        A = int(rng.integers(0, M + 1))
        nb = (P + M + ps - 1) // ps + 2
        table = rng.permutation(1000)[:nb].astype(np.int32)[None]
        t2, freed = oracle.commit_paged_table(table, ps, 1000, [P], [M], [P + A], [0])
        for i in range(nb):
            evicted = t2[0, i] == -1
            start = i * ps
            # evicted exactly when the block starts at or past the new length inside the tree
            assert evicted == (start >= P + A and start < P + M)
        assert sorted(table[0][t2[0] == -1].tolist()) == freed
