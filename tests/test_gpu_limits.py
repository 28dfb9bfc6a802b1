"""Device parity at the largest trees the library accepts (M_max = D_max = 128): a
128-deep chain, a 128-child star and an empty tree side by side, through every stage
that depends on the tree's size -- ancestor tables, attention masks up to tree slot 127,
greedy paths deeper than the entries kept on chip, and sampling walks that consume a
random word per node."""
import numpy as np
import pytest
import torch

import tmv_inputs as ti
from tests.harness import DeviceStep, oracle_tables
from tests.test_gpu_accept import _greedy_parity, _sample_parity
from tests.test_gpu_parity import _attention_parity, small_attention_workload

pytestmark = pytest.mark.gpu

M_MAX = 128


def _case(name):
    print("\n[gpu case] %s" % name, flush=True)


def _max_trees():
    """Rows of a [3][M_MAX+1] parents table: chain of 128, star of 128, empty."""
    parents = np.zeros((3, M_MAX + 1), np.int32)
    parents[0] = ti.tree_chain(M_MAX)
    return parents, np.array([M_MAX, M_MAX, 0], np.int32)


def test_build_ancestors_128_deep(ref):
    _case("build: 128-deep chain, 128-child star, empty tree; D_max 128 and 127")
    parents, n = _max_trees()
    for D_max in (128, 127):
        w = ti.Workload("limits", ti.F32, 3, 1, 1, 64, M_MAX, D_max, 1, 1, "greedy", parents, n, n * 0, n * 0)
        dev = DeviceStep(w)
        dev.build()
        a, d, s = dev.tables()
        ra, rd, rs = oracle_tables(ref, w)
        assert np.array_equal(s, rs) and np.array_equal(a, ra) and np.array_equal(d, rd)
        assert s.tolist() == ([0, 0, 0] if D_max == 128 else [ref.ERR_DEPTH, 0, 0])


@pytest.mark.parametrize("d", [128, 64])
def test_attention_128_node_trees(ref, d):
    _case("attention: 128-deep chain / 128-child star / empty tree, d=%d" % d)
    parents, n = _max_trees()
    w = small_attention_workload(700 + d, 3, 8, 2, d, M_MAX, [40, 0, 20], n.tolist(), q_scale=4.0, max_depth=M_MAX,
                                 labelled=False)
    w.parents[:] = parents
    assert int(oracle_tables(ref, w)[1].max()) == M_MAX
    _attention_parity(ref, w, 2e-2, 1e-2)


def test_greedy_paths_beyond_eight(ref):
    """Two 128-deep chains whose draft tokens match the teacher's argmax down to depth 128
    and 99: the accepted paths are longer than the ancestor entries the select kernel
    keeps on chip, so their tails come from the ancestor table."""
    _case("greedy: accepted paths of depth 128 and 99")
    rng = np.random.default_rng(710)
    B, V = 3, 1000
    parents = np.zeros((B, M_MAX + 1), np.int32)
    parents[0] = ti.tree_chain(M_MAX)
    parents[1] = ti.tree_chain(M_MAX)
    n = np.array([M_MAX, M_MAX, 0], np.int32)
    logits = rng.standard_normal((B, M_MAX + 1, V)).astype(np.float32)
    tokens = np.zeros((B, M_MAX + 1), np.int32)
    for b in range(2):
        for c in range(1, M_MAX + 1):
            tokens[b, c] = int(np.argmax(logits[b, c - 1]))
    tokens[1, 100] = (tokens[1, 100] + 1) % V                 # first mismatch at depth 100
    w = ti.Workload("greedy-limits", ti.F32, B, 0, 1, 64, M_MAX, M_MAX, 1, V, "greedy", parents, n,
                    np.zeros(B, np.int32), tokens, logits=logits)
    A, st = _greedy_parity(ref, w)
    assert st.tolist() == [0, 0, 0] and A.tolist() == [128, 99, 0]


def test_sampling_128_deep_and_128_children(ref):
    """A 128-deep chain whose teacher and draft rows agree (every node accepted: 128 words
    and one bonus draw) and a 128-child star whose draft row is far from the teacher's
    (a long run of refusals against one draft row)."""
    _case("sampling: 128-deep accepted chain and 128-child star")
    rng = np.random.default_rng(720)
    B, V = 2, 5000
    parents = np.zeros((B, M_MAX + 1), np.int32)
    parents[0] = ti.tree_chain(M_MAX)
    n = np.array([M_MAX, M_MAX], np.int32)
    zp = rng.standard_normal((B, M_MAX + 1, V)) * 2.0
    zq = rng.standard_normal((B, M_MAX + 1, V)) * 2.0
    p = np.exp(zp) / np.exp(zp).sum(-1, keepdims=True)
    q = np.exp(zq) / np.exp(zq).sum(-1, keepdims=True)
    q[0] = p[0]                                               # chain: q == p, always accepted
    p, q = p.astype(np.float32), q.astype(np.float32)
    tokens = np.zeros((B, M_MAX + 1), np.int32)
    for c in range(1, M_MAX + 1):
        tokens[0, c] = int(np.argmax(q[0, c - 1]))
        tokens[1, c] = int(np.argmax(q[1, 0]) + c) % V        # star: mostly low-p tokens
    A, st = _sample_parity(ref, parents, n, tokens, p, q, 11, 0, M_MAX)
    assert st.tolist() == [0, 0] and A[0] == 128
