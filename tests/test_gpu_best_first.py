"""Device parity of tree_best_first (BASTION summary, sections 1-3) against the oracle.

Parents, tokens, node counts and status must be bit-identical, and the fp64 path
scores too: both sides form them as the same fp64 products in depth order."""
import numpy as np
import pytest
import torch

import tmv_inputs as ti

pytestmark = pytest.mark.gpu


def _case(name):
    print("\n[gpu case] %s" % name, flush=True)


def _device_best_first(q, N, cost=None, l_ar=1.0, status=None):
    import tree_masked_verification_amd as tmv
    B, D, V = q.shape
    qd = torch.from_numpy(q).cuda()
    parents = torch.full((B, N + 1), -7, dtype=torch.int32, device="cuda")
    tokens = torch.full((B, N + 1), -7, dtype=torch.int32, device="cuda")
    n = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    rho = torch.full((B, N + 1), float("nan"), dtype=torch.float64, device="cuda")
    st = torch.from_numpy(np.zeros(B, np.int32) if status is None else status.copy()).cuda()
    cd = None if cost is None else torch.from_numpy(np.asarray(cost, np.float64)).cuda()
    tmv.tree_best_first(qd, N, parents, tokens, n, rho, st, cost=cd, l_ar=l_ar)
    torch.cuda.synchronize()
    return tuple(t.cpu().numpy() for t in (parents, tokens, n, rho, st))


def _parity(ref, q, N, cost=None, l_ar=1.0, status=None):
    got = _device_best_first(q, N, cost, l_ar, status)
    want = ref.tree_best_first(q, N, cost=cost, l_ar=l_ar, status=status)
    for g, w, name in zip(got, want, ("parents", "tokens", "n_nodes", "rho", "status")):
        assert np.array_equal(g, w), (name, g, w)
    return got


@pytest.mark.parametrize("D,V,N,levels", [(1, 5, 7, 4), (3, 100, 64, 6), (8, 20000, 128, None), (2, 50, 128, 3),
                                          (4, 40000, 96, None), (8, 7, 128, 2), (3, 20000, 128, 3),
                                          (2, 200000, 128, None), (1, 262144, 128, 5)])
def test_random_marginals(ref, D, V, N, levels):
    """Shapes across the limits: fewer tokens than the budget (V = 5, 50, 7), several
    32768-entry segments per row (V = 40000, 200000, up to the 262144 maximum, whose rows
    merge more keys than the merge holds one per thread), coarse values with many equal
    scores (V = 20000 with 4 levels: more candidates per segment than one per thread)."""
    _case("best-first: D=%d V=%d N=%d levels=%s" % (D, V, N, levels))
    rng = np.random.default_rng(1200 + D * 7 + V)
    q = ti.draft_marginals(rng, 6, D, V, sigma=2.0, levels=levels)
    parents, tokens, n, rho, st = _parity(ref, q, N)
    assert np.all(st == 0) and np.all(n == min(N, sum(min(V, N) ** d for d in range(1, D + 1))))


def test_workload3_shape(ref):
    """Workload 3's drafter shape: 16 sequences, 8 positions, 128256 tokens, budget 128."""
    _case("best-first: B16 D8 V128256 N128")
    rng = np.random.default_rng(1300)
    q = ti.draft_marginals(rng, 16, 8, 128256, sigma=3.0)
    parents, tokens, n, rho, st = _parity(ref, q, 128)
    assert np.all(st == 0) and np.all(n == 128) and np.all(parents[:, 1:] < np.arange(1, 129))


def test_budget_controller(ref):
    """A cost table: affine cost per node, so S(n) rises while the marginal score exceeds
    the marginal cost and stops at different sizes for different sequences."""
    _case("best-first: controller with a cost table")
    rng = np.random.default_rng(1310)
    q = ti.draft_marginals(rng, 8, 6, 3000, sigma=np.linspace(0.5, 4.0, 8)[:, None, None] * np.ones((1, 1, 1)))
    cost = 20.0 + 0.35 * np.arange(1, 129)
    parents, tokens, n, rho, st = _parity(ref, q, 128, cost=cost, l_ar=12.0)
    assert np.all(st == 0) and len(set(n.tolist())) > 1 and np.all(n >= 1)


def test_errors_and_failed_sequences(ref):
    _case("best-first: malformed rows and failed sequences")
    rng = np.random.default_rng(1320)
    q = ti.draft_marginals(rng, 5, 3, 300, sigma=2.0)
    q[0, 2, 17] = -1e-3
    q[1, 0, 299] = np.nan
    q[2, 1, 0] = 1.25
    st_in = np.array([0, 0, 0, 5, 0], np.int32)
    parents, tokens, n, rho, st = _parity(ref, q, 32, status=st_in)
    assert st.tolist() == [6, 6, 6, 5, 0] and n.tolist() == [0, 0, 0, 0, 32]


def test_negative_zero_marginals(ref):
    """-0.0 is a valid probability equal to 0: it ranks with the zeros, ties broken by
    token, exactly as the oracle's comparisons do."""
    _case("best-first: marginals with -0.0 entries")
    rng = np.random.default_rng(1400)
    q = ti.draft_marginals(rng, 3, 3, 300, sigma=2.0, levels=4)
    # most entries are zero, half of them -0.0, so the tree needs zero-scored nodes and
    # their order (by token) mixes both signs
    zeros = rng.random(q.shape) < 0.99
    neg = rng.random(q.shape) < 0.5
    q[zeros & neg] = -0.0
    q[zeros & ~neg] = 0.0
    assert np.signbit(q).any()
    parents, tokens, n, rho, st = _parity(ref, q, 96)
    assert np.all(st == 0)
