"""Device parity of greedy acceptance from the LM head (argmax fused into the LM-head
product; roofline section of "Speculative Decoding Hierarquico").  The device takes the
argmax of fp32-accumulated logits, the oracle computes them in fp64: a device choice x^ of
row u is accepted iff logit64[x^] >= logit64[x*] - (eps[x^] + eps[x*]), eps = K 2^-24
sum_k |h w| (the accumulation bound pinned in test_oracle_lm_head), and it must equal the
oracle's x* wherever the top two differ by more than their two bounds.  The path rule is
then checked bit-exactly against the oracle's greedy rule on the device's choices, and
against the pure oracle where every live row's choice is unambiguous."""
import numpy as np
import pytest
import torch

import oracle
import tmv_inputs as ti
from tests.harness import dev_tensor, host_bits

pytestmark = pytest.mark.gpu


def _case(name):
    print("\n[gpu case] %s" % name, flush=True)


def _tables(parents, n_nodes, M_max, D_max):
    return oracle.build_ancestors(parents, n_nodes, M_max, D_max)


def _run(hidden_bits, w_bits, parents, n_nodes, tokens, M_max, D_max, ws=None):
    import tree_masked_verification_amd as tmv
    B = hidden_bits.shape[0]
    hid = dev_tensor(hidden_bits, True)
    W = dev_tensor(w_bits, True)
    par = dev_tensor(parents.astype(np.int32))
    nn = dev_tensor(n_nodes.astype(np.int32))
    tok = dev_tensor(tokens.astype(np.int32))
    i32 = dict(dtype=torch.int32, device="cuda")
    anc = torch.full((B, M_max + 1, D_max + 1), -7, **i32)
    dep = torch.full((B, M_max + 1), -7, **i32)
    st = torch.full((B,), -7, **i32)
    tmv.tree_build_ancestors(par, nn, anc, dep, st)
    A = torch.full((B,), -7, **i32)
    path = torch.full((B, D_max), -7, **i32)
    nxt = torch.full((B,), -7, **i32)
    targ = torch.full((B, M_max + 1), -7, **i32)
    tmv.tree_accept_lm_head(tok, hid, W, nn, anc, dep, st, A, path, nxt, row_argmax=targ, workspace=ws)
    torch.cuda.synchronize()
    return [host_bits(x) for x in (A, path, nxt, st, targ)]


def _check_choices(t_dev, h_rows, w_bits, K):
    """t_dev [n] device choices of the rows h_rows [n][K]; returns (ok, clear) per row."""
    logits, bound = oracle.lm_head_logits(h_rows, w_bits)
    eps = K * 2.0 ** -24 * bound
    clear = []
    for i, x in enumerate(t_dev):
        xs = int(np.argmax(logits[i]))          # smallest index on ties
        assert 0 <= x < logits.shape[1]
        assert logits[i, x] >= logits[i, xs] - (eps[i, x] + eps[i, xs]), (i, x, xs)
        order = np.argsort(-logits[i], kind="stable")
        top2 = int(order[1])
        is_clear = logits[i, xs] - logits[i, top2] > eps[i, xs] + eps[i, top2]
        if is_clear:
            assert x == xs, (i, x, xs)
        clear.append(is_clear)
    return np.array(clear), logits


def _one_hot_accept(t_rows, tokens, parents, n_nodes, M_max, D_max, V):
    """The oracle's greedy rule on given per-row choices (one-hot rows)."""
    B = tokens.shape[0]
    anc, depth, st = _tables(parents, n_nodes, M_max, D_max)
    logits = np.zeros((B, M_max + 1, V), np.float32)
    for b in range(B):
        for u in range(M_max + 1):
            if t_rows[b, u] >= 0:
                logits[b, u, t_rows[b, u]] = 1.0
    return oracle.accept_greedy(tokens, logits, n_nodes, anc, depth, st)


def _small_case(seed, B, M_max, D_max, K, V, sigma_w, alpha=0.8):
    rng = np.random.default_rng(seed)
    parents = np.zeros((B, M_max + 1), np.int32)
    n_nodes = rng.integers(max(1, M_max // 2), M_max + 1, B).astype(np.int32)
    for b in range(B):
        parents[b, :n_nodes[b] + 1] = ti.tree_random(rng, int(n_nodes[b]), D_max)
    hidden = ti.bf16_bits(rng.standard_normal((B, M_max + 1, K), dtype=np.float32))
    w = ti.lm_head_weights(rng, V, K, sigma_w)
    # plant draft tokens on the oracle's choices
    tokens = np.zeros((B, M_max + 1), np.int32)
    t_or = np.zeros((B, M_max + 1), np.int64)
    for b in range(B):
        lg, _ = oracle.lm_head_logits(hidden[b], w, with_bound=False)
        t_or[b] = np.argmax(lg, axis=1)
        ti.plant_from_argmax(rng, parents[b], int(n_nodes[b]), V, t_or[b], tokens[b], alpha)
    return parents, n_nodes, hidden, w, tokens


@pytest.mark.parametrize("B,M_max,D_max,K,V", [(2, 6, 3, 512, 3000), (3, 20, 5, 1024, 1000), (1, 1, 1, 512, 257),
                                               # more than 64 rows: 272-row blocks (one, one, two)
                                               (2, 40, 5, 1024, 900), (4, 64, 6, 512, 2000), (3, 100, 8, 512, 700)])
def test_lm_head_accept_small(B, M_max, D_max, K, V):
    _case("lm-head accept: B%d M%d K%d V%d" % (B, M_max, K, V))
    parents, n_nodes, hidden, w, tokens = _small_case(300 + V, B, M_max, D_max, K, V, 0.05)
    A, path, nxt, st, targ = _run(hidden, w, parents, n_nodes, tokens, M_max, D_max)
    assert np.array_equal(st, np.zeros(B, np.int32))
    anc, depth, _ = _tables(parents, n_nodes, M_max, D_max)
    all_clear = True
    for b in range(B):
        live = [u for u in range(n_nodes[b] + 1) if u == 0 or depth[b, u] >= 1]
        assert np.all(targ[b, [u for u in range(M_max + 1) if u not in live]] == -1)
        clear, _ = _check_choices(targ[b, live], hidden[b, live], w, K)
        all_clear &= bool(clear.all())
    # the path rule on the device's choices, bit-exact
    rA, rpath, rnxt, rst = _one_hot_accept(targ, tokens, parents, n_nodes, M_max, D_max, V)
    assert np.array_equal(A, rA) and np.array_equal(path, rpath) and np.array_equal(nxt, rnxt)
    if M_max > 1:
        assert A.max() > 0
    if all_clear:
        # every choice unambiguous: the whole result equals the oracle's on its own fp64 logits
        oA = []
        for b in range(B):
            lg, _ = oracle.lm_head_logits(hidden[b], w, with_bound=False)
            oA.append(lg.astype(np.float32))
        lg = np.stack(oA)
        oA, opath, onxt, ost = oracle.accept_greedy(tokens, lg, n_nodes, anc, depth, np.zeros(B, np.int32))
        assert np.array_equal(A, oA) and np.array_equal(path, opath) and np.array_equal(nxt, onxt)


@pytest.mark.parametrize("M_max", [6, 40])
def test_lm_head_nan_and_workspace_reuse(M_max):
    _case("lm-head accept: NaN row rejects its sequence; the workspace is left zero (M_max %d)" % M_max)
    import tree_masked_verification_amd as tmv
    B, D_max, K, V = 3, 3, 512, 700
    parents, n_nodes, hidden, w, tokens = _small_case(311, B, M_max, D_max, K, V, 0.05)
    ws = torch.zeros(tmv.tree_accept_lm_head_workspace(B, M_max), dtype=torch.uint8, device="cuda")
    first = _run(hidden, w, parents, n_nodes, tokens, M_max, D_max, ws=ws)
    assert not ws.any()
    again = _run(hidden, w, parents, n_nodes, tokens, M_max, D_max, ws=ws)
    assert all(np.array_equal(x, y) for x, y in zip(first, again))
    bad = hidden.copy()
    bad[1, 0, 5] = 0x7FC0                        # NaN in sequence 1's root row
    A, path, nxt, st, targ = _run(bad, w, parents, n_nodes, tokens, M_max, D_max, ws=ws)
    assert st[1] == tmv.ERR_INPUT and A[1] == 0 and nxt[1] == 0 and np.all(path[1] == 0)
    assert st[0] == tmv.OK and st[2] == tmv.OK
    assert A[0] == first[0][0] and A[2] == first[0][2]
    assert not ws.any()


def test_lm_head_accept_llama8b_shape():
    """61 rows of the 8B-shaped step against a 128256 x 4096 head: rows built to favour
    one planted token each (hidden = 30 W[x_u] + noise), sampled rows checked against the
    oracle's fp64 logits, the whole path against the greedy rule on those choices."""
    _case("lm-head accept: 8B-shaped step, 61 x 4096 x 128256")
    rng = np.random.default_rng(1002)
    K, V, M_max, D_max = 4096, 128256, 60, 6
    parents = ti.tree_rank_sum()[None, :].astype(np.int32)
    n_nodes = np.array([60], np.int32)
    w = ti.lm_head_weights(rng, V, K, 0.03)
    x_u = rng.integers(0, V, M_max + 1)
    wf = ti.bf16_to_f32(w[x_u])
    hidden = ti.bf16_bits(30.0 * wf + rng.standard_normal((M_max + 1, K), dtype=np.float32))[None]
    tokens = np.zeros((1, M_max + 1), np.int32)
    ti.plant_from_argmax(rng, parents[0], 60, V, x_u, tokens[0], 0.7)
    A, path, nxt, st, targ = _run(hidden, w, parents, n_nodes, tokens, M_max, D_max)
    assert st[0] == 0
    assert np.array_equal(targ[0], x_u)
    rows = [0, 17, 60]
    clear, _ = _check_choices(targ[0, rows], hidden[0, rows], w, K)
    assert clear.all()
    rA, rpath, rnxt, rst = _one_hot_accept(targ, tokens, parents, n_nodes, M_max, D_max, V)
    assert np.array_equal(A, rA) and np.array_equal(path, rpath) and np.array_equal(nxt, rnxt)
    print("    accepted %d nodes" % int(A[0]), flush=True)
