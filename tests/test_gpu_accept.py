"""Device parity of tree_accept (greedy and sampling) against the oracle: accepted length,
path, next token and status must be bit-identical."""
import numpy as np
import pytest
import torch

import tmv_inputs as ti
from tests.harness import DeviceStep, dev_tensor, host_bits, oracle_tables
from tests.test_oracle_build import random_labelled_tree

pytestmark = pytest.mark.gpu


def _case(name):
    print("\n[gpu case] %s" % name, flush=True)


def _greedy_parity(ref, w, logits_dev=None, row_dtype=0, logits_host=None):
    dev = DeviceStep(w)
    dev.build()
    if logits_dev is not None:
        dev.logits = logits_dev
    dev.accept()
    torch.cuda.synchronize()
    ra, rd, rs = oracle_tables(ref, w)
    lh = w.logits if logits_host is None else logits_host
    A, path, nxt, st = ref.accept_greedy(w.tokens, lh, w.n_nodes, ra, rd, rs, row_dtype=row_dtype)
    got = [host_bits(t) for t in (dev.accept_len, dev.path, dev.next_token, dev.status)]
    for g, e, name in zip(got, (A, path, nxt, st), ("accept_len", "path", "next_token", "status")):
        assert np.array_equal(g, e), (name, g, e)
    return A, st


def small_greedy(seed, B, M_max, D_max, V, tie_levels=None, alpha=0.8):
    rng = np.random.default_rng(seed)
    n = rng.integers(0, M_max + 1, size=B).astype(np.int32)
    parents = np.zeros((B, M_max + 1), np.int32)
    for b in range(B):
        parents[b, : n[b] + 1] = random_labelled_tree(rng, int(n[b]), D_max)
    if tie_levels:
        # integer logits: every row has many tied maxima; most children carry the first
        # maximum of their parent's row (numpy argmax), so accepted paths go through ties
        logits = rng.integers(0, tie_levels, size=(B, M_max + 1, V)).astype(np.float32)
        tokens = rng.integers(0, V, size=(B, M_max + 1)).astype(np.int32)
        for b in range(B):
            for c in range(1, int(n[b]) + 1):
                if rng.random() < 0.7:
                    tokens[b, c] = int(np.argmax(logits[b, parents[b, c]]))
    else:
        logits = rng.standard_normal((B, M_max + 1, V)).astype(np.float32)
        tokens = np.zeros((B, M_max + 1), np.int32)
        for b in range(B):
            ti.plant_greedy(rng, parents[b], int(n[b]), V, logits[b], tokens[b], alpha)
    return ti.Workload("greedy-small", ti.F32, B, 0, 1, 64, M_max, D_max, 1, V, "greedy", parents, n,
                       np.zeros(B, np.int32), tokens, logits=logits)


@pytest.mark.parametrize("V,ties", [(5, 3), (37, None), (8192, None), (20000, 4), (128256, None)])
def test_greedy_small_trees(ref, V, ties):
    _case("greedy: random trees V=%d ties=%s" % (V, ties))
    w = small_greedy(300 + V, 24 if V < 100000 else 6, 20, 8, V, ties)
    A, st = _greedy_parity(ref, w)
    assert np.all(st == 0) and np.any(A > 0)


def test_greedy_bf16_rows_and_strided_rows(ref):
    _case("greedy: bf16 logits; padded row stride")
    w = small_greedy(310, 16, 12, 6, 1000)
    lb = ti.bf16_bits(w.logits)
    _greedy_parity(ref, w, logits_dev=dev_tensor(lb, bf16=True), row_dtype=1, logits_host=lb)
    # rows 3 elements apart from the vocabulary size (unaligned row starts)
    pad = np.zeros((w.B, w.M_max + 1, w.V + 3), np.float32)
    pad[:, :, : w.V] = w.logits
    view = dev_tensor(pad)[:, :, : w.V]
    _greedy_parity(ref, w, logits_dev=view)


def test_greedy_errors_and_degenerate(ref):
    _case("greedy: NaN rows, bad tokens, failed sequences, empty trees")
    w = small_greedy(311, 8, 10, 6, 300)
    w.n_nodes[:] = 10
    parents = np.zeros((8, 11), np.int32)
    rng = np.random.default_rng(5)
    for b in range(8):
        parents[b] = ti.tree_random(rng, 10, 6)
    w.parents = parents
    w.logits[1, 0, 17] = np.nan                       # root row
    w.logits[2, 4, 3] = np.nan                        # a live node's row
    w.tokens[3, 2] = 300                              # token == V
    w.tokens[4, 7] = -1
    w.parents[5, 3] = 3                               # cycle -> failed sequence upstream
    w.n_nodes[6] = 0                                  # empty tree
    A, st = _greedy_parity(ref, w)
    assert st[1] == ref.ERR_INPUT and st[2] == ref.ERR_INPUT and st[3] == ref.ERR_INPUT
    assert st[4] == ref.ERR_INPUT and st[5] == ref.ERR_CYCLE and st[6] == 0 and A[6] == 0
    # M_max = 0: only the root row
    w0 = ti.Workload("m0", ti.F32, 2, 0, 1, 64, 0, 0, 1, 7, "greedy", np.zeros((2, 1), np.int32),
                     np.zeros(2, np.int32), np.zeros(2, np.int32), np.zeros((2, 1), np.int32),
                     logits=np.array([[[0, 1, 5, 5, 2, 0, 0]], [[9, 1, 5, 5, 2, 0, 9]]], np.float32))
    _greedy_parity(ref, w0)


@pytest.mark.parametrize("V", [300, 9000])
def test_greedy_signed_zero_ties(ref, V):
    """Rows whose maximum is a -0.0 and a +0.0: the two compare equal, so the first of them
    is the argmax (in one chunk, or in different chunks of the scan); fp32 and bf16 rows."""
    _case("greedy: -0.0 / +0.0 maxima, V=%d" % V)
    from tests.test_oracle_greedy import signed_zero_rows
    rng = np.random.default_rng(330 + V)
    B, M_max = 6, 8
    parents, tokens, logits, first = signed_zero_rows(rng, B, M_max, V)
    w = ti.Workload("signed-zeros", ti.F32, B, 0, 1, 64, M_max, M_max, 1, V, "greedy", parents,
                    np.full(B, M_max, np.int32), np.zeros(B, np.int32), tokens, logits=logits)
    A, st = _greedy_parity(ref, w)
    assert np.all(st == 0) and np.any(A > 1)
    lb = ti.bf16_bits(logits)
    assert np.array_equal(np.argmax(ti.bf16_to_f32(lb), axis=2), first)
    _greedy_parity(ref, w, logits_dev=dev_tensor(lb, bf16=True), row_dtype=1, logits_host=lb)


@pytest.mark.parametrize("c", [1, 2, 4])
def test_greedy_workloads(ref, c):
    _case("greedy: workload %d" % c)
    A, st = _greedy_parity(ref, ti.workload(c))
    assert np.all(st == 0)
    print("    accept lengths", A.tolist(), flush=True)


def test_greedy_determinism_and_workspace_reuse():
    _case("greedy: repeated calls on one workspace")
    import tree_masked_verification_amd as tmv
    w = ti.workload(2)
    dev = DeviceStep(w)
    dev.build()
    ws = torch.zeros(tmv.tree_accept_workspace(tmv.ACCEPT_GREEDY, 1, w.M_max, w.V), dtype=torch.uint8, device="cuda")
    dev.accept(workspace=ws)
    first = [host_bits(t).copy() for t in (dev.accept_len, dev.path, dev.next_token)]
    for _ in range(5):
        dev.accept(workspace=ws)
        assert all(np.array_equal(host_bits(t), f) for t, f in zip((dev.accept_len, dev.path, dev.next_token), first))


# ------------------------------------------------------------------ sampling
def _sample_parity(ref, parents, n, tokens, p, q, seed, step, D_max, status_override=None, workspace=None):
    B, R, V = p.shape
    w = ti.Workload("sample", ti.F32, B, 0, 1, 64, R - 1, D_max, 1, V, "sample", parents, n,
                    np.zeros(B, np.int32), tokens, p=p, qd=q, seed=seed, step=step)
    dev = DeviceStep(w)
    dev.build()
    if status_override is not None:
        dev.status.copy_(torch.from_numpy(status_override).cuda())
    dev.accept(workspace=workspace)
    torch.cuda.synchronize()
    ra, rd, rs = oracle_tables(ref, w)
    if status_override is not None:
        rs = status_override.copy()
    A, path, nxt, st = ref.accept_sample(tokens, p, q, seed, step, n, ra, rd, rs)
    got = [host_bits(t) for t in (dev.accept_len, dev.path, dev.next_token, dev.status)]
    for g, e, name in zip(got, (A, path, nxt, st), ("accept_len", "path", "next_token", "status")):
        assert np.array_equal(g, e), (name, g, e)
    return A, st


@pytest.mark.parametrize("V,overlap", [(6, 0.9), (50, 0.95), (1000, 0.9), (5000, None), (128256, 0.97)])
def test_sampling_small(ref, V, overlap):
    _case("sampling: V=%d overlap=%s" % (V, overlap))
    rng = np.random.default_rng(400 + V)
    B = 64 if V <= 1000 else 8
    parents, n, tokens, p, q = ti.small_sampling_case(rng, B, 12, V, 5, overlap=overlap)
    for step in (0, 1):
        A, st = _sample_parity(ref, parents, n, tokens, p, q, 77, step, 5)
        assert np.all(st == 0)
    if V <= 1000:
        assert np.any(A >= 2)


def test_sampling_beside_a_busy_device(ref):
    """Long fp32 GEMMs on a second stream hold compute units while the walk runs, so the
    K workgroups of a sequence may not all be resident at once.  Every sequence then either
    matches the oracle bit for bit or fails with TMV_ERR_DEVICE and zero outputs; every
    kernel exits; the workspace is left zero, and the next call on it (not zero-filled
    again) is bit-exact."""
    _case("sampling: walk beside GEMMs on another stream")
    import tree_masked_verification_amd as tmv
    rng = np.random.default_rng(450)
    B, M, V, D = 16, 12, 50000, 5
    parents, n, tokens, p, q = ti.small_sampling_case(rng, B, M, V, D, overlap=0.95)
    w = ti.Workload("sample", ti.F32, B, 0, 1, 64, M, D, 1, V, "sample", parents, n, np.zeros(B, np.int32), tokens,
                    p=p, qd=q, seed=91, step=3)
    ra, rd, rs = oracle_tables(ref, w)
    want = ref.accept_sample(tokens, p, q, w.seed, w.step, n, ra, rd, rs)
    dev = DeviceStep(w)
    ws = torch.zeros(tmv.tree_accept_workspace(tmv.ACCEPT_SAMPLE, B, M, V), dtype=torch.uint8, device="cuda")
    big = torch.randn((6144, 6144), device="cuda")
    prod = torch.empty_like(big)
    side = torch.cuda.Stream()
    dev.build()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        for _ in range(4):
            torch.mm(big, big, out=prod)
    dev.accept(workspace=ws)
    torch.cuda.synchronize()
    got = [host_bits(t) for t in (dev.accept_len, dev.path, dev.next_token, dev.status)]
    failed = 0
    for b in range(B):
        if got[3][b] == tmv.ERR_DEVICE:
            failed += 1
            assert got[0][b] == 0 and got[2][b] == 0 and not got[1][b].any(), b
        else:
            assert all(np.array_equal(g[b], e[b]) for g, e in zip(got, want)), b
    print("    sequences that gave up waiting: %d of %d" % (failed, B), flush=True)
    assert int(ws.count_nonzero()) == 0
    dev.build()
    dev.accept(workspace=ws)
    torch.cuda.synchronize()
    got = [host_bits(t) for t in (dev.accept_len, dev.path, dev.next_token, dev.status)]
    assert all(np.array_equal(g, e) for g, e in zip(got, want))


@pytest.mark.parametrize("wait_us", [0, 5])
def test_sampling_gives_up_cleanly(ref, wait_us):
    """The walk's wait bound forced from the host (tmv_tree_accept_wait) down to nothing or
    a few microseconds: workgroups give up waiting for slices not yet resident.  Each
    sequence then matches the oracle bit for bit or ends with TMV_ERR_DEVICE and zero
    outputs, every kernel exits, the workspace is left zero, and a call with the default
    bound on that same workspace is bit-exact."""
    _case("sampling: wait bound %d us" % wait_us)
    import tree_masked_verification_amd as tmv
    rng = np.random.default_rng(460 + wait_us)
    B, M, V, D = 24, 12, 60000, 5
    parents, n, tokens, p, q = ti.small_sampling_case(rng, B, M, V, D, overlap=0.95)
    w = ti.Workload("sample", ti.F32, B, 0, 1, 64, M, D, 1, V, "sample", parents, n, np.zeros(B, np.int32), tokens,
                    p=p, qd=q, seed=92, step=4)
    ra, rd, rs = oracle_tables(ref, w)
    want = ref.accept_sample(tokens, p, q, w.seed, w.step, n, ra, rd, rs)
    dev = DeviceStep(w)
    ws = torch.zeros(tmv.tree_accept_workspace(tmv.ACCEPT_SAMPLE, B, M, V), dtype=torch.uint8, device="cuda")
    failed = 0
    for rep in range(3):
        dev.build()
        tmv.tree_accept(tmv.ACCEPT_SAMPLE, dev.tokens, dev.p, dev.n_nodes, dev.anc, dev.depth, dev.status,
                        dev.accept_len, dev.path, dev.next_token, draft_q=dev.qd, seed=w.seed, step=w.step,
                        workspace=ws, wait_us=wait_us)
        torch.cuda.synchronize()
        got = [host_bits(t) for t in (dev.accept_len, dev.path, dev.next_token, dev.status)]
        for b in range(B):
            if got[3][b] == tmv.ERR_DEVICE:
                failed += 1
                assert got[0][b] == 0 and got[2][b] == 0 and not got[1][b].any(), b
            else:
                assert all(np.array_equal(g[b], e[b]) for g, e in zip(got, want)), b
        assert int(ws.count_nonzero()) == 0
    print("    sequences that gave up waiting: %d of %d" % (failed, 3 * B), flush=True)
    if wait_us == 0:
        assert failed > 0
    dev.build()
    dev.accept(workspace=ws)
    torch.cuda.synchronize()
    got = [host_bits(t) for t in (dev.accept_len, dev.path, dev.next_token, dev.status)]
    assert all(np.array_equal(g, e) for g, e in zip(got, want))


def test_sampling_unnormalised_and_edge_rows(ref):
    """Rows that do not sum to 1 (the integer rule renormalises), rows with zeros,
    a p row equal to q (empty residual), exact 0/1 probabilities."""
    _case("sampling: unnormalised and degenerate rows")
    rng = np.random.default_rng(410)
    V = 40
    parents, n, tokens, p, q = ti.small_sampling_case(rng, 48, 9, V, 4, overlap=0.8)
    p = p.copy()
    q = q.copy()
    p[0:8] *= 0.37                                   # unnormalised
    q[8:16, :, ::2] = 0.0                            # zeros in the draft rows
    p[16:24] = q[16:24]                              # p == q: residual may vanish
    p[24:32] = 0.0
    p[24:32, :, 5] = 1.0                             # one-hot teacher
    p[32:40] = np.minimum(1.0, p[32:40] * 40.0)      # rows summing to far above 1
    A, st = _sample_parity(ref, parents, n, tokens, p, q, 3, 0, 4)
    assert np.all(st == 0)


def test_sampling_errors(ref):
    _case("sampling: malformed rows and failed sequences")
    rng = np.random.default_rng(411)
    V = 64
    parents, n, tokens, p, q = ti.small_sampling_case(rng, 8, 6, V, 3, overlap=0.9)
    p = p.copy(); q = q.copy(); tokens = tokens.copy()
    p[0, 0, 1] = -0.01
    p[1, 0, 2] = np.nan
    q[2, 0] = 0.0
    tokens[3, 1] = V
    p[4, 0, 0] = 1.5
    st_in = np.zeros(8, np.int32)
    st_in[5] = 3
    A, st = _sample_parity(ref, parents, n, tokens, p, q, 9, 0, 3, status_override=st_in)
    assert st[:6].tolist() == [ref.ERR_INPUT] * 5 + [3] and st[6] == 0 and st[7] == 0


def test_sampling_workload5(ref):
    _case("sampling: workload 5 (B32, V128256)")
    w = ti.workload(5)
    A, st = _sample_parity(ref, w.parents, w.n_nodes, w.tokens, w.p, w.qd, w.seed, w.step, w.D_max)
    assert np.all(st == 0)
    print("    accept lengths", A.tolist(), flush=True)


@pytest.mark.parametrize("B,seed", [(300, 420), (2, 421)])
def test_sampling_slice_shapes_and_workspace(ref, B, seed):
    """B = 300: one workgroup per sequence whose 20000-entry slice is longer than the
    registers hold (the rest is re-read on every pass); B = 2: many slices per sequence
    meeting at the barrier.  Both: parity on two calls sharing one workspace, which every
    completed call leaves zero."""
    import tree_masked_verification_amd as tmv
    _case("sampling: B=%d V=20000 (slice shapes, workspace left zero)" % B)
    rng = np.random.default_rng(seed)
    V = 20000
    parents, n, tokens, p, q = ti.small_sampling_case(rng, B, 10, V, 4, overlap=0.9)
    ws = torch.zeros(tmv.tree_accept_workspace(tmv.ACCEPT_SAMPLE, B, 10, V), dtype=torch.uint8, device="cuda")
    for step in (0, 1):
        A, st = _sample_parity(ref, parents, n, tokens, p, q, 5, step, 4, workspace=ws)
        assert np.all(st == 0)
        assert int(torch.count_nonzero(ws)) == 0
