"""Device parity: the HIP path through the C ABI against the oracle on the same seeded
inputs.  Bit-exact for ancestor tables, statuses, accepted lengths, paths and next
tokens; attention within 2e-2 absolute (bf16) / 1e-5 (fp32), plus a relative-L2
diagnostic and mask-sensitive variants (empty prefix, sharpened queries) that a wrong
mask cannot pass."""
import os

import numpy as np
import pytest
import torch

import tmv_inputs as ti
from tests.harness import DeviceStep, attention_error, host_bits, oracle_attention, oracle_tables
from tests.test_oracle_build import random_labelled_tree

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _case(name):
    print("\n[gpu case] %s" % name, flush=True)


def small_attention_workload(seed, B, Hq, Hkv, d, M_max, prefixes, n_nodes, dtype=ti.BF16, q_scale=1.0,
                             sigma=0.5, max_depth=6, labelled=True):
    rng = np.random.default_rng(seed)
    parents = np.zeros((B, M_max + 1), np.int32)
    for b in range(B):
        m = int(n_nodes[b])
        parents[b, : m + 1] = random_labelled_tree(rng, m, max_depth) if labelled else ti.tree_random(rng, m, max_depth)
    L_cap = int(max(np.asarray(prefixes) + np.asarray(n_nodes))) + 5
    mk = lambda shape, s: rng.standard_normal(shape).astype(np.float32) * np.float32(s)
    q = mk((B, M_max, Hq, d), sigma * q_scale)
    k = mk((B, Hkv, L_cap, d), sigma)
    v = mk((B, Hkv, L_cap, d), sigma)
    if dtype == ti.BF16:
        q, k, v = ti.bf16_bits(q), ti.bf16_bits(k), ti.bf16_bits(v)
    return ti.Workload("small", dtype, B, Hq, Hkv, d, M_max, max(max_depth, 1), L_cap, 16, "greedy", parents,
                       np.asarray(n_nodes, np.int32), np.asarray(prefixes, np.int32),
                       np.zeros((B, M_max + 1), np.int32), q, k, v)


# ------------------------------------------------------------------ stage 1
def test_build_ancestors_random_trees(ref):
    _case("build: random labelled trees")
    rng = np.random.default_rng(101)
    for M_max, D_max in [(8, 8), (60, 6), (128, 8), (128, 128)]:
        B = 40
        n = rng.integers(0, M_max + 1, size=B).astype(np.int32)
        parents = np.zeros((B, M_max + 1), np.int32)
        for b in range(B):
            parents[b, : n[b] + 1] = random_labelled_tree(rng, int(n[b]), min(D_max + (b % 3 == 0), 12))
        w = ti.Workload("build", ti.F32, B, 1, 1, 64, M_max, D_max, 1, 1, "greedy", parents, n, n * 0, n * 0)
        dev = DeviceStep(w)
        dev.build()
        a, d, s = dev.tables()
        ra, rd, rs = oracle_tables(ref, w)
        assert np.array_equal(s, rs) and np.array_equal(a, ra) and np.array_equal(d, rd)


def test_build_ancestors_malformed_and_formats(ref):
    _case("build: malformed fixtures, NEG1, valid masks")
    cases = []
    for line in open(os.path.join(GOLD, "malformed_trees.txt")):
        if line.strip() and line[0] != "#":
            cases.append([f.strip() for f in line.split("|")])
    M_max, D_max = 6, 4
    B = len(cases)
    parents = np.zeros((B, M_max + 1), np.int32)
    valid = np.ones((B, M_max + 1), np.uint8)
    n = np.zeros(B, np.int32)
    for b, (name, M, D, pars, vmask, want) in enumerate(cases):
        n[b] = int(M)
        if int(M):
            parents[b, 1:int(M) + 1] = [int(x) for x in pars.split()]
        if vmask != "-":
            valid[b, 1:int(M) + 1] = [int(x) for x in vmask.split()]
    for D in (3, 4):
        w = ti.Workload("bad", ti.F32, B, 1, 1, 64, M_max, D, 1, 1, "greedy", parents, n, n * 0, n * 0)
        dev = DeviceStep(w)
        dev.build(valid=torch.from_numpy(valid).cuda())
        a, d, s = dev.tables()
        ra, rd, rs = ref.build_ancestors(parents, n, M_max, D, valid=valid)
        assert np.array_equal(s, rs) and np.array_equal(a, ra) and np.array_equal(d, rd)
    # NEG1 form and out-of-range node counts
    rng = np.random.default_rng(102)
    B, M_max = 12, 20
    n = rng.integers(0, M_max + 1, size=B).astype(np.int32)
    n[0], n[1] = -1, M_max + 1
    neg1 = np.zeros((B, M_max), np.int32)
    for b in range(2, B):
        par = ti.tree_random(rng, int(n[b]), 5)
        neg1[b, : n[b]] = par[1:] - 1
    neg1[5, 0] = -3
    w = ti.Workload("neg1", ti.F32, B, 1, 1, 64, M_max, 5, 1, 1, "greedy", neg1, n, n * 0, n * 0)
    dev = DeviceStep(w)
    dev.build(parent_format=1)
    a, d, s = dev.tables()
    ra, rd, rs = ref.build_ancestors(neg1, n, M_max, 5, parent_format=ref.PARENTS_NEG1)
    assert np.array_equal(s, rs) and np.array_equal(a, ra) and np.array_equal(d, rd)


# ------------------------------------------------------------------ stage 2
def _attention_parity(ref, w, tol, rel_tol, rows=None, plan=None):
    dev = DeviceStep(w)
    dev.build()
    dev.attention(plan=plan)
    a, d, s = dev.tables()
    ra, rd, rs = oracle_tables(ref, w)
    assert np.array_equal(s, rs) and np.array_equal(a, ra)
    ref_out, ref_st = oracle_attention(ref, w, ra, rd, rs, row_select=rows)
    out = host_bits(dev.out)
    assert np.array_equal(host_bits(dev.status), ref_st)
    mask = None
    if rows is not None:
        mask = np.zeros(out.shape, bool)
        mask[rows.astype(bool)] = True
    err, rel = attention_error(out, ref_out, w.dtype, mask)
    print("    max|err| %.3g  relL2 %.3g" % (err, rel), flush=True)
    assert err <= tol and rel <= rel_tol
    if rows is None:
        assert not np.any(np.isnan(out.astype(np.float64) if w.dtype == ti.F32 else ti.bf16_to_f32(out)))
    return dev


def test_attention_tiny_fp32_workload(ref):
    _case("attention: tiny fp32 workload (config 1)")
    _attention_parity(ref, ti.workload(1), 1e-5, 1e-6)


@pytest.mark.parametrize("variant", ["plain", "empty_prefix", "sharpened", "tiny_prefix_sharp"])
def test_attention_bf16_small_ragged(ref, variant):
    _case("attention: bf16 ragged small, %s" % variant)
    B, Hq, Hkv, d, M_max = 3, 8, 2, 128, 37
    n_nodes = [37, 20, 1]
    prefixes = {"plain": [700, 33, 5], "empty_prefix": [0, 0, 0], "sharpened": [300, 64, 1],
                "tiny_prefix_sharp": [1, 2, 0]}[variant]
    q_scale = 8.0 if "sharp" in variant else 1.0
    w = small_attention_workload(200, B, Hq, Hkv, d, M_max, prefixes, n_nodes, q_scale=q_scale)
    _attention_parity(ref, w, 2e-2, 1e-2)


@pytest.mark.parametrize("d", [128, 64])
def test_attention_bf16_late_outlier_scores(ref, d):
    """Keys planted late in the prefix and in the tree so that some rows' scores there exceed
    everything in the first chunks by far more than 2^32 in base 2: the kernels' first pass
    detects it and redoes the split against the exact row maxima.  Rows that never see a
    planted key are unaffected; the planted ones must come out as the planted tokens' V."""
    _case("attention: bf16 late outlier scores d=%d" % d)
    B, Hq, Hkv, M_max = 2, 8, 2, 20
    prefixes, n_nodes = [600, 130], [20, 12]
    w = small_attention_workload(230 + d, B, Hq, Hkv, d, M_max, prefixes, n_nodes)
    qf = ti.bf16_to_f32(w.q)
    kf = ti.bf16_to_f32(w.k)
    g = Hq // Hkv
    rng = np.random.default_rng(231)
    for b in range(B):
        for kvh in range(Hkv):
            # a prefix slot in the last chunks gets 40 x a query row of node 1 (head kvh*g):
            # that row's score there is ~ 40 |q|^2 / sqrt(d) above its others
            t = prefixes[b] - 1 - int(rng.integers(0, 20))
            kf[b, kvh, t] = 40.0 * qf[b, 0, kvh * g]
            # and the tree slot of the last node, for the rows that see it
            kf[b, kvh, prefixes[b] + n_nodes[b] - 1] = 30.0 * qf[b, n_nodes[b] - 1, kvh * g + 1]
    w.k = ti.bf16_bits(kf)
    _attention_parity(ref, w, 2e-2, 1e-2)


@pytest.mark.parametrize("d", [128, 64])
def test_attention_bf16_deep_paths(ref, d):
    # ancestor paths longer than the entries a row fetches up front (the kernels' deep-row
    # branch): chains and deep random trees, with and without a prefix
    _case("attention: bf16 deep paths d=%d" % d)
    w = small_attention_workload(206 + d, 3, 8, 2, d, 70, [0, 45, 3], [70, 52, 33], q_scale=6.0, max_depth=70,
                                 labelled=False)
    w.parents[0, :71] = ti.tree_chain(70)
    assert int(oracle_tables(ref, w)[1].max()) > 16
    _attention_parity(ref, w, 2e-2, 1e-2)


@pytest.mark.parametrize("Hq,Hkv,d", [(4, 4, 128), (16, 2, 64), (12, 4, 64), (64, 8, 128)])
def test_attention_bf16_head_shapes(ref, Hq, Hkv, d):
    _case("attention: bf16 Hq=%d Hkv=%d d=%d" % (Hq, Hkv, d))
    w = small_attention_workload(201 + Hq, 2, Hq, Hkv, d, 24, [129, 0], [24, 17], q_scale=4.0)
    _attention_parity(ref, w, 2e-2, 1e-2)


def test_attention_fp32_general(ref):
    _case("attention: fp32 general shapes")
    w = small_attention_workload(205, 3, 6, 2, 128, 30, [90, 0, 257], [30, 11, 4], dtype=ti.F32, sigma=1.0)
    _attention_parity(ref, w, 1e-5, 1e-6)


def test_attention_llama8b_layer_full(ref):
    _case("attention: 8B-shaped layer, every row (config 2)")
    w = ti.workload(2)
    _attention_parity(ref, w, 2e-2, 1e-2)
    # the same tree with an empty prefix and sharpened queries: mask errors become O(1)
    w2 = ti.workload(2)
    w2.prefix = np.array([0], np.int32)
    w2.q = ti.bf16_bits(ti.bf16_to_f32(w2.q) * 8.0)
    _attention_parity(ref, w2, 2e-2, 1e-2)


def test_attention_determinism():
    _case("attention: bit-identical reruns")
    w = ti.workload(2)
    dev = DeviceStep(w)
    dev.build()
    dev.attention()
    first = host_bits(dev.out).copy()
    for _ in range(3):
        dev.out.fill_(float("nan"))
        dev.attention()
        assert np.array_equal(host_bits(dev.out), first)


def test_workspace_reuse_across_calls_and_shapes():
    _case("attention and greedy accept: zero-filled workspaces reused across calls and shapes")
    import tree_masked_verification_amd as tmv
    w = ti.workload(2)
    dev = DeviceStep(w)
    dev.build()
    n_attn = tmv.tree_verify_attention_workspace(tmv.BF16, w.B, w.M_max, w.Hq, w.Hkv, w.d, w.L_cap)
    small = small_attention_workload(207, 3, 8, 2, 128, 37, [700, 33, 5], [37, 20, 1], q_scale=4.0)
    n_small = tmv.tree_verify_attention_workspace(tmv.BF16, small.B, small.M_max, small.Hq, small.Hkv, small.d,
                                                  small.L_cap)
    wa = torch.zeros(max(n_attn, n_small), dtype=torch.uint8, device="cuda")
    dev.attention(workspace=wa)
    dev.accept()
    ref_out = host_bits(dev.out).copy()
    ref_acc = [host_bits(t).copy() for t in (dev.accept_len, dev.path, dev.next_token)]
    # a different split plan on the same workspace, then the first shape again: the
    # arrival counters must have come back to zero after every call
    ds = DeviceStep(small)
    ds.build()
    # logits for the small shape: two vocabulary chunks, the second one partial
    g = torch.Generator(device="cpu").manual_seed(208)
    ds.logits = torch.randn((small.B, small.M_max + 1, 5000), generator=g).cuda()
    ds.tokens = torch.randint(0, 5000, (small.B, small.M_max + 1), generator=g, dtype=torch.int32).cuda()
    for _ in range(2):
        ds.attention(workspace=wa)
    ds.accept()
    torch.cuda.synchronize()
    s1 = host_bits(ds.out).copy()
    s1_acc = [host_bits(t).copy() for t in (ds.accept_len, ds.path, ds.next_token)]
    # the greedy accept's keys and counters: one zero-filled workspace for both shapes,
    # left zero by every call
    n_acc = max(tmv.tree_accept_workspace(tmv.ACCEPT_GREEDY, w.B, w.M_max, w.V),
                tmv.tree_accept_workspace(tmv.ACCEPT_GREEDY, small.B, small.M_max, 5000))
    wc = torch.zeros(n_acc, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        dev.out.fill_(float("nan"))
        dev.accept_len.fill_(-7)
        dev.attention(workspace=wa)
        dev.accept(workspace=wc)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(dev.out), ref_out)
        assert all(np.array_equal(host_bits(t), r) for t, r in zip((dev.accept_len, dev.path, dev.next_token), ref_acc))
        assert int(wc.count_nonzero()) == 0
        ds.out.fill_(float("nan"))
        ds.accept_len.fill_(-7)
        ds.attention(workspace=wa)
        ds.accept(workspace=wc)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(ds.out), s1)
        assert all(np.array_equal(host_bits(t), r) for t, r in zip((ds.accept_len, ds.path, ds.next_token), s1_acc))
        assert int(wc.count_nonzero()) == 0


def test_attention_after_kernels_of_odd_grid_sizes(ref):
    """The splits of a row block (equal workgroup ids mod 8) exchange their partials through
    the L2 of the XCD the hardware deals them to, whatever ran before: after kernels of
    assorted grid sizes the rows must stay bit-identical (and no block may be rejected)."""
    _case("attention: 8B-shaped layer after kernels of odd grid sizes")
    w = ti.workload(2)
    dev = _attention_parity(ref, w, 2e-2, 1e-2)
    first = host_bits(dev.out).copy()
    scratch = torch.empty(1 << 20, device="cuda")
    for n in (1, 3, 70001, 5, 123457, 7, 9000, 333333):
        dev.out.fill_(float("nan"))
        scratch[:n].fill_(1.0)
        dev.attention()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(dev.out), first), n


def test_attention_splits_spread_over_xcds_rejected(ref):
    """A test-only placement deals each row block's splits to different XCDs, whose L2s do not
    see each other's partials: the merge must refuse (every row 0, status ERR_DEVICE), never
    merge stale data, and leave the workspace ready -- the next call on it is bit-identical
    to one on a fresh workspace."""
    _case("attention: row blocks spread over XCDs are rejected")
    import tree_masked_verification_amd as tmv
    w = ti.workload(2)
    dev = DeviceStep(w)
    dev.build()
    n = tmv.tree_verify_attention_plan_workspace(tmv.BF16, w.B, w.M_max, w.Hq, w.Hkv, w.d, w.L_cap, 64, 8)
    wa = torch.zeros(n, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        dev.out.fill_(float("nan"))
        dev.attention(workspace=wa, plan=(64, 8 | tmv.PLAN_SCATTER_XCD))
        torch.cuda.synchronize()
        assert host_bits(dev.status).tolist() == [tmv.ERR_DEVICE]
        assert not np.any(host_bits(dev.out))
        assert int(wa[:32768].count_nonzero()) == 0          # arrival words left zero
        dev.build()                                           # status back to OK
    dev.out.fill_(float("nan"))
    dev.attention(workspace=wa, plan=(64, 8))
    torch.cuda.synchronize()
    after = host_bits(dev.out).copy()
    dev.out.fill_(float("nan"))
    dev.attention(workspace=torch.zeros(n, dtype=torch.uint8, device="cuda"), plan=(64, 8))
    torch.cuda.synchronize()
    assert host_bits(dev.status).tolist() == [tmv.OK]
    assert np.array_equal(host_bits(dev.out), after)
    # a shape whose pairs do not fill whole XCD groups cannot be scattered
    small = small_attention_workload(207, 3, 8, 2, 128, 37, [700, 33, 5], [37, 20, 1])
    ds = DeviceStep(small)
    ds.build()
    with pytest.raises(tmv.TmvError):
        ds.attention(plan=(64, 4 | tmv.PLAN_SCATTER_XCD))


# a ragged batch shaped for the adaptive plan (16 sequences, 8 KV heads, two 256-row groups
# per head at M_max 96 fill one workgroup per CU): the sequences with the most chunks have
# few nodes, so the row groups they leave free go to second splits; node counts 0 and 1, an
# empty prefix and a sequence failed by a cycle (status set by the build) ride along
ADAPTIVE_PREFIX = [200, 100, 300, 50, 0, 150, 250, 100, 1400, 1300, 1200, 1100, 1000, 0, 900, 800]
ADAPTIVE_NODES = [96, 90, 80, 70, 65, 96, 66, 75, 40, 30, 20, 10, 1, 0, 64, 50]


def adaptive_workload(seed, q_scale=1.0):
    w = small_attention_workload(seed, 16, 32, 8, 128, 96, ADAPTIVE_PREFIX, ADAPTIVE_NODES, q_scale=q_scale)
    w.parents[6, 3], w.parents[6, 4] = 4, 3       # sequence 6 fails the build (a cycle)
    return w


@pytest.mark.parametrize("q_scale", [1.0, 6.0])
def test_attention_adaptive_splits_ragged_batch(ref, q_scale):
    """Every row of a ragged batch under the default (adaptive) plan: split and unsplit
    sequences, row groups past a sequence's last node, a failed and an empty sequence."""
    _case("attention: ragged batch with per-sequence splits, q x%g" % q_scale)
    w = adaptive_workload(290, q_scale)
    dev = _attention_parity(ref, w, 2e-2, 1e-2)
    first = host_bits(dev.out).copy()
    for _ in range(2):
        dev.out.fill_(float("nan"))
        dev.attention()
        assert np.array_equal(host_bits(dev.out), first)


@pytest.mark.parametrize("plan", [(64, 1), (64, 3), (64, 8), (128, 1), (128, 4), (128, 16), (256, 1), (256, 6),
                                  (32, 1), (128, 5)])
def test_attention_launch_plans(ref, plan):
    # every launch plan (row-group width : token splits) must give the same rows: the
    # split merge, the row-group combine and the per-wave chunk assignment all change
    # (widths 32 and 128 with head dim 64 run the streaming kernel)
    _case("attention: 8B-shaped layer under plan %s" % (plan,))
    if plan[0] != 32:
        w = ti.workload(2)
        _attention_parity(ref, w, 2e-2, 1e-2, plan=plan)
        w3 = small_attention_workload(208, 3, 8, 2, 128, 37, [700, 33, 5], [37, 20, 1], q_scale=4.0)
        _attention_parity(ref, w3, 2e-2, 1e-2, plan=plan)
    if plan[0] in (32, 128):
        w4 = small_attention_workload(209, 3, 12, 4, 64, 37, [700, 33, 5], [37, 20, 1], q_scale=4.0)
        _attention_parity(ref, w4, 2e-2, 1e-2, plan=plan)
