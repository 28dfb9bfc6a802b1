"""Device parity of the paged-cache calls (runtime-memory question of the hierarchical
speculative decoding blog: vLLM-style pages, shared ancestor pages, only the accepted path
kept).  The pages hold exactly the contiguous cache's slots, so the oracle's contiguous
results are the reference: attention within the bf16 tolerance (and bit-identical to the
contiguous kernel over the same capacity, which runs the same launch plan), commit
bit-exact after gathering the pages back."""
import numpy as np
import pytest
import torch

import tmv_inputs as ti
from tests.harness import DeviceStep, attention_error, dev_tensor, host_bits, oracle_attention, oracle_tables
from tests.test_gpu_commit import _path_of
from tests.test_gpu_parity import adaptive_workload, small_attention_workload
from tests.test_oracle_build import random_labelled_tree

pytestmark = pytest.mark.gpu


def _case(name):
    print("\n[gpu case] %s" % name, flush=True)


def _padded(w, L):
    """The same workload with its caches padded (zeros) to capacity L."""
    pad = lambda a: np.concatenate([a, np.zeros(a.shape[:2] + (L - a.shape[2], a.shape[3]), a.dtype)], axis=2)
    return ti.Workload(w.name, w.dtype, w.B, w.Hq, w.Hkv, w.d, w.M_max, w.D_max, L, w.V, w.mode, w.parents, w.n_nodes,
                       w.prefix, w.tokens, w.q, pad(w.k), pad(w.v))


def _paged_attention(w, page_size, rng, alias=(), table_edit=None, plan=None):
    """Runs tree_verify_attention_paged on w's caches laid out in pages; returns the step
    (tables, status) and the output bits."""
    import tree_masked_verification_amd as tmv
    (kp, vp), table = ti.paged_layout(rng, [w.k, w.v], page_size, alias=alias)
    if table_edit is not None:
        table_edit(table)
    dev = DeviceStep(w)
    dev.build()
    kpd, vpd = dev_tensor(kp, True), dev_tensor(vp, True)
    tab = torch.from_numpy(table).cuda()
    dev.out.fill_(float("nan"))
    tmv.tree_verify_attention_paged(dev.q, kpd, vpd, tab, dev.prefix, dev.n_nodes, dev.anc, dev.depth, dev.status,
                                    dev.out, scale=w.scale, plan=plan)
    torch.cuda.synchronize()
    return dev, host_bits(dev.out)


def _check_against_oracle(ref, w, dev, out):
    a, d, s = dev.tables()
    ra, rd, rs = oracle_tables(ref, w)
    ref_out, ref_st = oracle_attention(ref, w, ra, rd, rs)
    assert np.array_equal(host_bits(dev.status), ref_st)
    err, rel = attention_error(out, ref_out, w.dtype)
    print("    max|err| %.3g  relL2 %.3g" % (err, rel), flush=True)
    assert err <= 2e-2 and rel <= 1e-2
    assert not np.any(np.isnan(ti.bf16_to_f32(out)))


def _contiguous_bits(w, plan=None):
    dev = DeviceStep(w)
    dev.build()
    dev.out.fill_(float("nan"))
    dev.attention(plan=plan)
    torch.cuda.synchronize()
    return host_bits(dev.out)


@pytest.mark.parametrize("page_size", [16, 32, 64, 256])
def test_paged_attention_ragged_batch(ref, page_size):
    """Prefixes 700 / 33 / 5 with 37 / 20 / 1 nodes: chunks that straddle pages, a visible
    range ending inside a page, pages past the end holding random bits (NaN included)."""
    _case("paged attention: ragged batch, page %d" % page_size)
    w = small_attention_workload(230 + page_size, 3, 8, 2, 128, 37, [700, 33, 5], [37, 20, 1], q_scale=4.0)
    dev, out = _paged_attention(w, page_size, np.random.default_rng(240 + page_size))
    _check_against_oracle(ref, w, dev, out)
    L = -(-w.L_cap // page_size) * page_size
    assert np.array_equal(out, _contiguous_bits(_padded(w, L)))


def test_paged_attention_8b_layer(ref):
    _case("paged attention: 8B-shaped layer, 16-token pages")
    w = ti.workload(2)
    dev, out = _paged_attention(w, 16, np.random.default_rng(250))
    _check_against_oracle(ref, w, dev, out)
    L = -(-w.L_cap // 16) * 16
    assert np.array_equal(out, _contiguous_bits(_padded(w, L)))


def test_paged_attention_shared_prefix_pages(ref):
    """Sequences 1-3 read sequence 0's first 20 pages (the shared ancestors' pages)."""
    _case("paged attention: shared prefix pages")
    w = small_attention_workload(260, 4, 8, 2, 128, 24, [400, 360, 330, 500], [24, 10, 3, 17], q_scale=2.0)
    for b in (1, 2, 3):
        w.k[b, :, :320] = w.k[0, :, :320]
        w.v[b, :, :320] = w.v[0, :, :320]
    dev, out = _paged_attention(w, 16, np.random.default_rng(261), alias=((0, 1, 20), (0, 2, 20), (0, 3, 20)))
    _check_against_oracle(ref, w, dev, out)


def test_paged_attention_invalid_pages(ref):
    """An invalid entry under a visible slot rejects its sequence (zero rows, INPUT); invalid
    entries past the visible range are ignored."""
    _case("paged attention: invalid table entries")
    w = _padded(small_attention_workload(270, 3, 8, 2, 128, 16, [100, 100, 100], [16, 16, 16], q_scale=2.0), 400)
    nblk = -(-w.L_cap // 16)                              # 25 pages, 8 of them visible

    def edit(table):
        table[0, 3] = -1                                  # slot 48..63: visible
        table[1, 100 // 16 + 2:] = 1 << 30                # past slot 116 + page: never visible
        table[2, 0] = table.max() + 100                   # beyond the pool

    dev, out = _paged_attention(w, 16, np.random.default_rng(271), table_edit=edit)
    st = host_bits(dev.status)
    assert st.tolist() == [ref.ERR_INPUT, 0, ref.ERR_INPUT]
    o = ti.bf16_to_f32(out)
    assert np.all(o[0] == 0) and np.all(o[2] == 0) and not np.any(np.isnan(o[1]))
    ra, rd, rs = oracle_tables(ref, w)
    ref_out, _ = oracle_attention(ref, w, ra, rd, rs)
    err, _ = attention_error(out[1:2], ref_out[1:2], w.dtype)
    assert err <= 2e-2 and nblk == 25


@pytest.mark.parametrize("page_size,nl", [(16, 2), (4, 1), (1, 1)])
def test_paged_commit(ref, page_size, nl):
    _case("paged commit: page %d, %d layers" % (page_size, nl))
    import tree_masked_verification_amd as tmv
    rng = np.random.default_rng(280 + page_size + nl)
    B, Hkv, M_max, D_max, d = 7, 2, 24, 10, 128
    n = rng.integers(1, M_max + 1, size=B).astype(np.int32)
    P = rng.integers(0, 70, size=B).astype(np.int32)
    L_cap = int((P + n).max()) + 3
    parents = np.zeros((B, M_max + 1), np.int32)
    A = np.zeros(B, np.int32)
    path = np.zeros((B, D_max), np.int32)
    for b in range(B):
        parents[b, : n[b] + 1] = random_labelled_tree(rng, int(n[b]), D_max)
        pn = _path_of(parents[b], int(rng.integers(0, n[b] + 1)))
        A[b], path[b, : len(pn)] = len(pn), pn
    kh = rng.integers(0, 65536, size=(nl, B, Hkv, L_cap, d)).astype(np.uint16)
    vh = rng.integers(0, 65536, size=(nl, B, Hkv, L_cap, d)).astype(np.uint16)
    (kp, vp), table = ti.paged_layout(rng, [kh, vh], page_size)
    bad = B - 1                                         # a moving row's page is invalid
    w = ti.Workload("commit", ti.BF16, B, 0, Hkv, d, M_max, D_max, L_cap, 1, "greedy", parents, n, P,
                    np.zeros((B, M_max + 1), np.int32))
    dev = DeviceStep(w)
    dev.build()
    moving = [j for j in range(A[bad]) if path[bad, j] - 1 != j]
    if moving:
        table[bad, (P[bad] + moving[0]) // page_size] = -3
    dev.accept_len.copy_(torch.from_numpy(A).cuda())
    dev.path.copy_(torch.from_numpy(path).cuda())
    kpd, vpd = dev_tensor(kp, True), dev_tensor(vp, True)
    tmv.kv_commit_path_paged(kpd, vpd, torch.from_numpy(table).cuda(), dev.prefix, dev.n_nodes, dev.accept_len,
                             dev.path, dev.status, dev.new_len, M_max)
    torch.cuda.synchronize()
    ra, rd, rs = oracle_tables(ref, w)
    kr, vr = kh.copy(), vh.copy()
    if moving:
        rs = rs.copy()
        rs[bad] = ref.ERR_INPUT                          # the oracle leaves a failed sequence alone
    new_len, st = ref.commit(kr, vr, P, n, A, path, rs, M_max)
    kg, vg = host_bits(kpd), host_bits(vpd)
    assert np.array_equal(host_bits(dev.new_len), new_len) and np.array_equal(host_bits(dev.status), st)
    for b in range(B):
        for t in range(L_cap):
            pg, r = table[b, t // page_size], t % page_size
            if pg < 0:
                continue
            assert np.array_equal(kg[:, pg, :, r], kr[:, b, :, t]) and np.array_equal(vg[:, pg, :, r], vr[:, b, :, t])


@pytest.mark.parametrize("page_size,capacity", [(16, 1000), (4, 1000), (1, 1000), (4, 3)])
def test_paged_commit_evict(ref, page_size, capacity):
    """The commit with block eviction: rows as the oracle's commit through the kept entries,
    the rewritten table and the freed pages as the oracle's eviction rule (or, with a short
    free list, exactly the entries that fit)."""
    _case("paged commit with eviction: page %d, free-list capacity %d" % (page_size, capacity))
    import tree_masked_verification_amd as tmv
    rng = np.random.default_rng(330 + page_size + capacity)
    B, Hkv, M_max, D_max, d, nl = 6, 2, 24, 10, 128, 2
    n = rng.integers(1, M_max + 1, size=B).astype(np.int32)
    P = rng.integers(0, 70, size=B).astype(np.int32)
    L_cap = int((P + n).max()) + 3
    parents = np.zeros((B, M_max + 1), np.int32)
    A = np.zeros(B, np.int32)
    path = np.zeros((B, D_max), np.int32)
    for b in range(B):
        parents[b, : n[b] + 1] = random_labelled_tree(rng, int(n[b]), D_max)
        pn = _path_of(parents[b], int(rng.integers(0, n[b] + 1)))
        A[b], path[b, : len(pn)] = len(pn), pn
    kh = rng.integers(0, 65536, size=(nl, B, Hkv, L_cap, d)).astype(np.uint16)
    vh = rng.integers(0, 65536, size=(nl, B, Hkv, L_cap, d)).astype(np.uint16)
    (kp, vp), table = ti.paged_layout(rng, [kh, vh], page_size)
    w = ti.Workload("commit", ti.BF16, B, 0, Hkv, d, M_max, D_max, L_cap, 1, "greedy", parents, n, P,
                    np.zeros((B, M_max + 1), np.int32))
    dev = DeviceStep(w)
    dev.build()
    dev.accept_len.copy_(torch.from_numpy(A).cuda())
    dev.path.copy_(torch.from_numpy(path).cuda())
    kpd, vpd = dev_tensor(kp, True), dev_tensor(vp, True)
    tab = torch.from_numpy(table.copy()).cuda()
    freed = torch.full((capacity,), -5, dtype=torch.int32, device="cuda")
    count = torch.zeros((1,), dtype=torch.int32, device="cuda")
    tmv.kv_commit_path_paged_evict(kpd, vpd, tab, dev.prefix, dev.n_nodes, dev.accept_len, dev.path, dev.status,
                                   dev.new_len, M_max, freed, count)
    torch.cuda.synchronize()
    ra, rd, rs = oracle_tables(ref, w)
    kr, vr = kh.copy(), vh.copy()
    new_len, st = ref.commit(kr, vr, P, n, A, path, rs, M_max)
    assert np.array_equal(host_bits(dev.new_len), new_len) and np.array_equal(host_bits(dev.status), st)
    rtab, rfreed = ref.commit_paged_table(table, page_size, kp.shape[1], P, n, new_len, st)
    t2, fr, cnt = host_bits(tab), host_bits(freed), int(host_bits(count)[0])
    assert cnt == len(rfreed)
    if capacity >= len(rfreed):
        assert np.array_equal(t2, rtab) and sorted(fr[:cnt].tolist()) == rfreed
    else:
        # the first `capacity` evictions happened, the rest kept their entries
        cleared = (t2 == -1) & (table != -1)
        assert int(cleared.sum()) == capacity
        assert sorted(table[cleared].tolist()) == sorted(fr.tolist())
        assert np.all((t2 == table) | cleared) and np.all(rtab[cleared] == -1)
    # every kept slot below the new length holds the committed rows
    kg, vg = host_bits(kpd), host_bits(vpd)
    for b in range(B):
        for t in range(int(new_len[b])):
            pg, r = t2[b, t // page_size], t % page_size
            assert pg >= 0
            assert np.array_equal(kg[:, pg, :, r], kr[:, b, :, t]) and np.array_equal(vg[:, pg, :, r], vr[:, b, :, t])


@pytest.mark.parametrize("plan", [(64, 3), (128, 1), (128, 2), (256, 5), (64, 16)])
def test_paged_attention_launch_plans(ref, plan):
    """Every row-group width of the paged kernel (a pinned plan), against the oracle and
    bit-identical to the contiguous kernel under the same plan."""
    _case("paged attention: plan %s" % (plan,))
    w = small_attention_workload(290, 2, 16, 2, 128, 40, [600, 70], [40, 33], q_scale=3.0)
    dev, out = _paged_attention(w, 16, np.random.default_rng(291), plan=plan)
    _check_against_oracle(ref, w, dev, out)
    L = -(-w.L_cap // 16) * 16
    assert np.array_equal(out, _contiguous_bits(_padded(w, L), plan=plan))


def test_paged_attention_deep_trees(ref):
    """Trees deeper than the ancestor entries fetched in the prologue (the deep kernels)."""
    _case("paged attention: a 48-deep chain and a random tree, 32-token pages")
    w = small_attention_workload(295, 2, 8, 2, 128, 48, [300, 45], [48, 30], q_scale=3.0, max_depth=48)
    w.parents[0] = ti.tree_chain(48)
    dev, out = _paged_attention(w, 32, np.random.default_rng(296))
    _check_against_oracle(ref, w, dev, out)
    assert int(dev.tables()[1].max()) > 16


@pytest.mark.parametrize("page_size", [16, 128])
def test_paged_attention_adaptive_splits(ref, page_size):
    """The ragged batch of the adaptive plan (per-sequence splits) through the block table:
    against the oracle and bit-identical to the contiguous kernel."""
    _case("paged attention: ragged batch with per-sequence splits, page %d" % page_size)
    w = adaptive_workload(300 + page_size)
    L = -(-w.L_cap // page_size) * page_size
    wp = _padded(w, L)
    dev, out = _paged_attention(wp, page_size, np.random.default_rng(310 + page_size))
    _check_against_oracle(ref, wp, dev, out)
    assert np.array_equal(out, _contiguous_bits(wp))
