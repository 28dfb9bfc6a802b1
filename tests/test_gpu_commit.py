"""Device parity of kv_commit_path against the oracle: the committed cache layout must be
bit-identical (every row of small caches; windows around the tree rows, plus the whole
prefix against its known contents, for the 32-layer sampling workload)."""
import numpy as np
import pytest
import torch

import tmv_inputs as ti
from tests.harness import DeviceStep, dev_tensor, host_bits, oracle_tables
from tests.test_oracle_build import random_labelled_tree

pytestmark = pytest.mark.gpu


def _case(name):
    print("\n[gpu case] %s" % name, flush=True)


def _path_of(par, leaf):
    out = []
    while leaf:
        out.append(leaf)
        leaf = int(par[leaf])
    return out[::-1]


@pytest.mark.parametrize("dtype,d,nl", [(ti.BF16, 128, 3), (ti.F32, 64, 2), (ti.BF16, 64, 1), (ti.F32, 128, 1)])
def test_commit_small_caches(ref, dtype, d, nl):
    _case("commit: dtype=%d d=%d layers=%d" % (dtype, d, nl))
    rng = np.random.default_rng(500 + d + nl)
    B, Hkv, M_max, D_max = 9, 3, 24, 10
    n = rng.integers(0, M_max + 1, size=B).astype(np.int32)
    P = rng.integers(0, 50, size=B).astype(np.int32)
    L_cap = int((P + n).max()) + 7
    parents = np.zeros((B, M_max + 1), np.int32)
    A = np.zeros(B, np.int32)
    path = np.zeros((B, D_max), np.int32)
    for b in range(B):
        parents[b, : n[b] + 1] = random_labelled_tree(rng, int(n[b]), D_max)     # ids not topological
        leaf = int(rng.integers(0, n[b] + 1))
        pn = _path_of(parents[b], leaf)
        A[b] = len(pn)
        path[b, : len(pn)] = pn
    # a fully accepted chain (nothing moves) and a misfit sequence
    parents[0, :] = 0
    parents[0, : 11] = ti.tree_chain(10)
    n[0], A[0] = 10, 10
    path[0] = np.arange(1, 11)
    P[8] = L_cap - 1                                  # P + M > L_cap -> INPUT
    edt = np.float32 if dtype == ti.F32 else np.uint16
    shape = (nl, B, Hkv, L_cap, d)
    if dtype == ti.F32:
        kh = rng.standard_normal(shape).astype(np.float32)
        vh = rng.standard_normal(shape).astype(np.float32)
    else:
        kh = rng.integers(0, 65536, size=shape).astype(np.uint16)
        vh = rng.integers(0, 65536, size=shape).astype(np.uint16)
    w = ti.Workload("commit", dtype, B, 0, Hkv, d, M_max, D_max, L_cap, 1, "greedy", parents, n, P,
                    np.zeros((B, M_max + 1), np.int32))
    dev = DeviceStep(w)
    dev.build()
    dev.accept_len.copy_(torch.from_numpy(A).cuda())
    dev.path.copy_(torch.from_numpy(path).cuda())
    kd, vd = dev_tensor(kh, dtype == ti.BF16), dev_tensor(vh, dtype == ti.BF16)
    dev.commit(kd, vd)
    torch.cuda.synchronize()
    ra, rd, rs = oracle_tables(ref, w)
    kr, vr = kh.copy(), vh.copy()
    new_len, st = ref.commit(kr, vr, P, n, A, path, rs, M_max)
    assert np.array_equal(host_bits(dev.new_len), new_len) and np.array_equal(host_bits(dev.status), st)
    assert st[8] == ref.ERR_INPUT
    assert np.array_equal(host_bits(kd), kr) and np.array_equal(host_bits(vd), vr)
    assert np.array_equal(kr[:, 0], kh[:, 0])        # full chain accept moved nothing


@pytest.mark.parametrize("dtype,A_len", [(ti.BF16, 17), (ti.BF16, 40), (ti.F32, 9), (ti.F32, 30)])
def test_commit_long_paths_take_several_passes(ref, dtype, A_len):
    """Paths long enough that a (layer, sequence)'s moving rows over its 8 KV heads and both
    caches do not fit one LDS snapshot: more than 16 rows of bf16 d128 or 8 rows of fp32
    d128 are snapshotted and written in several passes."""
    _case("commit: %d-row path, dtype=%d, 8 KV heads, d128" % (A_len, dtype))
    rng = np.random.default_rng(600 + A_len + dtype)
    B, Hkv, d, nl = 3, 8, 128, 2
    M_max, D_max = 64, 48
    n = np.array([M_max, 50, A_len], np.int32)
    P = np.array([5, 0, 33], np.int32)
    L_cap = int((P + n).max()) + 4
    parents = np.zeros((B, M_max + 1), np.int32)
    A = np.zeros(B, np.int32)
    path = np.zeros((B, D_max), np.int32)
    for b in range(B):
        # a chain of A_len nodes under random labels (so almost every row moves), the rest
        # hanging off it
        labels = rng.permutation(np.arange(1, n[b] + 1))
        chain = labels[:A_len]
        par = np.zeros(n[b] + 1, np.int32)
        for i, c in enumerate(chain):
            par[c] = 0 if i == 0 else chain[i - 1]
        for c in labels[A_len:]:
            par[c] = chain[int(rng.integers(0, min(A_len, D_max - 1)))]
        parents[b, : n[b] + 1] = par
        A[b] = A_len
        path[b, :A_len] = chain
    edt = np.float32 if dtype == ti.F32 else np.uint16
    shape = (nl, B, Hkv, L_cap, d)
    if dtype == ti.F32:
        kh = rng.standard_normal(shape).astype(np.float32)
        vh = rng.standard_normal(shape).astype(np.float32)
    else:
        kh = rng.integers(0, 65536, size=shape).astype(np.uint16)
        vh = rng.integers(0, 65536, size=shape).astype(np.uint16)
    w = ti.Workload("commit", dtype, B, 0, Hkv, d, M_max, D_max, L_cap, 1, "greedy", parents, n, P,
                    np.zeros((B, M_max + 1), np.int32))
    dev = DeviceStep(w)
    dev.build()
    dev.accept_len.copy_(torch.from_numpy(A).cuda())
    dev.path.copy_(torch.from_numpy(path).cuda())
    kd, vd = dev_tensor(kh, dtype == ti.BF16), dev_tensor(vh, dtype == ti.BF16)
    dev.commit(kd, vd)
    torch.cuda.synchronize()
    ra, rd, rs = oracle_tables(ref, w)
    assert np.all(rs == 0) and np.all(rd.max(axis=1) >= A_len)
    kr, vr = kh.copy(), vh.copy()
    new_len, st = ref.commit(kr, vr, P, n, A, path, rs, M_max)
    moving = [int(np.sum(path[b, :A_len] - 1 != np.arange(A_len))) for b in range(B)]
    row_bytes = d * (4 if dtype == ti.F32 else 2)
    assert max(moving) * row_bytes * 2 * Hkv > 64 * 1024      # several snapshot passes
    assert np.array_equal(host_bits(dev.new_len), new_len) and np.array_equal(host_bits(dev.status), st)
    assert np.array_equal(host_bits(kd), kr) and np.array_equal(host_bits(vd), vr)


def test_commit_no_layers_publishes_lengths(ref):
    _case("commit: zero layers")
    import tree_masked_verification_amd as tmv
    B = 3
    empty = torch.zeros((0, B, 2, 8, 64), dtype=torch.bfloat16, device="cuda")
    P = torch.tensor([3, 4, 5], dtype=torch.int32, device="cuda")
    n = torch.tensor([2, 2, 2], dtype=torch.int32, device="cuda")
    A = torch.tensor([1, 2, 0], dtype=torch.int32, device="cuda")
    path = torch.tensor([[1, 0], [1, 2], [0, 0]], dtype=torch.int32, device="cuda")
    st = torch.zeros(B, dtype=torch.int32, device="cuda")
    nl = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    tmv.kv_commit_path(empty, empty, P, n, A, path, st, nl, M_max=2)
    assert nl.tolist() == [4, 6, 5] and st.tolist() == [0, 0, 0]


def _fill_pattern(cache, layer_offset=0):
    """cache [L][B][H][S][d] bf16 filled with tmv_inputs.cache_pattern_value (exact)."""
    L, B, H, S, d = cache.shape
    dev = cache.device
    bb = torch.arange(B, device=dev).view(B, 1, 1, 1)
    hh = torch.arange(H, device=dev).view(1, H, 1, 1)
    ss = torch.arange(S, device=dev).view(1, 1, S, 1)
    dd = torch.arange(d, device=dev).view(1, 1, 1, d)
    for l in range(L):
        val = ((l + layer_offset) * 7 + bb * 5 + hh * 3 + ss) % 251 - 125 + (dd % 2) * 0.5
        cache[l].copy_(val.to(torch.bfloat16))


def test_commit_sampling_workload_32_layers(ref):
    """Workload 5: accept by sampling, then commit over 32 layers x 32 sequences x 8 KV
    heads x 4128 slots x d128 (two 8.66 GB caches)."""
    _case("commit: workload 5, 32 layers")
    w = ti.workload(5)
    dev = DeviceStep(w)
    dev.build()
    dev.accept()
    L, B, H, d = w.n_layers, w.B, w.Hkv, w.d
    S = w.L_cap
    kc = torch.empty((L, B, H, S, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    _fill_pattern(kc)
    _fill_pattern(vc, layer_offset=100)
    P0, M = int(w.prefix[0]), w.M_max
    lo, hi = P0 - 1, P0 + M                           # window [P-1, P+M] of every (layer, b, head)
    win_k = host_bits(kc[:, :, :, lo:hi + 1]).copy()
    win_v = host_bits(vc[:, :, :, lo:hi + 1]).copy()
    dev.commit(kc, vc)
    torch.cuda.synchronize()
    ra, rd, rs = oracle_tables(ref, w)
    A, path, nxt, st = ref.accept_sample(w.tokens, w.p, w.qd, w.seed, w.step, w.n_nodes, ra, rd, rs)
    assert np.array_equal(host_bits(dev.accept_len), A) and np.array_equal(host_bits(dev.path), path)
    # the window holds slot P-1 at index 0, so its committed prefix length is 1
    wk, wv = np.ascontiguousarray(win_k), np.ascontiguousarray(win_v)
    new_len, st2 = ref.commit(wk, wv, np.ones(B, np.int32), w.n_nodes, A, path, st, M)
    assert np.array_equal(host_bits(dev.new_len), new_len + P0 - 1)
    assert np.array_equal(host_bits(kc[:, :, :, lo:hi + 1]), wk)
    assert np.array_equal(host_bits(vc[:, :, :, lo:hi + 1]), wv)
    # everything outside the windows is untouched: compare against the known pattern
    ref_k = torch.empty((1, B, H, S, d), dtype=torch.bfloat16, device="cuda")
    for l in range(L):
        _fill_pattern(ref_k, layer_offset=l)
        assert torch.equal(kc[l, :, :, :lo], ref_k[0, :, :, :lo]) and torch.equal(kc[l, :, :, hi + 1:], ref_k[0, :, :, hi + 1:])
        _fill_pattern(ref_k, layer_offset=100 + l)
        assert torch.equal(vc[l, :, :, :lo], ref_k[0, :, :, :lo])
    print("    mean accept length %.3f" % float(A.mean()), flush=True)
