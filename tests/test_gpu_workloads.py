"""Full-size workloads in the launch configuration the benchmark uses.

The oracle cannot afford every attention row of the long-prefix workloads, so:
  * sampled nodes (all their query heads) are compared against the oracle row by row;
  * the same trees with an empty prefix (where a mask error changes outputs by O(1))
    are compared on every row;
  * properties that hold at any size are checked on every row: inert rows are exactly
    zero, live rows are finite."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import tmv_inputs as ti
from tests.harness import DeviceStep, attention_error, host_bits, oracle_attention, oracle_tables

pytestmark = pytest.mark.gpu


def _case(name):
    print("\n[gpu case] %s" % name, flush=True)


def _sampled_rows(w, anc, depth, per_seq, seed):
    """The deepest node of every sequence plus `per_seq` random live nodes."""
    rng = np.random.default_rng(seed)
    sel = np.zeros((w.B, w.M_max), np.uint8)
    for b in range(w.B):
        live = [j for j in range(1, int(w.n_nodes[b]) + 1) if depth[b, j] >= 1]
        deepest = max(live, key=lambda j: (depth[b, j], -j))
        sel[b, deepest - 1] = 1
        for j in rng.choice(live, size=min(per_seq, len(live)), replace=False):
            sel[b, int(j) - 1] = 1
    return sel


def _oracle_rows(ref, w, ra, rd, rs, sel, threads=8):
    """The oracle on the selected rows, dealt round-robin to threads (the oracle's C
    routine runs without the interpreter lock)."""
    rows = np.argwhere(sel)
    n = max(1, min(threads, len(rows)))
    parts = []
    for t in range(n):
        s = np.zeros_like(sel)
        for b, j in rows[t::n]:
            s[b, j] = 1
        parts.append(s)

    def one(s):
        return s, oracle_attention(ref, w, ra, rd, rs, row_select=s)[0]

    out = None
    with ThreadPoolExecutor(len(parts)) as ex:
        for s, o in ex.map(one, parts):
            if out is None:
                out = o
            else:
                out[s.astype(bool)] = o[s.astype(bool)]
    return out


def _run(ref, w, per_seq, seed, all_rows=False, only_seq=None, threads=8):
    dev = DeviceStep(w)
    dev.build()
    dev.attention()
    a, d, s = dev.tables()
    ra, rd, rs = oracle_tables(ref, w)
    assert np.array_equal(a, ra) and np.array_equal(s, rs) and np.all(rs == 0)
    out = host_bits(dev.out)
    outf = ti.bf16_to_f32(out)
    live = np.zeros((w.B, w.M_max), bool)
    for b in range(w.B):
        for j in range(1, w.M_max + 1):
            live[b, j - 1] = j <= w.n_nodes[b] and rd[b, j] >= 1
    assert np.all(outf[~live] == 0) and np.all(np.isfinite(outf[live]))
    sel = np.ones((w.B, w.M_max), np.uint8) * live if all_rows else _sampled_rows(w, ra, rd, per_seq, seed)
    if only_seq is not None:
        sel[np.arange(w.B) != only_seq] = 0
    ref_out = _oracle_rows(ref, w, ra, rd, rs, sel, threads)
    mask = np.zeros(out.shape, bool)
    mask[sel.astype(bool)] = True
    err, rel = attention_error(out, ref_out, w.dtype, mask)
    print("    rows %d  max|err| %.3g  relL2 %.3g" % (int(sel.sum()), err, rel), flush=True)
    assert err <= 2e-2 and rel <= 1e-2


def test_batched_dynamic_trees_sampled(ref):
    _case("attention: batched dynamic trees (config 3), sampled nodes")
    w = ti.workload(3, with_rows=False)
    _run(ref, w, per_seq=6, seed=31)


def test_batched_dynamic_trees_all_rows(ref):
    """Every row of the batched workload with its prefixes: the ragged plan's per-sequence
    splits and split merges at full size."""
    _case("attention: batched dynamic trees (config 3), every row")
    w = ti.workload(3, with_rows=False)
    _run(ref, w, 0, 0, all_rows=True)


def test_batched_dynamic_trees_empty_prefix_all_rows(ref):
    _case("attention: batched dynamic trees, empty prefix, sharpened, every row")
    w = ti.workload(3, with_rows=False)
    w.prefix[:] = 0
    w.q = ti.bf16_bits(ti.bf16_to_f32(w.q) * 8.0)
    _run(ref, w, 0, 0, all_rows=True)


def test_long_context_70b_sampled(ref):
    _case("attention: 70B-shaped layer, prefix 32768 (config 4), sampled nodes")
    w = ti.workload(4, with_rows=False)
    _run(ref, w, per_seq=4, seed=41)


def test_long_context_70b_one_sequence_all_rows(ref):
    """Every row of one sequence (64 nodes x 64 query heads) with its whole 32768-token
    prefix, the oracle's rows dealt over 16 threads."""
    _case("attention: 70B-shaped layer, prefix 32768 (config 4), every row of sequence 1")
    w = ti.workload(4, with_rows=False)
    _run(ref, w, 0, 0, all_rows=True, only_seq=1, threads=16)


def test_long_context_70b_empty_prefix_all_rows(ref):
    _case("attention: 70B-shaped layer, empty prefix, sharpened, every row")
    w = ti.workload(4, with_rows=False)
    w.prefix[:] = 0
    w.q = ti.bf16_bits(ti.bf16_to_f32(w.q) * 8.0)
    _run(ref, w, 0, 0, all_rows=True)


def test_greedy_batched_dynamic(ref):
    _case("greedy: batched dynamic trees (config 3)")
    w = ti.workload(3)
    dev = DeviceStep(w)
    dev.build()
    dev.accept()
    torch.cuda.synchronize()
    ra, rd, rs = oracle_tables(ref, w)
    A, path, nxt, st = ref.accept_greedy(w.tokens, w.logits, w.n_nodes, ra, rd, rs)
    assert np.array_equal(host_bits(dev.accept_len), A) and np.array_equal(host_bits(dev.path), path)
    assert np.array_equal(host_bits(dev.next_token), nxt) and np.array_equal(host_bits(dev.status), st)
    print("    accept lengths", A.tolist(), flush=True)
