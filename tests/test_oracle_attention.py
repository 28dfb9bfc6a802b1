"""Pins of the oracle's tree-masked attention.

Independent evidence: torch's scaled_dot_product_attention (CPU, float64) over the
linear sequence prefix + path(k) with an ordinary causal mask, which must equal tree
attention for every node on the path; closed forms (P = 0 gives the node's own V);
relabelling and head-repetition invariances."""
import numpy as np
import torch

import tmv_inputs as ti


def path_of(par, i):
    out = []
    while i:
        out.append(i)
        i = int(par[i])
    return out[::-1]            # depth-1 node first


def make_case(rng, B, Hq, Hkv, d, M, P_list, L_cap, max_depth=5, sigma=1.0):
    trees = [ti.tree_random(rng, M, max_depth) for _ in range(B)]
    parents = np.zeros((B, M + 1), np.int32)
    for b in range(B):
        parents[b] = trees[b]
    q = rng.standard_normal((B, M, Hq, d)).astype(np.float32) * sigma
    k = rng.standard_normal((B, Hkv, L_cap, d)).astype(np.float32) * sigma
    v = rng.standard_normal((B, Hkv, L_cap, d)).astype(np.float32) * sigma
    return parents, np.full(B, M, np.int32), np.array(P_list, np.int32), q, k, v


def run_oracle(ref, parents, n, P, q, k, v, D_max, dtype=0):
    B, M = parents.shape[0], parents.shape[1] - 1
    anc, depth, st = ref.build_ancestors(parents, n, M, D_max)
    assert np.all(st == 0)
    Hkv = k.shape[1]
    d = q.shape[3]
    out, st2 = ref.tree_attention(q, k, v, P, n, anc, depth, st, 1.0 / np.sqrt(d), dtype, Hkv)
    return out, st2


def test_linear_sequence_equivalence(ref):
    rng = np.random.default_rng(11)
    B, Hq, Hkv, d, M = 3, 4, 2, 16, 12
    P = [0, 5, 37]
    L_cap = 37 + M + 3
    parents, n, Pa, q, k, v = make_case(rng, B, Hq, Hkv, d, M, P, L_cap)
    out, _ = run_oracle(ref, parents, n, Pa, q, k, v, D_max=6)
    g = Hq // Hkv
    for b in range(B):
        for i in range(1, M + 1):
            path = path_of(parents[b], i)
            slots = list(range(P[b])) + [P[b] + j - 1 for j in path]
            L = len(slots)
            for h in range(Hq):
                kv = h // g
                Kseq = torch.tensor(k[b, kv, slots], dtype=torch.float64)[None, None]
                Vseq = torch.tensor(v[b, kv, slots], dtype=torch.float64)[None, None]
                Qp = torch.tensor(np.stack([q[b, j - 1, h] for j in path]), dtype=torch.float64)[None, None]
                # query r (the node at depth r+1) sees keys 0 .. P+r: plain causal order
                mask = torch.zeros(len(path), L, dtype=torch.bool)
                for r in range(len(path)):
                    mask[r, : P[b] + r + 1] = True
                ref_out = torch.nn.functional.scaled_dot_product_attention(Qp, Kseq, Vseq, attn_mask=mask,
                                                                           scale=1.0 / np.sqrt(d))[0, 0]
                for r, j in enumerate(path):
                    np.testing.assert_allclose(out[b, j - 1, h], ref_out[r].numpy(), rtol=0, atol=1e-12)


def test_chain_is_full_causal_attention(ref):
    rng = np.random.default_rng(12)
    M, P, d = 9, 6, 8
    parents = ti.tree_chain(M)[None, :]
    q = rng.standard_normal((1, M, 1, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, P + M, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, P + M, d)).astype(np.float32)
    out, _ = run_oracle(ref, parents, np.array([M]), np.array([P]), q, k, v, D_max=M)
    Q = torch.zeros(1, 1, P + M, d, dtype=torch.float64)
    Q[0, 0, P:] = torch.tensor(q[0, :, 0], dtype=torch.float64)
    Kt = torch.tensor(k, dtype=torch.float64)
    Vt = torch.tensor(v, dtype=torch.float64)
    full = torch.nn.functional.scaled_dot_product_attention(Q, Kt, Vt, is_causal=True, scale=1 / np.sqrt(d))
    np.testing.assert_allclose(out[0, :, 0], full[0, 0, P:].numpy(), rtol=0, atol=1e-12)


def test_empty_prefix_depth_one_sees_only_itself(ref):
    rng = np.random.default_rng(13)
    parents, n, _, q, k, v = make_case(rng, 2, 2, 1, 8, 10, [0, 0], 10)
    out, _ = run_oracle(ref, parents, n, np.zeros(2, np.int32), q, k, v, D_max=5)
    for b in range(2):
        for i in range(1, 11):
            if parents[b, i] == 0:
                for h in range(2):
                    assert np.array_equal(out[b, i - 1, h], v[b, 0, i - 1].astype(np.float64))


def test_relabelling_permutes_outputs(ref):
    rng = np.random.default_rng(14)
    M, P, d = 11, 7, 8
    parents, n, Pa, q, k, v = make_case(rng, 1, 2, 2, d, M, [P], P + M)
    perm = np.concatenate([[0], rng.permutation(M) + 1])        # node i -> perm[i]
    par2 = np.zeros_like(parents)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for i in range(1, M + 1):
        par2[0, perm[i]] = perm[parents[0, i]]
        q2[0, perm[i] - 1] = q[0, i - 1]
        k2[0, :, P + perm[i] - 1] = k[0, :, P + i - 1]
        v2[0, :, P + perm[i] - 1] = v[0, :, P + i - 1]
    o1, _ = run_oracle(ref, parents, n, Pa, q, k, v, D_max=6)
    o2, _ = run_oracle(ref, par2, n, Pa, q2, k2, v2, D_max=6)
    for i in range(1, M + 1):
        np.testing.assert_allclose(o2[0, perm[i] - 1], o1[0, i - 1], rtol=0, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv(ref):
    rng = np.random.default_rng(15)
    parents, n, Pa, q, k, v = make_case(rng, 2, 6, 2, 8, 8, [3, 9], 20)
    o1, _ = run_oracle(ref, parents, n, Pa, q, k, v, D_max=5)
    o2, _ = run_oracle(ref, parents, n, Pa, q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), D_max=5)
    assert np.array_equal(o1, o2)


def test_bf16_inputs_widen_exactly(ref):
    rng = np.random.default_rng(16)
    parents, n, Pa, q, k, v = make_case(rng, 1, 4, 2, 16, 9, [20], 32)
    qb, kb, vb = ti.bf16_bits(q), ti.bf16_bits(k), ti.bf16_bits(v)
    o_bf, _ = run_oracle(ref, parents, n, Pa, qb, kb, vb, D_max=5, dtype=1)
    o_f, _ = run_oracle(ref, parents, n, Pa, ti.bf16_to_f32(qb), ti.bf16_to_f32(kb), ti.bf16_to_f32(vb), D_max=5)
    assert np.array_equal(o_bf, o_f)


def test_inert_rows_and_prefix_overflow(ref):
    rng = np.random.default_rng(17)
    parents, n, Pa, q, k, v = make_case(rng, 3, 2, 1, 8, 6, [2, 2, 2], 10)
    anc, depth, st = ref.build_ancestors(parents, np.array([6, 3, 6]), 6, 6)
    st = st.copy()
    st[2] = ref.ERR_CYCLE                                      # an upstream failure
    out, st2 = ref.tree_attention(q, k, v, np.array([2, 2, 5]), np.array([6, 3, 6]), anc, depth, st,
                                  0.3, 0, 1)
    assert np.all(out[1, 3:] == 0) and np.any(out[1, :3] != 0)  # nodes beyond M_b are inert
    assert np.all(out[2] == 0) and st2[2] == ref.ERR_CYCLE
    out, st3 = ref.tree_attention(q, k, v, np.array([2, 2, 5]), np.array([6, 3, 6]), anc, depth,
                                  np.zeros(3, np.int32), 0.3, 0, 1)
    assert st3.tolist() == [0, 0, ref.ERR_INPUT] and np.all(out[2] == 0)   # 5 + 6 > L_cap = 10
