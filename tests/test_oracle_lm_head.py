"""Pins of the oracle's LM-head logits (the projection whose per-row argmax is the
teacher's greedy choice; roofline section of "Speculative Decoding Hierarquico" for why it
is fused with the argmax).  The oracle's sums are checked against exact integer
arithmetic, against numpy's fp64 product, on a hand case, and the accumulation-error
bound the device comparison uses is checked against simulated fp32 accumulations."""
import numpy as np

import oracle
import tmv_inputs as ti


def _bf16(a):
    return ti.bf16_bits(np.asarray(a, np.float32))


def test_hand_case():
    h = _bf16([[1.0, 2.0]])
    w = _bf16([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [-1.0, 3.0]])
    logits, bound = oracle.lm_head_logits(h, w)
    assert logits.tolist() == [[1.0, 2.0, 3.0, 5.0]]
    assert bound.tolist() == [[1.0, 2.0, 3.0, 7.0]]


def test_small_integers_are_exact():
    # integers of magnitude <= 16 are exact in bf16 and every partial sum is exact in fp64
    rng = np.random.default_rng(71)
    h = rng.integers(-16, 17, (5, 96)).astype(np.float32)
    w = rng.integers(-16, 17, (333, 96)).astype(np.float32)
    logits, bound = oracle.lm_head_logits(_bf16(h), _bf16(w))
    ref = h.astype(np.int64) @ w.astype(np.int64).T
    assert np.array_equal(logits, ref.astype(np.float64))
    assert np.array_equal(bound, (np.abs(h).astype(np.int64) @ np.abs(w).astype(np.int64).T).astype(np.float64))


def test_matches_numpy_fp64_product():
    rng = np.random.default_rng(72)
    hb = _bf16(rng.standard_normal((7, 256)))
    wb = _bf16(rng.standard_normal((1000, 256)) * 0.05)
    logits, bound = oracle.lm_head_logits(hb, wb)
    ref = ti.bf16_to_f32(hb).astype(np.float64) @ ti.bf16_to_f32(wb).astype(np.float64).T
    assert np.all(np.abs(logits - ref) <= 1e-12 * bound)
    # ties: equal weight rows give equal logits; argmax takes the smallest index
    w2 = np.concatenate([wb[:3], wb[1:2]], axis=0)
    l2, _ = oracle.lm_head_logits(hb[:1], w2)
    assert l2[0, 1] == l2[0, 3] and int(np.argmax(l2[0])) in (0, 1, 2)


def test_fp32_accumulation_stays_within_the_bound():
    # any fp32 accumulation order (sequential, reversed, pairwise blocks of 32 like one MFMA
    # k-step) differs from the fp64 sum by at most K * 2^-24 * sum |h w|
    rng = np.random.default_rng(73)
    K = 512
    hb = _bf16(rng.standard_normal((3, K)))
    wb = _bf16(rng.standard_normal((200, K)) * 0.05)
    logits, bound = oracle.lm_head_logits(hb, wb)
    h = ti.bf16_to_f32(hb)
    w = ti.bf16_to_f32(wb)
    eps = K * 2.0 ** -24 * bound
    prods = h[:, None, :] * w[None, :, :]                      # exact in fp32 (bf16 x bf16)
    seq = np.zeros(prods.shape[:2], np.float32)
    for k in range(K):
        seq = seq + prods[:, :, k]
    rev = np.zeros(prods.shape[:2], np.float32)
    for k in reversed(range(K)):
        rev = rev + prods[:, :, k]
    blk = np.zeros(prods.shape[:2], np.float32)
    for k0 in range(0, K, 32):
        blk = blk + prods[:, :, k0:k0 + 32].sum(axis=2, dtype=np.float32)
    for acc in (seq, rev, blk):
        assert np.all(np.abs(acc.astype(np.float64) - logits) <= eps)
