"""Seeded synthetic inputs for the tree-verification step.

This module only draws random numbers and lays them out; it holds none of the method's
arithmetic (no ancestor walks, no masking, no softmax attention, no acceptance rule, no
commit).  Both the oracle-side tests and the device-side tests and benchmark take their
inputs from here, so the two sides see the same bytes.

Layouts (shared by every consumer):
  parents   int32 [B][M_max+1]     virtual-root form: column 0 unused, parent of node i
  n_nodes   int32 [B]              M_b
  prefix    int32 [B]              committed prefix length P_b
  q         [B][M_max][Hq][d]      query of node r+1 in row r
  k, v      [B][Hkv][L_cap][d]     node j's K/V at slot P_b + j - 1
  logits    f32 [B][M_max+1][V]    teacher logits; row 0 follows the prefix, row u node u
  tokens    int32 [B][M_max+1]     draft token of node i (column 0 unused)
  p, qd     f32 [B][M_max+1][V]    teacher / draft distributions (sampling workloads)
bf16 tensors are stored as uint16 bit patterns (round to nearest even from fp32).

The five workloads follow the configuration list of the benchmark specification
(sizes, distributions and tree shapes); ``workload(c)`` builds number ``c`` (1..5).
Random streams: ``numpy.random.default_rng(1000 + c)`` unless a seed is given.
"""
from __future__ import annotations

import heapq
import itertools
from dataclasses import dataclass, field

import numpy as np

F32, BF16 = 0, 1


# ------------------------------------------------------------------ bf16 bit patterns
def bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest even; NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # finite values cannot overflow 32 bits here (largest is 0xFF7FFFFF + 0x8000)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    out[np.isnan(x)] = 0x7FC0
    return out


def bf16_to_f32(bits) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ tree shapes
def tree_complete(branching: int, levels: int) -> np.ndarray:
    """Complete tree with `levels` levels below (and including) one draft root node,
    hung under the virtual root 0.  IDs breadth-first.  Returns parents[0..M]."""
    parents = [0, 0]
    frontier = [1]
    for _ in range(levels):
        nxt = []
        for u in frontier:
            for _ in range(branching):
                parents.append(u)
                nxt.append(len(parents) - 1)
        frontier = nxt
    return np.array(parents, np.int32)


def tree_rank_sum(branching=(4, 3, 2, 2, 1, 1), n: int = 60) -> np.ndarray:
    """Static EAGLE-style tree: rank tuples (r_1..r_d), r_k < branching[k-1], ordered by
    (sum of ranks, depth, lexicographic); the first n form the tree (prefix-closed).
    IDs are assigned in (depth, lexicographic) order.  Returns parents[0..n]."""
    tuples = []
    for dpt in range(1, len(branching) + 1):
        for t in itertools.product(*[range(b) for b in branching[:dpt]]):
            tuples.append(t)
    tuples.sort(key=lambda t: (sum(t), len(t), t))
    chosen = tuples[:n]
    chosen.sort(key=lambda t: (len(t), t))
    ids = {t: i + 1 for i, t in enumerate(chosen)}
    parents = np.zeros(n + 1, np.int32)
    for t, i in ids.items():
        parents[i] = 0 if len(t) == 1 else ids[t[:-1]]
    return parents


def tree_random(rng, M: int, max_depth: int) -> np.ndarray:
    """Random tree: node i's depth is uniform on 1..min(max_depth, 1 + deepest so far),
    its parent uniform over the existing nodes one level up (the virtual root for depth 1).
    IDs are in creation order.  Returns parents[0..M]."""
    parents = np.zeros(M + 1, np.int32)
    by_depth = {0: [0]}
    deepest = 0
    for i in range(1, M + 1):
        dpt = int(rng.integers(1, min(max_depth, deepest + 1) + 1))
        parents[i] = by_depth[dpt - 1][int(rng.integers(0, len(by_depth[dpt - 1])))]
        by_depth.setdefault(dpt, []).append(i)
        deepest = max(deepest, dpt)
    return parents


def tree_chain(M: int) -> np.ndarray:
    parents = np.arange(-1, M, dtype=np.int32)
    parents[0] = 0
    return parents


def tree_best_first(marginals_sorted: np.ndarray, budget: int):
    """Best-first prefix tree over per-position draft marginals (block-diffusion drafter
    of the BASTION page): a node at depth d with rank tuple (r_1..r_d) has path score
    rho = prod_k marg[k-1][r_k]; nodes are taken in decreasing rho (ties: shallower, then
    lexicographic) until `budget` nodes exist.  marginals_sorted[k] must be sorted in
    decreasing order.  Returns (parents[0..budget], ranks list of tuples in id order).

    Enumeration: popping a tuple pushes its first child and its next sibling, which
    visits tuples in exactly decreasing rho because each position is sorted."""
    K, topk = marginals_sorted.shape

    def rho(t):
        r = 1.0
        for pos, rank in enumerate(t):
            r *= float(marginals_sorted[pos][rank])
        return r

    heap = [(-rho((0,)), 1, (0,))]
    order = []
    while heap and len(order) < budget:
        _, dpt, t = heapq.heappop(heap)
        order.append(t)
        if dpt < K:
            child = t + (0,)
            heapq.heappush(heap, (-rho(child), dpt + 1, child))
        if t[-1] + 1 < topk:
            sib = t[:-1] + (t[-1] + 1,)
            heapq.heappush(heap, (-rho(sib), dpt, sib))
    ids = {t: i + 1 for i, t in enumerate(order)}
    parents = np.zeros(len(order) + 1, np.int32)
    for t, i in ids.items():
        parents[i] = 0 if len(t) == 1 else ids[t[:-1]]
    return parents, order


def draft_marginals(rng, B: int, D: int, V: int, sigma: float = 3.0, levels: int | None = None) -> np.ndarray:
    """Per-position draft marginals of a block-diffusion drafter, float32 [B][D][V]:
    softmax of N(0, sigma) logits per (sequence, position) -- workload 3's recipe.  With
    `levels`, values are instead drawn from {0, 1/levels, ..., 1}, so many are equal."""
    if levels:
        return (rng.integers(0, levels + 1, size=(B, D, V)) / levels).astype(np.float32)
    return _softmax_rows(rng.standard_normal(size=(B, D, V)) * sigma).astype(np.float32)


def children_lists(parents: np.ndarray, M: int):
    kids = {u: [] for u in range(M + 1)}
    for i in range(1, M + 1):
        kids[int(parents[i])].append(i)
    return kids


# ------------------------------------------------------------------ token planting
def plant_greedy(rng, parents, M, V, logits_b, tokens_b, alpha=0.7):
    """Draft tokens for greedy verification.  At each node u with children, with
    probability alpha one uniformly chosen child gets a token x and the teacher row u is
    raised so that x is its unique maximum (logits[u][x] = max + 1); the other children
    get distinct random tokens different from x (when the vocabulary allows it).
    logits_b [M_max+1][V] is modified in place."""
    kids = children_lists(parents, M)
    for u in range(M + 1):
        ch = kids[u]
        if not ch:
            continue
        toks = rng.choice(V, size=len(ch) + 1, replace=len(ch) + 1 > V)
        x = int(toks[0])
        star = -1
        if rng.random() < alpha:
            star = int(rng.integers(0, len(ch)))
            logits_b[u, x] = logits_b[u].max() + 1.0
        for ci, c in enumerate(ch):
            tokens_b[c] = x if ci == star else int(toks[1 + ci])


# ------------------------------------------------------------------ workloads
@dataclass
class Workload:
    name: str
    dtype: int                      # F32 or BF16 for q/k/v
    B: int
    Hq: int
    Hkv: int
    d: int
    M_max: int
    D_max: int
    L_cap: int
    V: int
    mode: str                       # "greedy" or "sample"
    parents: np.ndarray
    n_nodes: np.ndarray
    prefix: np.ndarray
    tokens: np.ndarray
    q: np.ndarray | None = None
    k: np.ndarray | None = None
    v: np.ndarray | None = None
    logits: np.ndarray | None = None
    p: np.ndarray | None = None
    qd: np.ndarray | None = None
    seed: int = 0
    step: int = 0
    n_layers: int = 1
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


def _normal(rng, shape, sigma, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)
    return x if dtype == F32 else bf16_bits(x)


def _pad_parents(trees, M_max):
    out = np.zeros((len(trees), M_max + 1), np.int32)
    for b, t in enumerate(trees):
        out[b, : len(t)] = t
    return out


def _attention_tensors(rng, B, Hq, Hkv, d, M_max, L_cap, sigma, dtype):
    q = _normal(rng, (B, M_max, Hq, d), sigma, dtype)
    k = _normal(rng, (B, Hkv, L_cap, d), sigma, dtype)
    v = _normal(rng, (B, Hkv, L_cap, d), sigma, dtype)
    return q, k, v


def _greedy_rows(rng, trees, n_nodes, M_max, V, sigma, alpha):
    B = len(trees)
    logits = rng.standard_normal(size=(B, M_max + 1, V), dtype=np.float32) * np.float32(sigma)
    tokens = np.zeros((B, M_max + 1), np.int32)
    for b in range(B):
        plant_greedy(rng, trees[b], int(n_nodes[b]), V, logits[b], tokens[b], alpha)
    return logits, tokens


def _softmax_rows(z):
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def paged_layout(rng, caches, page_size: int, spare: int = 3, alias=()):
    """Page pools holding contiguous caches [..., B, Hkv, L, d] (same shape, any element
    dtype): every sequence's slots [0, L) go to max_blocks = ceil(L / page_size) pages at
    random places of a pool of B * max_blocks + spare pages; slots past L and unused pages
    hold random bits.  alias = ((b_src, b_dst, n), ...) points b_dst's first n table entries
    at b_src's pages (the caller makes those slots' contents equal).  Returns the pools
    [..., num_pages, Hkv, page_size, d] and the table int32 [B][max_blocks]."""
    lead = caches[0].shape[:-4]
    B, H, L, d = caches[0].shape[-4:]
    nblk = -(-L // page_size)
    num_pages = B * nblk + spare
    table = rng.permutation(num_pages)[: B * nblk].reshape(B, nblk).astype(np.int32)
    for bs, bd, n in alias:
        table[bd, :n] = table[bs, :n]
    pools = []
    for c in caches:
        bits = np.dtype(c.dtype).itemsize * 8
        garbage = rng.integers(0, 1 << min(bits, 16), size=lead + (num_pages, H, page_size, d))
        pool = garbage.astype(np.uint16).view(np.uint16).astype(c.dtype) if bits == 16 else \
            rng.standard_normal(lead + (num_pages, H, page_size, d)).astype(c.dtype)
        pad = np.zeros(lead + (B, H, nblk * page_size, d), c.dtype)
        pad[..., :L, :] = c
        for b in range(B):
            for j in range(nblk):
                pool[..., table[b, j], :, :, :] = pad[..., b, :, j * page_size:(j + 1) * page_size, :]
        pools.append(pool)
    return pools, table


def budget_workload(M: int, D_max: int, seed: int, alpha: float = 0.7) -> Workload:
    """Workload 2's layer (bf16, 32/8 heads, d128, prefix 2048, vocabulary 128256, greedy)
    with a random tree of M nodes and depth at most D_max (tree_random): the inputs of the
    verify-cost sweep over tree size and depth."""
    rng = np.random.default_rng(seed)
    parents = tree_random(rng, M, D_max)
    P = 2048
    L_cap = P + (M + 63) // 64 * 64
    q, k, v = _attention_tensors(rng, 1, 32, 8, 128, M, L_cap, 0.5, BF16)
    logits, tokens = _greedy_rows(rng, [parents], [M], M, 128256, 2.0, alpha)
    return Workload("budget-sweep bf16 B1 H32/8 d128 P2048 M%d D%d V128256" % (M, D_max), BF16, 1, 32, 8, 128, M,
                    D_max, L_cap, 128256, "greedy", _pad_parents([parents], M), np.array([M], np.int32),
                    np.array([P], np.int32), tokens, q, k, v, logits)


def workload(c: int, seed: int | None = None, *, alpha: float = 0.7, with_rows: bool = True) -> Workload:
    """Workload number c (1..5).  `seed` overrides the default stream 1000 + c (used to
    make many distinct input sets of the same shape)."""
    rng = np.random.default_rng(1000 + c if seed is None else seed)
    if c == 1:
        # tiny fp32 step: 1 head, d64, prefix 128, complete binary tree of 7 nodes
        parents = tree_complete(2, 2)
        M = 7
        q, k, v = _attention_tensors(rng, 1, 1, 1, 64, M, 128 + M, 1.0, F32)
        logits, tokens = _greedy_rows(rng, [parents], [M], M, 32, 1.0, alpha) if with_rows else (None, np.zeros((1, M + 1), np.int32))
        return Workload("tiny-fp32 B1 H1/1 d64 P128 M7 V32", F32, 1, 1, 1, 64, M, 3, 128 + M, 32, "greedy",
                        _pad_parents([parents], M), np.array([M], np.int32), np.array([128], np.int32),
                        tokens, q, k, v, logits)
    if c == 2:
        # Llama-3-8B-shaped layer: 32/8 heads, d128, prefix 2048, 60-node static tree
        parents = tree_rank_sum((4, 3, 2, 2, 1, 1), 60)
        M, P, L_cap = 60, 2048, 2112
        q, k, v = _attention_tensors(rng, 1, 32, 8, 128, M, L_cap, 0.5, BF16)
        logits, tokens = _greedy_rows(rng, [parents], [M], M, 128256, 2.0, alpha) if with_rows else (None, np.zeros((1, M + 1), np.int32))
        return Workload("llama3-8b-layer bf16 B1 H32/8 d128 P2048 M60 V128256", BF16, 1, 32, 8, 128, M, 6, L_cap,
                        128256, "greedy", _pad_parents([parents], M), np.array([M], np.int32),
                        np.array([P], np.int32), tokens, q, k, v, logits)
    if c == 3:
        # batched dynamic trees: 16 sequences, ragged prefixes and budgets, best-first trees
        B, V, K, topk, M_max = 16, 128256, 8, 128, 128
        prefix = rng.integers(512, 4096 + 1, size=B).astype(np.int32)
        budgets = rng.integers(16, 128 + 1, size=B).astype(np.int32)
        trees, tok_rows = [], np.zeros((B, M_max + 1), np.int32)
        for b in range(B):
            marg = _softmax_rows(rng.standard_normal(size=(K, V)) * 3.0)
            top = np.argsort(-marg, axis=1, kind="stable")[:, :topk]
            ms = np.take_along_axis(marg, top, axis=1)
            par, order = tree_best_first(ms, int(budgets[b]))
            trees.append(par)
            for i, t in enumerate(order):
                tok_rows[b, i + 1] = top[len(t) - 1, t[-1]]
        n_nodes = np.array([len(t) - 1 for t in trees], np.int32)
        L_cap = 4096 + M_max
        q, k, v = _attention_tensors(rng, B, 32, 8, 128, M_max, L_cap, 0.5, BF16)
        logits = None
        tokens = tok_rows
        if with_rows:
            logits = rng.standard_normal(size=(B, M_max + 1, V), dtype=np.float32) * np.float32(2.0)
            # the drafter's tokens are kept; the teacher agrees with one child per node
            # with probability alpha (its row maximum is raised onto that child's token)
            for b in range(B):
                kids = children_lists(trees[b], int(n_nodes[b]))
                for u, ch in kids.items():
                    if ch and rng.random() < alpha:
                        x = int(tokens[b, ch[int(rng.integers(0, len(ch)))]])
                        logits[b, u, x] = logits[b, u].max() + 1.0
        return Workload("batched-dynamic bf16 B16 H32/8 d128 P~U[512,4096] M~U[16,128] V128256", BF16, B, 32, 8,
                        128, M_max, K, L_cap, V, "greedy", _pad_parents(trees, M_max), n_nodes, prefix, tokens,
                        q, k, v, logits)
    if c == 4:
        # long-context 70B-shaped layer: 64/8 heads, d128, 4 sequences of prefix 32768
        B, M, P, V = 4, 64, 32768, 128256
        trees = [tree_random(rng, M, 8) for _ in range(B)]
        L_cap = P + M
        q, k, v = _attention_tensors(rng, B, 64, 8, 128, M, L_cap, 0.5, BF16)
        logits, tokens = _greedy_rows(rng, trees, [M] * B, M, V, 2.0, alpha) if with_rows else (None, np.zeros((B, M + 1), np.int32))
        return Workload("llama3-70b-layer bf16 B4 H64/8 d128 P32768 M64 V128256", BF16, B, 64, 8, 128, M, 8, L_cap,
                        V, "greedy", _pad_parents(trees, M), np.full(B, M, np.int32), np.full(B, P, np.int32),
                        tokens, q, k, v, logits)
    if c == 5:
        # sampling verification: 32 sequences, 32-node trees, p and q over 128256 tokens,
        # commit over 32 layers of 8 KV heads x d128 bf16 (cache made on the device)
        B, M, V, P = 32, 32, 128256, 4096
        trees = [tree_random(rng, M, 6) for _ in range(B)]
        p = np.empty((B, M + 1, V), np.float32)
        qd = np.empty((B, M + 1, V), np.float32)
        tokens = np.zeros((B, M + 1), np.int32)
        for b in range(B):
            p[b] = _softmax_rows(rng.standard_normal(size=(M + 1, V)) * 2.0 / 0.8)
            qd[b] = _softmax_rows(rng.standard_normal(size=(M + 1, V)) * 2.0 / 0.8)
            kids = children_lists(trees[b], M)
            for u, ch in kids.items():
                if ch:
                    w = qd[b, u].astype(np.float64)
                    tokens[b, ch] = rng.choice(V, size=len(ch), p=w / w.sum())
        return Workload("sampling B32 M32 V128256 + commit 32 layers H8 d128 P4096", BF16, B, 0, 8, 128, M, 6,
                        P + M, V, "sample", _pad_parents(trees, M), np.full(B, M, np.int32),
                        np.full(B, P, np.int32), tokens, p=p, qd=qd, seed=5, step=0, n_layers=32)
    raise ValueError("workload %d" % c)


def small_sampling_case(rng, B, M, V, max_depth, overlap=None, dist_sigma=2.0, temp=0.8):
    """Random trees with p / q rows over a small vocabulary and children drawn i.i.d.
    from q of their parent.  `overlap` in (0,1) correlates the draft logits with the
    teacher's (z_q = overlap*z_p + sqrt(1-overlap^2)*z')."""
    trees = [tree_random(rng, M, max_depth) for _ in range(B)]
    zp = rng.standard_normal(size=(B, M + 1, V)) * dist_sigma
    zq = rng.standard_normal(size=(B, M + 1, V)) * dist_sigma
    if overlap is not None:
        zq = overlap * zp + np.sqrt(1 - overlap * overlap) * zq
    p = _softmax_rows(zp / temp).astype(np.float32)
    q = _softmax_rows(zq / temp).astype(np.float32)
    tokens = np.zeros((B, M + 1), np.int32)
    for b in range(B):
        for u, ch in children_lists(trees[b], M).items():
            if ch:
                w = q[b, u].astype(np.float64)
                tokens[b, ch] = rng.choice(V, size=len(ch), p=w / w.sum())
    return _pad_parents(trees, M), np.full(B, M, np.int32), tokens, p, q


def lm_head_weights(rng, V: int, K: int, sigma: float, chunk: int = 8192) -> np.ndarray:
    """Synthetic LM-head weights [V][K] as bf16 bits: N(0, sigma) drawn in fp32, in chunks
    of rows (the full 8B-shaped head is 1 GiB of bf16)."""
    out = np.empty((V, K), np.uint16)
    for v0 in range(0, V, chunk):
        v1 = min(V, v0 + chunk)
        out[v0:v1] = bf16_bits(rng.standard_normal((v1 - v0, K), dtype=np.float32) * np.float32(sigma))
    return out


def plant_from_argmax(rng, parents, M, V, t_row, tokens_b, alpha=0.7):
    """Draft tokens of one tree given the teacher's choices t_row[u]: at each node with
    children, with probability alpha one child gets t_row[u]; the other children get
    distinct tokens different from it."""
    kids = children_lists(parents, M)
    for u in range(M + 1):
        ch = kids[u]
        if not ch:
            continue
        x = int(t_row[u])
        star = int(rng.integers(0, len(ch))) if rng.random() < alpha else -1
        others = [y for y in rng.choice(V, size=min(V, len(ch) + 2), replace=False).tolist() if y != x]
        for ci, c in enumerate(ch):
            tokens_b[c] = x if ci == star else others[ci % len(others)]


def cache_pattern_value(layer, b, head, slot, dim):
    """Deterministic cache contents for the multi-layer commit workload: every row is
    tagged by its coordinates, so a row moved to the wrong place is visible.  Values are
    small integers, exact in bf16."""
    return ((layer * 7 + b * 5 + head * 3 + slot) % 251) - 125 + (dim % 2) * 0.5
