"""CPU oracle for the tree-verification step (TEST INFRASTRUCTURE ONLY).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its binding) never loads it, and
the two share no code: the arithmetic lives in ``tmv_oracle.c`` (plain C, fp64 and
exact integers), this module only marshals numpy arrays through ctypes.

Every function mirrors one entry point of the C ABI on host arrays:

``build_ancestors``   virtual-root remap, ancestor table, invariant checks
                      (EAGLE-Pangu Chinese technical summary, section 2.2)
``tree_attention``    tree-masked attention: prefix + own ancestor path incl. itself
                      (same page, section 2.3; Medusa section of the hierarchical
                      speculative decoding blog)
``accept_greedy``     deepest matching path under the teacher's argmax
                      (blog, Medusa section: the longest valid path is kept)
``accept_sample``     modified rejection sampling with min(1,p/q) and the normalised
                      max(0,p-q) residual (blog, modified rejection sampling section)
``commit``            prefix-sharing path-index commit (Chinese summary, section 2.1)
``tree_best_first``   best-first prefix tree from per-position draft marginals and the
                      budget controller (BASTION summary, sections 1-3)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tmv_oracle.c")
_LIB = os.path.join(_HERE, "libtmv_oracle.so")
# a sanitizer build of the same source (tests/test_oracle_sanitized.py) is loaded instead
# when TMV_ORACLE_LIB names it
_LIB_OVERRIDE = os.environ.get("TMV_ORACLE_LIB")

OK, ERR_ARG, ERR_RANGE, ERR_CYCLE, ERR_DEPTH, ERR_CLOSURE, ERR_INPUT = range(7)
PARENTS_VROOT, PARENTS_NEG1 = 0, 1
F32, BF16 = 0, 1


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no HIP, no shared sources)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=gnu99", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I, I64, U64, D = ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
        lib.tmvref_build_ancestors.argtypes = [I, I, I, I, P, P, P, P, P, P]
        lib.tmvref_tree_attention.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, I,
                                              P, P, P, P, P, D, P, P]
        lib.tmvref_accept_greedy.argtypes = [I, I, I, I, P, I, P, I64, I64, P, P, P, P, P, P, P]
        lib.tmvref_accept_sample.argtypes = [I, I, I, I, P, P, P, U64, U64, P, P, P, P, P, P, P]
        lib.tmvref_commit.argtypes = [I, I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P]
        lib.tmvref_lm_head_logits.argtypes = [I, I, I, P, P, I64, P, P]
        lib.tmvref_philox_words.argtypes = [U64, U64, I64, P]
        lib.tmvref_philox_words.restype = None
        lib.tmvref_sample_accept_test.argtypes = [U64, U64, U64, U64, U64, U64, U64]
        lib.tmvref_sample_draw.argtypes = [P, P, I, U64]
        lib.tmvref_tree_best_first.argtypes = [I, I, I, I, P, P, D, P, P, P, P, P]
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc):
    if rc != OK:
        raise ValueError("oracle rejected its arguments (code %d)" % rc)


def build_ancestors(parents, n_nodes, M_max, D_max, parent_format=PARENTS_VROOT, valid=None):
    """Returns (anc [B][M_max+1][D_max+1], depth [B][M_max+1], status [B]) as int32."""
    parents = _c(parents, np.int32)
    n_nodes = _c(n_nodes, np.int32)
    B = n_nodes.shape[0]
    want = (B, M_max + 1) if parent_format == PARENTS_VROOT else (B, M_max)
    assert parents.shape == want, (parents.shape, want)
    if valid is not None:
        valid = _c(valid, np.uint8)
        assert valid.shape == (B, M_max + 1)
    anc = np.zeros((B, M_max + 1, D_max + 1), np.int32)
    depth = np.zeros((B, M_max + 1), np.int32)
    status = np.zeros((B,), np.int32)
    _check(_load().tmvref_build_ancestors(B, M_max, D_max, parent_format, _p(parents), _p(valid),
                                          _p(n_nodes), _p(anc), _p(depth), _p(status)))
    return anc, depth, status


def tree_attention(q, k, v, prefix_len, n_nodes, anc, depth, status, scale, dtype,
                   Hkv, row_select=None):
    """q [B][M_max][Hq][d]; k, v [B][Hkv][L_cap][d] (float32, or uint16 bf16 bits).

    Returns (out fp64 [B][M_max][Hq][d], status after the stage)."""
    edt = np.float32 if dtype == F32 else np.uint16
    q, k, v = _c(q, edt), _c(k, edt), _c(v, edt)
    B, M_max, Hq, d = q.shape
    assert k.shape[0] == B and k.shape[1] == Hkv and k.shape[3] == d and v.shape == k.shape
    L_cap = k.shape[2]
    D_max = anc.shape[2] - 1
    qs = np.array([M_max * Hq * d, Hq * d, d], np.int64)
    ks = np.array([Hkv * L_cap * d, L_cap * d, d], np.int64)
    st = _c(status, np.int32).copy()
    out = np.zeros((B, M_max, Hq, d), np.float64)
    if row_select is not None:
        row_select = _c(row_select, np.uint8)
        assert row_select.shape == (B, M_max)
    _check(_load().tmvref_tree_attention(B, M_max, D_max, Hq, Hkv, d, dtype, _p(q), _p(qs), _p(k), _p(v),
                                         _p(ks), L_cap, _p(_c(prefix_len, np.int32)),
                                         _p(_c(n_nodes, np.int32)), _p(_c(anc, np.int32)),
                                         _p(_c(depth, np.int32)), _p(st), float(scale), _p(row_select),
                                         _p(out)))
    return out, st


def accept_greedy(tokens, logits, n_nodes, anc, depth, status, row_dtype=F32):
    """logits [B][M_max+1][V] (float32 or uint16 bf16 bits); tokens [B][M_max+1].

    Returns (accept_len [B], path [B][D_max], next_token [B], status)."""
    edt = np.float32 if row_dtype == F32 else np.uint16
    logits = _c(logits, edt)
    B, R, V = logits.shape
    M_max, D_max = R - 1, anc.shape[2] - 1
    st = _c(status, np.int32).copy()
    A = np.zeros((B,), np.int32)
    path = np.zeros((B, D_max), np.int32)
    nxt = np.zeros((B,), np.int32)
    _check(_load().tmvref_accept_greedy(B, M_max, D_max, V, _p(_c(tokens, np.int32)), row_dtype, _p(logits),
                                        R * V, V, _p(_c(n_nodes, np.int32)), _p(_c(anc, np.int32)),
                                        _p(_c(depth, np.int32)), _p(st), _p(A), _p(path), _p(nxt)))
    return A, path, nxt, st


def commit_paged_table(table, page_size, num_pages, prefix_len, n_nodes, new_len, status):
    """Block eviction after a paged commit (the runtime-memory question of the hierarchical
    speculative decoding blog: discarded branches' blocks are evicted, only the accepted
    path is kept).  For every sequence with status OK, the blocks of its tree slots
    [P, P + M) that start at or beyond new_len and hold a valid page are cleared to -1 and
    their pages freed.  Returns (new table, sorted list of freed pages)."""
    table = np.array(table, np.int32, copy=True)
    freed = []
    for b in range(table.shape[0]):
        if int(status[b]) != OK:
            continue
        P, M, nl = int(prefix_len[b]), int(n_nodes[b]), int(new_len[b])
        first = -(-nl // page_size)                   # first block starting at or after new_len
        last = -(-(P + M) // page_size)               # one past the tree's last block
        for i in range(first, min(last, table.shape[1])):
            pg = int(table[b, i])
            if 0 <= pg < num_pages:
                freed.append(pg)
                table[b, i] = -1
    return table, sorted(freed)


def lm_head_logits(h_bits, w_bits, with_bound=True):
    """fp64 logits of the rows h_bits [n][K] (bf16 bit patterns) against the LM head
    w_bits [V][K]: (logits [n][V], bound [n][V] = sum_k |h w| or None)."""
    h = _c(h_bits, np.uint16)
    w = _c(w_bits, np.uint16)
    n, K = h.shape
    V = w.shape[0]
    assert w.shape[1] == K
    logits = np.zeros((n, V), np.float64)
    bound = np.zeros((n, V), np.float64) if with_bound else None
    _check(_load().tmvref_lm_head_logits(n, K, V, _p(h), _p(w), K, _p(logits), _p(bound) if with_bound else None))
    return logits, bound


def accept_sample(tokens, p, q, seed, step, n_nodes, anc, depth, status):
    """p, q float32 [B][M_max+1][V].  Returns (accept_len, path, next_token, status)."""
    p, q = _c(p, np.float32), _c(q, np.float32)
    B, R, V = p.shape
    assert q.shape == p.shape
    M_max, D_max = R - 1, anc.shape[2] - 1
    st = _c(status, np.int32).copy()
    A = np.zeros((B,), np.int32)
    path = np.zeros((B, D_max), np.int32)
    nxt = np.zeros((B,), np.int32)
    _check(_load().tmvref_accept_sample(B, M_max, D_max, V, _p(_c(tokens, np.int32)), _p(p), _p(q),
                                        int(seed), int(step), _p(_c(n_nodes, np.int32)),
                                        _p(_c(anc, np.int32)), _p(_c(depth, np.int32)), _p(st), _p(A),
                                        _p(path), _p(nxt)))
    return A, path, nxt, st


def commit(k_cache, v_cache, prefix_len, n_nodes, accept_len, path, status, M_max):
    """In place on k_cache / v_cache [n_layers][B][Hkv][L_cap][d] (float32 or uint16).

    Returns (new_len [B], status)."""
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous and k_cache.shape == v_cache.shape
    nl, B, Hkv, L_cap, d = k_cache.shape
    es = k_cache.dtype.itemsize
    D_max = path.shape[1]
    stride = np.array([B * Hkv * L_cap * d, Hkv * L_cap * d, L_cap * d, d], np.int64)
    st = _c(status, np.int32).copy()
    new_len = np.zeros((B,), np.int32)
    _check(_load().tmvref_commit(nl, B, Hkv, d, L_cap, M_max, D_max, es, _p(k_cache), _p(v_cache),
                                 _p(stride), _p(_c(prefix_len, np.int32)), _p(_c(n_nodes, np.int32)),
                                 _p(_c(accept_len, np.int32)), _p(_c(path, np.int32)), _p(st),
                                 _p(new_len)))
    return new_len, st


def philox_words(seed, stream, n):
    out = np.zeros((n,), np.uint64)
    _load().tmvref_philox_words(int(seed), int(stream), int(n), _p(out))
    return out


def sample_accept_test(u24, wq_x, T, r_x, SQ) -> bool:
    """U * WQ(x) * T < R(x) * SQ * 2^24 on Python integers (T, r_x < 2^128)."""
    m = (1 << 64) - 1
    return bool(_load().tmvref_sample_accept_test(int(u24), int(wq_x), int(T) & m, int(T) >> 64, int(r_x) & m,
                                                  int(r_x) >> 64, int(SQ)))


def sample_draw(w, word) -> int:
    """Inverse-CDF draw over integer weights w (Python ints < 2^128)."""
    m = (1 << 64) - 1
    lo = np.array([int(x) & m for x in w], np.uint64)
    hi = np.array([int(x) >> 64 for x in w], np.uint64)
    return int(_load().tmvref_sample_draw(_p(lo), _p(hi), len(w), int(word)))


def tree_best_first(q, N_max, cost=None, l_ar=1.0, status=None):
    """q float32 [B][D][V] (row k = marginal of position k+1); cost float64 [N_max] or None.
    Returns (parents [B][N_max+1], tokens [B][N_max+1], n_nodes [B], rho [B][N_max+1], status)."""
    q = _c(q, np.float32)
    B, D, V = q.shape
    R = N_max + 1
    st = np.zeros((B,), np.int32) if status is None else _c(status, np.int32).copy()
    parents = np.zeros((B, R), np.int32)
    tokens = np.zeros((B, R), np.int32)
    n = np.zeros((B,), np.int32)
    rho = np.zeros((B, R), np.float64)
    c = None if cost is None else _c(cost, np.float64)
    _check(_load().tmvref_tree_best_first(B, D, V, int(N_max), _p(q), _p(c), float(l_ar), _p(parents), _p(tokens),
                                          _p(n), _p(rho), _p(st)))
    return parents, tokens, n, rho, st
