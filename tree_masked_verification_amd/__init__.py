"""tree_masked_verification_amd -- MI355X (gfx950) tree-verification step.

Thin ctypes binding of libtmv.so (see include/tmv.h for the C ABI).  Every function
only marshals torch tensors into pointers, strides and the current HIP stream; all
work runs in the library's HIP kernels.  If the library is not built, importing this
package raises ImportError -- there is no fallback.

Stages of one verify step, in order:
  tree_build_ancestors   parents -> (anc, depth, status)
  tree_verify_attention  tree-masked attention of all draft nodes
  tree_accept            greedy longest matching path, or modified rejection sampling
  kv_commit_path         prefix-sharing in-place compaction of the accepted K/V rows
and, on the drafting side of a step:
  tree_best_first        best-first prefix tree from per-position draft marginals, sized
                         by the budget controller
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtmv.so")

OK, ERR_ARG, ERR_RANGE, ERR_CYCLE, ERR_DEPTH, ERR_CLOSURE, ERR_INPUT, ERR_DEVICE = range(8)
F32, BF16 = 0, 1
PARENTS_VROOT, PARENTS_NEG1 = 0, 1
ACCEPT_GREEDY, ACCEPT_SAMPLE = 0, 1
# ORed into the pinned split count of a plan: each row block's splits on different XCDs
# (a placement the attention's partial exchange rejects: zero rows, ERR_DEVICE; tests)
PLAN_SCATTER_XCD = 0x100

if not os.path.exists(LIB_PATH):
    raise ImportError("libtmv.so is not built (run `python tree_masked_verification_amd/build.py`); "
                      "the tree-verification path has no CPU fallback")

_lib = ctypes.CDLL(LIB_PATH)
_P, _I, _I64, _U64, _F, _SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float,
                               ctypes.c_size_t)
_lib.tmv_status_string.argtypes = [_I]
_lib.tmv_status_string.restype = ctypes.c_char_p
_lib.tmv_abi_version.restype = _I
_lib.tmv_tree_build_ancestors.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]
_lib.tmv_tree_verify_attention_workspace.argtypes = [_I, _I, _I, _I, _I, _I, _I]
_lib.tmv_tree_verify_attention_workspace.restype = _SZ
_lib.tmv_tree_verify_attention.argtypes = [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P,
                                           _F, _P, _P, _P, _SZ, _P]
_lib.tmv_tree_verify_attention_plan_workspace.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, _I]
_lib.tmv_tree_verify_attention_plan_workspace.restype = _SZ
_lib.tmv_tree_verify_attention_plan.argtypes = [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P,
                                                _F, _P, _P, _I, _I, _P, _SZ, _P]
_lib.tmv_tree_verify_attention_noalloc.argtypes = [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P,
                                                   _P, _F, _P, _P, _P]
_lib.tmv_tree_accept_workspace.argtypes = [_I, _I, _I, _I]
_lib.tmv_tree_accept_workspace.restype = _SZ
_lib.tmv_tree_accept.argtypes = [_I, _I, _I, _I, _I, _P, _I, _P, _I64, _I64, _P, _I64, _I64, _U64, _U64,
                                 _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
_lib.tmv_tree_accept_wait.argtypes = [_I, _I, _I, _I, _I, _P, _I, _P, _I64, _I64, _P, _I64, _I64, _U64, _U64,
                                      _P, _P, _P, _P, _P, _P, _P, _P, _SZ, ctypes.c_uint32, _P]
_lib.tmv_tree_accept_lm_head_workspace.argtypes = [_I, _I]
_lib.tmv_tree_accept_lm_head_workspace.restype = _SZ
_lib.tmv_tree_accept_lm_head.argtypes = [_I, _I, _I, _I, _I, _P, _P, _I64, _I64, _P, _I64, _P, _P, _P, _P, _P, _P, _P,
                                         _P, _P, _SZ, _P]
_lib.tmv_kv_commit_path.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
_lib.tmv_tree_verify_attention_paged_workspace.argtypes = [_I, _I, _I, _I, _I, _I, _I]
_lib.tmv_tree_verify_attention_paged_workspace.restype = _SZ
_lib.tmv_tree_verify_attention_paged.argtypes = [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _I, _P, _I64, _I,
                                                 _P, _P, _P, _P, _P, _F, _P, _P, _P, _SZ, _P]
_lib.tmv_tree_verify_attention_paged_plan_workspace.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, _I]
_lib.tmv_tree_verify_attention_paged_plan_workspace.restype = _SZ
_lib.tmv_tree_verify_attention_paged_plan.argtypes = [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _I, _P, _I64,
                                                      _I, _P, _P, _P, _P, _P, _F, _P, _P, _I, _I, _P, _SZ, _P]
_lib.tmv_kv_commit_path_paged.argtypes = [_I, _I, _I, _I, _I, _I, _I, _P, _I64, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P,
                                          _P, _P, _P]
_lib.tmv_kv_commit_path_paged_evict.argtypes = [_I, _I, _I, _I, _I, _I, _I, _P, _I64, _I, _I, _I, _P, _P, _P, _P, _P,
                                                _P, _P, _P, _P, _P, _P, _I, _P]
_lib.tmv_tree_best_first_workspace.argtypes = [_I, _I, _I, _I]
_lib.tmv_tree_best_first_workspace.restype = _SZ
_lib.tmv_tree_best_first.argtypes = [_I, _I, _I, _I, _P, _I64, _I64, _P, ctypes.c_double, _P, _P, _P, _P, _P, _P,
                                     _SZ, _P]

EXPORTED = ("tmv_status_string", "tmv_abi_version", "tmv_tree_build_ancestors",
            "tmv_tree_verify_attention_workspace", "tmv_tree_verify_attention", "tmv_tree_accept_workspace",
            "tmv_tree_accept", "tmv_kv_commit_path", "tmv_tree_best_first_workspace", "tmv_tree_best_first",
            "tmv_tree_verify_attention_paged_workspace", "tmv_tree_verify_attention_paged",
            "tmv_kv_commit_path_paged", "tmv_tree_verify_attention_plan_workspace",
            "tmv_tree_verify_attention_plan", "tmv_tree_verify_attention_paged_plan_workspace",
            "tmv_tree_verify_attention_paged_plan", "tmv_tree_verify_attention_noalloc",
            "tmv_tree_accept_lm_head_workspace", "tmv_tree_accept_lm_head", "tmv_kv_commit_path_paged_evict",
            "tmv_tree_accept_wait")


class TmvError(RuntimeError):
    def __init__(self, code, what):
        super().__init__("%s: %s (code %d)" % (what, status_string(code), code))
        self.code = code


def status_string(code: int) -> str:
    return _lib.tmv_status_string(int(code)).decode()


def abi_version() -> int:
    return int(_lib.tmv_abi_version())


def library():
    """The loaded ctypes handle (for callers that need the raw ABI)."""
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _torch_stream(stream):
    return torch.cuda.current_stream() if stream is None else stream


def _stream(stream):
    return ctypes.c_void_p(_torch_stream(stream).cuda_stream)


def _temp_workspace(nbytes, device, stream, zero):
    """A workspace for one call, allocated (and zero-filled) on the call's own stream: the
    fill is ordered before the launch, and the caching allocator does not hand the block
    to other work until everything queued on that stream up to its release has run."""
    with torch.cuda.stream(_torch_stream(stream)):
        alloc = torch.zeros if zero else torch.empty
        return alloc(max(256, int(nbytes)), dtype=torch.uint8, device=device)


def _shape(t, shape, name):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _vec(n, name, *ts):
    for t in ts:
        if t is not None and t.numel() != n:
            raise ValueError("%s: expected %d entries, got %d" % (name, n, t.numel()))


def _strides(t, dims):
    return (ctypes.c_int64 * len(dims))(*[t.stride(i) for i in dims])


def _dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("unsupported dtype %s" % t.dtype)


def _check(rc, what):
    if rc != OK:
        raise TmvError(rc, what)


# TMV_DEBUG=1: after every call, synchronise its stream and report on stderr each sequence
# whose status is not OK (debugging only: it adds a host synchronisation to every call, so it
# must stay off under graph capture and in timed runs; the computation is the same)
DEBUG = os.environ.get("TMV_DEBUG", "") not in ("", "0")


def _debug(what, status, stream=None):
    if not DEBUG:
        return []
    if status.is_cuda:
        _torch_stream(stream).synchronize()
    codes = status.cpu().tolist()
    bad = [(i, status_string(int(c))) for i, c in enumerate(codes) if c != OK]
    if bad:
        import sys
        print("tmv debug: %s: %d of %d sequences not OK: %s" % (what, len(bad), len(codes), bad[:16]),
              file=sys.stderr, flush=True)
    return bad


def _i32(*ts):
    for t in ts:
        if t is not None and (t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous()):
            raise TypeError("expected contiguous int32 device tensors")


# ------------------------------------------------------------------------ stage 1
def tree_build_ancestors(parents, n_nodes, anc, depth, status, parent_format=PARENTS_VROOT, valid=None,
                         stream=None):
    """parents int32 [B][M_max+1] (VROOT) or [B][M_max] (NEG1); anc [B][M_max+1][D_max+1],
    depth [B][M_max+1], status [B] (outputs); valid uint8 [B][M_max+1] or None."""
    _i32(parents, n_nodes, anc, depth, status)
    B, R, W = anc.shape
    if valid is not None and (valid.dtype != torch.uint8 or not valid.is_contiguous()):
        raise TypeError("valid must be contiguous uint8")
    _shape(parents, (B, R if parent_format == PARENTS_VROOT else R - 1), "parents")
    _shape(depth, (B, R), "depth")
    _shape(valid, (B, R), "valid")
    _vec(B, "n_nodes / status", n_nodes, status)
    _check(_lib.tmv_tree_build_ancestors(B, R - 1, W - 1, parent_format, _ptr(parents), _ptr(valid), _ptr(n_nodes),
                                         _ptr(anc), _ptr(depth), _ptr(status), _stream(stream)),
           "tree_build_ancestors")
    _debug("tree_build_ancestors", status, stream)


# ------------------------------------------------------------------------ stage 2
def tree_verify_attention_workspace(dtype, B, M_max, Hq, Hkv, d, L_cap) -> int:
    return int(_lib.tmv_tree_verify_attention_workspace(dtype, B, M_max, Hq, Hkv, d, L_cap))


def tree_verify_attention_plan_workspace(dtype, B, M_max, Hq, Hkv, d, L_cap, rows_per_group, splits) -> int:
    return int(_lib.tmv_tree_verify_attention_plan_workspace(dtype, B, M_max, Hq, Hkv, d, L_cap, rows_per_group,
                                                             splits))


def _check_tree_tables(B, M_max, anc, depth, what):
    if anc.dim() != 3 or anc.shape[0] != B or anc.shape[1] != M_max + 1:
        raise ValueError("%s: anc must be [B][M_max+1][D_max+1]" % what)
    _shape(depth, (B, M_max + 1), "depth")


def tree_verify_attention(q, k_cache, v_cache, prefix_len, n_nodes, anc, depth, status, out, scale=None,
                          workspace=None, stream=None, plan=None):
    """q, out [B][M_max][Hq][d]; k_cache, v_cache [B][Hkv][L_cap][d] (same dtype, d contiguous).
    plan = (rows per group, token splits) pins the launch plan (tuning and tests); None lets
    the library choose."""
    _i32(prefix_len, n_nodes, anc, depth, status)
    dt = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype or out.dtype != q.dtype:
        raise TypeError("q, k_cache, v_cache and out must share a dtype")
    if k_cache.shape != v_cache.shape or k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must have the same shape and strides")
    B, M_max, Hq, d = q.shape
    if k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError("k_cache must be [B][Hkv][L_cap][d]")
    Hkv, L_cap = k_cache.shape[1], k_cache.shape[2]
    if tuple(out.shape) != tuple(q.shape) or q.stride(3) != 1 or k_cache.stride(3) != 1 or out.stride(3) != 1:
        raise ValueError("bad q / out / cache layout")
    _check_tree_tables(B, M_max, anc, depth, "tree_verify_attention")
    _vec(B, "prefix_len / n_nodes / status", prefix_len, n_nodes, status)
    D_max = anc.shape[2] - 1
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    rows, splits = (0, 0) if plan is None else (int(plan[0]), int(plan[1]))
    if workspace is None:
        workspace = _temp_workspace(tree_verify_attention_plan_workspace(dt, B, M_max, Hq, Hkv, d, L_cap, rows, splits),
                                    q.device, stream, zero=True)
    args = (dt, B, M_max, D_max, Hq, Hkv, d, _ptr(q), _strides(q, (0, 1, 2)), _ptr(k_cache), _ptr(v_cache),
            _strides(k_cache, (0, 1, 2)), L_cap, _ptr(prefix_len), _ptr(n_nodes), _ptr(anc), _ptr(depth), _ptr(status),
            float(scale), _ptr(out), _strides(out, (0, 1, 2)))
    tail = (_ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if plan is None:
        _check(_lib.tmv_tree_verify_attention(*args, *tail), "tree_verify_attention")
    else:
        _check(_lib.tmv_tree_verify_attention_plan(*args, rows, splits, *tail), "tree_verify_attention_plan")
    _debug("tree_verify_attention", status, stream)


def tree_verify_attention_paged_workspace(B, M_max, Hq, Hkv, d, page_size, max_blocks) -> int:
    return int(_lib.tmv_tree_verify_attention_paged_workspace(B, M_max, Hq, Hkv, d, page_size, max_blocks))


def tree_verify_attention_paged(q, k_pages, v_pages, block_table, prefix_len, n_nodes, anc, depth, status, out,
                                scale=None, workspace=None, stream=None, plan=None):
    """q, out [B][M_max][Hq][d] bf16; k_pages, v_pages [num_pages][Hkv][page_size][d] bf16;
    block_table int32 [B][max_blocks] (logical slot t of sequence b: page block_table[b][t //
    page_size], row t % page_size)."""
    _i32(block_table, prefix_len, n_nodes, anc, depth, status)
    if k_pages.dtype != q.dtype or v_pages.dtype != q.dtype or out.dtype != q.dtype:
        raise TypeError("q, k_pages, v_pages and out must share a dtype")
    if k_pages.shape != v_pages.shape or k_pages.stride() != v_pages.stride():
        raise ValueError("k_pages and v_pages must have the same shape and strides")
    B, M_max, Hq, d = q.shape
    num_pages, Hkv, page_size = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    max_blocks = block_table.shape[1]
    if tuple(out.shape) != tuple(q.shape) or q.stride(3) != 1 or k_pages.stride(3) != 1 or out.stride(3) != 1:
        raise ValueError("bad q / out / page layout")
    if k_pages.dim() != 4 or k_pages.shape[3] != d or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("k_pages must be [num_pages][Hkv][page_size][d] and block_table [B][max_blocks]")
    _check_tree_tables(B, M_max, anc, depth, "tree_verify_attention_paged")
    _vec(B, "prefix_len / n_nodes / status", prefix_len, n_nodes, status)
    D_max = anc.shape[2] - 1
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    rows, splits = (0, 0) if plan is None else (int(plan[0]), int(plan[1]))
    if workspace is None:
        workspace = _temp_workspace(_lib.tmv_tree_verify_attention_paged_plan_workspace(
            B, M_max, Hq, Hkv, d, page_size, max_blocks, rows, splits), q.device, stream, zero=True)
    args = (_dtype_code(q), B, M_max, D_max, Hq, Hkv, d, _ptr(q), _strides(q, (0, 1, 2)), _ptr(k_pages),
            _ptr(v_pages), _strides(k_pages, (0, 1, 2)), num_pages, page_size, _ptr(block_table), block_table.stride(0),
            max_blocks, _ptr(prefix_len), _ptr(n_nodes), _ptr(anc), _ptr(depth), _ptr(status), float(scale), _ptr(out),
            _strides(out, (0, 1, 2)))
    tail = (_ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if plan is None:
        _check(_lib.tmv_tree_verify_attention_paged(*args, *tail), "tree_verify_attention_paged")
    else:
        _check(_lib.tmv_tree_verify_attention_paged_plan(*args, rows, splits, *tail),
               "tree_verify_attention_paged_plan")
    _debug("tree_verify_attention_paged", status, stream)


# ------------------------------------------------------------------------ stage 3
def tree_accept_workspace(mode, B, M_max, V) -> int:
    return int(_lib.tmv_tree_accept_workspace(mode, B, M_max, V))


def tree_accept(mode, tokens, teacher, n_nodes, anc, depth, status, accept_len, path, next_token, draft_q=None,
                seed=0, step=0, workspace=None, stream=None, wait_us=None):
    """teacher [B][M_max+1][V]: logits (GREEDY, f32/bf16) or p (SAMPLE, f32); draft_q the
    same shape (SAMPLE).  Outputs accept_len [B], path [B][D_max], next_token [B].
    wait_us: the sampling walk's wait bound (tmv_tree_accept_wait); None = the default."""
    _i32(tokens, n_nodes, anc, depth, status, accept_len, path, next_token)
    B, R, V = teacher.shape
    _check_tree_tables(B, R - 1, anc, depth, "tree_accept")
    D_max = anc.shape[2] - 1
    _shape(tokens, (B, R), "tokens")
    _shape(path, (B, D_max), "path")
    _vec(B, "n_nodes / status / accept_len / next_token", n_nodes, status, accept_len, next_token)
    if teacher.stride(2) != 1:
        raise ValueError("teacher rows must be contiguous")
    if mode == ACCEPT_SAMPLE:
        if draft_q is None or draft_q.dtype != torch.float32 or draft_q.shape != teacher.shape or draft_q.stride(2) != 1:
            raise ValueError("sampling needs a float32 draft_q shaped like teacher")
        qs = (draft_q.stride(0), draft_q.stride(1))
    else:
        qs = (0, 0)
    if workspace is None:
        workspace = _temp_workspace(tree_accept_workspace(mode, B, R - 1, V), teacher.device, stream, zero=True)
    args = (mode, B, R - 1, D_max, V, _ptr(tokens), _dtype_code(teacher), _ptr(teacher), teacher.stride(0),
            teacher.stride(1), _ptr(draft_q), qs[0], qs[1], ctypes.c_uint64(seed), ctypes.c_uint64(step), _ptr(n_nodes),
            _ptr(anc), _ptr(depth), _ptr(status), _ptr(accept_len), _ptr(path), _ptr(next_token), _ptr(workspace),
            workspace.numel() * workspace.element_size())
    if wait_us is None:
        _check(_lib.tmv_tree_accept(*args, _stream(stream)), "tree_accept")
    else:
        if not 0 <= int(wait_us) < 1 << 32:
            raise ValueError("wait_us out of range")
        _check(_lib.tmv_tree_accept_wait(*args, int(wait_us), _stream(stream)), "tree_accept")
    _debug("tree_accept", status, stream)


def tree_accept_lm_head_workspace(B, M_max) -> int:
    return int(_lib.tmv_tree_accept_lm_head_workspace(B, M_max))


def tree_accept_lm_head(tokens, hidden, lm_head, n_nodes, anc, depth, status, accept_len, path, next_token,
                        row_argmax=None, workspace=None, stream=None):
    """Greedy acceptance from the LM head: hidden bf16 [B][M_max+1][K], lm_head bf16 [V][K]
    (K contiguous).  Outputs as tree_accept; row_argmax int32 [B][M_max+1] (optional)."""
    _i32(tokens, n_nodes, anc, depth, status, accept_len, path, next_token, row_argmax)
    if hidden.dtype != torch.bfloat16 or lm_head.dtype != torch.bfloat16:
        raise TypeError("hidden and lm_head must be bfloat16")
    if hidden.dim() != 3 or lm_head.dim() != 2 or hidden.stride(2) != 1 or lm_head.stride(1) != 1:
        raise ValueError("hidden [B][M_max+1][K] and lm_head [V][K] with K contiguous")
    B, R, K = hidden.shape
    V = lm_head.shape[0]
    if lm_head.shape[1] != K:
        raise ValueError("lm_head must be [V][K]")
    _check_tree_tables(B, R - 1, anc, depth, "tree_accept_lm_head")
    D_max = anc.shape[2] - 1
    _shape(tokens, (B, R), "tokens")
    _shape(path, (B, D_max), "path")
    _shape(row_argmax, (B, R), "row_argmax")
    _vec(B, "n_nodes / status / accept_len / next_token", n_nodes, status, accept_len, next_token)
    if workspace is None:
        workspace = _temp_workspace(tree_accept_lm_head_workspace(B, R - 1), hidden.device, stream, zero=True)
    _check(_lib.tmv_tree_accept_lm_head(B, R - 1, D_max, K, V, _ptr(tokens), _ptr(hidden), hidden.stride(0),
                                        hidden.stride(1), _ptr(lm_head), lm_head.stride(0), _ptr(n_nodes), _ptr(anc),
                                        _ptr(depth), _ptr(status), _ptr(accept_len), _ptr(path), _ptr(next_token),
                                        _ptr(row_argmax), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                        _stream(stream)),
           "tree_accept_lm_head")
    _debug("tree_accept_lm_head", status, stream)


# ------------------------------------------------------------------------ stage 4
def kv_commit_path(k_cache, v_cache, prefix_len, n_nodes, accept_len, path, status, new_len, M_max, stream=None):
    """In place on k_cache / v_cache [n_layers][B][Hkv][L_cap][d]."""
    _i32(prefix_len, n_nodes, accept_len, path, status, new_len)
    if k_cache.dim() == 4:
        k_cache, v_cache = k_cache.unsqueeze(0), v_cache.unsqueeze(0)
    if k_cache.shape != v_cache.shape or k_cache.stride() != v_cache.stride() or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must match")
    nl, B, Hkv, L_cap, d = k_cache.shape
    if k_cache.stride(4) != 1:
        raise ValueError("d must be contiguous")
    if path.dim() != 2 or path.shape[0] != B:
        raise ValueError("path must be [B][D_max]")
    _vec(B, "prefix_len / n_nodes / accept_len / status / new_len", prefix_len, n_nodes, accept_len, status, new_len)
    _check(_lib.tmv_kv_commit_path(_dtype_code(k_cache), nl, B, Hkv, d, L_cap, int(M_max), path.shape[1],
                                   _ptr(k_cache), _ptr(v_cache), _strides(k_cache, (0, 1, 2, 3)), _ptr(prefix_len),
                                   _ptr(n_nodes), _ptr(accept_len), _ptr(path), _ptr(status), _ptr(new_len),
                                   _stream(stream)),
           "kv_commit_path")
    _debug("kv_commit_path", status, stream)


def kv_commit_path_paged(k_pages, v_pages, block_table, prefix_len, n_nodes, accept_len, path, status, new_len, M_max,
                         stream=None):
    """In place on k_pages / v_pages [n_layers][num_pages][Hkv][page_size][d] (or without the
    layer dimension); block_table int32 [B][max_blocks], shared by every layer."""
    _i32(block_table, prefix_len, n_nodes, accept_len, path, status, new_len)
    if k_pages.dim() == 4:
        k_pages, v_pages = k_pages.unsqueeze(0), v_pages.unsqueeze(0)
    if k_pages.shape != v_pages.shape or k_pages.stride() != v_pages.stride() or k_pages.dtype != v_pages.dtype:
        raise ValueError("k_pages and v_pages must match")
    nl, num_pages, Hkv, page_size, d = k_pages.shape
    if k_pages.stride(4) != 1:
        raise ValueError("d must be contiguous")
    B = prefix_len.numel()
    if path.dim() != 2 or path.shape[0] != B or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("path must be [B][D_max] and block_table [B][max_blocks]")
    _vec(B, "n_nodes / accept_len / status / new_len", n_nodes, accept_len, status, new_len)
    _check(_lib.tmv_kv_commit_path_paged(_dtype_code(k_pages), nl, prefix_len.shape[0], Hkv, d, num_pages, page_size,
                                         _ptr(block_table), block_table.stride(0), block_table.shape[1], int(M_max),
                                         path.shape[1], _ptr(k_pages), _ptr(v_pages), _strides(k_pages, (0, 1, 2, 3)),
                                         _ptr(prefix_len), _ptr(n_nodes), _ptr(accept_len), _ptr(path), _ptr(status),
                                         _ptr(new_len), _stream(stream)),
           "kv_commit_path_paged")
    _debug("kv_commit_path_paged", status, stream)


def kv_commit_path_paged_evict(k_pages, v_pages, block_table, prefix_len, n_nodes, accept_len, path, status, new_len,
                               M_max, freed_pages, freed_count, stream=None):
    """kv_commit_path_paged, then block eviction: block_table (int32 [B][max_blocks], in/out)
    loses the tree blocks wholly past new_len, whose pages are appended to freed_pages
    (int32 device array) at indices counted by freed_count (int32 [1], in/out)."""
    _i32(block_table, prefix_len, n_nodes, accept_len, path, status, new_len, freed_pages, freed_count)
    if k_pages.dim() == 4:
        k_pages, v_pages = k_pages.unsqueeze(0), v_pages.unsqueeze(0)
    if k_pages.shape != v_pages.shape or k_pages.stride() != v_pages.stride() or k_pages.dtype != v_pages.dtype:
        raise ValueError("k_pages and v_pages must match")
    nl, num_pages, Hkv, page_size, d = k_pages.shape
    if k_pages.stride(4) != 1:
        raise ValueError("d must be contiguous")
    B = prefix_len.numel()
    if path.dim() != 2 or path.shape[0] != B or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("path must be [B][D_max] and block_table [B][max_blocks]")
    _vec(B, "n_nodes / accept_len / status / new_len", n_nodes, accept_len, status, new_len)
    _vec(1, "freed_count", freed_count)
    _check(_lib.tmv_kv_commit_path_paged_evict(_dtype_code(k_pages), nl, B, Hkv, d, num_pages, page_size,
                                               _ptr(block_table), block_table.stride(0), block_table.shape[1],
                                               int(M_max), path.shape[1], _ptr(k_pages), _ptr(v_pages),
                                               _strides(k_pages, (0, 1, 2, 3)), _ptr(prefix_len), _ptr(n_nodes),
                                               _ptr(accept_len), _ptr(path), _ptr(status), _ptr(new_len),
                                               _ptr(freed_pages), _ptr(freed_count), freed_pages.numel(),
                                               _stream(stream)),
           "kv_commit_path_paged_evict")
    _debug("kv_commit_path_paged_evict", status, stream)


# ------------------------------------------------------------------------ tree construction
def tree_best_first_workspace(B, D, V, N_max) -> int:
    return int(_lib.tmv_tree_best_first_workspace(B, D, V, N_max))


def tree_best_first(q, N_max, parents, tokens, n_nodes, rho, status, cost=None, l_ar=1.0, workspace=None,
                    stream=None):
    """q float32 [B][D][V] (vocabulary contiguous); parents, tokens int32 [B][N_max+1], n_nodes
    int32 [B], rho float64 [B][N_max+1] (outputs); status int32 [B] (in/out); cost float64
    [N_max] device tensor or None."""
    _i32(parents, tokens, n_nodes, status)
    if q.dtype != torch.float32 or q.stride(2) != 1 or not q.is_cuda:
        raise ValueError("q must be a float32 device tensor with a contiguous vocabulary")
    if rho.dtype != torch.float64 or not rho.is_contiguous():
        raise TypeError("rho must be contiguous float64")
    if cost is not None and (cost.dtype != torch.float64 or not cost.is_contiguous() or cost.numel() < N_max):
        raise ValueError("cost must be a contiguous float64 tensor of N_max entries")
    B, D, V = q.shape
    if tuple(parents.shape) != (B, N_max + 1) or tuple(tokens.shape) != (B, N_max + 1) or \
            tuple(rho.shape) != (B, N_max + 1):
        raise ValueError("outputs must be [B][N_max+1]")
    _vec(B, "n_nodes / status", n_nodes, status)
    if workspace is None:
        workspace = _temp_workspace(tree_best_first_workspace(B, D, V, N_max), q.device, stream, zero=False)
    _check(_lib.tmv_tree_best_first(B, D, V, int(N_max), _ptr(q), q.stride(0), q.stride(1), _ptr(cost),
                                    ctypes.c_double(l_ar), _ptr(parents), _ptr(tokens), _ptr(n_nodes), _ptr(rho),
                                    _ptr(status), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)),
           "tree_best_first")
    _debug("tree_best_first", status, stream)


class Workspaces:
    """Workspaces cached by size and device, zero-filled when created (the attention
    workspace's arrival counters must start at zero; every call leaves them at zero)."""

    def __init__(self):
        self._cache = {}

    def get(self, nbytes, device):
        key = (int(nbytes), str(device))
        ws = self._cache.get(key)
        if ws is None:
            ws = torch.zeros(max(256, int(nbytes)), dtype=torch.uint8, device=device)
            self._cache[key] = ws
        return ws
