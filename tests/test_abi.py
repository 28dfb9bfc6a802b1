"""The C ABI library loads and exports every symbol declared in include/tmv.h; host-side
argument checks reject bad calls before anything is launched (these calls touch no GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "tmv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tmv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_stages():
    names = declared_functions()
    for n in ("tmv_tree_build_ancestors", "tmv_tree_verify_attention", "tmv_tree_accept", "tmv_kv_commit_path"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import tree_masked_verification_amd as tmv
    lib = ctypes.CDLL(tmv.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(tmv.EXPORTED)


def test_status_strings_and_version():
    import tree_masked_verification_amd as tmv
    assert tmv.abi_version() == 2
    names = {tmv.status_string(c) for c in range(8)}
    assert len(names) == 8 and tmv.status_string(99) == "unknown status"


def test_workspace_sizes_are_host_only():
    import tree_masked_verification_amd as tmv
    assert tmv.tree_verify_attention_workspace(tmv.BF16, 1, 60, 32, 8, 128, 2112) >= 256
    assert tmv.tree_verify_attention_workspace(tmv.F32, 1, 7, 1, 1, 64, 135) == 256
    big = tmv.tree_accept_workspace(tmv.ACCEPT_GREEDY, 16, 128, 128256)
    assert big >= 16 * 129 * 16 * 8
    # sampling: one synchronisation block (4224 bytes) per sequence, nothing per vocabulary entry
    assert 32 * 4224 <= tmv.tree_accept_workspace(tmv.ACCEPT_SAMPLE, 32, 32, 128256) < 32 * 8192


def test_argument_checks_return_before_launch():
    import tree_masked_verification_amd as tmv
    lib = tmv.library()
    P = ctypes.c_void_p
    fake = P(0x1000)
    s3 = (ctypes.c_int64 * 3)(1, 1, 1)
    s4 = (ctypes.c_int64 * 4)(8, 8, 8, 8)
    # build: M_max > 128, bad format, null outputs
    assert lib.tmv_tree_build_ancestors(1, 129, 4, 0, fake, None, fake, fake, fake, fake, None) == tmv.ERR_ARG
    assert lib.tmv_tree_build_ancestors(1, 8, 4, 7, fake, None, fake, fake, fake, fake, None) == tmv.ERR_ARG
    assert lib.tmv_tree_build_ancestors(1, 8, 4, 0, fake, None, fake, None, fake, fake, None) == tmv.ERR_ARG
    assert lib.tmv_tree_build_ancestors(0, 8, 4, 0, None, None, None, None, None, None, None) == tmv.OK
    # attention: head_dim, GQA ratio, dtype, workspace too small
    args = lambda dt, Hq, Hkv, d, ws, wsb: (dt, 1, 8, 4, Hq, Hkv, d, fake, s3, fake, fake, s3, 64, fake, fake, fake,
                                          fake, fake, ctypes.c_float(0.1), fake, s3, ws, wsb, None)
    assert lib.tmv_tree_verify_attention(*args(tmv.BF16, 8, 2, 96, fake, 1 << 20)) == tmv.ERR_ARG
    assert lib.tmv_tree_verify_attention(*args(tmv.BF16, 9, 2, 128, fake, 1 << 20)) == tmv.ERR_ARG
    assert lib.tmv_tree_verify_attention(*args(5, 8, 2, 128, fake, 1 << 20)) == tmv.ERR_ARG
    assert lib.tmv_tree_verify_attention(*args(tmv.BF16, 8, 2, 128, fake, 16)) == tmv.ERR_ARG
    assert lib.tmv_tree_verify_attention(*args(tmv.BF16, 8, 2, 128, None, 1 << 20)) == tmv.ERR_ARG
    # accept: unknown mode, sampling without q, workspace too small
    acc = lambda mode, rd, q, wsb: (mode, 1, 8, 4, 100, fake, rd, fake, 900, 100, q, 900, 100, ctypes.c_uint64(1),
                                    ctypes.c_uint64(0), fake, fake, fake, fake, fake, fake, fake, fake, wsb, None)
    assert lib.tmv_tree_accept(*acc(3, 0, None, 1 << 20)) == tmv.ERR_ARG
    assert lib.tmv_tree_accept(*acc(tmv.ACCEPT_SAMPLE, 0, None, 1 << 20)) == tmv.ERR_ARG
    assert lib.tmv_tree_accept(*acc(tmv.ACCEPT_GREEDY, 0, None, 8)) == tmv.ERR_ARG
    assert lib.tmv_tree_accept(*acc(tmv.ACCEPT_GREEDY, 4, None, 1 << 20)) == tmv.ERR_ARG
    big_v = (tmv.ACCEPT_SAMPLE, 1, 8, 4, (1 << 24) + 1, fake, 0, fake, 9 * ((1 << 24) + 1), (1 << 24) + 1, fake,
             9 * ((1 << 24) + 1), (1 << 24) + 1, ctypes.c_uint64(1), ctypes.c_uint64(0), fake, fake, fake, fake, fake,
             fake, fake, fake, 1 << 20, None)
    assert lib.tmv_tree_accept(*big_v) == tmv.ERR_ARG                 # sampling vocabulary above 2^24
    # best-first: depth, vocabulary and budget limits, workspace too small
    bf = lambda D, V, N, wsb: (1, D, V, N, fake, 0, 0, None, ctypes.c_double(1.0), fake, fake, fake, fake, fake, fake,
                                wsb, None)
    assert lib.tmv_tree_best_first(*bf(0, 100, 8, 1 << 20)) == tmv.ERR_ARG
    assert lib.tmv_tree_best_first(*bf(9, 100, 8, 1 << 20)) == tmv.ERR_ARG
    assert lib.tmv_tree_best_first(*bf(4, 262145, 8, 1 << 30)) == tmv.ERR_ARG
    assert lib.tmv_tree_best_first(*bf(4, 100, 129, 1 << 20)) == tmv.ERR_ARG
    assert lib.tmv_tree_best_first(*bf(4, 100, 0, 1 << 20)) == tmv.ERR_ARG
    assert lib.tmv_tree_best_first(*bf(4, 100, 8, 16)) == tmv.ERR_ARG
    # commit: row bytes not a multiple of 16 / too large, misaligned strides
    com = lambda dt, d, st: (dt, 2, 1, 8, d, 64, 8, 4, fake, fake, st, fake, fake, fake, fake, fake, fake, None)
    assert lib.tmv_kv_commit_path(*com(tmv.BF16, 4, s4)) == tmv.ERR_ARG
    assert lib.tmv_kv_commit_path(*com(tmv.F32, 256, s4)) == tmv.ERR_ARG
    assert lib.tmv_kv_commit_path(*com(tmv.BF16, 128, (ctypes.c_int64 * 4)(8, 8, 8, 3))) == tmv.ERR_ARG
    # paged attention: bf16 d128 only; page size a power of two >= 16; table sizes
    s3p = (ctypes.c_int64 * 3)(8 * 16 * 128, 16 * 128, 128)
    pa = lambda dt, d, ps, nblk, ts, npg, wsb: (dt, 1, 8, 4, 8, 2, d, fake, s3, fake, fake, s3p, npg, ps, fake,
                                                ctypes.c_int64(ts), nblk, fake, fake, fake, fake, fake,
                                                ctypes.c_float(0.1), fake, s3, fake, wsb, None)
    ok_ws = tmv.tree_verify_attention_paged_workspace(1, 8, 8, 2, 128, 16, 64)
    assert ok_ws >= 1024
    assert lib.tmv_tree_verify_attention_paged(*pa(tmv.F32, 128, 16, 64, 64, 100, ok_ws)) == tmv.ERR_ARG
    assert lib.tmv_tree_verify_attention_paged(*pa(tmv.BF16, 64, 16, 64, 64, 100, ok_ws)) == tmv.ERR_ARG
    assert lib.tmv_tree_verify_attention_paged(*pa(tmv.BF16, 128, 24, 64, 64, 100, ok_ws)) == tmv.ERR_ARG
    assert lib.tmv_tree_verify_attention_paged(*pa(tmv.BF16, 128, 8, 64, 64, 100, ok_ws)) == tmv.ERR_ARG
    assert lib.tmv_tree_verify_attention_paged(*pa(tmv.BF16, 128, 16, 4097, 4097, 100, 1 << 30)) == tmv.ERR_ARG
    assert lib.tmv_tree_verify_attention_paged(*pa(tmv.BF16, 128, 16, 64, 63, 100, ok_ws)) == tmv.ERR_ARG
    assert lib.tmv_tree_verify_attention_paged(*pa(tmv.BF16, 128, 16, 64, 64, 0, ok_ws)) == tmv.ERR_ARG
    assert lib.tmv_tree_verify_attention_paged(*pa(tmv.BF16, 128, 16, 64, 64, 100, 16)) == tmv.ERR_ARG
    # paged commit: page size, table width, row bytes
    s4p = (ctypes.c_int64 * 4)(100 * 8 * 16 * 128, 8 * 16 * 128, 16 * 128, 128)
    pc = lambda ps, nblk, ts, d: (tmv.BF16, 2, 1, 8, d, 100, ps, fake, ctypes.c_int64(ts), nblk, 8, 4, fake, fake, s4p,
                                  fake, fake, fake, fake, fake, fake, None)
    assert lib.tmv_kv_commit_path_paged(*pc(12, 8, 8, 128)) == tmv.ERR_ARG
    assert lib.tmv_kv_commit_path_paged(*pc(16, 8, 7, 128)) == tmv.ERR_ARG
    assert lib.tmv_kv_commit_path_paged(*pc(16, 0, 8, 128)) == tmv.ERR_ARG
    assert lib.tmv_kv_commit_path_paged(*pc(16, 8, 8, 4)) == tmv.ERR_ARG


def test_package_fails_loudly_without_library(tmp_path):
    """Importing the binding with the library missing raises ImportError (no fallback)."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "tree_masked_verification_amd"
    shutil.copytree(os.path.join(ROOT, "tree_masked_verification_amd"), pkg,
                    ignore=shutil.ignore_patterns("*.so", "_build", "__pycache__"))
    r = subprocess.run([sys.executable, "-c", "import tree_masked_verification_amd"], cwd=tmp_path,
                       capture_output=True, text=True)
    assert r.returncode != 0 and "ImportError" in r.stderr and "no CPU fallback" in r.stderr


def test_debug_mode_reports_failed_sequences(capsys, monkeypatch):
    """TMV_DEBUG=1 makes the binding report, after a call, every sequence whose status is not
    OK (here on a host status array: no GPU call is made)."""
    import torch
    import tree_masked_verification_amd as tmv
    st = torch.tensor([tmv.OK, tmv.ERR_CYCLE, tmv.OK, tmv.ERR_DEVICE], dtype=torch.int32)
    monkeypatch.setattr(tmv, "DEBUG", False)
    assert tmv._debug("tree_verify_attention", st) == []
    assert capsys.readouterr().err == ""
    monkeypatch.setattr(tmv, "DEBUG", True)
    bad = tmv._debug("tree_verify_attention", st)
    assert [i for i, _ in bad] == [1, 3]
    err = capsys.readouterr().err
    assert "tree_verify_attention: 2 of 4 sequences not OK" in err and tmv.status_string(tmv.ERR_CYCLE) in err
