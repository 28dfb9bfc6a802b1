"""The allocation-free attention entry point, called through the C ABI: its rows must be
bit-identical to the workspace entry point's on the same inputs (same kernels and plan),
on two calls in a row, the second with a smaller input (then the first shape again)."""
import ctypes

import numpy as np
import pytest
import torch

import tmv_inputs as ti
from tests.harness import DeviceStep, host_bits
from tests.test_gpu_parity import small_attention_workload

pytestmark = pytest.mark.gpu


def _noalloc(dev):
    import tree_masked_verification_amd as tmv
    lib = tmv.library()
    w = dev.w
    q, k, out = dev.q, dev.k, dev.out
    B, M_max, Hq, d = q.shape
    Hkv, L_cap = k.shape[1], k.shape[2]
    st = lambda t: (ctypes.c_int64 * 3)(*[t.stride(i) for i in range(3)])
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = lib.tmv_tree_verify_attention_noalloc(
        1 if w.dtype == ti.BF16 else 0, B, M_max, dev.anc.shape[2] - 1, Hq, Hkv, d, p(q), st(q), p(k), p(dev.v),
        st(k), L_cap, p(dev.prefix), p(dev.n_nodes), p(dev.anc), p(dev.depth), p(dev.status), ctypes.c_float(w.scale),
        p(out), st(out), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return rc


def _compare(w):
    dev = DeviceStep(w)
    dev.build()
    dev.out.fill_(float("nan"))
    dev.attention()                              # the workspace entry point
    torch.cuda.synchronize()
    ref = host_bits(dev.out).copy()
    dev.out.fill_(float("nan"))
    assert _noalloc(dev) == 0
    torch.cuda.synchronize()
    got = host_bits(dev.out)
    assert np.array_equal(got, ref)
    assert np.array_equal(host_bits(dev.status), np.zeros(w.B, np.int32))


def test_noalloc_matches_workspace_entry_twice():
    print("\n[gpu case] attention no-alloc: 8B-shaped layer, then a smaller ragged batch", flush=True)
    _compare(ti.workload(2))
    _compare(small_attention_workload(401, 3, 8, 2, 128, 37, [700, 33, 5], [37, 20, 1], q_scale=4.0))
    # and the large one again on the scratch the smaller call left behind
    _compare(ti.workload(2))
