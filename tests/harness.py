"""Shared plumbing of the GPU tests: move a tmv_inputs workload to the device, run the
four stages through the C ABI binding, and run the same bytes through the oracle."""
from __future__ import annotations

import numpy as np
import torch

import tmv_inputs as ti


GUARD_BYTES = 4096          # canary band on each side of a guarded device buffer
GUARD_FILL = 0xA5


class Guards:
    """Device buffers with canary bands: each lives in the middle of a larger allocation
    whose first and last GUARD_BYTES hold GUARD_FILL, and check() fails if any band changed
    -- a write past either end of an output or a cache."""

    def __init__(self):
        self.bufs = []

    def alloc(self, shape, dtype, fill=None, like=None):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        raw = torch.full((n + 2 * GUARD_BYTES,), GUARD_FILL, dtype=torch.uint8, device="cuda")
        t = raw[GUARD_BYTES:GUARD_BYTES + n].view(dtype).view(tuple(shape))
        if like is not None:
            t.copy_(like)
        elif fill is not None:
            t.fill_(fill)
        self.bufs.append((raw, n))
        return t

    def check(self):
        for raw, n in self.bufs:
            lo = raw[:GUARD_BYTES].cpu().numpy()
            hi = raw[GUARD_BYTES + n:].cpu().numpy()
            assert np.all(lo == GUARD_FILL) and np.all(hi == GUARD_FILL), "a canary band was overwritten"


def dev_tensor(a, bf16=False):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if bf16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def host_bits(t):
    """Device tensor -> numpy (bf16 as uint16 bit patterns)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_f64(bits):
    return ti.bf16_to_f32(bits).astype(np.float64)


class DeviceStep:
    """The device tensors of one workload and its per-stage outputs."""

    def __init__(self, w: ti.Workload):
        import tree_masked_verification_amd as tmv
        self.tmv = tmv
        self.w = w
        B, M, D = w.B, w.M_max, w.D_max
        bf = w.dtype == ti.BF16
        self.guards = Guards()
        g = self.guards
        self.parents = dev_tensor(w.parents.astype(np.int32))
        self.n_nodes = dev_tensor(w.n_nodes.astype(np.int32))
        self.prefix = dev_tensor(w.prefix.astype(np.int32))
        self.tokens = dev_tensor(w.tokens.astype(np.int32))
        i32 = torch.int32
        self.anc = g.alloc((B, M + 1, D + 1), i32, fill=-7)
        self.depth = g.alloc((B, M + 1), i32, fill=-7)
        self.status = g.alloc((B,), i32, fill=-7)
        if w.q is not None:
            self.q = dev_tensor(w.q, bf)
            # the caches are written by the commit: guarded too
            self.k = g.alloc(w.k.shape, torch.bfloat16 if bf else torch.float32, like=dev_tensor(w.k, bf))
            self.v = g.alloc(w.v.shape, torch.bfloat16 if bf else torch.float32, like=dev_tensor(w.v, bf))
            self.out = g.alloc(w.q.shape, torch.bfloat16 if bf else torch.float32, fill=float("nan"))
        if w.logits is not None:
            self.logits = dev_tensor(w.logits)
        if w.p is not None:
            self.p = dev_tensor(w.p)
            self.qd = dev_tensor(w.qd)
        self.accept_len = g.alloc((B,), i32, fill=-7)
        self.path = g.alloc((B, D), i32, fill=-7)
        self.next_token = g.alloc((B,), i32, fill=-7)
        self.new_len = g.alloc((B,), i32, fill=-7)

    def build(self, valid=None, parent_format=0, parents=None):
        self.tmv.tree_build_ancestors(self.parents if parents is None else parents, self.n_nodes, self.anc,
                                      self.depth, self.status, parent_format=parent_format, valid=valid)
        self.guards.check()

    def attention(self, workspace=None, plan=None):
        self.tmv.tree_verify_attention(self.q, self.k, self.v, self.prefix, self.n_nodes, self.anc, self.depth,
                                       self.status, self.out, scale=self.w.scale, workspace=workspace, plan=plan)
        self.guards.check()

    def accept(self, workspace=None):
        w = self.w
        if w.mode == "greedy":
            self.tmv.tree_accept(self.tmv.ACCEPT_GREEDY, self.tokens, self.logits, self.n_nodes, self.anc,
                                 self.depth, self.status, self.accept_len, self.path, self.next_token,
                                 workspace=workspace)
        else:
            self.tmv.tree_accept(self.tmv.ACCEPT_SAMPLE, self.tokens, self.p, self.n_nodes, self.anc, self.depth,
                                 self.status, self.accept_len, self.path, self.next_token, draft_q=self.qd,
                                 seed=w.seed, step=w.step, workspace=workspace)
        self.guards.check()

    def commit(self, k_cache=None, v_cache=None):
        kc = self.k if k_cache is None else k_cache
        vc = self.v if v_cache is None else v_cache
        self.tmv.kv_commit_path(kc, vc, self.prefix, self.n_nodes, self.accept_len, self.path, self.status,
                                self.new_len, self.w.M_max)
        self.guards.check()

    def tables(self):
        torch.cuda.synchronize()
        return host_bits(self.anc), host_bits(self.depth), host_bits(self.status)


def oracle_tables(ref, w, valid=None):
    return ref.build_ancestors(w.parents, w.n_nodes, w.M_max, w.D_max, valid=valid)


def oracle_attention(ref, w, anc, depth, status, row_select=None):
    return ref.tree_attention(w.q, w.k, w.v, w.prefix, w.n_nodes, anc, depth, status, w.scale, w.dtype, w.Hkv,
                              row_select=row_select)


def attention_error(dev_out_bits, ref_out, dtype, mask_rows=None):
    """max |dev - ref| and relative L2 over the compared rows."""
    dev = bf16_f64(dev_out_bits) if dtype == ti.BF16 else dev_out_bits.astype(np.float64)
    if mask_rows is not None:
        dev = dev[mask_rows]
        ref_out = ref_out[mask_rows]
    diff = np.abs(dev - ref_out)
    rel = np.linalg.norm(dev - ref_out) / max(np.linalg.norm(ref_out), 1e-300)
    return float(diff.max()) if diff.size else 0.0, float(rel)
