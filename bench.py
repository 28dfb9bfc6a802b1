#!/usr/bin/env python3
"""Benchmark of the tree-verification step on one MI355X.

A step is one pass of the whole verify path over one batch of synthetic, seeded input:
tree_build_ancestors, tree_verify_attention, tree_accept and kv_commit_path.  The default
workload (the one the headline metric is quoted on) is the Llama-3-8B-shaped single layer:
bf16, 32 query / 8 KV heads, head_dim 128, batch 1, prefix 2048, 60-node static tree of
depth 6, vocabulary 128256, greedy acceptance.  `--workload N` measures the others:
  1  tiny fp32 step (1 head, d64, prefix 128, 7-node tree, vocabulary 32)
  3  batch 16 of ragged prefixes (512..4096) and best-first trees of 16..128 nodes
  4  70B-shaped layer: 64 / 8 heads, batch 4, prefix 32768, 64-node random trees
  5  sampling acceptance (batch 32, 32-node trees, p and q over 128256 tokens) and the
     commit of the accepted paths over 32 layers of 8 KV heads x d128 (no attention)
Inputs are resident in HBM before timing and rotated over enough distinct sets that
reads miss the 256 MB Infinity Cache (each set of workloads 3-5 is larger than it).

Timed regions (both after --warmup untimed steps):
  1. throughput: --steps steps, bracketed by torch.cuda.synchronize(); the steps run as
     replays of one HIP graph that holds a step on every input set in turn (plus one graph
     for the remainder); value = verified node-tokens per second.
  2. kernel durations: for each stage, one HIP graph of back-to-back launches over the
     rotating sets (device copies added until the stage's own inputs exceed the Infinity
     Cache 2.5 times), timed with HIP events recorded on the stream the kernels run on;
     the average launch duration feeds the roofline figures.
  3. workload 3 only: device best-first tree construction at its drafter shape (16
     sequences, 8 positions, vocabulary 128256, budget 128), reported as "drafting" beside
     the step (it builds the trees a step verifies; it is not part of the step).
  4. workloads 2-4: the paged-cache attention and commit on the same sets (K/V in pools
     of 16-token pages at random places), timed like region 2, reported as "paged".
  5. a streaming ceiling of the device (the better of torch.amax over 4 GiB and a 2 GiB
     device copy), reported as "stream_read_ceiling"; every kernel's GB/s is also given as
     a fraction of it.
  6. workloads 2 and 4: greedy acceptance straight from the LM head (hidden 4096 / 8192,
     vocabulary 128256, synthetic bf16 weights): the fused product + argmax against a
     library GEMM that writes the logits followed by tree_accept, reported as "lm_head".
The oracle (tests-only CPU implementation) is timed on a bounded sample of the same
workload for the cpu_baseline field: once on one thread, then as one process per host
thread (at most 16) running the sample concurrently.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
MALL_BYTES = 256 << 20          # Infinity Cache
ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "tree-verify node-tokens/s and achieved HBM GB/s (% of peak) at 1 MI355X"


# ---------------------------------------------------------------- roofline helpers
def ridge_point(peak_flops, peak_bytes_per_s):
    """FLOP per byte where a kernel turns from bandwidth- to compute-bound."""
    return peak_flops / peak_bytes_per_s


def read_time_s(nbytes, bytes_per_s):
    return nbytes / bytes_per_s


def attention_work(M_nodes_depths, P, Hq, Hkv, d, elem=2):
    """Algorithmic bytes and flops of one tree-attention launch for one sequence:
    Q and O once, each KV head's prefix + tree rows once; flops over visible keys only."""
    M = len(M_nodes_depths)
    q_bytes = M * Hq * d * elem
    kv_bytes = 2 * Hkv * (P + M) * d * elem
    flops = 4 * d * Hq * sum(P + dep for dep in M_nodes_depths)
    return 2 * q_bytes + kv_bytes, flops


def workload_work(w, depth, accept_len):
    """Algorithmic bytes and flops per launch of every stage of one step of workload w,
    given the device-built depths [B][M_max+1] and the accepted lengths [B]."""
    elem = 4 if w.dtype == 0 else 2
    nodes = [int(n) for n in w.n_nodes]
    work = {"build": (w.B * (w.M_max + 1) * 4 * (w.D_max + 3), 0)}
    if w.mode == "greedy":
        ab, af = 0, 0
        for b in range(w.B):
            nb, fl = attention_work(depth[b, 1:nodes[b] + 1].tolist(), int(w.prefix[b]), w.Hq, w.Hkv, w.d, elem)
            ab += nb + (w.M_max + 1) * (w.D_max + 2) * 4                 # ancestor table + depths
            af += fl
        work["attention"] = (ab, af)
        # every live row of the teacher's logits once (row 0 plus the nodes)
        work["accept"] = (sum(n + 1 for n in nodes) * w.V * 4 + w.B * (w.M_max + 1) * 4, 0)
    else:
        # the sampling walk reads the teacher's and the draft's row of every visited node
        visited = int(np.sum(accept_len)) + w.B
        work["accept"] = (visited * w.V * 4 * 2, 0)
    # every accepted row of K and V read and written once, per layer and KV head
    work["commit"] = (int(2 * 2 * w.n_layers * w.Hkv * w.d * elem * int(np.sum(accept_len))), 0)
    return work


# ---------------------------------------------------------------- workload sets
class StepSet:
    """Device tensors of one input set and its stage outputs."""

    def __init__(self, tmv, torch, w, ws_attn, ws_acc, caches=None):
        dev = "cuda"
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        self.tmv, self.torch = tmv, torch
        self.w = w
        self.parents = t(w.parents.astype(np.int32))
        self.n_nodes = t(w.n_nodes.astype(np.int32))
        self.prefix = t(w.prefix.astype(np.int32))
        self.tokens = t(w.tokens.astype(np.int32))
        if w.mode == "greedy":
            bf = w.dtype == 1
            self.q, self.k, self.v = (t(a).view(torch.bfloat16) if bf else t(a) for a in (w.q, w.k, w.v))
            self.out = torch.zeros_like(self.q)
            self.logits = t(w.logits)
        else:
            self.p, self.qd = t(w.p), t(w.qd)
            self.k, self.v = caches
        B, M, D = w.B, w.M_max, w.D_max
        i32 = dict(dtype=torch.int32, device=dev)
        self.anc = torch.zeros((B, M + 1, D + 1), **i32)
        self.depth = torch.zeros((B, M + 1), **i32)
        self.status = torch.zeros((B,), **i32)
        self.accept_len = torch.zeros((B,), **i32)
        self.path = torch.zeros((B, D), **i32)
        self.next_token = torch.zeros((B,), **i32)
        self.new_len = torch.zeros((B,), **i32)
        self.ws_attn, self.ws_acc = ws_attn, ws_acc

    def build(self):
        self.tmv.tree_build_ancestors(self.parents, self.n_nodes, self.anc, self.depth, self.status)

    def attention(self):
        self.tmv.tree_verify_attention(self.q, self.k, self.v, self.prefix, self.n_nodes, self.anc, self.depth,
                                       self.status, self.out, scale=self.w.scale, workspace=self.ws_attn)

    def accept(self):
        if self.w.mode == "greedy":
            self.tmv.tree_accept(self.tmv.ACCEPT_GREEDY, self.tokens, self.logits, self.n_nodes, self.anc, self.depth,
                                 self.status, self.accept_len, self.path, self.next_token, workspace=self.ws_acc)
        else:
            self.tmv.tree_accept(self.tmv.ACCEPT_SAMPLE, self.tokens, self.p, self.n_nodes, self.anc, self.depth,
                                 self.status, self.accept_len, self.path, self.next_token, draft_q=self.qd,
                                 seed=self.w.seed, step=self.w.step, workspace=self.ws_acc)

    def commit(self):
        self.tmv.kv_commit_path(self.k, self.v, self.prefix, self.n_nodes, self.accept_len, self.path, self.status,
                                self.new_len, self.w.M_max)

    def clone(self):
        """A copy of this set at new device addresses (inputs copied, outputs fresh)."""
        other = object.__new__(StepSet)
        other.__dict__.update(self.__dict__)
        names = ["parents", "n_nodes", "prefix", "tokens", "anc", "depth", "status", "accept_len", "path",
                 "next_token", "new_len"]
        names += ["q", "k", "v", "out", "logits"] if self.w.mode == "greedy" else ["p", "qd"]
        for n in names:
            setattr(other, n, getattr(self, n).clone())
        return other

    def stages(self):
        names = ["build", "attention", "accept", "commit"] if self.w.mode == "greedy" else ["build", "accept", "commit"]
        return {n: getattr(self, n) for n in names}

    def step(self):
        for fn in self.stages().values():
            fn()


def set_bytes(w):
    if w.mode == "greedy":
        return w.q.nbytes + w.k.nbytes + w.v.nbytes + w.logits.nbytes + w.q.nbytes
    return w.p.nbytes + w.qd.nbytes


# ---------------------------------------------------------------- counters from profiles/
# the sources each timed stage is compiled from (its kernels plus the shared device header
# and the C ABI header)
STAGE_SOURCES = {
    "build": ["build_ancestors.hip"],
    "attention": ["verify_attention.hip"],
    "accept": ["accept.hip"],
    "commit": ["commit.hip"],
    "lm_head": ["accept.hip"],
}


def stage_source_digest(stage):
    h = hashlib.sha256()
    src = os.path.join(ROOT, "tree_masked_verification_amd", "csrc")
    for name in STAGE_SOURCES[stage] + ["tmv_device.hpp"]:
        with open(os.path.join(src, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    with open(os.path.join(ROOT, "include", "tmv.h"), "rb") as f:
        h.update(b"tmv.h\0" + f.read())
    return h.hexdigest()


def traffic_from_profiles(stage, workload):
    """HBM bytes per launch of `stage` from the committed rocprofv3 counter runs of this
    workload, or None when none was taken or the stage's sources changed since."""
    path = os.path.join(ROOT, "profiles", "hbm_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    k = rec.get("workloads", {}).get(str(workload), {}).get(stage)
    if k is None or k.get("source_sha256") != stage_source_digest(stage):
        return None
    return k.get("hbm_bytes_per_launch")


STAGE_KERNELS = {
    "build": ("build_ancestors_kernel",),
    "attention": ("tree_attn_bf16_kernel", "tree_attn_bf16_stream_kernel", "tree_attn_merge_kernel",
                  "tree_attn_f32_kernel"),
    "accept": ("greedy_accept_kernel", "greedy_scan_kernel", "greedy_select_kernel", "sample_walk_kernel"),
    "commit": ("commit_kernel",),
}


def stage_of(kernel_name):
    """The timed stage a dispatched kernel belongs to; None for the paged-cache variants
    (block-table template argument true), library kernels and everything else."""
    import re
    if re.search(r"tree_attn_bf16_kernel<\d+, \d+, (true|false), true\b", kernel_name) or "commit_kernel<true>" in kernel_name:
        return None
    for stage, names in STAGE_KERNELS.items():
        if any(re.search(r"\b%s\b" % n, kernel_name) for n in names):
            return stage
    return None


def ingest_counters(workload, fetch_csv, write_csv, command):
    """HBM bytes per launch of each stage from two rocprofv3 --pmc runs of this script with
    --copy-probe (FETCH_SIZE, then WRITE_SIZE; per-dispatch KiB), each counter scaled by the
    factor that makes it read the copy probe's known 256 MiB, into profiles/hbm_counters.json
    under this workload, with each stage's source digest."""
    import csv
    import collections
    import re

    def per_kernel(path):
        agg = collections.defaultdict(list)
        with open(path) as f:
            for r in csv.DictReader(f):
                agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in agg.items()}

    fe, wr = per_kernel(fetch_csv), per_kernel(write_csv)
    probe_kib = (256 << 20) / 1024
    probe = [k for k in fe if "AUnaryFunctor" in k or "BUnaryFunctor" in k]
    if len(probe) != 1:
        raise RuntimeError("copy probe kernel not found once in the counter run: %s" % probe)
    fscale, wscale = probe_kib / fe[probe[0]], probe_kib / wr[probe[0]]
    stages = {}
    for k in fe:
        st = stage_of(k)
        if st is None:
            continue
        e = stages.setdefault(st, {"fetch_kib": 0.0, "write_kib": 0.0, "kernels": []})
        e["fetch_kib"] += fe[k]
        e["write_kib"] += wr.get(k, 0.0)
        m = re.search(r"(\w+_kernel(<[^>]*>)?)", k)
        e["kernels"].append(m.group(1) if m else k[:80])
    for st, e in stages.items():
        e["hbm_bytes_per_launch"] = (e["fetch_kib"] * fscale + e["write_kib"] * wscale) * 1024
        e["source_sha256"] = stage_source_digest(st)
    path = os.path.join(ROOT, "profiles", "hbm_counters.json")
    rec = {"workloads": {}}
    if os.path.exists(path):
        with open(path) as f:
            rec = json.load(f)
        rec.setdefault("workloads", {})
    rec["copy_probe_bytes"] = 256 << 20
    rec["how"] = ("rocprofv3 FETCH_SIZE and WRITE_SIZE per dispatch (KiB), each scaled by the copy probe's "
                  "known size, summed over the stage's kernels (one dispatch each per launch)")
    rec["workloads"][str(workload)] = {"fetch_scale": fscale, "write_scale": wscale, "command": command, **stages}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    return rec["workloads"][str(workload)]


# ---------------------------------------------------------------- CPU baseline
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def host_threads():
    """CPU threads this process may use, at most 16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def slice_workload(w, seqs):
    """The sequences `seqs` of workload w as a workload of their own (same layer)."""
    import dataclasses
    sl = lambda a: None if a is None else np.ascontiguousarray(a[seqs])
    return dataclasses.replace(w, B=len(seqs), parents=sl(w.parents), n_nodes=sl(w.n_nodes), prefix=sl(w.prefix),
                               tokens=sl(w.tokens), q=sl(w.q), k=sl(w.k), v=sl(w.v), logits=sl(w.logits),
                               p=sl(w.p), qd=sl(w.qd))


def cpu_sample(c, w):
    """The bounded sample of workload c the oracle is timed on: (sample workload, attention
    rows to compute or None for all, the factor from sampled to whole-step attention time,
    layers of cache the commit sample moves, the factor to the workload's layers, words)."""
    if c in (1, 2):
        return w, None, 1.0, 1, 1.0, "whole verify steps of the workload"
    if c == 3:
        s = slice_workload(w, [0])
        return s, None, 1.0, 1, 1.0, ("verify steps of sequence 0 of the batch (prefix %d, %d nodes)"
                                      % (int(s.prefix[0]), int(s.n_nodes[0])))
    if c == 4:
        s = slice_workload(w, [0])
        rows = np.zeros((1, s.M_max), np.uint8)
        rows[0, ::8] = 1
        return s, rows, s.M_max / int(rows.sum()), 1, 1.0, (
            "verify steps of sequence 0 of the batch with the attention over every 8th tree node (%d of %d, its "
            "time scaled by %d)" % (int(rows.sum()), s.M_max, s.M_max // int(rows.sum())))
    s = slice_workload(w, [0, 1, 2, 3])
    return s, None, 1.0, 1, float(w.n_layers), ("sampling acceptance of sequences 0-3 of the batch and their "
                                                "commit over 1 of the %d layers (its time scaled by %d)"
                                                % (w.n_layers, w.n_layers))


def oracle_worker(args):
    """Oracle verify steps on a sample for about budget_s seconds; returns (steps, seconds
    per stage).  Runs in a worker process of its own (the oracle is single-threaded)."""
    w, rows, layers, budget_s = args
    import oracle
    t = {"build": 0.0, "attention": 0.0, "accept": 0.0, "commit": 0.0}
    if w.mode == "greedy":
        k, v = w.k.copy()[None], w.v.copy()[None]
    else:
        shape = (layers, w.B, w.Hkv, w.L_cap, w.d)
        k, v = np.zeros(shape, np.uint16), np.ones(shape, np.uint16)
    steps, t0 = 0, time.perf_counter()
    while True:
        a = time.perf_counter()
        anc, depth, st = oracle.build_ancestors(w.parents, w.n_nodes, w.M_max, w.D_max)
        b = time.perf_counter()
        t["build"] += b - a
        if w.mode == "greedy":
            out, st = oracle.tree_attention(w.q, k[0], v[0], w.prefix, w.n_nodes, anc, depth, st, w.scale, w.dtype,
                                            w.Hkv, row_select=rows)
            a = time.perf_counter()
            t["attention"] += a - b
            A, path, nxt, st = oracle.accept_greedy(w.tokens, w.logits, w.n_nodes, anc, depth, st)
        else:
            a = time.perf_counter()
            A, path, nxt, st = oracle.accept_sample(w.tokens, w.p, w.qd, w.seed, w.step, w.n_nodes, anc, depth, st)
        b = time.perf_counter()
        t["accept"] += b - a
        oracle.commit(k, v, w.prefix, w.n_nodes, A, path, st, w.M_max)
        t["commit"] += time.perf_counter() - b
        steps += 1
        if time.perf_counter() - t0 >= budget_s or steps >= 1000:
            break
    return steps, t


def cpu_baseline(c, w, budget_s):
    """The oracle, as it stands, on a bounded sample of workload c: once on one thread, then
    as one process per host thread (up to 16) running the same sample concurrently; the
    value is the concurrent aggregate in node-tokens/s of the whole workload."""
    import multiprocessing as mp
    import oracle
    oracle.build()
    s, rows, attn_scale, layers, commit_scale, words = cpu_sample(c, w)
    nodes = int(s.n_nodes.sum())

    def rate(steps, t):
        step_s = (t["build"] + t["attention"] * attn_scale + t["accept"] + t["commit"] * commit_scale) / steps
        return nodes / step_s, step_s

    steps1, t1 = oracle_worker((s, rows, layers, budget_s))
    v1, step1 = rate(steps1, t1)
    n = host_threads()
    with mp.get_context("spawn").Pool(n) as pool:
        res = pool.map(oracle_worker, [(s, rows, layers, budget_s)] * n)
    vn = sum(rate(st, t)[0] for st, t in res)
    return {"value": round(vn, 2), "unit": "node-tokens/s", "cores": n, "kind": "oracle", "cpu": cpu_model(),
            "sample": "%s; the oracle on %d processes at once (one per host thread), each about %.0f s; the "
                      "single-thread leg ran %d step(s) at %.3g s per step" % (words, n, budget_s, steps1, step1),
            "single_thread": {"value": round(v1, 2), "cores": 1, "s_per_step": float("%.4g" % step1)}}


# ---------------------------------------------------------------- LM head with fused argmax
def time_lm_head(torch, tmv, s, stream, K, reps=20):
    """Greedy acceptance straight from the LM head on the first input set's trees: the fused
    bf16 product + argmax (logits never written) against a library bf16 GEMM that writes the
    logits followed by the greedy accept on them.  Hidden states N(0,1) and weights
    N(0, 0.03^2) bf16 from a seeded device generator; the weight matrix (K x vocabulary,
    1 GB at K 4096) is larger than the Infinity Cache, so every launch streams it from HBM."""
    w = s.w
    g = torch.Generator(device="cuda")
    g.manual_seed(777)
    W = (torch.randn((w.V, K), generator=g, device="cuda") * 0.03).to(torch.bfloat16)
    H = torch.randn((w.B, w.M_max + 1, K), generator=g, device="cuda").to(torch.bfloat16)
    i32 = dict(dtype=torch.int32, device="cuda")
    A, path, nxt = torch.zeros((w.B,), **i32), torch.zeros((w.B, w.D_max), **i32), torch.zeros((w.B,), **i32)
    A2, path2, nxt2 = torch.zeros_like(A), torch.zeros_like(path), torch.zeros_like(nxt)
    ws = torch.zeros(tmv.tree_accept_lm_head_workspace(w.B, w.M_max), dtype=torch.uint8, device="cuda")
    ws2 = torch.zeros(tmv.tree_accept_workspace(tmv.ACCEPT_GREEDY, w.B, w.M_max, w.V), dtype=torch.uint8,
                      device="cuda")
    logits = torch.empty((w.B, w.M_max + 1, w.V), dtype=torch.bfloat16, device="cuda")
    st = s.status
    torch.cuda.synchronize()            # weights and zeroed workspaces were made on torch's stream

    def fused():
        tmv.tree_accept_lm_head(s.tokens, H, W, s.n_nodes, s.anc, s.depth, st, A, path, nxt, workspace=ws,
                                stream=stream)

    def gemm():
        torch.matmul(H.view(-1, K), W.t(), out=logits.view(-1, w.V))

    def scan():
        tmv.tree_accept(tmv.ACCEPT_GREEDY, s.tokens, logits, s.n_nodes, s.anc, s.depth, st, A2, path2, nxt2,
                        workspace=ws2, stream=stream)

    def timed(fn):
        with torch.cuda.stream(stream):
            for _ in range(3):
                fn()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=stream):
                for _ in range(reps):
                    fn()
            gr.replay()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            gr.replay()
            e1.record(stream)
            e1.synchronize()
        del gr
        return e0.elapsed_time(e1) * 1e3 / reps

    us_f, us_g, us_s = timed(fused), timed(gemm), timed(scan)
    torch.cuda.synchronize()
    if int(st.abs().sum()) != 0:
        raise RuntimeError("tree_accept_lm_head reported a non-OK status")
    nb = w.V * K * 2 + H.numel() * 2
    fl = 2.0 * w.V * K * H.shape[0] * H.shape[1]
    gbs = nb / (us_f * 1e-6) / 1e9
    del W, H, logits
    torch.cuda.empty_cache()
    return {"hidden": K, "rows": w.B * (w.M_max + 1), "vocab": w.V,
            "fused_argmax": {"avg_us": round(us_f, 3), "bytes": int(nb), "GB/s": round(gbs, 1),
                             "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                             "TFLOP/s": round(fl / (us_f * 1e-6) / 1e12, 1)},
            "library_gemm_then_accept": {"avg_us": round(us_g + us_s, 3), "gemm_us": round(us_g, 3),
                                         "accept_us": round(us_s, 3),
                                         "how": "torch.matmul bf16 into bf16 logits, then tree_accept greedy"},
            "speedup": round((us_g + us_s) / us_f, 3)}


# ---------------------------------------------------------------- main
def time_best_first(torch, tmv, ti, stream, B=16, D=8, V=128256, N=128):
    """Device best-first tree construction (drafting side, not part of the verify step) at
    workload 3's drafter shape: per-position marginals softmax(N(0,3)) over the vocabulary,
    sets rotated past the Infinity Cache, one HIP graph of back-to-back launches timed with
    HIP events on its capture stream."""
    set_bytes = B * D * V * 4
    n_sets = max(2, math.ceil(2.5 * MALL_BYTES / set_bytes))
    rng = np.random.default_rng(3300)
    qs = [torch.from_numpy(ti.draft_marginals(rng, B, D, V)).cuda() for _ in range(n_sets)]
    parents = torch.zeros((B, N + 1), dtype=torch.int32, device="cuda")
    tokens = torch.zeros_like(parents)
    n_nodes = torch.zeros((B,), dtype=torch.int32, device="cuda")
    rho = torch.zeros((B, N + 1), dtype=torch.float64, device="cuda")
    status = torch.zeros((B,), dtype=torch.int32, device="cuda")
    ws = torch.empty(tmv.tree_best_first_workspace(B, D, V, N), dtype=torch.uint8, device="cuda")
    run = lambda q: tmv.tree_best_first(q, N, parents, tokens, n_nodes, rho, status, workspace=ws, stream=stream)
    reps = 40
    torch.cuda.synchronize()            # inputs were made on torch's stream
    with torch.cuda.stream(stream):
        for q in qs:
            run(q)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for r in range(reps):
                run(qs[r % n_sets])
        g.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        e1.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    if int(status.abs().sum()) != 0 or int(n_nodes.min()) != N:
        raise RuntimeError("tree_best_first: unexpected status or size")
    nb = set_bytes + B * (N + 1) * (4 + 4 + 8) + B * 4
    gbs = nb / (us * 1e-6) / 1e9
    del g
    return {"tree_best_first": {"avg_us": round(us, 3), "bytes": int(nb), "GB/s": round(gbs, 1),
                                "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                                "shape": "B%d positions %d vocab %d budget %d" % (B, D, V, N),
                                "input_sets": n_sets}}


def stream_read_ceiling(torch, stream, nbytes=4 << 30, reps=5):
    """A measured streaming ceiling of this device, the better of two plain library kernels,
    best of `reps` each, HIP events on the launch stream: the maximum over a 4 GiB fp32 tensor
    (every byte read once) and a 2 GiB device-to-device copy (bytes read + bytes written)."""
    def best_ms(fn):
        best = None
        with torch.cuda.stream(stream):
            fn()
            for _ in range(reps):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                e1.synchronize()
                ms = e0.elapsed_time(e1)
                best = ms if best is None else min(best, ms)
        return best
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    read = nbytes / (best_ms(lambda: torch.amax(x)) * 1e-3) / 1e9
    half = x[: x.numel() // 2]
    y = torch.empty_like(half)
    copy = nbytes / (best_ms(lambda: y.copy_(half)) * 1e-3) / 1e9
    del x, y, half
    torch.cuda.empty_cache()
    return {"GB/s": round(max(read, copy), 1), "read_GB/s": round(read, 1), "copy_GB/s": round(copy, 1),
            "how": "max of torch.amax over 4 GiB fp32 (bytes read) and a 2 GiB device copy (bytes read + written), "
                   "best of %d each" % reps}


def time_paged(torch, tmv, sets, stream, durations, page_size=16, reps=None):
    """The paged-cache calls on the same input sets: every set's K/V laid out in a pool of
    page_size-token pages at a random permutation (made on the device), the attention and
    commit timed like the contiguous stages (one HIP graph of back-to-back launches over
    the rotating sets, HIP events on its capture stream)."""
    g = torch.Generator(device="cpu").manual_seed(4242)
    paged = []
    w0 = sets[0].w
    ws = torch.zeros(tmv.tree_verify_attention_paged_workspace(w0.B, w0.M_max, w0.Hq, w0.Hkv, w0.d, page_size,
                                                               -(-w0.L_cap // page_size)),
                     dtype=torch.uint8, device="cuda")
    for s in sets:
        B, H, L, d = s.k.shape
        nblk = -(-L // page_size)
        perm = torch.randperm(B * nblk + 3, generator=g)[: B * nblk].to(torch.int32)
        table = perm.view(B, nblk).cuda()
        pad = torch.zeros((B, H, nblk * page_size, d), dtype=s.k.dtype, device="cuda")
        pools = []
        for c in (s.k, s.v):
            pad[:, :, :L] = c
            pool = torch.zeros((B * nblk + 3, H, page_size, d), dtype=c.dtype, device="cuda")
            pool[table.view(-1).long()] = pad.view(B, H, nblk, page_size, d).permute(0, 2, 1, 3, 4).reshape(
                B * nblk, H, page_size, d)
            pools.append(pool)
        paged.append((s, pools[0], pools[1], table))
    del pad

    def attn(e):
        s, kp, vp, tab = e
        tmv.tree_verify_attention_paged(s.q, kp, vp, tab, s.prefix, s.n_nodes, s.anc, s.depth, s.status, s.out,
                                        scale=s.w.scale, workspace=ws)

    def commit(e):
        s, kp, vp, tab = e
        tmv.kv_commit_path_paged(kp, vp, tab, s.prefix, s.n_nodes, s.accept_len, s.path, s.status, s.new_len,
                                 s.w.M_max)

    reps = reps or (40 if w0.B * w0.L_cap > 100000 else 400)
    out = {}
    torch.cuda.synchronize()            # the pools were filled on torch's stream
    with torch.cuda.stream(stream):
        for name, fn in (("attention", attn), ("commit", commit)):
            for e in paged:
                fn(e)
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=stream):
                for r in range(reps):
                    fn(paged[r % len(paged)])
            gr.replay()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            gr.replay()
            e1.record(stream)
            e1.synchronize()
            out[name] = e0.elapsed_time(e1) * 1e3 / reps
            del gr
    torch.cuda.synchronize()
    if int(torch.stack([s.status for s in sets]).abs().sum()) != 0:
        raise RuntimeError("a paged call reported a non-OK status")
    return {"page_size": page_size, "input_sets": len(paged),
            "tree_verify_attention_paged": {"avg_us": round(out["attention"], 3),
                                            "vs_contiguous": round(out["attention"] / durations["attention"], 3)},
            "kv_commit_path_paged": {"avg_us": round(out["commit"], 3),
                                     "vs_contiguous": round(out["commit"] / durations["commit"], 3)}}


def make_sets(c, ti, tmv, torch):
    """The rotating input sets of workload c (and the workspaces and caches they share)."""
    return make_sets_from(ti.workload(c), lambda i: ti.workload(c, seed=20000 + 100 * c + i), c, tmv, torch)


def make_sets_from(w0, gen, c, tmv, torch, quiet=False, max_gen=64):
    """Rotating input sets: w0 and gen(1), gen(2), ... (same shape, at most max_gen
    generated), then device copies."""
    per_set = set_bytes(w0)
    if c == 5:
        n_sets = 1                                           # p and q: 1.08 GB per set
    else:
        n_sets = min(max_gen, max(2 if per_set > MALL_BYTES else 16, math.ceil(2.5 * MALL_BYTES / per_set)))
    dt = tmv.BF16 if w0.dtype == 1 else tmv.F32
    ws_attn = None
    if w0.mode == "greedy":
        ws_attn = torch.zeros(tmv.tree_verify_attention_workspace(dt, w0.B, w0.M_max, w0.Hq, w0.Hkv, w0.d, w0.L_cap),
                              dtype=torch.uint8, device="cuda")
    mode = tmv.ACCEPT_GREEDY if w0.mode == "greedy" else tmv.ACCEPT_SAMPLE
    ws_acc = torch.zeros(tmv.tree_accept_workspace(mode, w0.B, w0.M_max, w0.V), dtype=torch.uint8, device="cuda")
    caches = None
    if c == 5:
        # [layer][b][head][slot][d] bf16 K and V caches (8.66 GB each), made on the device
        shape = (w0.n_layers, w0.B, w0.Hkv, w0.L_cap, w0.d)
        caches = (torch.zeros(shape, dtype=torch.bfloat16, device="cuda"),
                  torch.ones(shape, dtype=torch.bfloat16, device="cuda"))
    sets = [StepSet(tmv, torch, w0, ws_attn, ws_acc, caches)]
    for i in range(1, n_sets):
        sets.append(StepSet(tmv, torch, gen(i), ws_attn, ws_acc, caches))
    # a stage timed alone must also rotate its own inputs through more than the Infinity
    # Cache holds: add device copies of the generated sets (the same values at new
    # addresses) until the smallest stage's inputs do
    n_gen = n_sets
    if c != 5 and per_set <= MALL_BYTES:
        stage_bytes = min(w0.q.nbytes * 2 + w0.k.nbytes + w0.v.nbytes, w0.logits.nbytes)
        n_total = min(96, max(n_sets, math.ceil(2.5 * MALL_BYTES / stage_bytes)))
        for i in range(n_sets, n_total):
            sets.append(sets[i % n_gen].clone())
    if not quiet:
        print("bench: workload %d, %d input set(s) of %.1f MB (%d generated, %.0f MB total)"
              % (c, len(sets), per_set / 1e6, n_gen, len(sets) * per_set / 1e6), file=sys.stderr, flush=True)
    return w0, sets


def time_steps(sets, steps, warmup, torch):
    """us per verify step: graph replays of a step on every set in turn (as in the main loop)."""
    n_sets = len(sets)
    for i in range(max(min(warmup, 4 * n_sets), n_sets)):
        sets[i % n_sets].step()
    torch.cuda.synchronize()
    st = torch.stack([s.status for s in sets]).cpu()
    if int(st.abs().sum()) != 0:
        raise RuntimeError("a verify step reported a non-OK status")
    stream = torch.cuda.Stream()
    reps, rem = divmod(steps, n_sets)
    with torch.cuda.stream(stream):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for s in sets:
                s.step()
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for _ in range(max(1, reps)):
            g.replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / (max(1, reps) * n_sets) * 1e6
    del g
    return us


def stage_durations(sets, stream, reps, torch):
    """us per launch of each stage: one HIP graph of `reps` back-to-back launches over the
    rotating sets per stage, replayed on its capture stream and timed with HIP events
    recorded on that stream (the kernels' own stream)."""
    durations = {}
    with torch.cuda.stream(stream):
        for name in sets[0].stages():
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for r in range(reps):
                    sets[r % len(sets)].stages()[name]()
            g.replay()                      # warm
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            e1.synchronize()
            durations[name] = e0.elapsed_time(e1) * 1e3 / reps      # us per launch
            del g
    torch.cuda.synchronize()
    return durations


def controller_from_sweep(out, ti, tmv, torch, B=16, D=8, V=128256, N=128):
    """The budget controller fed by the measured cost: C(n) = verify-step us at n nodes,
    interpolated linearly between the swept sizes (mean over the depth limits; flat below
    the smallest), L_AR = the step at the smallest size.  Device best-first construction
    over workload 3's drafter marginals then picks each sequence's budget."""
    Ms = sorted({r["M"] for r in out})
    t = [float(np.mean([r["us_per_step"] for r in out if r["M"] == m])) for m in Ms]
    cost = np.interp(np.arange(1, N + 1), Ms, t)
    q = torch.from_numpy(ti.draft_marginals(np.random.default_rng(3300), B, D, V)).cuda()
    i32 = dict(dtype=torch.int32, device="cuda")
    parents, tokens = torch.zeros((B, N + 1), **i32), torch.zeros((B, N + 1), **i32)
    n_nodes, status = torch.zeros((B,), **i32), torch.zeros((B,), **i32)
    rho = torch.zeros((B, N + 1), dtype=torch.float64, device="cuda")
    tmv.tree_best_first(q, N, parents, tokens, n_nodes, rho, status, cost=torch.from_numpy(cost).cuda(), l_ar=t[0])
    torch.cuda.synchronize()
    if int(status.abs().sum()) != 0:
        raise RuntimeError("tree_best_first reported a non-OK status")
    n = n_nodes.cpu().numpy()
    r = rho.cpu().numpy()
    a_hat = [float(r[b, 1:n[b] + 1].sum()) for b in range(B)]
    return {"cost_us_at": dict(zip(map(str, Ms), [round(x, 2) for x in t])), "l_ar_us": round(t[0], 2),
            "drafter": "B%d positions %d vocab %d budget <= %d, marginals softmax(N(0,3))" % (B, D, V, N),
            "chosen_n": n.tolist(), "mean_n": float(n.mean()),
            "mean_expected_accepted": round(float(np.mean(a_hat)), 3),
            "mean_S_at_chosen_n": round(float(np.mean([a * t[0] / cost[k - 1] for a, k in zip(a_hat, n)])), 3)}


def budget_sweep(args, ti, tmv, torch):
    """Verify-step cost over tree size M and depth limit D_max on workload 2's layer (the
    pages' budget sweet-spot experiment, without a model): the cost table C(N) that the
    best-first budget controller takes."""
    out = []
    for M in (8, 16, 32, 64, 96, 128):
        for D in (2, 4, 8, 16):
            w0, sets = make_sets_from(ti.budget_workload(M, D, 50000 + 97 * M + D),
                                      lambda i: ti.budget_workload(M, D, 50000 + 97 * M + D + 7919 * i), 2, tmv, torch,
                                      quiet=True, max_gen=6)
            us = time_steps(sets, args.steps if args.steps is not None else 600, args.warmup, torch)
            stages = stage_durations(sets, torch.cuda.Stream(), 200, torch)
            depth = int(max(np.max(s.depth.cpu().numpy()) for s in sets[:4]))
            out.append({"M": M, "D_max": D, "depth": depth, "us_per_step": round(us, 2),
                        "stage_us": {k: round(v, 2) for k, v in stages.items()}, "input_sets": len(sets)})
            print("bench: sweep M=%d D_max=%d (deepest %d): %.2f us/step (%s)"
                  % (M, D, depth, us, ", ".join("%s %.2f" % kv for kv in stages.items())), file=sys.stderr, flush=True)
            del sets
            torch.cuda.empty_cache()
    line = {"metric": "verify step us by tree size and depth (budget sweep)", "unit": "us/step", "n_gpus": 1,
            "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "llama3-8b-layer bf16 B1 H32/8 d128 P2048 V128256, random trees (M nodes, depth "
                                   "<= D_max), greedy"},
            "sweep": out, "controller": controller_from_sweep(out, ti, tmv, torch)}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the step line: verify-step cost over tree size and depth (one JSON line)")
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 2000; 200 for workloads 3-5)")
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-lm-head", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain copy kernel of known size (for counter scaling)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/hbm_counters.json for --workload from two rocprofv3 --pmc runs "
                         "(FETCH_SIZE, WRITE_SIZE) of this script with --copy-probe, and exit")
    ap.add_argument("--counter-command", default="", help="the profiled command, recorded with --ingest-counters")
    ap.add_argument("--record", default="", metavar="JSONL",
                    help="also append this run's record (the JSON line, the command, host and device, the input "
                         "seeds and sizes) to this JSON-lines file")
    args = ap.parse_args()
    if args.ingest_counters:
        print(json.dumps(ingest_counters(args.workload, args.ingest_counters[0], args.ingest_counters[1],
                                         args.counter_command), indent=1))
        return
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only; --gpus %d is not supported "
              "(the multi-GPU sharding is described in the design notes, not run)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    c = args.workload
    big = c in (3, 4, 5)
    steps = args.steps if args.steps is not None else (200 if big else 2000)

    import torch
    import tmv_inputs as ti
    import tree_masked_verification_amd as tmv

    torch.cuda.init()
    if args.sweep:
        budget_sweep(args, ti, tmv, torch)
        return
    w0, sets = make_sets(c, ti, tmv, torch)
    n_sets = len(sets)
    torch.cuda.synchronize()

    # eager warm-up (also validates every stage once per set)
    for i in range(max(min(args.warmup, 4 * n_sets), n_sets)):
        sets[i % n_sets].step()
    torch.cuda.synchronize()
    st = torch.stack([s.status for s in sets]).cpu()
    if int(st.abs().sum()) != 0:
        raise RuntimeError("a verify step reported a non-OK status: %s" % st.flatten().tolist())
    mean_accept = float(torch.stack([s.accept_len for s in sets]).float().mean())

    # ---- the step loop as HIP graphs: one graph runs a step on each input set in turn
    # (n_sets steps back to back), a second one the first `rem` of them, so that exactly
    # `steps` steps are timed with one replay per n_sets steps
    stream = torch.cuda.Stream()

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                sets[i].step()
        return g

    full_reps, rem = divmod(steps, n_sets)
    with torch.cuda.stream(stream):
        g_all = capture(n_sets)
        g_rem = capture(rem) if rem else None
    torch.cuda.synchronize()
    # replays go to the stream the graphs were captured on (a replay on another stream
    # measured ~20 % slower per step)
    with torch.cuda.stream(stream):
        for _ in range(max(1, args.warmup // n_sets)):
            g_all.replay()
    torch.cuda.synchronize()

    # ---- timed region 1: throughput
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for _ in range(full_reps):
            g_all.replay()
        if g_rem is not None:
            g_rem.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec_per_step = (t1 - t0) / steps
    nodes = int(w0.n_nodes.sum())
    value = nodes / sec_per_step
    print("bench: %.2f us/step, %.4g node-tokens/s, mean accept length %.2f"
          % (sec_per_step * 1e6, value, mean_accept), file=sys.stderr, flush=True)

    # ---- timed region 2: per-stage launch durations.  For each stage, one HIP graph of
    # back-to-back launches over the rotating sets, replayed on its capture stream and timed
    # with HIP events recorded on that stream (the kernels' own stream).
    durations = stage_durations(sets, stream, 40 if big else 400, torch)

    # ---- algorithmic work per launch (averaged over the input sets)
    works = [workload_work(s.w, s.depth.cpu().numpy(), s.accept_len.cpu().numpy()) for s in sets]
    work = {k: (sum(x[k][0] for x in works) / n_sets, sum(x[k][1] for x in works) / n_sets) for k in works[0]}
    kernels = {}
    for name, us in durations.items():
        nb, fl = work[name]
        gbs = nb / (us * 1e-6) / 1e9
        kernels[name] = {"avg_us": round(us, 3), "bytes": int(nb), "GB/s": round(gbs, 1),
                         "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
        if fl:
            tf = fl / (us * 1e-6) / 1e12
            kernels[name]["flops"] = int(fl)
            kernels[name]["TFLOP/s"] = round(tf, 1)
            kernels[name]["frac_mfma"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)

    def roofline(name):
        """The stage against the roof that bounds it: MFMA when its flops take longer at
        peak than its bytes do, HBM otherwise."""
        nb, fl = work[name]
        us = durations[name]
        if fl and fl / (MFMA_BF16_PEAK_TFLOPS * 1e12) > nb / (HBM_PEAK_GBS * 1e9):
            ach = fl / (us * 1e-6) / 1e12
            return {"bound": "mfma", "kernel": name, "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": traffic_from_profiles(name, c)}
        ach = nb / (us * 1e-6) / 1e9
        return {"bound": "hbm", "kernel": name, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic_from_profiles(name, c)}

    dominant = max((k for k in durations if k != "build"), key=lambda k: durations[k])
    ceiling = stream_read_ceiling(torch, stream)
    for k in kernels.values():
        k["frac_stream_ceiling"] = round(k["GB/s"] / ceiling["GB/s"], 4)
    drafting = time_best_first(torch, tmv, ti, stream) if c == 3 else None
    paged = time_paged(torch, tmv, sets, stream, durations) if c in (2, 3, 4) else None
    if paged:
        print("bench: paged (%d-token pages): attention %.2f us (x%.3f), commit %.2f us"
              % (paged["page_size"], paged["tree_verify_attention_paged"]["avg_us"],
                 paged["tree_verify_attention_paged"]["vs_contiguous"], paged["kv_commit_path_paged"]["avg_us"]),
              file=sys.stderr, flush=True)
    if drafting:
        print("bench: tree_best_first %.2f us per launch (%s)" % (drafting["tree_best_first"]["avg_us"],
                                                                   drafting["tree_best_first"]["shape"]),
              file=sys.stderr, flush=True)

    if args.copy_probe:
        n = 256 << 20
        x = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            torch.mul(x, 1.0, out=y)
        torch.cuda.synchronize()
        print("bench: copy probe %d bytes read, %d bytes written per launch (3 launches)" % (n, n),
              file=sys.stderr, flush=True)

    lm_head = None
    if c in (2, 4) and not args.no_lm_head:
        lm_head = time_lm_head(torch, tmv, sets[0], stream, 4096 if c == 2 else 8192)
        print("bench: LM head + greedy accept: fused %.2f us, library GEMM + accept %.2f us"
              % (lm_head["fused_argmax"]["avg_us"], lm_head["library_gemm_then_accept"]["avg_us"]),
              file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(c, w0, args.cpu_budget)
        print("bench: oracle %.4g node-tokens/s on %d processes (%.4g on one)"
              % (cpu["value"], cpu["cores"], cpu["single_thread"]["value"]), file=sys.stderr, flush=True)

    config = {"workload": w0.name, "batch": w0.B,
              "prefix": int(w0.prefix[0]) if w0.B == 1 else [int(x) for x in w0.prefix],
              "tree_nodes": nodes, "tree_depth": w0.D_max, "heads_q_kv": [w0.Hq, w0.Hkv], "head_dim": w0.d,
              "vocab": w0.V, "accept": w0.mode, "layers": w0.n_layers, "input_sets": n_sets,
              "mean_accept_len": round(mean_accept, 3)}
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "node-tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(sec_per_step * 1e3, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32" if w0.dtype == 0 else "bf16", "data": "synthetic",
        "config": config,
        "roofline": roofline(dominant),
        "attention_roofline": roofline("attention") if "attention" in durations else None,
        "stream_read_ceiling": ceiling,
        "kernels": kernels,
        "drafting": drafting,
        "paged": paged,
        "lm_head": lm_head,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    if args.record:
        append_record(args.record, line, run_record(w0, c, torch.cuda.get_device_name(0)))


def run_record(w0, c, gpu_name):
    """What a JSON-lines run record holds beside the bench line: the command, when, where
    (host CPU, its thread count, the device), the code (the git commit when the tree has one)
    and the workload's seeds and sizes."""
    head = None
    try:
        with open(os.path.join(ROOT, ".git", "HEAD")) as f:
            ref = f.read().strip()
        if ref.startswith("ref: "):
            with open(os.path.join(ROOT, ".git", ref[5:])) as f:
                head = f.read().strip()
        else:
            head = ref
    except OSError:
        pass
    return {"time_utc": time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime()), "argv": sys.argv[1:],
            "git_head": head, "host_cpu": cpu_model(), "host_threads": host_threads(), "gpu": gpu_name,
            "workload": c, "seed": 1000 + c, "extra_set_seeds": "20000 + 100 * workload + i",
            "sizes": {"B": w0.B, "M_max": w0.M_max, "D_max": w0.D_max, "Hq": w0.Hq, "Hkv": w0.Hkv, "d": w0.d,
                      "L_cap": w0.L_cap, "V": w0.V, "layers": w0.n_layers}}


def append_record(path, line, meta):
    """Append one JSON line {..meta, "result": line} to `path`."""
    with open(path, "a") as f:
        f.write(json.dumps(dict(meta, result=line)) + "\n")


if __name__ == "__main__":
    main()
