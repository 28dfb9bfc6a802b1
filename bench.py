#!/usr/bin/env python3
"""Benchmark of the tree-verification step on one MI355X.

A step is one pass of the whole verify path over one batch: tree_build_ancestors,
tree_verify_attention, tree_accept (greedy) and kv_commit_path, on the Llama-3-8B-shaped
single-layer workload (bf16, 32 query / 8 KV heads, head_dim 128, batch 1, prefix 2048,
60-node static tree of depth 6, vocabulary 128256).  Inputs are synthetic and seeded
(tmv_inputs), resident in HBM before timing, and rotated over enough distinct sets that
reads miss the 256 MB Infinity Cache.

Timed regions (both after --warmup untimed steps):
  1. throughput: --steps steps, bracketed by torch.cuda.synchronize(); the steps run as
     replays of one HIP graph that holds a step on every input set in turn (plus one graph
     for the remainder); value = verified node-tokens per second.
  2. kernel durations: for each stage, one HIP graph of back-to-back launches over the
     rotating sets, timed with HIP events recorded on the stream the kernels run on;
     the average launch duration feeds the roofline figures.
The oracle (tests-only CPU implementation) is timed on a bounded sample of the same
workload for the cpu_baseline field.

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


# ---------------------------------------------------------------- workload sets
class StepSet:
    """Device tensors of one input set and its stage outputs."""

    def __init__(self, tmv, torch, w, ws_attn, ws_acc):
        dev = "cuda"
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        self.tmv, self.torch = tmv, torch
        self.w = w
        self.parents = t(w.parents.astype(np.int32))
        self.n_nodes = t(w.n_nodes.astype(np.int32))
        self.prefix = t(w.prefix.astype(np.int32))
        self.tokens = t(w.tokens.astype(np.int32))
        self.q = t(w.q).view(torch.bfloat16)
        self.k = t(w.k).view(torch.bfloat16)
        self.v = t(w.v).view(torch.bfloat16)
        self.logits = t(w.logits)
        B, M, D = w.B, w.M_max, w.D_max
        i32 = dict(dtype=torch.int32, device=dev)
        self.anc = torch.zeros((B, M + 1, D + 1), **i32)
        self.depth = torch.zeros((B, M + 1), **i32)
        self.status = torch.zeros((B,), **i32)
        self.out = torch.zeros_like(self.q)
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
        self.tmv.tree_accept(self.tmv.ACCEPT_GREEDY, self.tokens, self.logits, self.n_nodes, self.anc, self.depth,
                             self.status, self.accept_len, self.path, self.next_token, workspace=self.ws_acc)

    def commit(self):
        self.tmv.kv_commit_path(self.k, self.v, self.prefix, self.n_nodes, self.accept_len, self.path, self.status,
                                self.new_len, self.w.M_max)

    def step(self):
        self.build()
        self.attention()
        self.accept()
        self.commit()


def set_bytes(w):
    return w.q.nbytes + w.k.nbytes + w.v.nbytes + w.logits.nbytes + w.q.nbytes


# ---------------------------------------------------------------- counters from profiles/
def kernel_source_digest():
    h = hashlib.sha256()
    src = os.path.join(ROOT, "tree_masked_verification_amd", "csrc")
    for name in sorted(os.listdir(src)):
        with open(os.path.join(src, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def traffic_from_profiles(kernel_key):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when the
    kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_source_digest():
        return None
    k = rec.get("kernels", {}).get(kernel_key)
    return None if k is None else k.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------- CPU baseline
def cpu_baseline(w, budget_s):
    """The oracle, as it stands, on whole verify steps of the same workload."""
    import oracle
    oracle.build()
    k = w.k.copy()
    v = w.v.copy()
    steps = 0
    t0 = time.perf_counter()
    while True:
        anc, depth, st = oracle.build_ancestors(w.parents, w.n_nodes, w.M_max, w.D_max)
        out, st = oracle.tree_attention(w.q, k, v, w.prefix, w.n_nodes, anc, depth, st, w.scale, w.dtype, w.Hkv)
        A, path, nxt, st = oracle.accept_greedy(w.tokens, w.logits, w.n_nodes, anc, depth, st)
        oracle.commit(k[None], v[None], w.prefix, w.n_nodes, A, path, st, w.M_max)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 1000:
            break
    node_tokens = steps * int(w.n_nodes.sum())
    return {"value": node_tokens / el, "unit": "node-tokens/s", "cores": 1, "kind": "oracle",
            "sample": "%d full verify steps of the same 8B-layer workload (build, attention over all 1920 "
                      "query rows, greedy accept over 61 x 128256 logits, commit), single thread, %.1f s"
                      % (steps, el),
            "ms_per_step": 1e3 * el / steps}


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--kernel-reps", type=int, default=400, help="launches per stage in the duration graphs")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain copy kernel of known size (for counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only; --gpus %d is not supported "
              "(the multi-GPU sharding is described in the design notes, not run)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import tmv_inputs as ti
    import tree_masked_verification_amd as tmv

    torch.cuda.init()
    w0 = ti.workload(2)
    per_set = set_bytes(w0)
    n_sets = max(16, math.ceil(2.5 * MALL_BYTES / per_set))
    print("bench: %d input sets of %.1f MB (%.0f MB total)" % (n_sets, per_set / 1e6, n_sets * per_set / 1e6),
          file=sys.stderr, flush=True)

    ws_attn = torch.zeros(tmv.tree_verify_attention_workspace(tmv.BF16, w0.B, w0.M_max, w0.Hq, w0.Hkv, w0.d, w0.L_cap),
                          dtype=torch.uint8, device="cuda")
    ws_acc = torch.zeros(tmv.tree_accept_workspace(tmv.ACCEPT_GREEDY, w0.B, w0.M_max, w0.V), dtype=torch.uint8,
                         device="cuda")
    sets = [StepSet(tmv, torch, w0, ws_attn, ws_acc)]
    for i in range(1, n_sets):
        sets.append(StepSet(tmv, torch, ti.workload(2, seed=20000 + i), ws_attn, ws_acc))
    torch.cuda.synchronize()

    # eager warm-up (also validates every stage once per set)
    for i in range(max(args.warmup, n_sets)):
        sets[i % n_sets].step()
    torch.cuda.synchronize()
    st = torch.stack([s.status for s in sets]).cpu()
    if int(st.abs().sum()) != 0:
        raise RuntimeError("a verify step reported a non-OK status: %s" % st.flatten().tolist())
    mean_accept = float(torch.stack([s.accept_len for s in sets]).float().mean())

    # ---- the step loop as HIP graphs: one graph runs a step on each input set in turn
    # (n_sets steps back to back), a second one the first `rem` of them, so that exactly
    # --steps steps are timed with one replay per n_sets steps
    stream = torch.cuda.Stream()

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                sets[i].step()
        return g

    full_reps, rem = divmod(args.steps, n_sets)
    with torch.cuda.stream(stream):
        g_all = capture(n_sets)
        g_rem = capture(rem) if rem else None
    torch.cuda.synchronize()
    for _ in range(max(1, args.warmup // n_sets)):
        g_all.replay()
    torch.cuda.synchronize()

    # ---- timed region 1: throughput
    t0 = time.perf_counter()
    for _ in range(full_reps):
        g_all.replay()
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec_per_step = (t1 - t0) / args.steps
    nodes = int(w0.n_nodes.sum())
    value = nodes / sec_per_step
    print("bench: %.2f us/step, %.3g node-tokens/s, mean accept length %.2f"
          % (sec_per_step * 1e6, value, mean_accept), file=sys.stderr, flush=True)

    # ---- timed region 2: per-stage launch durations (HIP events on the launch stream)
    reps = args.kernel_reps
    stages = {"build": lambda s: s.build, "attention": lambda s: s.attention, "accept": lambda s: s.accept,
              "commit": lambda s: s.commit}
    durations = {}
    with torch.cuda.stream(stream):
        for name, fn in stages.items():
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for r in range(reps):
                    fn(sets[r % n_sets])()
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

    # ---- algorithmic work per launch
    depth = sets[0].depth.cpu().numpy()[0, 1:nodes + 1].tolist()
    attn_bytes, attn_flops = attention_work(depth, int(w0.prefix[0]), w0.Hq, w0.Hkv, w0.d)
    attn_bytes += (w0.M_max + 1) * (w0.D_max + 2) * 4                  # ancestor table + depths
    acc_bytes = (nodes + 1) * w0.V * 4 + (w0.M_max + 1) * 4
    build_bytes = (w0.M_max + 1) * 4 * (w0.D_max + 3)
    commit_bytes = int(round(2 * 2 * w0.Hkv * w0.d * 2 * mean_accept))   # rows read + written, K and V
    work = {"build": (build_bytes, 0), "attention": (attn_bytes, attn_flops), "accept": (acc_bytes, 0),
            "commit": (commit_bytes, 0)}
    kernels = {}
    for name, (nb, fl) in work.items():
        us = durations[name]
        gbs = nb / (us * 1e-6) / 1e9
        kernels[name] = {"avg_us": round(us, 3), "bytes": nb, "GB/s": round(gbs, 1),
                         "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
        if fl:
            tf = fl / (us * 1e-6) / 1e12
            kernels[name]["flops"] = fl
            kernels[name]["TFLOP/s"] = round(tf, 1)
            kernels[name]["frac_mfma"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)
    dominant = max(("attention", "accept"), key=lambda k: durations[k])
    nb = work[dominant][0]
    achieved = nb / (durations[dominant] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profiles(dominant)}
    attention_roofline = {"bound": "hbm", "kernel": "attention",
                          "achieved": kernels["attention"]["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": kernels["attention"]["frac_hbm"], "traffic": traffic_from_profiles("attention")}

    if args.copy_probe:
        n = 256 << 20
        x = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            torch.mul(x, 1.0, out=y)
        torch.cuda.synchronize()
        print("bench: copy probe %d bytes read, %d bytes written per launch (3 launches)" % (n, n),
              file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w0, args.cpu_budget)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "node-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(sec_per_step * 1e3, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w0.name, "batch": w0.B, "prefix": int(w0.prefix[0]), "tree_nodes": nodes,
                   "tree_depth": w0.D_max, "heads_q_kv": [w0.Hq, w0.Hkv], "head_dim": w0.d, "vocab": w0.V,
                   "accept": "greedy", "input_sets": n_sets, "mean_accept_len": round(mean_accept, 3)},
        "roofline": roofline,
        "attention_roofline": attention_roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
