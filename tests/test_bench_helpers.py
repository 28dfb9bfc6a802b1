"""Known-answer checks of the benchmark's roofline arithmetic against the worked H100
example printed in the roofline section of the hierarchical speculative decoding blog,
and of its algorithmic-work accounting against a direct count."""
import os

import numpy as np

import bench
import tmv_inputs as ti

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def golden():
    vals = {}
    for line in open(os.path.join(GOLD, "h100_roofline.txt")):
        if line.strip() and line[0] != "#":
            k, v, _ = line.split()
            vals[k] = float(v)
    return vals


def test_h100_worked_example():
    g = golden()
    ridge = bench.ridge_point(g["peak_bf16"] * 1e12, g["hbm_bw"] * 1e12)
    assert round(ridge, 1) == g["ridge"]
    assert round(100 * 1.0 / ridge, 2) == g["decode_util"]          # 1 FLOP/B at B=1
    t = bench.read_time_s(g["weights_70b"] * 1e9, g["hbm_bw"] * 1e12)
    assert round(t * 1e3, 1) == g["read_time"]
    assert round(1.0 / t, 1) == g["tokens_per_s"]


def test_attention_work_matches_direct_count():
    w = ti.workload(2, with_rows=False)
    par = w.parents[0]
    depths = []
    for i in range(1, 61):
        d, h = 0, i
        while h:
            h = par[h]
            d += 1
        depths.append(d)
    nbytes, flops = bench.attention_work(depths, 2048, 32, 8, 128)
    # K and V rows of 8 heads over prefix + 60 tree slots, plus Q and O (bf16)
    assert nbytes == 2 * 8 * (2048 + 60) * 128 * 2 + 2 * 60 * 32 * 128 * 2
    # QK^T and PV over visible keys only: each (node, head) sees 2048 + depth keys
    assert flops == sum(4 * 128 * 32 * (2048 + d) for d in depths)
    assert sum(depths) == 242


def test_budget_sweep_inputs():
    """The sweep's trees hold M nodes no deeper than D_max, the cache has room for the
    prefix and every tree slot, and the greedy rows are the layer's vocabulary."""
    for M, D in ((8, 2), (64, 16), (128, 4)):
        w = ti.budget_workload(M, D, 7)
        par = w.parents[0]
        assert par.shape == (M + 1,) and np.all(par[1:] < np.arange(1, M + 1))
        depth = np.zeros(M + 1, np.int64)
        for i in range(1, M + 1):
            depth[i] = depth[par[i]] + 1
        assert depth.max() <= D and w.D_max == D
        assert w.L_cap >= w.prefix[0] + M and w.logits.shape == (1, M + 1, 128256)
        assert (w.B, w.Hq, w.Hkv, w.d, w.mode) == (1, 32, 8, 128, "greedy")


def test_paged_layout_places_every_slot():
    """The page pools hold each sequence's slot t at page table[b][t // page], row t % page,
    for every layer and head; aliased table entries point at the source sequence's pages;
    the table is a permutation of distinct pages apart from the aliases."""
    rng = np.random.default_rng(11)
    k = rng.integers(0, 65536, size=(2, 3, 2, 70, 8)).astype(np.uint16)       # [layer][B][H][L][d]
    v = rng.integers(0, 65536, size=(2, 3, 2, 70, 8)).astype(np.uint16)
    k[:, 2, :, :32] = k[:, 0, :, :32]
    v[:, 2, :, :32] = v[:, 0, :, :32]
    (kp, vp), table = ti.paged_layout(rng, [k, v], 16, spare=2, alias=((0, 2, 2),))
    assert kp.shape == (2, 3 * 5 + 2, 2, 16, 8) and table.shape == (3, 5)
    for b in range(3):
        for t in range(70):
            pg, r = table[b, t // 16], t % 16
            assert np.array_equal(kp[:, pg, :, r], k[:, b, :, t]) and np.array_equal(vp[:, pg, :, r], v[:, b, :, t])
    assert np.array_equal(table[2, :2], table[0, :2])
    rest = np.concatenate([table[0], table[1], table[2, 2:]])
    assert len(set(rest.tolist())) == rest.size and rest.max() < kp.shape[1]


def test_counter_kernels_map_to_stages():
    """Counter ingestion attributes each dispatched kernel to its stage: the paged-cache
    attention (block-table template argument true) and paged commit belong to none."""
    import bench
    ns = "void (anonymous namespace)::"
    assert bench.stage_of(ns + "tree_attn_bf16_kernel<128, 2, false, false, false>(unsigned short const*)") == "attention"
    assert bench.stage_of(ns + "tree_attn_bf16_kernel<128, 8, true, false, true>(unsigned short const*)") == "attention"
    assert bench.stage_of(ns + "tree_attn_bf16_kernel<128, 2, false, true, false>(unsigned short const*)") is None
    assert bench.stage_of(ns + "tree_attn_bf16_kernel<128, 8, true, true, true>(unsigned short const*)") is None
    assert bench.stage_of(ns + "tree_attn_f32_kernel<64>(int, int)") == "attention"
    assert bench.stage_of(ns + "greedy_accept_kernel<0>(int, int)") == "accept"
    assert bench.stage_of(ns + "greedy_scan_kernel<0>(int, int)") == "accept"
    assert bench.stage_of(ns + "greedy_select_kernel(int, int)") == "accept"
    assert bench.stage_of(ns + "sample_walk_kernel(int, int)") == "accept"
    assert bench.stage_of(ns + "lm_select_kernel(int, int)") is None
    assert bench.stage_of(ns + "commit_kernel<false>(int, int)") == "commit"
    assert bench.stage_of(ns + "commit_kernel<true>(int, int)") is None
    assert bench.stage_of(ns + "build_ancestors_kernel(int, int)") == "build"
    assert bench.stage_of("Cijk_Alik_Bljk_BBS_BH_MT128x128x64") is None


def test_run_record_appends_json_lines(tmp_path):
    """--record appends one self-contained JSON line per run: the bench line under "result"
    beside the command, host, device and the workload's seeds and sizes."""
    import json
    w = ti.workload(1)
    meta = bench.run_record(w, 1, "test-device")
    path = tmp_path / "runs.jsonl"
    for v in (1.0, 2.0):
        bench.append_record(str(path), {"metric": "m", "value": v}, meta)
    recs = [json.loads(l) for l in open(path)]
    assert [r["result"]["value"] for r in recs] == [1.0, 2.0]
    r = recs[0]
    assert r["gpu"] == "test-device" and r["workload"] == 1 and r["seed"] == 1001
    assert r["sizes"]["B"] == 1 and r["sizes"]["d"] == 64 and r["sizes"]["V"] == 32
    assert r["host_threads"] >= 1 and "time_utc" in r
