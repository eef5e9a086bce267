"""Benchmark: HSA forward over an HKV active set, ms per chunk-layer, on one MI355X.

One step is one hsa_forward call (retrieval + gather, pooling + selection,
low-rank branch, block-sparse attention with the fused gate) over the
Wan-1.3B-shaped 480p chunk-layer (H=12, d=128, Lq=4680, pages of
12480 tokens, 32-page pool, Kp=4, r=256, Binter=128, Bintra=64), with every
input already resident in HBM. Inputs are seeded synthetic values with the
workload's shapes and laws (clustered keys, tau_h ~ U[0.35, 1)).

Prints one JSON line. Extra fields: per-stage times from the separate entry
points, the roofline of the dominant kernel (block-sparse attention, bf16
MFMA) and of the gather (HBM), and the float64 CPU oracle timed on a bounded
sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan1.3b-480p")
    ap.add_argument("--tau-min", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stages", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle sparse-attention rows in the CPU baseline sample")
    ap.add_argument("--policy", default="two_stage",
                    choices=["two_stage", "page_only", "prompt_only", "recent", "random", "mismatched"],
                    help="retrieval policy of the forward (the method's is two_stage)")
    ap.add_argument("--seed", type=int, default=0, help="seed of the random retrieval policy")
    ap.add_argument("--sweep", default=None, choices=["psize-kp", "policies", "tiers"],
                    help="instead of the benchmark line, one JSON line per configuration: "
                         "(Psize, Kp) at a fixed history length, or every retrieval policy on the "
                         "60 s workload")
    return ap.parse_args()


def main() -> int:
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; "
                          f"--gpus {a.gpus} is not supported (the path shards by heads, "
                          "see the design notes, but only the one-GPU share is built)"}))
        return 2
    import torch

    import synth
    from block_sparse_rank_amd import hsakv as hs

    if a.sweep:
        return sweep(a)
    over = {} if a.tau_min is None else {"tau_min": a.tau_min}
    s = synth.shape(a.workload, **over)
    run = time_forward(s, a.steps, a.warmup, a.policy, a.seed)
    d, T, ch, pool_k, pool_v = run["d"], run["T"], run["ch"], run["pool_k"], run["pool_v"]
    page_kmean, tau, stream = run["page_kmean"], run["tau"], run["stream"]
    n_sel, sel_count, sel_idx = run["n_sel"], run["sel_count"], run["sel_idx"]
    ms_med, ms_p10, ms_p90, warm_ms, wall_ms = (run[k] for k in ("ms_med", "ms_p10", "ms_p90", "warm_ms",
                                                                  "wall_ms"))

    # selection actually taken: algorithmic work of the sparse attention
    # (4 d flops per selected (query, key) pair: QK^T and PV, 2 flops per MAC)
    density, sparse_flops, n = density_of(s, d, n_sel, sel_count, sel_idx)
    eb = 2 if s.dtype == "bf16" else 4
    gather_bytes = 2.0 * 2 * n * s.Tp * s.H * s.d * eb       # K and V, read + write
    floor_us, floor_parts = forward_floor(s, n, sparse_flops)

    result = {
        "metric": "HSA fwd ms per chunk-layer (1.3B-shape 480p, Kp=4) + % HBM/MFMA roofline",
        "value": round(ms_med, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_med, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": s.dtype,
        "data": "synthetic",
        "config": {"workload": s.name, "H": s.H, "d": s.d, "Lq": s.Lq, "Tp": s.Tp, "P": s.P,
                   "Kp": s.Kp, "r": s.r, "Binter": s.Binter, "Bintra": s.Bintra, "Bq": s.Bq,
                   "tau_min": s.tau_min, "selected_block_density": round(density, 4),
                   "parallelism": "single-gpu"},
        "timing": {"headline": "median of per-step HIP-event times, 1 GiB written before each step "
                               "(cold MALL and L2)",
                   "median_ms": round(ms_med, 4), "p10_ms": round(ms_p10, 4),
                   "p90_ms": round(ms_p90, 4), "warm_mean_ms": round(warm_ms, 4),
                   "wall_ms_per_step_incl_flush": round(wall_ms, 4),
                   "graph_replay_median_ms": round(run["graph_ms_med"], 4),
                   "graph_replay_warm_mean_ms": round(run["graph_warm_ms"], 4)},
        "forward_roofline": {"floor_us": round(floor_us, 1),
                             "frac": round(floor_us * 1e-3 / ms_med, 4),
                             "floor_parts_us": {k: round(v, 1) for k, v in floor_parts.items()},
                             "basis": "sum over stages of max(algorithmic bytes / 8 TB/s, "
                                      "algorithmic flops / dense peak) at the measured selection"},
    }

    if not a.no_stages:
        result.update(stage_times(a, s, d, T, page_kmean, tau, hs, torch, stream, sparse_flops,
                                  gather_bytes))
        result["page_commit"] = commit_time(a, s, T, hs, torch, stream)

    if a.policy != "two_stage":
        result["config"]["retrieval_policy"] = a.policy
    if not a.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(s, ch, pool_k, pool_v, a.cpu_budget)
        result["cpu_baseline"]["ratio_to_gpu"] = round(result["cpu_baseline"]["value"] / ms_med, 1)
    hs.fork_destroy(run["fork"])
    print(json.dumps(result), flush=True)
    return 0


def time_forward(s, steps, warmup, policy="two_stage", seed=0):
    """Upload the synthetic chunk-layer `s`, then time hsa_forward on it: each
    step alone by HIP events on the launch stream, 1 GiB written before it
    (outside the events) so that no input or intermediate is left in the
    256 MB MALL or the L2 caches; then the same steps back to back (warm)."""
    import torch

    import synth
    from block_sparse_rank_amd import hsakv as hs

    d = hs.make_dims(H=s.H, d=s.d, Lq=s.Lq, tokens_per_frame=s.tokens_per_frame, Psize=s.Psize,
                     P=s.P, Kp=s.Kp, Binter=s.Binter, Bintra=s.Bintra, Bq=s.Bq, r=s.r,
                     dtype=s.dtype)
    assert hs.validate(d) == hs.OK
    t0 = time.time()
    ch = synth.draw_chunk(s)
    pool_k, pool_v = synth.draw_pool(s)
    print(f"# inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")

    def up(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    tdt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    T = {k: up(ch[k]) for k in ("q", "k_intra", "v_intra", "E", "F", "w_g", "b_g", "page_prompt")}
    T["pool_k"], T["pool_v"] = up(pool_k), up(pool_v)
    page_kmean = torch.empty((s.P, s.H, s.d), dtype=torch.float32, device=dev)
    hs.hkv_page_summary(d, T["pool_k"], page_kmean)          # commit-time metadata, untimed

    out = torch.empty((s.Lq, s.H, s.d), dtype=tdt, device=dev)
    sel_count = torch.empty((s.H, d.NQB), dtype=torch.int32, device=dev)
    sel_idx = torch.empty((s.H, d.NQB, d.NB_max), dtype=torch.int32, device=dev)
    n_sel = torch.empty((1,), dtype=torch.int32, device=dev)
    ws_fwd = torch.empty(hs.workspace_bytes(d, hs.ENTRY_FORWARD), dtype=torch.uint8, device=dev)
    ins = {k: T[k] for k in ("q", "k_intra", "v_intra", "pool_k", "pool_v", "E", "F", "w_g",
                             "b_g", "page_prompt")}
    ins["page_kmean"] = page_kmean
    outs = {"out": out, "sel_count": sel_count, "sel_idx": sel_idx, "n_sel": n_sel}
    tau = ch["tau"]
    stream = torch.cuda.current_stream()
    fork = hs.fork_create()          # the caller-owned second stream of the forward

    def step():
        hs.hsa_forward(d, tau, s.cur_prompt, ins, outs, ws_fwd, stream=stream, fork=fork,
                       policy=policy, seed=seed)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(steps):
        flush.fill_(k & 0xff)
        evs[k][0].record(stream)
        step()
        evs[k][1].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_start) * 1e3 / steps
    cold = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    ms_med, ms_p10, ms_p90 = (float(np.percentile(cold, q)) for q in (50, 10, 90))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(steps):
        step()
    ev[1].record(stream)
    torch.cuda.synchronize()
    warm_ms = ev[0].elapsed_time(ev[1]) / steps
    # the same step captured once in a HIP graph and replayed: same protocol
    # (1 GiB written before each replay, outside the events), then back to back
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.graph(graph, stream=cap):
        hs.hsa_forward(d, tau, s.cur_prompt, ins, outs, ws_fwd, stream=cap, fork=fork, policy=policy, seed=seed)
    torch.cuda.synchronize()
    gevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for k in range(steps):
        flush.fill_(k & 0xff)
        gevs[k][0].record(stream)
        graph.replay()
        gevs[k][1].record(stream)
    torch.cuda.synchronize()
    gcold = np.array([e0.elapsed_time(e1) for e0, e1 in gevs])
    ev[0].record(stream)
    for _ in range(steps):
        graph.replay()
    ev[1].record(stream)
    torch.cuda.synchronize()
    graph_warm_ms = ev[0].elapsed_time(ev[1]) / steps
    del graph
    del flush
    return {"d": d, "T": T, "ch": ch, "pool_k": pool_k, "pool_v": pool_v, "page_kmean": page_kmean,
            "tau": tau, "stream": stream, "fork": fork, "n_sel": n_sel, "sel_count": sel_count,
            "sel_idx": sel_idx, "ms_med": ms_med, "ms_p10": ms_p10, "ms_p90": ms_p90,
            "warm_ms": warm_ms, "wall_ms": wall_ms, "graph_ms_med": float(np.median(gcold)),
            "graph_warm_ms": graph_warm_ms}


def density_of(s, d, n_sel, sel_count, sel_idx):
    """Selected-block density and algorithmic sparse flops of the selection taken."""
    n = int(n_sel.cpu()[0])
    cnt = sel_count.cpu().numpy()
    ids = sel_idx.cpu().numpy()
    Lh = n * s.Tp
    NBh = -(-Lh // s.Binter)
    blen = np.array([min(s.Binter, Lh - b * s.Binter) for b in range(NBh)] +
                    [min(s.Bintra, s.Lq - j * s.Bintra) for j in range(d.NBc)], dtype=np.int64)
    qlen = np.array([min(s.Bq, s.Lq - i * s.Bq) for i in range(d.NQB)], dtype=np.int64)
    pairs, nb = 0, 0
    for h in range(s.H):
        for i in range(d.NQB):
            c = int(cnt[h, i])
            nb += c
            pairs += int(qlen[i]) * int(blen[ids[h, i, :c]].sum())
    return nb / (s.H * d.NQB * (NBh + d.NBc)), 4.0 * s.d * pairs, n


def sweep(a):
    """One JSON line per configuration (not the benchmark contract line).

    psize-kp: the Wan-1.3B 480p chunk-layer with Psize in {4, 8, 16} frames
    and Kp in {2, 4, 8}, the pool holding the same 256 frames of history
    (P = 256 / Psize pages); the open (Psize, Kp) question of the pages,
    timing and density only.
    policies: the 60 s workload (6 prompt segments of 16 pages, the current
    prompt's pages non-recent) under each retrieval policy.
    """
    from block_sparse_rank_amd import hsakv as hs

    import synth
    if a.sweep == "tiers":
        return sweep_tiers(a)
    if a.sweep == "psize-kp":
        base = synth.shape("wan1.3b-480p")
        confs = [(dict(Psize=ps, P=256 // ps, Kp=kp), "two_stage") for ps in (4, 8, 16) for kp in (2, 4, 8)
                 if ps * kp <= 64]
    else:
        base = synth.shape("wan1.3b-480p-60s")
        confs = [({}, pol) for pol in ("two_stage", "page_only", "prompt_only", "recent", "random",
                                       "mismatched")]
    for over, pol in confs:
        s = base.with_(**over)
        run = time_forward(s, a.steps, a.warmup, pol, a.seed)
        dens, flops, n = density_of(s, run["d"], run["n_sel"], run["sel_count"], run["sel_idx"])
        line = {"sweep": a.sweep, "workload": s.name, "Psize": s.Psize, "Kp": s.Kp, "P": s.P,
                "Tp": s.Tp, "policy": pol, "n_sel": n, "selected_block_density": round(dens, 4),
                "median_ms": round(run["ms_med"], 4), "p10_ms": round(run["ms_p10"], 4),
                "p90_ms": round(run["ms_p90"], 4), "warm_mean_ms": round(run["warm_ms"], 4),
                "sparse_tflops": round(flops / (run["ms_med"] * 1e-3) / 1e12, 1)}
        hs.fork_destroy(run["fork"])
        print(json.dumps(line), flush=True)
    return 0


def commit_time(a, s, T, hs, torch, stream):
    """hkv_page_commit of this chunk's K and V into a two-page pool, placed so
    that it completes page 0 (the copy plus one page-mean pass); HIP events
    on the launch stream, mean over the repetitions."""
    dev = T["q"].device
    d2 = hs.make_dims(H=s.H, d=s.d, Lq=s.Lq, tokens_per_frame=s.tokens_per_frame, Psize=s.Psize, P=2,
                      Kp=min(s.Kp, 2), Binter=s.Binter, Bintra=s.Bintra, Bq=s.Bq, r=s.r, dtype=s.dtype)
    pk = torch.zeros((2, s.Tp, s.H, s.d), dtype=T["q"].dtype, device=dev)
    pv = torch.zeros_like(pk)
    km = torch.zeros((2, s.H, s.d), dtype=torch.float32, device=dev)
    pp = torch.zeros(2, dtype=torch.int32, device=dev)
    fill = max(0, s.Tp - s.Lq // 4)
    n = min(s.Lq, 2 * s.Tp - fill)
    ws = torch.empty(hs.workspace_bytes(d2, hs.ENTRY_COMMIT), dtype=torch.uint8, device=dev)

    def once():
        hs.hkv_page_commit(d2, pk, pv, km, pp, T["k_intra"], T["v_intra"], n, fill, 0, ws=ws, stream=stream)

    once()
    torch.cuda.synchronize()
    reps = max(3, a.steps)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        once()
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    eb = 2 if s.dtype == "bf16" else 4
    completes = (fill + n) // s.Tp - fill // s.Tp
    nbytes = 2.0 * 2 * n * s.H * s.d * eb + completes * s.Tp * s.H * s.d * eb
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "tokens": n, "pages_completed": completes, "bound": "hbm",
            "algorithmic_bytes": nbytes, "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4)}


def sweep_tiers(a):
    """Tiered pages: every page in the pinned host store, 8 HBM slots, on the
    Wan-1.3B 480p chunk-layer at two horizons (32 and 96 pages of history).
    Per horizon: the forward with the whole pool in HBM (reference), with
    the retrieved pages read from the host store over the bus, and with them
    in HBM slots after the planner promoted them; the promotion itself; and
    the forward while another page is promoted on a second stream (the
    prefetch of a page the next chunk-layer retrieves). HBM held by the pool
    stays at the slots whatever the horizon."""
    import torch

    import synth
    from block_sparse_rank_amd import hsakv as hs
    for name in ("wan1.3b-480p", "wan1.3b-480p-60s"):
        s = synth.shape(name)
        run = time_forward(s, 2, 1)       # uploads the chunk-layer; its all-HBM times are the reference
        d, T, stream = run["d"], run["T"], run["stream"]
        del T["pool_k"], T["pool_v"]      # the pool now lives in host memory only
        torch.cuda.empty_cache()
        slots = 8
        hk = hs.HostStore(run["pool_k"].shape, run["pool_k"].dtype)
        hv = hs.HostStore(run["pool_v"].shape, run["pool_v"].dtype)
        hk.array[:] = run["pool_k"]
        hv.array[:] = run["pool_v"]
        pk = torch.zeros((slots, s.Tp, s.H, s.d), dtype=T["q"].dtype, device=T["q"].device)
        pv = torch.zeros_like(pk)
        table = torch.full((s.P,), -1, dtype=torch.int32, device=pk.device)
        tiers = hs.Tiers(table.data_ptr(), hk.device, hv.device)
        pl = hs.TierPlacement(s.P, slots)
        outs = {"out": torch.empty((s.Lq, s.H, s.d), dtype=T["q"].dtype, device=pk.device),
                "n_sel": run["n_sel"], "page_idx": torch.empty(s.Kp, dtype=torch.int32, device=pk.device)}
        ins = {k: T[k] for k in ("q", "k_intra", "v_intra", "E", "F", "w_g", "b_g", "page_prompt")}
        ins.update(pool_k=pk, pool_v=pv, page_kmean=run["page_kmean"])
        ws = torch.empty(hs.workspace_bytes(d, hs.ENTRY_FORWARD), dtype=torch.uint8, device=pk.device)

        def timed(fn, reps):
            fn()
            torch.cuda.synchronize()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            for _ in range(reps):
                fn()
            e[1].record(stream)
            torch.cuda.synchronize()
            return e[0].elapsed_time(e[1]) / reps

        fwd = lambda: hs.hsa_forward(d, run["tau"], s.cur_prompt, ins, outs, ws, stream=stream,  # noqa: E731
                                     fork=run["fork"], tiers=tiers)
        miss_ms = timed(fwd, max(2, a.steps // 4))
        torch.cuda.synchronize()
        n = int(outs["n_sel"].cpu()[0])
        pages = outs["page_idx"].cpu().tolist()[:n]
        pp, ps, up, uv = hs.hkv_tier_plan(pl, 1, pages)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        hs.hkv_tier_apply(d, tiers, pk, pv, slots, pp, ps, up, uv, stream=stream)
        e[1].record(stream)
        torch.cuda.synchronize()
        apply_ms = e[0].elapsed_time(e[1])
        hit_ms = timed(fwd, a.steps)

        # one more page promoted on a second stream while the forward runs:
        # the planner evicts the least recently used slot, never a page of
        # the forward (those were used last)
        side = torch.cuda.Stream()
        others = [p for p in range(s.P) if p not in pages]
        reps = max(3, a.steps // 2)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
        torch.cuda.synchronize()
        for k in range(reps):
            extra = others[k % len(others)]
            pp2, ps2, up2, uv2 = hs.hkv_tier_plan(pl, 2 + k, pages + [extra])
            assert len(pp2) == 1 and pp2[0] == extra
            ev[k][0].record(side)
            hs.hkv_tier_apply(d, tiers, pk, pv, slots, pp2, ps2, up2, uv2, stream=side)
            ev[k][1].record(side)
            ev[k][2].record(stream)
            fwd()
            ev[k][3].record(stream)
            torch.cuda.synchronize()
        fwd_beside_ms = sum(ev[k][2].elapsed_time(ev[k][3]) for k in range(reps)) / reps
        promote1_ms = sum(ev[k][0].elapsed_time(ev[k][1]) for k in range(reps)) / reps
        page_bytes = 2 * s.Tp * s.H * s.d * 2
        line = {"sweep": "tiers", "workload": s.name, "P": s.P, "hbm_slots": slots, "retrieved": pages,
                "forward_all_hbm_pool_ms": round(run["warm_ms"], 4),
                "forward_pages_in_hbm_slots_ms": round(hit_ms, 4),
                "forward_pages_from_host_store_ms": round(miss_ms, 4),
                "promote_pages_ms": round(apply_ms, 4), "promoted": len(pp),
                "promote_GBps": round(len(pp) * page_bytes / (apply_ms * 1e-3) / 1e9, 1),
                "forward_beside_one_page_promotion_ms": round(fwd_beside_ms, 4),
                "one_page_promotion_beside_forward_ms": round(promote1_ms, 4),
                "hbm_pool_bytes": slots * page_bytes, "history_bytes": s.P * page_bytes}
        hs.fork_destroy(run["fork"])
        torch.cuda.synchronize()
        hk.free()
        hv.free()
        del run, pk, pv, ins, outs, ws
        torch.cuda.empty_cache()
        print(json.dumps(line), flush=True)
    return 0


def forward_floor(s, n_sel, sparse_flops):
    """Lower bound of one chunk-layer on this chip, in microseconds: per stage
    the larger of its algorithmic HBM bytes at 8 TB/s and its algorithmic
    flops at the dense peak of the storage type, summed over the stages."""
    eb = 2 if s.dtype == "bf16" else 4
    peak = (PEAK_BF16_TFLOPS if s.dtype == "bf16" else PEAK_F32_TFLOPS) * 1e12
    bw = PEAK_HBM_GBS * 1e9
    Lh = n_sel * s.Tp
    tok = s.H * s.d * eb                      # bytes of one token row of one tensor
    L_act = Lh + s.Lq
    parts = {
        "retrieve": s.Lq * tok / bw,                                    # read q
        "gather": 4.0 * Lh * tok / bw,                                  # K and V, read + write
        "select": (L_act + s.Lq) * tok / bw,                            # read K_act and q
        "sparse_attn": sparse_flops / peak,
        "linear": max((2 * s.r * L_act * eb + 2 * L_act * tok + s.Lq * tok + s.Lq * s.H * s.d * 4) / bw,
                      (4.0 * s.r * L_act * s.H * s.d + 4.0 * s.Lq * s.r * s.H * s.d) / peak),
        "fuse": (2 * s.Lq * s.H * s.d * 4 + 2 * s.Lq * tok) / bw,     # o_s, o_l in; q in, out
    }
    parts = {k: v * 1e6 for k, v in parts.items()}
    return sum(parts.values()), parts


def stage_times(a, s, d, T, page_kmean, tau, hs, torch, stream, sparse_flops, gather_bytes):
    """Each stage through its own entry point, events on the launch stream."""
    dev = page_kmean.device
    tdt = T["q"].dtype
    page_idx = torch.empty((s.Kp,), dtype=torch.int32, device=dev)
    n_sel = torch.empty((1,), dtype=torch.int32, device=dev)
    k_hist = torch.empty((s.Kp * s.Tp, s.H, s.d), dtype=tdt, device=dev)
    v_hist = torch.empty_like(k_hist)
    cnt = torch.empty((s.H, d.NQB), dtype=torch.int32, device=dev)
    idx = torch.empty((s.H, d.NQB, d.NB_max), dtype=torch.int32, device=dev)
    o_s = torch.empty((s.Lq, s.H, s.d), dtype=torch.float32, device=dev)
    o_l = torch.empty_like(o_s)
    out = torch.empty((s.Lq, s.H, s.d), dtype=tdt, device=dev)
    W = {e: torch.empty(max(256, hs.workspace_bytes(d, e)), dtype=torch.uint8, device=dev)
         for e in (hs.ENTRY_GATHER, hs.ENTRY_SELECT, hs.ENTRY_SPARSE, hs.ENTRY_LINEAR)}
    stages = {
        "gather": lambda: hs.hkv_gather(d, T["pool_k"], T["pool_v"], page_kmean, T["page_prompt"],
                                        s.cur_prompt, T["q"], page_idx, n_sel, k_hist, v_hist,
                                        W[hs.ENTRY_GATHER], stream=stream),
        "select": lambda: hs.hsa_select(d, T["q"], k_hist, T["k_intra"], n_sel, tau, cnt, idx,
                                        None, None, W[hs.ENTRY_SELECT], stream=stream),
        "linear": lambda: hs.hsa_linear_branch(d, T["q"], k_hist, v_hist, T["k_intra"],
                                               T["v_intra"], n_sel, T["E"], T["F"], o_l, None,
                                               None, W[hs.ENTRY_LINEAR], stream=stream),
        # float32 has no separate plan: its whole entry point counts as the compute
        "sparse_plan": (lambda: hs.hsa_sparse_plan(d, n_sel, cnt, idx, W[hs.ENTRY_SPARSE], stream=stream))
        if s.dtype == "bf16" else (lambda: None),
        "sparse_compute": (lambda: hs.hsa_sparse_compute(d, T["q"], k_hist, v_hist, T["k_intra"],
                                                         T["v_intra"], n_sel, o_s, W[hs.ENTRY_SPARSE],
                                                         stream=stream))
        if s.dtype == "bf16" else
        (lambda: hs.hsa_sparse_attn(d, T["q"], k_hist, v_hist, T["k_intra"], T["v_intra"], n_sel, cnt, idx,
                                    o_s, W[hs.ENTRY_SPARSE], stream=stream)),
        "fuse": lambda: hs.hsa_fuse(d, T["q"], T["w_g"], T["b_g"], o_s, o_l, out, None,
                                    stream=stream),
    }
    for fn in stages.values():       # warm and produce each stage's inputs once
        fn()
    torch.cuda.synchronize()
    # each rep runs the stages in forward order, with an event between stages,
    # so every stage meets the caches as it does inside hsa_forward
    names = list(stages)
    reps = max(3, a.steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(reps)]
    for r in range(reps):
        evs[r][0].record(stream)
        for j, name in enumerate(names):
            stages[name]()
            evs[r][j + 1].record(stream)
    torch.cuda.synchronize()
    ms = {name: sum(evs[r][j].elapsed_time(evs[r][j + 1]) for r in range(reps)) / reps
          for j, name in enumerate(names)}
    peak = PEAK_BF16_TFLOPS if s.dtype == "bf16" else PEAK_F32_TFLOPS
    ms["sparse_attn"] = ms["sparse_plan"] + ms["sparse_compute"]     # the whole entry point
    att_tflops = sparse_flops / (ms["sparse_compute"] * 1e-3) / 1e12
    entry_tflops = sparse_flops / (ms["sparse_attn"] * 1e-3) / 1e12
    gather_gbs = gather_bytes / (ms["gather"] * 1e-3) / 1e9
    traffic = recorded_traffic("hsa_sparse_attn", s.name)
    bwd = backward_time(a, s, d, T, hs, torch, stream, k_hist, v_hist, n_sel, o_s)
    return {
        "backward": bwd,
        "stages_ms": {k: round(v, 4) for k, v in ms.items()},
        "roofline": {"kernel": "k_sparse_attn32 + k_sparse_combine (hsa_sparse_compute: the attention over "
                               "the plan and the merge of split groups)",
                     "bound": "mfma", "achieved": round(att_tflops, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(att_tflops / peak, 4),
                     "traffic": traffic, "algorithmic_flops": sparse_flops,
                     "entry_point_frac": round(entry_tflops / peak, 4),
                     "entry_point": "hsa_sparse_attn = hsa_sparse_plan + hsa_sparse_compute"},
        "gather_roofline": {"kernel": "k_gather (+ retrieval)", "bound": "hbm",
                            "achieved": round(gather_gbs, 1), "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": round(gather_gbs / PEAK_HBM_GBS, 4),
                            "traffic": recorded_traffic("hkv_gather", s.name),
                            "algorithmic_bytes": gather_bytes},
    }


def backward_time(a, s, d, T, hs, torch, stream, k_hist, v_hist, n_sel, o_s):
    """hsa_backward_params on this chunk-layer's saved forward values and a
    seeded upstream gradient; HIP events on the launch stream, mean over the
    repetitions. Its floor is the larger of its algorithmic bytes over the
    HBM peak and its algorithmic flops over the bf16 MFMA peak."""
    import synth
    if s.dtype != "bf16":
        return None
    dev = T["q"].device
    up = synth.draw_upstream(s)
    d_out = torch.from_numpy(up["d_out"].view(np.int16)).view(torch.bfloat16).to(dev)
    o_l = torch.empty((s.Lq, s.H, s.d), dtype=torch.float32, device=dev)
    k_low = torch.empty((s.r, s.H, s.d), dtype=torch.float32, device=dev)
    v_low = torch.empty_like(k_low)
    hs.hsa_linear_branch(d, T["q"], k_hist, v_hist, T["k_intra"], T["v_intra"], n_sel, T["E"], T["F"], o_l,
                         k_low, v_low, torch.empty(hs.workspace_bytes(d, hs.ENTRY_LINEAR), dtype=torch.uint8,
                                                   device=dev), stream=stream)
    d_wg = torch.empty((s.H, s.d), dtype=torch.float32, device=dev)
    d_bg = torch.empty((s.H,), dtype=torch.float32, device=dev)
    d_E = torch.empty((s.r, s.L), dtype=torch.float32, device=dev)
    d_F = torch.empty_like(d_E)
    ws = torch.empty(hs.workspace_bytes(d, hs.ENTRY_BACKWARD), dtype=torch.uint8, device=dev)
    fork = hs.fork_create()

    def once():
        hs.hsa_backward_params(d, T["q"], k_hist, v_hist, T["k_intra"], T["v_intra"], n_sel, T["w_g"], T["b_g"],
                               k_low, v_low, o_s, o_l, d_out, d_wg, d_bg, d_E, d_F, ws, stream=stream, fork=fork)

    once()
    torch.cuda.synchronize()
    reps = max(3, a.steps)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        once()
    ev[1].record(stream)
    torch.cuda.synchronize()
    hs.fork_destroy(fork)
    ms = ev[0].elapsed_time(ev[1]) / reps
    ns = int(n_sel.item())
    L_act = ns * s.Tp + s.Lq
    HD = s.H * s.d
    # dE = dK' K^T and dF = dV' V^T over the active keys, plus the low-rank
    # backward (four r x d x Lq products per head) and the gate terms
    flops = 2 * 2.0 * s.r * HD * L_act + 4 * 2.0 * s.r * s.d * s.Lq * s.H + 8.0 * s.Lq * HD
    nbytes = (2.0 * L_act * HD * 2            # K and V rows of the active keys
              + 2.0 * s.r * s.L * 4           # dE and dF
              + s.Lq * HD * (2 + 2 + 4 + 4)   # q, d_out, o_sparse, o_linear
              + 2.0 * s.r * HD * 4)           # K', V'
    floor_us = max(nbytes / (PEAK_HBM_GBS * 1e9), flops / (PEAK_BF16_TFLOPS * 1e12)) * 1e6
    return {"ms": round(ms, 4), "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
            "floor_us": round(floor_us, 1), "frac": round(floor_us * 1e-3 / ms, 4),
            "basis": "max(algorithmic bytes / 8 TB/s, algorithmic flops / 2.5 PFLOP/s bf16)"}


# Sources whose kernels a recorded HBM-traffic figure covers; a figure is only
# reported while the hash of these files matches the one recorded with it.
TRAFFIC_SOURCES = {
    "hsa_sparse_attn": ["block_sparse_rank_amd/csrc/k_sparse32.hip", "block_sparse_rank_amd/csrc/common.h"],
    "hkv_gather": ["block_sparse_rank_amd/csrc/k_hkv.hip", "block_sparse_rank_amd/csrc/common.h"],
}


def source_hash(entry: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES[entry]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(entry: str, workload: str):
    """HBM bytes per call of `entry` from the committed rocprofv3 counter record
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration), or None
    when there is no record for this workload or the kernels changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)[entry][workload]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_hash") != source_hash(entry):
        return None
    return rec.get("bytes_per_call")


def cpu_baseline(s, ch, pool_k, pool_v, budget_s):
    """The float64 oracle, as it stands, on a bounded sample of the same chunk-layer.

    Timed: retrieval, gather, pooling, selection, the low-rank branch and the
    gate for every head, then the sparse attention on random rows until
    `budget_s` seconds have passed; the sparse part is scaled to all rows by
    their selected (query, key) pairs. The page summary is commit-time
    metadata and is excluded.
    """
    import oracle
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max([i.get("num_threads", 1) for i in info] + [1])
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu_model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    km = np.stack([oracle.page_summary(oracle.as_f64(pool_k[p], s.dtype)[None])[0]
                   for p in range(s.P)])
    t0 = time.perf_counter()
    ref = oracle.forward(dtype=s.dtype, q=ch["q"], k_intra=ch["k_intra"], v_intra=ch["v_intra"],
                         pool_k=pool_k, pool_v=pool_v, page_prompt=ch["page_prompt"],
                         cur_prompt=s.cur_prompt, E=ch["E"], F=ch["F"], w_g=ch["w_g"],
                         b_g=ch["b_g"], tau=ch["tau"], Kp=s.Kp, Binter=s.Binter,
                         Bintra=s.Bintra, Bq=s.Bq, page_kmean=km, rows=[])
    t_dense = time.perf_counter() - t0
    blocks, qblocks = ref["blocks"], ref["qblocks"]
    NQB = len(qblocks)
    K = np.concatenate([oracle.as_f64(ref["k_hist"], s.dtype), oracle.as_f64(ch["k_intra"], s.dtype)])
    V = np.concatenate([oracle.as_f64(ref["v_hist"], s.dtype), oracle.as_f64(ch["v_intra"], s.dtype)])
    q = oracle.as_f64(ch["q"], s.dtype)

    def pairs_of(h, i):
        return (qblocks[i][1] - qblocks[i][0]) * sum(blocks[b][1] - blocks[b][0]
                                                     for b in ref["sel"][h][i])

    order = np.random.default_rng(0).permutation(s.H * NQB)
    sample_pairs, n_rows = 0, 0
    t1 = time.perf_counter()
    for r in order:
        h, i = divmod(int(r), NQB)
        oracle.sparse_attention_row(q, K, V, h, qblocks[i], ref["sel"][h][i], blocks)
        sample_pairs += pairs_of(h, i)
        n_rows += 1
        if time.perf_counter() - t1 >= budget_s:
            break
    t_sparse = time.perf_counter() - t1
    total_pairs = sum(pairs_of(h, i) for h in range(s.H) for i in range(NQB))
    est_s = t_dense + t_sparse * total_pairs / max(1, sample_pairs)
    return {"value": round(est_s * 1e3, 1), "unit": "ms", "cores": int(cores), "kind": "oracle",
            "sample": (f"oracle O2-O13 in full for all {s.H} heads ({t_dense:.1f} s) + sparse "
                       f"attention on {n_rows} of {s.H * NQB} random rows ({t_sparse:.1f} s), "
                       f"scaled by selected (query, key) pairs {sample_pairs} -> {total_pairs}"),
            "measured_s": round(t_dense + t_sparse, 1), "cpu_model": cpu_model, "blas": blas,
            "ratio_to_gpu": None}


if __name__ == "__main__":
    sys.exit(main())
