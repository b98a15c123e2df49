"""Benchmark of the DSA decode hot path (index + select + attend) on one MI355X.

One step = one dsa_decode_k call covering every row of the workload: index
scores for every cached token, exact top-k per row, FP8 paged gather-attend.
Inputs are seeded synthetic data already resident in HBM. To keep the timed
steps honest about HBM (the 256 MB Infinity Cache would otherwise hold much of
the working set), the keys and the latent pool are replicated and the steps
rotate through the replicas.

Prints one JSON line. `roofline` covers the dominant kernel (the in-step
index-score pass): algorithmic bytes per launch over its median duration,
measured with HIP events recorded on the step's stream around it
(dsa_decode_k_timed). `stage_us` gives the median of every stage the same
way, and `index_attend_roofline` puts the step's algorithmic bytes over the
indexer plus the gather-attend (attention and chunk merge). `cpu_baseline`
times the CPU oracle on a bounded sample of the same workload.
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

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DSA decode steps/sec (index+select+attend) at 1 GPU; % of HBM roofline"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "index_scores_long_traffic.json")
INDEX_SRC = os.path.join(ROOT, "sparse_attention_decode_03_amd", "csrc", "index_scores.hip")


def algorithmic_bytes(inputs: dict) -> dict:
    """Bytes the method must move per step (keys of every visible token,
    selected FP8 rows, query/output, indexer query and weights, block-table
    entries), split by stage."""
    lens = inputs["seq_lens"].astype(np.int64)
    K = inputs["rows_per_seq"]
    D, Hi, H, Dl = inputs["index_dim"], inputs["index_heads"], inputs["num_heads"], inputs["latent_dim"]
    k, ps = inputs["top_k"], inputs["page_size"]
    seq_max = lens.reshape(-1, K).max(axis=1)
    keys = int(seq_max.sum()) * D * 2                      # read once per sequence
    qw = len(lens) * Hi * (D * 2 + 4)
    n = np.minimum(lens, k)
    gather = int(n.sum()) * Dl
    qo = len(lens) * H * Dl * 2 * 2
    bt = int(np.minimum(n, (lens + ps - 1) // ps).sum()) * 4
    return dict(index=keys + qw, attend=gather + qo + bt, total=keys + qw + gather + qo + bt)


def kernel_sha() -> str:
    return hashlib.sha256(open(INDEX_SRC, "rb").read()).hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per index-kernel launch from the committed rocprofv3 counter
    runs: only for the workload they were taken on, and only while the kernel
    source still matches the one measured."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha") != kernel_sha():
        return None
    if rec.get("workload", "").split(":")[0].strip() != workload:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(inputs: dict, budget_s: float = 12.0) -> dict:
    """The oracle on the host cores: rows of the workload evaluated one after
    another (cycling over them) until about `budget_s` of CPU work, scaled to
    steps of the workload's row count."""
    import oracle
    K = inputs["rows_per_seq"]
    R = inputs["seq_lens"].shape[0]
    t0 = time.perf_counter()
    done = 0
    while True:
        oracle.decode(inputs, rows=[done % R])
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    rows_per_s = done / dt
    return {"value": rows_per_s / R, "unit": "steps/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{done} row evaluations cycling over the workload's {R} rows (each: fp64 "
                      f"scores over the row's whole context, full-sort top-k, two-pass softmax "
                      f"attention), {dt:.1f} s, scaled to steps of {R} rows",
            "rows_per_seq": K}


def bench_pooled(args, wlk, inputs: dict, sh) -> int:
    """Pooled selection alone at the workload's rows and lengths: seeded
    N(0,1) pool scores resident in HBM, top_k / kp pools per row; prints one
    JSON line (calls/s and the selected ids per second)."""
    import torch
    from sparse_attention_decode_03_amd import dsa
    kp = args.pooled_kp
    select_k = max(1, wlk.top_k // kp)
    psh = dsa.shape_of(inputs, top_k=select_k)
    R = psh.num_rows
    stride = dsa.pool_score_stride(psh, kp)
    rng = np.random.default_rng(1234)
    scores = torch.from_numpy(rng.standard_normal((R, stride)).astype(np.float32)).cuda()
    lens = torch.from_numpy(inputs["seq_lens"]).cuda()
    width = select_k * kp + kp - 1
    sel = torch.empty((R, width), dtype=torch.int32, device="cuda")
    ws = torch.empty(dsa.pooled_workspace_bytes(psh, kp), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            dsa.topk_select_pooled(psh, kp, scores, lens, sel, ws, stream=stream)
        ea = torch.cuda.Event(enable_timing=True)
        eb = torch.cuda.Event(enable_timing=True)
        ea.record(stream)
        for _ in range(args.steps):
            dsa.topk_select_pooled(psh, kp, scores, lens, sel, ws, stream=stream)
        eb.record(stream)
        torch.cuda.synchronize()
    ms = ea.elapsed_time(eb) / args.steps
    n_sel = int(np.minimum(inputs["seq_lens"] // kp, select_k).sum() * kp
                + (inputs["seq_lens"] % kp).sum())
    print(json.dumps({"metric": "pooled selection calls/sec", "value": 1e3 / ms, "unit": "calls/s",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_call": ms,
                      "higher_is_better": True, "data": "synthetic",
                      "config": {"workload": wlk.name, "rows": R, "pool_tokens": kp,
                                 "pools_per_row": select_k,
                                 "max_pools": int(inputs["max_len"]) // kp},
                      "selected_ids_per_s": n_sel * 1e3 / ms}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long",
                    choices=["tiny", "single", "batched", "kverify", "long", "rowgroup"])
    ap.add_argument("--replicas", type=int, default=4,
                    help="input copies the steps rotate through (1 = warm caches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--index-launches", type=int, default=50)
    ap.add_argument("--pooled-kp", type=int, default=0,
                    help="time the pooled selection (pools of this many tokens, top_k / kp "
                         "pools per row, synthetic pool scores) instead of the decode step")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only run four decode steps and a plain 256 MiB device copy four "
                         "times (for rocprofv3 counter passes), then exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); the path "
              "shards by sequence with no exchange between GPUs, so each GPU would run this "
              "same step on its own sequences", file=sys.stderr)
        return 2

    import torch
    from sparse_attention_decode_03_amd import dsa
    from sparse_attention_decode_03_amd import workloads as wl

    wlk = wl.WORKLOADS[args.workload]
    t_gen = time.perf_counter()
    inputs = wl.make_inputs(wlk)
    t_gen = time.perf_counter() - t_gen
    dsa.load()
    step = dsa.DeviceStep(inputs)
    sh = step.shape
    stream = torch.cuda.Stream()
    nrep = max(1, args.replicas)
    keys = [step.k_normed] + [step.k_normed.clone() for _ in range(nrep - 1)]
    pools = [step.kv_cache] + [step.kv_cache.clone() for _ in range(nrep - 1)]
    torch.cuda.synchronize()

    def run(i: int) -> None:
        dsa.decode_k(sh, step.q_idx, step.w, keys[i % nrep], step.q, pools[i % nrep],
                     step.block_tables, step.seq_lens, step.kv_scale, step.sm_scale,
                     step.scores, step.sel, step.out, step.ws, stream=stream)

    if args.pooled_kp > 0:
        return bench_pooled(args, wlk, inputs, sh)

    if args.traffic_probe:
        # HBM counters read per dispatch: four decode steps (their index pass
        # is the dominant kernel the roofline times), and a plain copy of
        # known size that calibrates the counter's scale
        copy_bytes = 256 << 20
        src = torch.ones(copy_bytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for i in range(4):
                dst.copy_(src)
            for i in range(4):
                run(i)
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": True, "copy_bytes": copy_bytes,
                          "index_algorithmic_bytes": algorithmic_bytes(inputs)["index"],
                          "index_kernel_sha": kernel_sha()}), flush=True)
        return 0

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            run(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            run(i)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0

        # warm figure: one replica, same steps
        wt0 = time.perf_counter()
        for i in range(args.steps):
            dsa.decode_k(sh, step.q_idx, step.w, keys[0], step.q, pools[0], step.block_tables,
                         step.seq_lens, step.kv_scale, step.sm_scale, step.scores, step.sel,
                         step.out, step.ws, stream=stream)
        torch.cuda.synchronize()
        warm = time.perf_counter() - wt0

        # per-step spread: the same rotating steps, each between HIP events
        # on the stream (a separate pass, so the timed loop above carries no
        # event records)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        evs[0].record(stream)
        for i in range(args.steps):
            run(i)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        step_us = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(args.steps)])

        # a plain streaming read on the same device (torch's row sums over
        # 2 GiB of bf16 in 4096-wide rows: reads 2 GiB, writes 1 MiB), the
        # practical HBM read ceiling the index kernel is held to
        big = torch.ones(1 << 30, dtype=torch.bfloat16, device="cuda").view(-1, 4096)
        big.sum(1)
        sa = torch.cuda.Event(enable_timing=True)
        sb = torch.cuda.Event(enable_timing=True)
        sa.record(stream)
        for _ in range(5):
            big.sum(1)
        sb.record(stream)
        torch.cuda.synchronize()
        read_ceiling = 5 * big.numel() * 2 / (sa.elapsed_time(sb) * 1e-3) / 1e9
        del big

        # per-kernel times inside the step: the same steps through
        # dsa_decode_k_timed, whose kernels are launched with start/stop HIP
        # events bound to their own dispatches (index, filter, finish,
        # attention, merge) on the step's stream
        nst = min(args.steps, 100)
        sev = [[torch.cuda.Event(enable_timing=True) for _ in range(10)] for _ in range(nst)]
        for evs6 in sev:
            for e in evs6:
                e.record(stream)  # creates the underlying event
        torch.cuda.synchronize()
        for i in range(nst):
            dsa.decode_k_timed(sh, step.q_idx, step.w, keys[i % nrep], step.q, pools[i % nrep],
                               step.block_tables, step.seq_lens, step.kv_scale, step.sm_scale,
                               step.scores, step.sel, step.out, step.ws, sev[i], stream=stream)
        torch.cuda.synchronize()
        stage_names = ["index", "select_filter", "select_finish", "attend", "merge"]
        stage_us = {nm: float(np.median([sev[i][2 * j].elapsed_time(sev[i][2 * j + 1]) * 1e3
                                         for i in range(nst)]))
                    for j, nm in enumerate(stage_names)}
        stage_mean_us = {nm: float(np.mean([sev[i][2 * j].elapsed_time(sev[i][2 * j + 1]) * 1e3
                                            for i in range(nst)]))
                         for j, nm in enumerate(stage_names)}
        # stages that launch no kernel for this shape (their events are
        # recorded back to back: the span is no kernel's)
        if int(inputs["max_len"]) <= dsa.SELECT_DIRECT_MAX:
            stage_us["select_filter"] = None  # the selection is one kernel (select_finish)
        if min(int(inputs["top_k"]), int(inputs["max_len"])) <= 256:
            stage_us["merge"] = None  # one attention chunk per row: no merge

        # dominant kernel, standalone: the index-score pass launched back to
        # back on rotating replicas between one pair of HIP events (a
        # cross-check of the in-step figure; it writes no group maxima)
        ev_a = torch.cuda.Event(enable_timing=True)
        ev_b = torch.cuda.Event(enable_timing=True)
        dsa.index_scores(sh, step.q_idx, step.w, keys[1 % nrep], step.seq_lens, step.scores,
                         stream=stream)
        ev_a.record(stream)
        for i in range(args.index_launches):
            dsa.index_scores(sh, step.q_idx, step.w, keys[i % nrep], step.seq_lens, step.scores,
                             stream=stream)
        ev_b.record(stream)
        torch.cuda.synchronize()
        idx_ms = ev_a.elapsed_time(ev_b) / args.index_launches

    ab = algorithmic_bytes(inputs)
    ms = elapsed / args.steps * 1e3
    idx_us = stage_us["index"]
    achieved = ab["index"] / (idx_us * 1e-6) / 1e9
    traffic = load_traffic(wlk.name)
    # the indexer plus the gather-attend (attention and chunk merge), against
    # every algorithmic byte of the step (keys, selected rows, q/out,
    # q_idx/w, block-table entries)
    ia_us = stage_us["index"] + stage_us["attend"] + (stage_us["merge"] or 0.0)
    ia_gbs = ab["total"] / (ia_us * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": args.steps / elapsed,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wlk.name,
            "num_seqs": wlk.num_seqs, "rows_per_seq": wlk.rows_per_seq,
            "context": int(inputs["max_len"]), "heads": wlk.num_heads, "latent_dim": wlk.latent_dim,
            "index_heads": wlk.index_heads, "index_dim": wlk.index_dim, "top_k": wlk.top_k,
            "page_size": wlk.page_size, "kv_cache": "fp8-e4m3", "keys": wlk.key_dist,
            "parallelism": "single-gpu", "replicas": nrep,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_index_scores (in-step: scores" + (" and group maxima)" if int(inputs["max_len"]) > dsa.SELECT_DIRECT_MAX else ")"),
            "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": ab["index"],
            "median_launch_us": idx_us,
            "mean_launch_us": stage_mean_us["index"],
            "standalone_mean_launch_us": idx_ms * 1e3,
        },
        "stage_us": stage_us,
        "index_attend_roofline": {
            "stages": "index + attend + merge", "us": ia_us,
            "algorithmic_bytes": ab["total"], "achieved_GBs": ia_gbs,
            "peak_GBs": HBM_PEAK_GBS, "frac": ia_gbs / HBM_PEAK_GBS,
        },
        "step_roofline": {
            "algorithmic_bytes": ab["total"],
            "achieved_GBs": ab["total"] / (ms * 1e-3) / 1e9,
            "frac": ab["total"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        },
        "rows_per_s": args.steps / elapsed * int(inputs["seq_lens"].shape[0]),
        "step_us": {"p10": float(np.percentile(step_us, 10)), "p50": float(np.median(step_us)),
                    "p90": float(np.percentile(step_us, 90))},
        "hbm_read_ceiling": {"GBs": read_ceiling, "kernel": "torch row sums over 2 GiB bf16",
                             "index_frac_of_ceiling": achieved / read_ceiling},
        "warm_value": args.steps / warm,
        "input_gen_s": round(t_gen, 2),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inputs)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
