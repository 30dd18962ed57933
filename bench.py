#!/usr/bin/env python3
"""Decode throughput of one CSA attention layer at 1M context on one MI355X.

One step is the whole CSA decode hot path for a batch of 4 sequences of 1,048,576 raw
tokens (262,144 compressed entries each), 64 query heads, top-1024, window 128:
  compress_kv (newest complete chunk) -> indexer_scores -> topk_select -> sparse_attn_decode,
issued as one csl_csa_decode_step call (the compression rides in the indexer's launch).
Inputs are synthetic (seeded N(0,1) bf16, indexer N(0,1/64)), resident in HBM before the
timed region. The compressed cache and the indexer keys are kept in several independent
copies that consecutive steps rotate through, so every step streams from HBM rather than
from the last-level cache.

The timed region replays a HIP graph that keeps M independent micro-batches in flight
(default 4), as a serving engine overlaps independent batches: each micro-batch is a chain
of consecutive whole steps on its own graph branch, with its own outputs and workspaces and
its own rotated input copies, so the latency-bound tail of one micro-batch's step (top-k
finish, attention, merge on a few compute units) runs beside another's HBM-bound indexer.
Every step is the whole hot path; the graph only saves host-side launches. Steps keep no
scores for rows whose top-k runs on candidate lists (csl.h, scores_on_demand: the ids and
outputs are the same; the in-flight time of steps that write every score is reported beside
it, and --with-scores times those instead). The time per step
of one micro-batch at a time (a chain of 32 dependent steps) and the latency of a step
captured and launched on its own are reported beside it. Prints one JSON line: queries/s,
ms per step, the
indexer kernel's achieved HBM bandwidth against the 8 TB/s peak (HIP events around 100
back-to-back launches), and the fp64 CPU oracle's rate on a bounded sample of the same
workload.

  python bench.py [--steps K] [--warmup W] [--copies R] [--inflight M] [--no-cpu-baseline]
  python bench.py --copy-calibration     # plain device copy of known size (for counters)
  python bench.py --run-workload NAME    # replay another configuration's step (for profiles;
                                         # prints its step time, not a bench line)
  python bench.py --report-configs       # every synthetic configuration: queries/s, GB/s and
                                         # roofline fraction beside the oracle (not a bench line)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "CSA/HCA decode queries/s at 1M ctx; achieved HBM GB/s vs MI355X peak"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published peak
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published peak
WORKLOAD = "csa_decode_1m"
# A timed graph replays GRAPH_ROUNDS rounds of the rotated-copy steps back to back (32 steps
# with 4 copies), as one replay of a model holds all of its layers' steps: the replay's own
# launch cost is then a small share of each step. The one-step-per-replay latency is reported
# beside it (step_us_one_graph_per_step).
GRAPH_ROUNDS = 8
# With micro-batches in flight, one replay holds this many steps in all (a chain of
# IN_FLIGHT_STEPS / M steps per micro-batch): the replay's start and end, where the chains
# fill and drain, are then a small share of each step.
IN_FLIGHT_STEPS = 64
COUNTER_FILE = os.path.join(ROOT, "profiles", "indexer_csa_decode_1m_counters.txt")
INDEXER_SOURCES = ["compressed_sparse_long_amd/csrc/indexer.hip", "compressed_sparse_long_amd/csrc/indexer_common.h",
                   "compressed_sparse_long_amd/csrc/device_common.h",
                   "compressed_sparse_long_amd/csrc/topk_common.h", "compressed_sparse_long_amd/csrc/compress_common.h"]


def in_flight_steps(lane_list, M: int, R: int):
    """The graph of M independent micro-batches in flight over ``lane_list`` (the lanes of one
    step, with R >= M rotated copies each): every lane of every micro-batch is a chain of
    IN_FLIGHT_STEPS / M consecutive steps on its own graph branch. Micro-batch i owns its
    outputs and workspaces (the first is the lane itself) and steps through the copies c with
    c mod M == i, so no two concurrent steps touch the same memory. Returns the graph, the
    steps per replay (a step being one pass of every lane over one micro-batch) and, per lane,
    its M micro-batches."""
    from compressed_sparse_long_amd import lanes
    mbs = [[lane] + [lane.micro_batch() for _ in range(M - 1)] for lane in lane_list]
    own = [[c for c in range(R) if c % M == i] for i in range(M)]
    per_chain = max(1, IN_FLIGHT_STEPS // M)
    g = lanes.in_flight_graph([[lambda mb=mbs[j][i], r=own[i][t % len(own[i])]: mb.step(r) for t in range(per_chain)]
                               for j in range(len(lane_list)) for i in range(M)])
    return g, per_chain * M, mbs


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2048)
    ap.add_argument("--warmup", type=int, default=256)
    ap.add_argument("--copies", type=int, default=4,
                    help="rotated input copies (>= 4 defeats the 256 MB MALL; at least 2 per micro-batch in flight)")
    ap.add_argument("--with-scores", action="store_true",
                    help="the timed steps write every score (default: scores on demand, see csl.h)")
    ap.add_argument("--inflight", type=int, default=4,
                    help="independent micro-batches whose step chains the timed graph runs concurrently")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="wall budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stages", action="store_true", help="skip the per-stage breakdown pass")
    ap.add_argument("--no-configs", action="store_true", help="skip the every-configuration pass")
    ap.add_argument("--config-cpu-seconds", type=float, default=3.0,
                    help="oracle sample per configuration in the every-configuration pass")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for HBM counters)")
    ap.add_argument("--report-configs", action="store_true",
                    help="time every synthetic configuration's step against its roofline and the oracle; one JSON "
                         "line per configuration")
    ap.add_argument("--run-workload", default=None,
                    help="replay --steps steps of another synthetic configuration (for profiling) and print "
                         "its mean step time")
    ap.add_argument("--inflight-workload", action="store_true",
                    help="with --run-workload: keep --inflight micro-batches in flight (default: one at a time)")
    ap.add_argument("--scoreless", action="store_true",
                    help="with --run-workload: CSA steps select with the indexer fused with top-k (no scores)")
    ap.add_argument("--paged", default=None, choices=("random", "interleaved"),
                    help="with --run-workload: page every lane's cache first (blocks in this order)")
    return ap.parse_args()


def sources_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic(launch_bytes_alg):
    """HBM bytes per indexer launch from committed counter runs, or None if the kernel
    source changed since they were taken."""
    if not os.path.exists(COUNTER_FILE):
        return None
    vals = {}
    with open(COUNTER_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != sources_hash(INDEXER_SOURCES):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 5}))


def host_machine():
    """The host the oracle runs on: cores this process may use, the CPU model and the BLAS
    thread count (the oracle's only parallelism)."""
    from threadpoolctl import threadpool_info
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = 1
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            blas = max(blas, int(info.get("num_threads", 1)))
    return {"affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": model, "blas_threads": blas,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(inp, seconds: float):
    """The fp64 oracle on whole decode queries of the same workload, on the host cores."""
    import numpy as np

    from oracle import csa

    li = inp.lanes[0]
    lane = li.lane
    B, m, k, W = lane.B, lane.m, lane.k, lane.W
    kv, z, q = inp.kv, inp.z, inp.q
    keys = [li.kI[lane.ent_off()[b]:lane.ent_off()[b + 1]].double().numpy() for b in range(B)]
    scale = 1.0 / np.sqrt(lane.D)
    t0 = time.perf_counter()
    n = 0
    while n == 0 or time.perf_counter() - t0 < seconds:
        b = n % B
        row0 = lane.kv_off()[b]
        N = lane.lengths[b]
        p = lane.q_pos[b]
        # newest complete chunk, then the query-side steps
        csa.compress(kv[row0 + N - m: row0 + N].double().numpy(), z[row0 + N - m: row0 + N].double().numpy(), m)
        s = csa.indexer(li.qI[b, 0].double().numpy(), li.w[b, 0].double().numpy(), keys[b][:csa.n_visible(p, m, N // m)])
        sel = csa.topk(s, k)
        sel = sel[sel >= 0]
        rows = (row0 + sel[:, None] * m + np.arange(m)[None, :]).reshape(-1)
        import torch
        rt = torch.from_numpy(rows)
        comp = csa.to_bf16_f64(csa.compress(kv.index_select(0, rt).double().numpy(),
                                            z.index_select(0, rt).double().numpy(), m))
        win = csa.window_rows(p, N, W)
        X = np.concatenate([comp, kv[row0 + win.start: row0 + win.stop].double().numpy()])
        csa.attend(q[b, 0].double().numpy(), X, scale)
        n += 1
    el = time.perf_counter() - t0
    mach = host_machine()
    return {"value": n / el, "unit": "queries/s", "cores": mach["blas_threads"], "kind": "oracle",
            "sample": f"{n} whole decode queries of {WORKLOAD} (fp64 numpy: newest-chunk compression, "
                      f"indexer over 262144 keys, top-1024, attention over 1152 rows) in {el:.1f} s",
            "machine": mach}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this path runs on a "
              f"single MI355X and has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.run_workload:
        run_workload(args.run_workload, args.steps, args.warmup, args.paged, args.copies, args.scoreless,
                     args.inflight if args.inflight_workload else 1, args.with_scores)
        return
    if args.report_configs:
        report_configs(args.copies, args.cpu_seconds, inflight=args.inflight, on_demand=not args.with_scores)
        return

    result = measure_headline(args)
    if not args.no_configs:
        # every synthetic configuration's whole step beside its roofline and the oracle (the
        # headline pass's buffers and graphs are released first)
        import gc
        gc.collect()
        torch.cuda.empty_cache()
        result["configs"] = {ln.pop("workload"): ln for ln in
                             report_configs(args.copies, args.config_cpu_seconds, emit=False,
                                            inflight=args.inflight, on_demand=not args.with_scores)}
    print(json.dumps(result), flush=True)


def measure_headline(args) -> dict:
    """The bench line's headline figures on the 1M-context CSA decode workload."""
    import torch
    import synth
    from compressed_sparse_long_amd import lanes

    t_gen = time.perf_counter()
    inp = synth.generate(WORKLOAD)
    (cl,) = lanes.build_lanes(inp)
    # the step keeps no scores for rows selected from candidate lists (csl.h, scores_on_demand):
    # the ids and outputs are those of the step with scores, which is timed beside it
    cl.scores_on_demand = not args.with_scores
    M = max(1, args.inflight)
    cl.rotate(max(args.copies, 2 * M))
    cl.compress_all()
    torch.cuda.synchronize()
    print(f"# inputs ready in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    lane = inp.lanes[0].lane
    B, T, E, HI, CI, H, D, k, W = lane.B, lane.T, lane.entries[0], lane.HI, lane.CI, lane.H, lane.D, lane.k, lane.W

    R = len(cl.ckv_copies)

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    def time_graphs(graphs, reps, per_replay=1):
        """Average device time per unit of `reps` back-to-back replays (round-robin)."""
        for i in range(min(reps, 2 * len(graphs))):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(reps):
            graphs[i % len(graphs)].replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (reps * per_replay) * 1e3  # microseconds

    # the timed loop replays one graph holding M independent micro-batches in flight: M chains
    # of consecutive decode steps on parallel graph branches, S = IN_FLIGHT_STEPS in all per
    # replay (in_flight_steps); every step is the whole hot path, the graph only saves host
    # launches
    multi, S, (mbs,) = in_flight_steps([cl], M, R)
    for i in range((args.warmup + S - 1) // S):
        multi.replay()
    torch.cuda.synchronize()

    reps = (args.steps + S - 1) // S
    K = reps * S
    # the same timed loop with every step writing its scores
    for mb in mbs:
        mb.scores_on_demand = False
    with_scores = in_flight_steps([cl], M, R)[0]
    with_scores.replay()
    torch.cuda.synchronize()
    ws_a, ws_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ws_a.record()
    for i in range(reps):
        with_scores.replay()
    ws_b.record()
    torch.cuda.synchronize()
    with_scores_us = ws_a.elapsed_time(ws_b) / K * 1e3
    del with_scores
    for mb in mbs:
        mb.scores_on_demand = not args.with_scores
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(reps):
        multi.replay()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / K
    queries = B * T * K
    value = queries / (total_ms / 1e3)

    # one micro-batch at a time: a graph of GRAPH_ROUNDS x 4 consecutive steps over 4 rotated
    # copies (each step waits for the one before), and a step launched on its own (one graph
    # per step, replayed back to back)
    serial = capture(lambda: [cl.step(r) for _ in range(GRAPH_ROUNDS) for r in range(4)])
    serial_us = time_graphs([serial], max(2, args.steps // (GRAPH_ROUNDS * 4)), per_replay=GRAPH_ROUNDS * 4)
    del serial
    singles = [capture(lambda r=r: cl.step(r)) for r in range(R)]
    single_us = time_graphs(singles, 200)

    # the dominant kernel (indexer): 100 back-to-back launches over the rotated copies per
    # replay, timed with events on the stream the kernels run on
    n_idx = 25 * R
    idx_graph = capture(lambda: [cl.index(i % R) for i in range(n_idx)])
    idx_us = time_graphs([idx_graph], 4, per_replay=n_idx)
    cl.select()  # consume the candidate lists the timing loop left behind
    torch.cuda.synchronize()
    # the same launches as two independent streams of launches on parallel graph branches
    # (two micro-batches' indexers, each with its own scores and candidate lists): one launch's
    # start and end then overlap the other's stream, which shows the kernel's sustained rate
    # without the per-launch fill and drain
    pair = mbs[:2] if M >= 2 else [cl, cl.micro_batch()]
    two = lanes.in_flight_graph([[lambda mb=pair[i], r=(i + 2 * j) % R: mb.index(r) for j in range(n_idx // 2)]
                                 for i in range(2)])
    idx_two_us = time_graphs([two], 4, per_replay=2 * (n_idx // 2))
    del two
    for mb in pair:
        mb.select()
    torch.cuda.synchronize()

    # algorithmic bytes (per step, and per indexer launch)
    idx_bytes = B * (E * CI * 2 + E * 4 + HI * CI * 2 + HI * 4)                # keys + scores + q + w
    step_bytes = (B * (E * CI * 2 + HI * CI * 2 + HI * 4)                       # indexer inputs
                  + B * (k * D * 2 + W * D * 2 + H * D * 2 + H * D * 4 + H * 4)  # gathers, q, out, lse
                  + B * (2 * lane.m * D * 2 + D * 2))                            # newest-chunk compress
    achieved = idx_bytes / (idx_us * 1e-6) / 1e9
    traffic = read_traffic(idx_bytes)
    # the indexer's contraction: algorithmic flops, and the flops its MFMAs issue (the B
    # operand holds 16 / HI query rows x HI heads, so with one query row per sequence the
    # remaining columns are padding)
    idx_flops = B * T * E * HI * CI * 2
    idx_issued = B * ((T + 16 // HI - 1) // (16 // HI)) * E * 16 * CI * 2

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "batch": B, "context_tokens": lane.lengths[0], "entries": E,
                   "heads": H, "head_dim": D, "m": lane.m, "top_k": k, "window": W, "indexer_heads": HI,
                   "indexer_dim": CI, "rotated_copies": R, "micro_batches_in_flight": M,
                   "scores_on_demand": not args.with_scores},
        "roofline": {"kernel": "indexer_decode_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "launch_us": round(idx_us, 3), "bytes_per_launch": idx_bytes,
                     "two_in_flight": {"us_per_launch": round(idx_two_us, 3),
                                       "achieved": round(idx_bytes / (idx_two_us * 1e-6) / 1e9, 1),
                                       "frac": round(idx_bytes / (idx_two_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}},
        "indexer_mfma": {"flops_per_launch": idx_flops, "issued_flops_per_launch": idx_issued,
                         "achieved": round(idx_flops / (idx_us * 1e-6) / 1e12, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(idx_flops / (idx_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5)},
        "step_us_with_scores": round(with_scores_us, 2),
        "step_us_serial": round(serial_us, 2),
        "step_us_one_graph_per_step": round(single_us, 2),
        "step_hbm": {"bytes": step_bytes, "GB_s": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
                     "frac": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }

    if not args.no_stages:
        # per-stage device time per launch: graphs of n back-to-back launches over the rotated
        # copies (top-k is timed with its indexer, as the difference)
        n = 25 * R
        g_comp = capture(lambda: [cl.compress_new(i % R) for i in range(n)])
        g_idx = capture(lambda: [cl.index(i % R) for i in range(n)])
        g_idx_topk = capture(lambda: [(cl.index(i % R), cl.select()) for i in range(n)])
        g_attn = capture(lambda: [cl.attend(i % R) for i in range(n)])
        t_idx = time_graphs([g_idx], 4, per_replay=n)
        cl.select()
        torch.cuda.synchronize()
        t_it = time_graphs([g_idx_topk], 4, per_replay=n)
        t_comp, t_attn = time_graphs([g_comp], 4, per_replay=n), time_graphs([g_attn], 4, per_replay=n)
        result["stages_us"] = {"compress_new": round(t_comp, 2), "indexer": round(t_idx, 2),
                               "topk": round(t_it - t_idx, 2), "attention": round(t_attn, 2)}
        # algorithmic HBM bytes of the streaming and gather stages over their per-launch times
        comp_bytes = B * (2 * lane.m * D * 2 + D * 2)
        attn_bytes = B * T * (k * 4 + (k + W) * D * 2 + H * D * 2 + H * D * 4 + H * 4)  # ids, rows, q, out, lse
        gbs = lambda nb, us: {"bytes": nb, "GB_s": round(nb / (us * 1e-6) / 1e9, 1),
                              "frac": round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        result["stages_hbm"] = {"compress_new": gbs(comp_bytes, t_comp), "indexer": gbs(idx_bytes, t_idx),
                                "attention": gbs(attn_bytes, t_attn)}
        # bulk compression of one whole 4 x 1M-token context (2 GiB read)
        g_bulk = [capture(lambda r=r: lanes.compress_kv(cl.kv, cl.z, cl.kv_off, cl.ent_off, cl.m, cl.ckv_copies[r],
                                                        max_new_entries=cl.max_entries)) for r in range(R)]
        cus = time_graphs(g_bulk, 8)
        cbytes = sum(lane.lengths) * D * 2 * 2 + sum(lane.entries) * D * 2
        result["compress_bulk"] = {"us": round(cus, 1), "bytes": cbytes, "GB_s": round(cbytes / (cus * 1e-6) / 1e9, 1),
                                   "frac": round(cbytes / (cus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        # overlapped (dual-series) compression of the same contexts: entry i pools its own
        # 4 rows of series a with the 4 rows of series b before it. Series b here is the raw
        # array reversed along the rows (its values do not change the work), and the entries
        # go to a scratch cache.
        kv_b, z_b = cl.kv.flip(0).contiguous(), cl.z.flip(0).contiguous()
        ckv_s = torch.empty_like(cl.ckv)
        g_ov_new = capture(lambda: [lanes.compress_kv_overlap(cl.kv, cl.z, kv_b, z_b, cl.kv_off, cl.ent_off, cl.m,
                                                              ckv_s, first_entry=cl.first_new,
                                                              max_new_entries=cl.n_new) for _ in range(n)])
        t_ov_new = time_graphs([g_ov_new], 4, per_replay=n)
        g_ov_bulk = capture(lambda: lanes.compress_kv_overlap(cl.kv, cl.z, kv_b, z_b, cl.kv_off, cl.ent_off, cl.m,
                                                              ckv_s, max_new_entries=cl.max_entries))
        t_ov_bulk = time_graphs([g_ov_bulk], 8)
        ov_rows = sum(e * lane.m + max(e - 1, 0) * lane.m for e in lane.entries)   # series a + series b rows read
        ov_bytes = ov_rows * D * 2 * 2 + sum(lane.entries) * D * 2
        result["stages_us"]["compress_overlap_new"] = round(t_ov_new, 2)
        result["stages_hbm"]["compress_overlap_new"] = gbs(B * (2 * 2 * lane.m * D * 2 + D * 2), t_ov_new)
        result["compress_overlap_bulk"] = {"us": round(t_ov_bulk, 1), "bytes": ov_bytes,
                                           "GB_s": round(ov_bytes / (t_ov_bulk * 1e-6) / 1e9, 1),
                                           "frac": round(ov_bytes / (t_ov_bulk * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        # the whole decode step with the method's options, timed like the headline loop:
        # overlapped compression (carried by the indexer launch), the attention sink with
        # partial RoPE on the last 64 dims, and both
        import synth.workloads as SW
        sink = SW.normal_f32(inp.workload.seed, SW.S_EXTRA + 7, (H,), std=2.0).cuda()

        def options_step(overlap: bool, extras: bool) -> float:
            cl.kv_b, cl.z_b = (kv_b, z_b) if overlap else (None, None)
            cl.sink, cl.rope_dims = (sink, 64) if extras else (None, 0)
            g = capture(lambda: [cl.step(r) for r in range(R)])
            t = time_graphs([g], max(1, 400 // R), per_replay=R)
            cl.kv_b = cl.z_b = cl.sink = None
            cl.rope_dims = 0
            return round(t, 2)

        # MXFP4 indexer keys (E2M1 codes + an E8M0 scale per 32 dims: 34 bytes per key) for
        # the same draws: the indexer launch and the whole step, over 16 rotated key copies
        # (570 MB, past the last-level cache)
        import synth as SY
        li4 = SY.generate(SW.with_lanes(inp.workload, kI_fp4=True), parts=("kI",)).lanes[0]
        saved = (cl.kI_copies, cl.k_scale_copies, cl.k_format)
        n4 = 16
        cl.kI_copies = [li4.kI.cuda()] + [None] * (n4 - 1)
        cl.k_scale_copies = [li4.k_scale.cuda()] + [None] * (n4 - 1)
        for i in range(1, n4):
            cl.kI_copies[i] = cl.kI_copies[0].clone()
            cl.k_scale_copies[i] = cl.k_scale_copies[0].clone()
        cl.k_format = "mxfp4"
        g4 = capture(lambda: [cl.index(i) for i in range(n4 * 4)])
        t4 = time_graphs([g4], 4, per_replay=n4 * 4)
        cl.select()
        torch.cuda.synchronize()
        g4s = capture(lambda: [cl.step(i) for i in range(n4)])
        t4s = time_graphs([g4s], max(1, 400 // n4), per_replay=n4)
        b4 = B * (E * (CI // 2 + CI // 32) + E * 4 + HI * CI * 2 + HI * 4)
        result["mxfp4_keys"] = {"indexer_us": round(t4, 2), "bytes_per_launch": b4,
                                "GB_s": round(b4 / (t4 * 1e-6) / 1e9, 1),
                                "frac": round(b4 / (t4 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                "step_us": round(t4s, 2), "queries_per_s": round(B / (t4s * 1e-6), 1)}
        cl.kI_copies, cl.k_scale_copies, cl.k_format = saved
        del g4, g4s

        # the same step with the cache paged (entries and keys in a pool of 32-entry blocks,
        # raw rows in 256-row rings), the blocks in a random order (a free list after churn)
        # or handed out round-robin over the sequences (concurrent growth); a separate lane
        # over the same inputs
        def paged_step(order: str) -> float:
            (pl,) = lanes.build_lanes(inp)
            pl.compress_all()
            pl.paginate(ring_rows=256, order=order)
            pl.rotate(R)
            gpg = capture(lambda: [pl.step(r) for r in range(R)])
            t = time_graphs([gpg], max(1, 400 // R), per_replay=R)
            del gpg, pl
            torch.cuda.empty_cache()
            return round(t, 2)

        paged_us = paged_step("random")
        paged_il_us = paged_step("interleaved")

        result["options_step_us"] = {"plain": round(serial_us, 2), "paged": paged_us,
                                     "paged_interleaved": paged_il_us,
                                     "overlap": options_step(True, False),
                                     "sink_rope64": options_step(False, True),
                                     "overlap_sink_rope64": options_step(True, True)}
        del kv_b, z_b, ckv_s

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    return result


def run_workload(name: str, steps: int, warmup: int, paged: str | None = None, copies: int = 4,
                 scoreless: bool = False, inflight: int = 1, with_scores: bool = False) -> None:
    """Replay one configuration's whole step (every lane) as a graph; print its mean time.
    Each graph holds ``copies`` steps over rotated copies of the large inputs (as in the main
    measurement); ``paged``: move every lane's cache into a block pool first, blocks in that
    order; ``inflight`` > 1: that many independent micro-batches in flight, each lane of each a
    chain of steps on its own graph branch over its own rotated copies (as the bench line)."""
    import torch
    import synth
    from compressed_sparse_long_amd import lanes

    inp = synth.generate(name)
    ls = lanes.build_lanes(inp, scoreless=scoreless)
    for lane in ls:  # as the bench line: CSA steps keep no scores for rows on candidate lists
        if hasattr(lane, "scores_on_demand"):
            lane.scores_on_demand = not with_scores
    M = max(1, inflight)
    R = max(1, copies, 2 * M if M > 1 else 1)
    for lane in ls:
        lane.compress_all()
        if paged:
            lane.paginate(ring_rows=256, order=paged)
        lane.rotate(R)
    torch.cuda.synchronize()
    if M > 1:
        if paged:
            raise SystemExit("--paged with --inflight > 1 is not supported (the micro-batches share one pool)")
        g, S, _ = in_flight_steps(ls, M, R)
    else:
        S = GRAPH_ROUNDS * R
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(GRAPH_ROUNDS):
                for r in range(R):
                    for lane in ls:
                        lane.step(r)
    for _ in range(max(1, (warmup + S - 1) // S)):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, (steps + S - 1) // S)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    print(f"workload {name}{' paged ' + paged if paged else ''}{' without scores' if scoreless else ''}"
          f"{f' with {M} micro-batches in flight' if M > 1 else ''}: {a.elapsed_time(b) / (reps * S) * 1e3:.1f} us per "
          f"step over {reps * S} steps ({R} rotated input copies)", flush=True)


def step_model(lane_list, D: int = 128):
    """Algorithmic HBM bytes and MFMA flops of one step of a configuration (all lanes).

    Per sequence: the step's newest compressed entries; for CSA the indexer keys once, per
    query row the indexer query and weights, the selected ids (written and read back), the
    gathered entries and window rows, q, the output and lse; for HCA every visible entry and
    the window. Prefill (T > 1) counts the score matrix's round trip (the top-k reads what the
    indexer writes) and the gathered rows once each (the rows of one sequence are shared by
    its query rows). Flops: indexer H_I*c^I*2 per (row, visible entry); attention H*D*4 per
    (row, key) for the logits and the value product.
    """
    nbytes = flops = queries = 0
    for lane in lane_list:
        m, W, H, T = lane.m, lane.W, lane.H, lane.T
        for b in range(lane.B):
            N, E, p0 = lane.lengths[b], lane.entries[b], lane.q_pos[b]
            first = max(0, min(p0 // m, E - 1)) if E else 0
            nbytes += (E - first) * (2 * m * D * 2 + D * 2)
            nv = [max(0, min((p0 + t) // m, E)) for t in range(T)]
            win = [max(0, min(p0 + t, N - 1) - max(0, min(p0 + t, N - 1) - W + 1) + 1) if N else 0 for t in range(T)]
            queries += T
            nbytes += T * (H * D * 2 + H * D * 4 + H * 4)
            if lane.kind == "csa":
                kb = (lane.CI + 4.0 / lane.scale_group) if lane.kI_fp8 else lane.CI * 2
                sel = [min(lane.k, n) for n in nv]
                nbytes += int(max(nv) * kb) + T * (lane.HI * lane.CI * 2 + lane.HI * 4) + T * lane.k * 4 * 2
                if T > 1:
                    nbytes += 2 * 4 * sum(nv) + (max(nv) + T + W - 1) * D * 2
                else:
                    nbytes += (sel[0] + win[0]) * D * 2
                flops += sum(nv) * lane.HI * lane.CI * 2 + sum(s + w for s, w in zip(sel, win)) * H * D * 4
            else:
                nbytes += ((max(nv) + T + W - 1) if T > 1 else (nv[0] + win[0])) * D * 2
                flops += sum(n + w for n, w in zip(nv, win)) * H * D * 4
    return int(nbytes), int(flops), queries


def oracle_rate(inp, seconds: float, D: int = 128):
    """The fp64 oracle's queries/s on the host: one sampled sequence per lane, its compressed
    cache built before the clock starts (as the GPU's is); per query the newest chunk's
    compression, then indexer, top-k and sparse attention (CSA) or dense attention (HCA)."""
    import numpy as np

    from oracle import csa, pipeline

    scale = 1.0 / np.sqrt(D)
    work = []
    for li in inp.lanes:
        lane = li.lane
        b = max(range(lane.B), key=lambda i: lane.lengths[i])  # the longest sequence of the lane
        r0, N, m = lane.kv_off()[b], lane.lengths[b], lane.m
        kvb = inp.kv[r0:r0 + N].double().numpy()
        zb = inp.z[r0:r0 + N].double().numpy() if inp.z is not None else None
        cache = csa.to_bf16_f64(csa.compress(kvb, zb, m))
        keys = None
        if lane.kind == "csa":
            e0, e1 = lane.ent_off()[b], lane.ent_off()[b + 1]
            if lane.kI_fp8:
                allk = pipeline.index_keys_f64(li.kI, li.k_scale, li.scale_off, lane.ent_off(), lane.scale_group)
                keys = allk[e0:e1]
            else:
                keys = li.kI[e0:e1].double().numpy()
        q = inp.q[li.q_slice][b].double().numpy()
        work.append((li, lane, b, kvb, zb, cache, keys, q))
    t0 = time.perf_counter()
    n = 0
    while n == 0 or time.perf_counter() - t0 < seconds:
        li, lane, b, kvb, zb, cache, keys, q = work[n % len(work)]
        t = (n // len(work)) % lane.T
        m, N = lane.m, lane.lengths[b]
        p = lane.q_pos[b] + t
        e_new = min(p // m, N // m) - 1
        if e_new >= 0:
            csa.compress(kvb[e_new * m:(e_new + 1) * m], None if zb is None else zb[e_new * m:(e_new + 1) * m], m)
        nv = csa.n_visible(p, m, N // m)
        win = csa.window_rows(p, N, lane.W)
        if lane.kind == "csa":
            s = csa.indexer(li.qI[b, t].double().numpy(), li.w[b, t].double().numpy(), keys[:nv])
            sel = csa.topk(s, lane.k)
            X = np.concatenate([cache[sel[sel >= 0]], kvb[win.start:win.stop]])
        else:
            X = np.concatenate([cache[:nv], kvb[win.start:win.stop]])
        csa.attend(q[t], X, scale)
        n += 1
    el = time.perf_counter() - t0
    mach = host_machine()
    return {"value": round(n / el, 2), "unit": "queries/s", "cores": mach["blas_threads"], "kind": "oracle",
            "sample": f"{n} queries ({len(work)} sampled sequence(s), fp64 numpy) in {el:.1f} s", "machine": mach}


def report_configs(copies: int, cpu_seconds: float, emit: bool = True, inflight: int = 4,
                   on_demand: bool = True) -> list:
    """Every synthetic configuration: whole-step time with ``inflight`` independent
    micro-batches in flight (each a chain of steps on its own graph branch, every lane of a
    micro-batch a chain of its own) and one micro-batch at a time (a graph of GRAPH_ROUNDS x
    `copies` consecutive steps), queries/s, algorithmic GB/s and roofline fraction, and the
    oracle's rate beside it. Returns one dict per configuration (and prints each as a JSON
    line when ``emit``)."""
    import torch
    import synth
    from compressed_sparse_long_amd import lanes

    def time_step(inp, scoreless: bool, M: int) -> float:
        ls = lanes.build_lanes(inp, scoreless=scoreless)
        for lane in ls:  # CSA steps keep no scores for rows on candidate lists (csl.h)
            if hasattr(lane, "scores_on_demand"):
                lane.scores_on_demand = on_demand
        R = max(copies, 2 * M) if M > 1 else copies
        for lane in ls:
            lane.rotate(R)
            lane.compress_all()
        torch.cuda.synchronize()
        if M > 1:
            g, steps, _ = in_flight_steps(ls, M, R)
        else:
            steps = GRAPH_ROUNDS * R
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(GRAPH_ROUNDS):
                    for r in range(R):
                        for lane in ls:
                            lane.step(r)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g.replay()
        torch.cuda.synchronize()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        reps = max(3, min(200, int(300.0 / max(a.elapsed_time(b), 1e-3))))  # about 0.3 s of replays
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        del g, ls
        torch.cuda.empty_cache()
        return a.elapsed_time(b) / (reps * steps) * 1e3

    lines = []
    # the prefill configuration last: its long MFMA-heavy replays would otherwise heat the chip
    # right before the next configuration's timing
    for name in sorted(synth.CONFIG_ORDER, key=lambda n: "prefill" in n):
        print(f"# configuration {name}: generating inputs", file=sys.stderr, flush=True)
        inp = synth.generate(name)
        step_us = time_step(inp, False, max(1, inflight))
        serial_us = time_step(inp, False, 1)
        nbytes, flops, queries = step_model([li.lane for li in inp.lanes])
        bound_us = max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e6
        extra = {}
        if any(li.lane.kind == "csa" and li.lane.T >= 16 for li in inp.lanes):
            # query batches: the same step with the indexer fused with top-k (no score matrix)
            nos_us = time_step(inp, True, max(1, inflight))
            extra = {"step_us_without_scores": round(nos_us, 2),
                     "queries_per_s_without_scores": round(queries / (nos_us * 1e-6), 1)}
        line = {"workload": name, "micro_batches_in_flight": max(1, inflight), "scores_on_demand": on_demand,
                "step_us": round(step_us, 2),
                "queries_per_s": round(queries / (step_us * 1e-6), 1), "step_us_serial": round(serial_us, 2),
                "queries_per_s_serial": round(queries / (serial_us * 1e-6), 1),
                "bytes": nbytes, "GB_s": round(nbytes / (step_us * 1e-6) / 1e9, 1),
                "hbm_frac": round(nbytes / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "flops": flops, "TFLOP_s": round(flops / (step_us * 1e-6) / 1e12, 2),
                "bound": "hbm" if nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) else "mfma",
                "roofline_us": round(bound_us, 2), "roofline_frac": round(bound_us / step_us, 4), **extra,
                "cpu_baseline": oracle_rate(inp, cpu_seconds)}
        del inp
        lines.append(line)
        if emit:
            print(json.dumps(line), flush=True)
        else:
            print(f"# configuration {name}: {line['step_us']} us per step", file=sys.stderr, flush=True)
    return lines


if __name__ == "__main__":
    main()
