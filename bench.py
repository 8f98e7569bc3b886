#!/usr/bin/env python3
"""Benchmark of index-selected sparse attention on one MI355X.

Default workload: batched decode, 64 sequences with contexts uniform in
[32768, 131072], one query each, indexer width 128, 32 query heads on one KV
head, top-2048, bf16 inputs (seed 0, synthetic). One step = one fused decode
call (score -> masked top-k -> paged gather -> attention) for the whole batch,
inputs already resident in HBM.

Prints ONE JSON line with the whole-job throughput (queries/s), the achieved
algorithmic HBM bandwidth of the whole path, the roofline of the dominant
kernel (the decode scorer: its average launch time from HIP events recorded
around it on its stream), and the CPU oracle timed on a bounded sample.

Other workloads (--workload): decode_4k, prefill_8k, block_pruned_256k,
long_decode_1m (append + decode per step, 256 steps in a stream), and
mxfp4_experts_4096x7168 (the online MXFP4 -> FP8 conversion of 8 selected
experts per step into one reused FP8 workspace).
"""
import argparse
import json
import math
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
METRIC = "queries/sec + achieved HBM GB/s, 128K-ctx decode top-2048 (bf16)"


def host_info():
    model = ""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
    except Exception:
        pass
    return {"nproc": os.cpu_count(), "cpu": model or platform.processor()}


def scorer_bytes(w):
    """Algorithmic bytes of one decode-scorer launch: every compressed key of
    every causal position (2*d_c bytes, read once for all indexer heads), one
    page-table entry per page, and the query's compressed row per indexer
    head."""
    cfg = w.config
    hi = cfg.num_idx_heads
    total = 0
    for L in w.seq_lens.tolist():
        total += L * 2 * cfg.d_c + math.ceil(L / cfg.block_size) * 4 + hi * 2 * cfg.d_c
    return total


def prefill_rows(w):
    """(candidates n, kept k) of every prefill query row: row i of sequence b
    sits at position q_start[b] + i and sees positions 0..that."""
    cfg = w.config
    out = []
    for b, L in enumerate(w.seq_lens.tolist()):
        q0 = int(w.q_start[b])
        for i in range(w.num_q):
            n = min(q0 + i, L - 1) + 1
            out.append((n, min(cfg.topk, n)))
    return out


def prefill_attend_work(w):
    """Algorithmic work of one prefill attention launch: 4*H*D flop per kept
    (row, key) (S = q.k and O += p.v for every head); bytes: q and out rows,
    the index lists, and each distinct K/V page once."""
    cfg = w.config
    rows = prefill_rows(w)
    flops = sum(4 * cfg.num_heads * cfg.head_dim * k for _, k in rows)
    dense = sum(4 * cfg.num_heads * cfg.head_dim * n for n, _ in rows)
    pages = sum(math.ceil(L / cfg.block_size) for L in w.seq_lens.tolist())
    nbytes = (len(rows) * (2 * cfg.num_heads * cfg.head_dim * 2 + cfg.topk * 4)
              + pages * cfg.block_size * cfg.head_dim * 2 * 2)
    return flops, dense, nbytes


def path_bytes_decode(w):
    """Algorithmic bytes of one decode step over the batch (per query: the
    compressed-key scan, page table, K/V rows of the selected positions, q and
    out, the compressed query and the index list)."""
    cfg = w.config
    hi = cfg.num_idx_heads
    total = 0
    for L in w.seq_lens.tolist():
        k = min(cfg.topk, L) if cfg.n_sel_pages == 0 else min(cfg.topk, cfg.n_sel_pages * 64, L)
        # per indexer head: its K/V rows, its compressed query and its index list
        total += (L * 2 * cfg.d_c + math.ceil(L / cfg.block_size) * 4
                  + hi * (k * 2 * cfg.head_dim * 2 + 2 * cfg.d_c + k * 4)
                  + 2 * cfg.num_heads * cfg.head_dim * 2)
    return total


def gather_bytes(w):
    """Algorithmic bytes of one decode gather-attend launch: per selection row,
    the K and V rows of its selected positions (2 * head_dim bf16 each), its
    index list, and the query rows of its query heads. (The split partial
    states that the launch writes for the merge are the design's own traffic,
    not counted here: the counter record shows them.)"""
    cfg = w.config
    hi = cfg.num_idx_heads
    total = 0
    for L in w.seq_lens.tolist():
        k = min(cfg.topk, L) if cfg.n_sel_pages == 0 else min(cfg.topk, cfg.n_sel_pages * 64, L)
        total += hi * (k * (2 * cfg.head_dim * 2 + 4)) + cfg.num_heads * cfg.head_dim * 2
    return total


def step_latencies(torch, step, n, flush):
    """Per-step latency in microseconds: median, 99th percentile (linear
    interpolation), mean and the count, from events recorded around each step
    on the stream the library uses. With `flush`, every step is preceded by a
    read of that buffer (outside the events), so that it starts with no input
    resident in L2 or the MALL (a read, not a write, so that no dirty lines
    are left to be written back during the step)."""
    import numpy as np
    evs = []
    for _ in range(n):
        if flush is not None:
            flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    t = np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in evs])
    return {"p50": float(np.percentile(t, 50)), "p99": float(np.percentile(t, 99)),
            "mean": float(t.mean()), "n": n}


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/traffic.json), if it was taken on the current kernel sources;
    else None."""
    from top_index_selection_amd.rocprof_summary import sources_sha
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))[workload][kernel]
        if rec.get("source_sha") != sources_sha(rec["sources"]):
            return None
        return rec["hbm_bytes_per_launch"]
    except Exception:
        return None


def mfma_from_profiles(kernel, workload):
    """Counter-measured MFMA busy fraction of the kernel (profiles/mfma.json),
    if it was taken on the current kernel sources; else None."""
    from top_index_selection_amd.rocprof_summary import sources_sha
    path = os.path.join(ROOT, "profiles", "mfma.json")
    try:
        rec = json.load(open(path))[workload][kernel]
        if rec.get("source_sha") != sources_sha(rec["sources"]):
            return None
        return rec["mfma_busy_frac"]
    except Exception:
        return None


def decode_scorer_kernel(w, torch):
    """The decode scorer the library launches for this table: the MFMA one for
    several indexer heads; for block pruning over a table that gives blocks of
    at least 16 pages in one round (three per compute unit, at most 128 pages
    each) the one that writes each block's scores at its end; else the
    streaming one."""
    cfg = w.config
    if cfg.num_idx_heads > 1:
        return "score_decode_mh_kernel"
    if cfg.n_sel_pages > 0:
        per_round = 3 * torch.cuda.get_device_properties(0).multi_processor_count
        ppb = -(-(cfg.batch * int(w.page_table.shape[1])) // per_round)
        ppb = min((ppb + 3) // 4 * 4, 128)
        if ppb >= 16:
            return "score_decode_pmax_kernel"
    return "score_decode_kernel"


def oracle_rows_problem(w, rows):
    """CPU arrays for the oracle: one single-query problem per sampled row (b, i).

    Entry r of the returned batch is query row i of sequence b, at position
    q_start[b] + i, with its own copy of b's page-table row; the caches keep
    only the pages of the sampled sequences (renumbered, contents unchanged).
    """
    import torch
    seqs = sorted({b for b, _ in rows})
    pt_all = w.page_table.cpu()
    n_pages = {b: int((pt_all[b] >= 0).sum()) for b in seqs}
    maxp = max(n_pages.values())
    base, pages, total = {}, [], 0
    for b in seqs:
        base[b] = total
        pages.append(pt_all[b, : n_pages[b]].long())
        total += n_pages[b]
    allp = torch.cat(pages).to(w.device)
    R = len(rows)
    pt = torch.full((R, maxp), -1, dtype=torch.int32)
    q_start = torch.empty(R, dtype=torch.int32)
    qs_all = w.q_start.cpu()
    for r, (b, i) in enumerate(rows):
        pt[r, : n_pages[b]] = torch.arange(base[b], base[b] + n_pages[b], dtype=torch.int32)
        q_start[r] = int(qs_all[b]) + i
    bi = torch.tensor([b for b, _ in rows], device=w.device)
    ii = torch.tensor([i for _, i in rows], device=w.device)
    return {"max_pages": maxp, "page_table": pt, "q_start": q_start,
            "q_comp": w.q_comp[bi, ii].unsqueeze(1).cpu(), "q": w.q[bi, ii].unsqueeze(1).cpu(),
            "k_comp_cache": w.k_comp_cache[allp].cpu(), "k_cache": w.k_cache[allp].cpu(),
            "v_cache": w.v_cache[allp].cpu()}


def cpu_baseline(w, rows, threads, min_seconds):
    """The oracle, as it stands, on a sample of the workload's query rows.

    The whole sample (scores, full-sort selection, attention, all in fp64) is
    evaluated repeatedly until at least `min_seconds` of wall time have passed;
    the rate is query rows per second. The oracle parallelises over rows, so it
    uses min(threads, rows) cores.
    """
    from oracle import oracle as O
    cfg = w.config
    pr = oracle_rows_problem(w, rows)
    R = len(rows)
    sh = O.shape(R, 1, cfg.d_c, cfg.num_heads, cfg.head_dim, cfg.block_size, pr["max_pages"],
                 cfg.num_idx_heads)
    O.set_threads(threads)
    passes, t0 = 0, time.perf_counter()
    while True:
        sc = O.index_scores(sh, pr["q_comp"], pr["k_comp_cache"], pr["page_table"], None,
                            pr["q_start"])
        sel = O.topk_select(sh, sc, None, pr["q_start"], cfg.topk, cfg.n_sel_pages)
        O.attend(sh, pr["q"], pr["k_cache"], pr["v_cache"], pr["page_table"], sel["idx"])
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": passes * R / dt, "unit": "queries/s", "cores": min(threads, R),
            "kind": "oracle",
            "sample": f"{R} query rows of {cfg.name} (seed {w.seed}) evaluated {passes} times: fp64 "
                      f"scores, full-sort top-{cfg.topk}"
                      + (f" inside the top {cfg.n_sel_pages} pages" if cfg.n_sel_pages else "")
                      + f", fp64 attention; {dt:.1f} s wall"}


def bench_mxfp4(args, torch, T, PL, W, dev):
    """One step = the MXFP4 -> FP8 conversion of one layer's 8 selected
    experts into the one FP8 workspace every layer reuses; the layers' picks
    are cycled. Returns the JSON record."""
    cfg = W.MXFP4_CONFIGS[args.workload]
    pool = W.make_mxfp4_pool(cfg, args.seed, device=dev)
    ws = PL.Fp8Workspace(cfg.n_sel, cfg.rows, cfg.cols, device=dev)
    E, R, K = cfg.num_experts, cfg.rows, cfg.cols
    state = {"l": 0}

    def step():
        layer = state["l"] % cfg.layers
        T.mxfp4_to_fp8_experts(pool.packed, pool.scales, E, R, K, pool.expert_ids[layer], ws.buf)
        state["l"] += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    T.stage_timing_read()
    T.stage_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    T.stage_timing_enable(False)
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    stages = T.stage_timing_read()
    stage_ms = {k: (v[0] / v[1] if v[1] else 0.0) for k, v in stages.items() if v[1]}
    latency = {"warm": step_latencies(torch, step, args.steps, None)}
    elems = cfg.n_sel * R * K
    # algorithmic bytes per launch: the selected experts' packed elements and
    # scales read once, the FP8 bytes written once, the router's ids
    abytes = cfg.n_sel * R * (K // 2 + K // 32) + elems + 4 * cfg.n_sel
    t_conv = stage_ms.get("convert", 0.0) / 1e3
    achieved = abytes / t_conv / 1e9 if t_conv else 0.0
    res = {
        "metric": "MXFP4 -> FP8 E4M3 expert-weight conversion: elements/sec + achieved HBM GB/s",
        "value": elems / (ms_per_step / 1e3), "unit": "elements/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": cfg.name, "num_experts": E, "rows": R, "cols": K,
                   "experts_per_step": cfg.n_sel, "layers_cycled": cfg.layers,
                   "scale_bytes": [cfg.scale_lo, cfg.scale_hi], "seed": args.seed,
                   "parallelism": "single GPU"},
        "hbm_gbps": abytes / (ms_per_step / 1e3) / 1e9,
        "stage_us": {k: v * 1e3 for k, v in stage_ms.items()},
        "step_latency_us": latency,
        "roofline": {"kernel": "mxfp4_to_fp8_kernel", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic_from_profiles("mxfp4_to_fp8_kernel", cfg.name),
                     "algorithmic_bytes_per_launch": abytes, "avg_launch_us": t_conv * 1e6},
        "wall_s_timed": wall, "host": host_info(),
    }
    if args.no_cpu_baseline:
        res["cpu_baseline"] = None
        return res
    from oracle import oracle as O
    threads = min(16, os.cpu_count() or 1)
    O.set_threads(threads)
    rows_s = 512
    e = int(pool.expert_ids[0, 0])
    pk = pool.packed[e, :rows_s].cpu().numpy()
    sc = pool.scales[e, :rows_s].cpu().numpy()
    passes, t0 = 0, time.perf_counter()
    while True:
        O.mxfp4_to_fp8(pk, sc, rows_s, K)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= args.cpu_seconds:
            break
    res["cpu_baseline"] = {
        "value": passes * rows_s * K / dt, "unit": "elements/s", "cores": threads,
        "kind": "oracle",
        "sample": f"the first {rows_s} rows of expert {e} ({rows_s * K} elements) converted "
                  f"{passes} times, fp64 values and one rounding each; {dt:.1f} s wall",
        "cpu_model": host_info()["cpu"]}
    O.set_threads(1)
    passes, t0 = 0, time.perf_counter()
    while True:
        O.mxfp4_to_fp8(pk[:64], sc[:64], 64, K)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= args.cpu_seconds / 2:
            break
    res["cpu_baseline"]["single_thread"] = {
        "value": passes * 64 * K / dt, "cores": 1,
        "sample": f"the first 64 rows of expert {e} converted {passes} times; {dt:.1f} s wall"}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 100 warm-up steps: the compute-bound prefill step needs tens of
    # milliseconds of GPU work before the clocks settle (after 10 steps it
    # still measures about 3% slow); the memory-bound decode steps do not
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="batched_decode_32k_128k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample", type=int, default=64,
                    help="query rows in the oracle's sample (decode: the first sequences; prefill: "
                         "rows spread evenly over the context; decode stream: the first query)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum wall time of the oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time the step as the replay of a HIP graph captured once (not for "
                         "the stream workload, whose step depends on the host's step index)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed steps, run a plain fp32 copy kernel (torch.neg) over "
                         "this many MiB three times: the known-size reference for the HBM byte "
                         "counters of a rocprofv3 --pmc run")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py: the library runs on exactly one GPU; sharding the path over "
                  "several GPUs (by sequence, or by page range for one long context) is not "
                  "implemented. Run with --gpus 1.",
                  file=sys.stderr)
        sys.exit(2)

    import torch
    from top_index_selection_amd import _lib as T
    from top_index_selection_amd import pipeline as PL
    from top_index_selection_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    T.lib()
    dev = "cuda:0"
    if args.workload in W.MXFP4_CONFIGS:
        print(json.dumps(bench_mxfp4(args, torch, T, PL, W, dev)), flush=True)
        return
    cfg = W.CONFIGS[args.workload]
    t_gen = time.perf_counter()
    w = W.make_workload(cfg, args.seed, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] workload {cfg.name} generated in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)

    sh = PL.shape_of(w)
    extra = {}
    if cfg.prefill:
        ws = torch.empty(max(T.workspace_size(sh, T.TIS_OP_TOPK_SELECT, cfg.topk, cfg.n_sel_pages),
                             1), dtype=torch.uint8, device=dev)
        rows = (cfg.batch, w.num_q)
        idx = torch.empty(rows + (cfg.topk,), dtype=torch.int32, device=dev)
        out = torch.empty(rows + (cfg.num_heads, cfg.head_dim), dtype=torch.bfloat16, device=dev)

        def step():
            T.sparse_topk_select(sh, w.q_comp, w.k_comp_cache, None, w.page_table, w.seq_lens,
                                 w.q_start, cfg.topk, cfg.n_sel_pages, idx, workspace=ws)
            T.paged_gather_attend(sh, T.TIS_PHASE_PREFILL, w.q, w.k_cache, w.v_cache, w.page_table,
                                  idx, cfg.topk, 0.0, out)
        queries_per_step = cfg.batch * w.num_q
    elif cfg.stream_steps > 0:
        ws = torch.empty(T.workspace_size(sh, T.TIS_OP_DECODE_STEP, cfg.topk, cfg.n_sel_pages),
                         dtype=torch.uint8, device=dev)
        outs = PL.decode_step(w, workspace=ws)
        L0 = w.seq_lens.clone()
        state = {"t": 0}

        def step():
            t = state["t"] % cfg.stream_steps
            if t == 0:
                w.seq_lens.copy_(L0)
            PL.append(w, t)
            wt = W.Workload(**{**w.__dict__, "q_comp": w.stream.q_comp[t], "q": w.stream.q[t]})
            PL.decode_step(wt, workspace=ws, outputs=outs)
            state["t"] += 1
        queries_per_step = cfg.batch
        extra["cache"] = "warm: the 268 MB compressed-key cache is re-read every step and may " \
                         "partly reside in the 256 MB MALL; step_latency_us.cold has it evicted"
    else:
        ws = torch.empty(T.workspace_size(sh, T.TIS_OP_DECODE_STEP, cfg.topk, cfg.n_sel_pages),
                         dtype=torch.uint8, device=dev)
        outs = PL.decode_step(w, workspace=ws)

        def step():
            PL.decode_step(w, workspace=ws, outputs=outs)
        queries_per_step = cfg.batch

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    run = step
    if args.graph:
        if cfg.stream_steps > 0:
            raise SystemExit("--graph: the stream workload's step depends on the host's step "
                             "index and is not captured")
        # captured once after a warm-up on a side stream (as torch's capture asks); the
        # replays run the same kernels on the same buffers
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()

    # timed region: exactly K steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = e0.elapsed_time(e1) / args.steps

    # second region, same K steps, HIP events around every kernel stage
    T.stage_timing_read()
    T.stage_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    T.stage_timing_enable(False)
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    stages = T.stage_timing_read()
    stage_ms = {k: (v[0] / v[1] if v[1] else 0.0) for k, v in stages.items() if v[1]}

    # third region, outside the timed one: events around every step, warm, and
    # cold (each step after a 512 MiB read that evicts L2 and the MALL)
    latency = {"warm": step_latencies(torch, run, args.steps, None)}
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    latency["cold"] = step_latencies(torch, run, args.steps, flush)
    del flush

    value = queries_per_step / (ms_per_step / 1e3)
    if cfg.prefill:
        # dominant kernel: the prefill attention (bf16 MFMA); the scorer is reported beside it
        flops, dense, abytes = prefill_attend_work(w)
        t_att = stage_ms.get("attend", 0.0) / 1e3
        achieved = flops / t_att / 1e12 if t_att else 0.0
        roof = {"kernel": "prefill_attend_kernel", "bound": "mfma", "achieved": achieved,
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                "traffic": traffic_from_profiles("prefill_attend_kernel", cfg.name),
                "algorithmic_flops_per_launch": flops,
                "algorithmic_bytes_per_launch": abytes,
                "dense_equivalent_tflops": dense / t_att / 1e12 if t_att else 0.0,
                "mfma_busy_counter": mfma_from_profiles("prefill_attend_kernel", cfg.name),
                "avg_launch_us": t_att * 1e6}
        # the scorer computes the rows whose scores the selection reads: without
        # block pruning, a row that sees at most topk positions keeps them all
        # unread (the step asks for no w)
        pairs = sum(n for n, _ in prefill_rows(w) if n > cfg.topk or cfg.n_sel_pages > 0)
        t_score = stage_ms.get("score", 0.0) / 1e3
        sc_tflops = 2 * cfg.d_c * pairs / t_score / 1e12 if t_score else 0.0
        sc_gbs = 4 * pairs / t_score / 1e9 if t_score else 0.0
        roof["scorer"] = {"kernel": "score_prefill_kernel", "avg_launch_us": t_score * 1e6,
                          "mfma_tflops": sc_tflops, "mfma_frac": sc_tflops / MFMA_BF16_PEAK_TFLOPS,
                          "score_write_gbps": sc_gbs, "score_write_hbm_frac": sc_gbs / HBM_PEAK_GBS,
                          "mfma_busy_counter": mfma_from_profiles("score_prefill_kernel", cfg.name),
                          "traffic": traffic_from_profiles("score_prefill_kernel", cfg.name)}
        path_gbs = None
    else:
        t_score = stage_ms.get("score", 0.0) / 1e3
        achieved = scorer_bytes(w) / t_score / 1e9 if t_score else 0.0
        roof_kernel = decode_scorer_kernel(w, torch)
        roof = {"kernel": roof_kernel, "bound": "hbm", "achieved": achieved,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                "traffic": traffic_from_profiles(roof_kernel, cfg.name),
                "algorithmic_bytes_per_launch": scorer_bytes(w),
                "avg_launch_us": t_score * 1e6}
        if cfg.num_idx_heads > 1:  # the MFMA scorer: its matrix cores' busy fraction too
            roof["mfma_busy_counter"] = mfma_from_profiles(roof_kernel, cfg.name)
        # the paged gather + attention of the selected rows, beside it
        t_att = stage_ms.get("attend", 0.0) / 1e3
        gb = gather_bytes(w)
        g_gbs = gb / t_att / 1e9 if t_att else 0.0
        roof["gather"] = {"kernel": "attend_kernel", "avg_launch_us": t_att * 1e6,
                          "algorithmic_bytes_per_launch": gb, "achieved_gbps": g_gbs,
                          "hbm_frac": g_gbs / HBM_PEAK_GBS,
                          "traffic": traffic_from_profiles("attend_kernel", cfg.name)}
        path_gbs = path_bytes_decode(w) / (ms_per_step / 1e3) / 1e9

    res = {
        "metric": METRIC,
        "value": value,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch,
                   "context": list(cfg.lengths[1:]) if cfg.lengths[0] != "list" else None,
                   "queries_per_step": queries_per_step, "topk": cfg.topk, "d_c": cfg.d_c,
                   "num_heads": cfg.num_heads, "num_idx_heads": cfg.num_idx_heads,
                   "head_dim": cfg.head_dim,
                   "block_size": cfg.block_size, "n_sel_pages": cfg.n_sel_pages,
                   "seed": args.seed, "parallelism": "single GPU",
                   "launch": "hip graph replay" if args.graph else "eager"},
        "hbm_gbps": path_gbs,
        "stage_us": {k: v * 1e3 for k, v in stage_ms.items()},
        "step_latency_us": latency,
        "roofline": roof,
        "wall_s_timed": wall,
        "host": host_info(),
    }
    res.update(extra)
    if not args.no_cpu_baseline:
        if cfg.prefill:
            n = min(args.cpu_sample, w.num_q)
            rows = [(0, int((k + 0.5) * w.num_q / n)) for k in range(n)]
        elif cfg.stream_steps > 0:
            rows = [(0, 0)]
        else:
            rows = [(b, 0) for b in range(min(args.cpu_sample, cfg.batch))]
        threads = min(16, os.cpu_count() or 1)
        res["cpu_baseline"] = cpu_baseline(w, rows, threads, args.cpu_seconds)
        # the same oracle on one thread, over the first rows of the sample
        one = cpu_baseline(w, rows[: max(1, min(len(rows), 4))], 1, args.cpu_seconds / 2)
        res["cpu_baseline"]["single_thread"] = {k: one[k] for k in ("value", "cores", "sample")}
        res["cpu_baseline"]["cpu_model"] = host_info()["cpu"]
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
