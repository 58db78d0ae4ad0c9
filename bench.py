"""Benchmark of the DSA-style sparse-attention hot path on one MI355X.

A step is one pass of the whole path over one batch: lightning indexer ->
top-k -> sparse MLA, through the fused sparse_attn_decode C entry point, on
seeded synthetic inputs already resident in HBM.

Default workload: batched decode, B = 32 sequences x 1 query, L = 32768 cached
tokens, indexer 64 heads x 128 (bf16), top-k 2048, MLA 128 heads, latent 512 +
RoPE 64 (bf16), 16 planted needle rows per sequence.  Metric: decode
queries/s; the whole step is also reported as a fraction of the HBM roofline
(algorithmic bytes per query / step time / 8 TB/s).

The JSON line carries, besides the contract fields:
  roofline      the dominant kernel (the indexer) timed live with HIP events on
                its own stream: algorithmic bytes per launch / mean duration,
                against MI355X's 8 TB/s; `traffic` is the HBM bytes per
                launch from rocprofv3 FETCH_SIZE/WRITE_SIZE counters, scaled
                by a plain copy of known size (profiles/), or null when the
                indexer source changed since they were taken;
  cpu_baseline  the CPU oracle on a bounded sample of the same workload.

Usage: python bench.py [--steps K] [--warmup W]
       [--workload decode_32k|decode_128k_fp8|prefill_16k|block_sparse_64k|csa_decode|
                   prefill_crossover]
       [--staged] [--fused-select] [--shared-choice] [--no-cpu-baseline] [--kernel-only]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes_per_query(wl):
    """Bytes one decode query must move at least once: indexer keys (+ fp8
    scales), indexer query and weights, the gathered latent rows, the MLA
    query and the fp32 output."""
    kb = 1 if wl.k_idx.dtype.itemsize == 1 else wl.k_idx.element_size()
    ki = wl.L * wl.dI * kb + (wl.L * 4 if wl.k_scale is not None else 0)
    qi = wl.HI * wl.dI * wl.q_idx.element_size() + wl.HI * 4
    gather = wl.topk * (wl.dc + wl.dR) * wl.kv.element_size()
    qm = wl.H * (wl.dc + wl.dR) * wl.q_lat.element_size()
    out = wl.H * wl.dc * 4
    return ki, qi, gather, qm, out


def make_workload(name):
    from top_indexer_sparse_amd import workloads
    if name == "decode_32k":
        return workloads.decode_32k()
    if name == "decode_128k_fp8":
        return workloads.decode_128k_fp8()
    raise SystemExit(f"unknown decode workload {name}")


def time_events(fn, iters, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters  # ms


def cpu_baseline(wl, budget_s=20.0):
    """The oracle (unchanged) on the same workload: whole sequences of the
    batch, `threads` at a time, until the batch is done or about `budget_s`
    seconds have passed.  Each chunk is timed end to end: decode of the stored
    bytes, indexer, top-k, sparse MLA."""
    import oracle
    threads = oracle.num_threads()
    step = max(1, threads)
    done, spent = 0, 0.0
    while done < wl.B and spent < budget_s:
        sub = wl.slice_batch(done, min(wl.B, done + step))
        t0 = time.perf_counter()
        s = oracle.indexer(sub.q_idx, sub.w, sub.k_idx, k_scale=sub.k_scale, kv_len=sub.kv_len)
        idx, _ = oracle.topk(s, sub.topk, kv_len=sub.kv_len)
        oracle.sparse_mla(sub.q_lat, sub.q_rope, sub.kv, idx, sub.sm_scale, dc=sub.dc)
        spent += time.perf_counter() - t0
        done += sub.B
    return {"value": round(done / spent, 3), "unit": "queries/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} of {wl.B} sequences of {wl.name} (full L={wl.L}, k={wl.topk}, "
                      f"H={wl.H}), fp64 C oracle, OpenMP over (query, head) on {threads} "
                      f"threads of {os.cpu_count()} ({cpu_model()}), {spent:.2f} s"}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_decode_32k_traffic.md")
# the decode score kernel's source: its translation unit and the headers it uses
INDEXER_SRC = [os.path.join(ROOT, "top_indexer_sparse_amd", "csrc", f)
               for f in ("indexer.hip", "index_core.hpp", "split_select.hpp", "select_core.hpp",
                         "launch.hpp", "common.hpp")]


def indexer_source_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in INDEXER_SRC:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per indexer launch from the committed rocprofv3 counter
    summary: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by the
    factor a plain device copy of known size gives.  None when the summary is
    missing or was taken on other indexer source."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("- ") and ":" in line:
            key, _, v = line[2:].partition(":")
            vals[key.strip()] = v.strip().strip("`")
    if vals.get("indexer_source_sha256") != indexer_source_sha256():
        return None
    try:
        fetch = float(vals["fetch_kib_per_launch"]) * 1024 * float(vals["fetch_scale"])
        write = float(vals["write_kib_per_launch"]) * 1024 * float(vals["write_scale"])
    except (KeyError, ValueError):
        return None
    return round(fetch + write)


def timed_after(step, fn, n, stream):
    """Mean duration of fn, each launch timed alone with HIP events on
    `stream` right after an untimed step (so caches hold what they hold
    inside the step loop)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        step()
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return sum(e0.elapsed_time(e1) for e0, e1 in ev) / n


def per_step_stats(step, n, stream, dev, flush_gib=1):
    """Each step timed alone with HIP events, after an untimed pass that evicts
    the 256 MB Infinity Cache: median, p10 and p90 of the step time in
    microseconds (cold caches, unlike the back-to-back steps of the headline
    number).  The pass reads flush_gib GiB of scratch (a sum), so that the
    cache is left holding clean lines: a write pass would leave dirty ones
    whose write-back the timed step would pay for."""
    import torch
    scratch = torch.ones(flush_gib << 28, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        torch.sum(scratch, dim=0, out=sink)
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
    del scratch

    def pct(p):
        return us[min(n - 1, int(round(p * (n - 1))))]
    return {"median_us": round(pct(0.5), 2), "p10_us": round(pct(0.1), 2),
            "p90_us": round(pct(0.9), 2), "iters": n,
            "cache_flush": f"{flush_gib} GiB scratch read before each step, not timed"}


def copy_peak_gbs(dev, mib=1024, iters=5):
    """Measured device-copy bandwidth: (bytes read + bytes written) / time of a
    plain mib-MiB device-to-device copy, the practical HBM ceiling."""
    import torch
    src = torch.empty(mib << 18, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / iters
    del src, dst
    return 2 * (mib << 20) / sec / 1e9


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_probe(mib, dev):
    import torch
    src = torch.empty(mib << 18, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy probe: 3 x {mib} MiB device copies")


def run_decode(args, api, dev):
    import torch
    log(f"generating {args.workload}")
    wl = make_workload(args.workload)
    t = wl.to(dev)
    B, L, k = wl.B, wl.L, wl.topk
    c_kv, k_rope = t.kv[..., :wl.dc], t.kv[..., wl.dc:]
    out = torch.empty((B, 1, wl.H, wl.dc), dtype=torch.float32, device=dev)
    lse = torch.empty((B, 1, wl.H), dtype=torch.float32, device=dev)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
    nws = api.sparse_attn_workspace_bytes(api.SA_OP_DECODE, B, 1, L, k, wl.H, wl.dc)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        api.sparse_attn_decode(t.q_idx, t.w, t.k_idx, t.k_scale, t.kv_len, k, t.q_lat,
                               t.q_rope, c_kv, k_rope, wl.sm_scale, out=out, lse=lse,
                               idx_out=idx, ws=ws, stream=stream)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    ms = time_events(step, args.steps, stream)
    wall = time.perf_counter() - t0
    torch.cuda.synchronize()
    qps = B / (ms * 1e-3)
    ki, qi, gather, qm, o = algorithmic_bytes_per_query(wl)
    per_q = ki + qi + gather + qm + o
    step_frac = per_q * qps / (HBM_PEAK_GBS * 1e9)
    log(f"{ms * 1e3:.1f} us/step, {qps:,.0f} queries/s, whole step {100 * step_frac:.1f}% "
        f"of HBM peak ({wall:.2f} s wall)")
    if args.copy_probe:
        copy_probe(args.copy_probe, dev)
    if args.kernel_only:
        return None

    # the indexer (the metric's HBM-bound stage) and the sparse MLA, each
    # timed launch by launch after an untimed fused step
    scores = torch.empty((B, 1, L), dtype=torch.float32, device=dev)
    mout = torch.empty_like(out)
    mlse = torch.empty_like(lse)
    mws = torch.empty(max(1, api.sparse_attn_workspace_bytes(api.SA_OP_MLA_FORWARD, B, 1, L, k,
                                                              wl.H, wl.dc)),
                      dtype=torch.uint8, device=dev)

    def idx_only():
        api.sparse_attn_indexer_scores(t.q_idx, t.w, t.k_idx, k_scale=t.k_scale,
                                       kv_len=t.kv_len, scores=scores, stream=stream)

    def mla_only():
        api.sparse_attn_mla_forward(t.q_lat, t.q_rope, c_kv, k_rope, idx, wl.sm_scale,
                                    out=mout, lse=mlse, ws=mws, stream=stream)

    idx_only()
    mla_only()
    n_roof = max(5, min(args.steps, 50))
    idx_ms = timed_after(step, idx_only, n_roof, stream)
    mla_ms = timed_after(step, mla_only, n_roof, stream)
    idx_bytes = B * (ki + qi)
    idx_gbs = idx_bytes / (idx_ms * 1e-3) / 1e9
    mla_bytes = B * (gather + qm + o)
    mla_flop = B * 2 * wl.H * k * ((wl.dc + wl.dR) + wl.dc)
    mla_tfs = mla_flop / (mla_ms * 1e-3) / 1e12
    log(f"indexer {idx_ms * 1e3:.1f} us/launch (each after a step), "
        f"{idx_gbs:,.0f} GB/s algorithmic")
    log(f"sparse MLA {mla_ms * 1e3:.1f} us/launch incl. split combine, "
        f"{mla_tfs:,.0f} TFLOP/s, {mla_bytes / (mla_ms * 1e-3) / 1e9:,.0f} GB/s")
    cold = per_step_stats(step, max(5, min(args.steps, 50)), stream, dev)
    log(f"cold-cache step: median {cold['median_us']} us (p10 {cold['p10_us']}, "
        f"p90 {cold['p90_us']})")
    copy_gbs = copy_peak_gbs(dev)
    log(f"device copy {copy_gbs:,.0f} GB/s (read + write); whole step "
        f"{100 * per_q * qps / (copy_gbs * 1e9):.1f}% of it")

    result = {
        "metric": "decode queries/s at L=32K,k=2048; indexer+gather % of HBM roofline",
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.k_idx.dtype == torch.bfloat16 else "bf16+fp8",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "L": L, "topk": k, "HI": wl.HI, "dI": wl.dI,
                   "H": wl.H, "dc": wl.dc, "dR": wl.dR,
                   "indexer_keys": str(wl.k_idx.dtype).replace("torch.", "")},
        "hbm_frac_step": round(step_frac, 4),
        "bytes_per_query": per_q,
        "copy_peak_gbs": round(copy_gbs, 1),
        "hbm_frac_step_vs_copy": round(per_q * qps / (copy_gbs * 1e9), 4),
        "per_step": cold,
        "roofline": {"bound": "hbm", "kernel": "indexer", "achieved": round(idx_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(idx_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic() if args.workload == "decode_32k" else None,
                     "launch_us": round(idx_ms * 1e3, 2),
                     "bytes_per_launch": idx_bytes},
        "roofline_mla": {"bound": "mfma", "kernel": "sparse MLA + split combine",
                         "achieved": round(mla_tfs, 1), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(mla_tfs / BF16_PEAK_TFLOPS, 4),
                         "hbm_frac": round(mla_bytes / (mla_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "launch_us": round(mla_ms * 1e3, 2), "flop_per_launch": mla_flop,
                         "bytes_per_launch": mla_bytes},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) on a sample")
        result["cpu_baseline"] = cpu_baseline(wl)
    return result


def prefill_indexer_flop(wl):
    """2 H^I d^I flop per (query t, candidate s <= t), over the causal triangle."""
    pairs = wl.T * (wl.T + 1) // 2
    return pairs * 2 * wl.HI * wl.dI


def prefill_mla_flop(wl, rows):
    """Flops of the sparse MLA over `rows` gathered rows summed over queries:
    per row and head, 2 (d_c + d_R) for the score and 2 d_c for the value."""
    return rows * wl.H * 2 * (2 * wl.dc + wl.dR)


def run_prefill(args, api, dev):
    """Causal prefill, T = L = 16384, through sparse_attn_prefill (sparse mode).
    At this size the entry point selects staged (the indexer scores of all T
    rows into its workspace, then the top-k), then runs the sparse MLA for
    every query; the roofline times that select as the same two calls.
    --staged times the three-call path (score tensor, top-k, MLA);
    --fused-select times the fused select (indexer scores and Top-K per query
    row, the row held on chip, no [T, L] score tensor) and the MLA."""
    import torch
    from top_indexer_sparse_amd import workloads
    log("generating prefill_16k")
    wl = workloads.prefill_16k()
    t = wl.to(dev)
    T, L, k = wl.T, wl.L, wl.topk
    c_kv, k_rope = t.kv[..., :wl.dc], t.kv[..., wl.dc:]
    idx = torch.empty((1, T, k), dtype=torch.int32, device=dev)
    cnt = torch.empty((1, T), dtype=torch.int32, device=dev)
    out = torch.empty((1, T, wl.H, wl.dc), dtype=torch.float32, device=dev)
    lse = torch.empty((1, T, wl.H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    mws = torch.empty(max(1, api.sparse_attn_workspace_bytes(api.SA_OP_MLA_FORWARD, 1, T, L, k,
                                                              wl.H, wl.dc)),
                      dtype=torch.uint8, device=dev)

    def mla():
        api.sparse_attn_mla_forward(t.q_lat, t.q_rope, c_kv, k_rope, idx, wl.sm_scale,
                                    out=out, lse=lse, ws=mws, stream=stream)

    if args.fused_select:
        def select():
            api.sparse_attn_prefill_select(t.q_idx, t.w, t.k_idx, k, q_pos=t.q_pos, idx=idx,
                                           count=cnt, stream=stream)

        def step():
            select()
            mla()
    else:
        scores = torch.empty((1, T, L), dtype=torch.float32, device=dev)
        tws = torch.empty(max(1, api.sparse_attn_workspace_bytes(api.SA_OP_TOPK, 1, T, L, k, 0, 0)),
                          dtype=torch.uint8, device=dev)

        def select():
            api.sparse_attn_indexer_scores(t.q_idx, t.w, t.k_idx, q_pos=t.q_pos, scores=scores,
                                           stream=stream)
            api.sparse_attn_topk(scores, k, q_pos=t.q_pos, idx=idx, count=cnt, ws=tws,
                                 stream=stream)

        if args.staged:
            def step():
                select()
                mla()
        else:
            ws = torch.empty(max(1, api.sparse_attn_workspace_bytes(api.SA_OP_PREFILL, 1, T, L, k,
                                                                     wl.H, wl.dc)),
                             dtype=torch.uint8, device=dev)

            def step():
                api.sparse_attn_prefill(t.q_idx, t.w, t.k_idx, k, t.q_lat, t.q_rope, c_kv,
                                        k_rope, wl.sm_scale, q_pos=t.q_pos,
                                        mode=api.SA_PREFILL_SPARSE, out=out, lse=lse,
                                        idx_out=idx, ws=ws, stream=stream)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    ms = time_events(step, args.steps, stream)
    qps = T / (ms * 1e-3)
    path = "fused_select" if args.fused_select else "staged" if args.staged else "sparse_attn_prefill"
    log(f"{ms:.2f} ms/step, {qps:,.0f} queries/s ({path})")
    if args.kernel_only:
        return None
    sel_ms = timed_after(step, select, max(3, min(args.steps, 10)), stream)
    flop = prefill_indexer_flop(wl)
    tfs = flop / (sel_ms * 1e-3) / 1e12
    what = "fused select (scores + top-k)" if args.fused_select else "indexer scores + top-k"
    log(f"{what} {sel_ms:.3f} ms: indexer flops at {tfs:,.0f} TFLOP/s = "
        f"{100 * tfs / BF16_PEAK_TFLOPS:.1f}% of bf16 MFMA peak")
    rows = int(torch.clamp(cnt, max=k).sum().item())
    mla_ms = ms - sel_ms
    mla_tfs = prefill_mla_flop(wl, rows) / (mla_ms * 1e-3) / 1e12
    log(f"sparse MLA ~{mla_ms:.2f} ms over {rows:,} rows: {mla_tfs:,.0f} TFLOP/s")
    result = {
        "metric": "prefill queries/s at T=L=16K, k=2048; select % of bf16 MFMA peak",
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": 1, "T": T, "L": L, "topk": k, "HI": wl.HI,
                   "dI": wl.dI, "H": wl.H, "dc": wl.dc, "dR": wl.dR,
                   "path": path},
        "roofline": {"bound": "mfma", "kernel": what, "achieved": round(tfs, 1),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tfs / BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "launch_us": round(sel_ms * 1e3, 1), "flop_per_launch": flop},
        "roofline_mla": {"bound": "mfma", "achieved": round(mla_tfs, 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(mla_tfs / BF16_PEAK_TFLOPS, 4),
                         "ms": round(mla_ms, 3), "rows": rows},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) on a sample")
        result["cpu_baseline"] = cpu_baseline_prefill(wl)
    return result


def run_crossover(args, api, dev):
    """Dense (every causal candidate) against sparse (fused select + k rows)
    prefill at T = L for L = 1K .. 16K, k = 2048, H = 128: the short-sequence
    crossover of the two modes of sparse_attn_prefill."""
    import torch
    from top_indexer_sparse_amd import workloads
    stream = torch.cuda.current_stream()
    table = []
    for L in (1024, 1536, 2048, 2560, 3072, 4096, 6144, 8192, 16384):
        wl = workloads.prefill_16k(L=L, n_needles=0)
        t = wl.to(dev)
        c_kv, k_rope = t.kv[..., :wl.dc], t.kv[..., wl.dc:]
        out = torch.empty((1, L, wl.H, wl.dc), dtype=torch.float32, device=dev)
        lse = torch.empty((1, L, wl.H), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, api.sparse_attn_workspace_bytes(api.SA_OP_PREFILL, 1, L, L,
                                                                 wl.topk, wl.H, wl.dc)),
                         dtype=torch.uint8, device=dev)
        row = {"L": L}
        for name, mode in (("sparse", api.SA_PREFILL_SPARSE), ("dense", api.SA_PREFILL_DENSE)):
            def step():
                api.sparse_attn_prefill(t.q_idx, t.w, t.k_idx, wl.topk, t.q_lat, t.q_rope, c_kv,
                                        k_rope, wl.sm_scale, q_pos=t.q_pos, mode=mode, out=out,
                                        lse=lse, ws=ws, stream=stream)
            for _ in range(2):
                step()
            n = max(3, min(args.steps, 20 if L <= 4096 else 5))
            row[f"{name}_ms"] = round(time_events(step, n, stream), 4)
        row["dense_over_sparse"] = round(row["dense_ms"] / row["sparse_ms"], 3)
        log(f"L={L:6d}: sparse {row['sparse_ms']:.3f} ms, dense {row['dense_ms']:.3f} ms "
            f"(dense/sparse {row['dense_over_sparse']:.2f})")
        table.append(row)
        del t, out, lse, ws
        torch.cuda.empty_cache()
    faster = [r["L"] for r in table if r["dense_ms"] <= r["sparse_ms"]]
    cross = max(faster) if faster else None
    last = table[-1]
    return {
        "metric": "prefill dense/sparse crossover (T=L, k=2048): longest L where dense is faster",
        "value": cross, "unit": "tokens", "n_gpus": 1, "steps": args.steps,
        "warmup": 2, "ms_per_step": last["sparse_ms"], "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill_crossover", "k": 2048, "H": 128, "HI": 64, "dI": 128},
        "sweep": table,
    }


def cpu_baseline_prefill(wl, stride=64):
    """The oracle on every `stride`-th query row of the prefill (full causal
    rows, top-k and sparse MLA), in queries/s."""
    import oracle
    import torch
    rows = torch.arange(stride - 1, wl.T, stride)
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    s = oracle.indexer(wl.q_idx[:, rows], wl.w[:, rows], wl.k_idx, q_pos=wl.q_pos[:, rows])
    idx, _ = oracle.topk(s, wl.topk, q_pos=wl.q_pos[:, rows])
    oracle.sparse_mla(wl.q_lat[:, rows], wl.q_rope[:, rows], wl.kv, idx, wl.sm_scale, dc=wl.dc)
    dt = time.perf_counter() - t0
    return {"value": round(len(rows) / dt, 3), "unit": "queries/s", "cores": threads,
            "kind": "oracle",
            "sample": f"every {stride}th query row of prefill_16k ({len(rows)} rows, causal "
                      f"L up to {wl.L}), fp64 C oracle on {threads} threads, {dt:.2f} s"}


def block_union_bytes(wl, blocks):
    """K and V bytes one step must read at least: per (sequence, KV head), the
    union over its query heads of the visible tokens (chosen blocks, sinks,
    window), each token's key and value row once."""
    import numpy as np
    bl = blocks.cpu().numpy()
    G = wl.Hq // wl.Hkv
    row = 2 * wl.d * 2  # key + value, bf16
    total = 0
    base = np.zeros(wl.L, dtype=bool)
    base[:min(wl.n_sink, wl.L)] = True
    base[max(0, wl.L - wl.n_win):] = True
    for b in range(wl.B):
        for g in range(wl.Hkv):
            vis = base.copy()
            for n in bl[b, g * G:(g + 1) * G].reshape(-1):
                if n >= 0:
                    vis[n * wl.blk:(n + 1) * wl.blk] = True
            total += int(vis.sum()) * row
    return total


def run_block(args, api, dev):
    """Block-sparse GQA decode, B=16, L=65536, 32 query / 8 KV heads: a step is
    block choice + attention over the visible set, on pooled keys that are
    built once beforehand (a cache-maintenance step, timed on its own)."""
    import torch
    from top_indexer_sparse_amd import workloads
    log("generating block_sparse_64k")
    wl = workloads.block_sparse_64k()
    t = wl.to(dev)
    stream = torch.cuda.current_stream()
    krep = torch.empty((wl.B, wl.L // wl.blk, wl.Hkv, wl.d), dtype=torch.bfloat16, device=dev)
    out = torch.empty((wl.B, wl.Hq, wl.d), dtype=torch.float32, device=dev)
    blocks = torch.empty((wl.B, wl.Hq, wl.nsel), dtype=torch.int32, device=dev)
    ws = torch.empty(api.sparse_attn_workspace_bytes(api.SA_OP_BLOCK_DECODE, wl.B, wl.Hq, wl.L,
                                                     wl.nsel, wl.Hkv, wl.d),
                     dtype=torch.uint8, device=dev)

    def pool():
        api.sparse_attn_block_pool(t.k, wl.blk, krep=krep, stream=stream)

    def step():
        api.sparse_attn_block_decode(t.q, t.k, t.v, krep, wl.blk, wl.nsel, wl.n_sink, wl.n_win,
                                     wl.sm_scale, out=out, blocks_out=blocks, ws=ws,
                                     stream=stream, shared_choice=args.shared_choice)

    pool()
    pool_ms = time_events(pool, 3, stream)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    ms = time_events(step, args.steps, stream)
    qps = wl.B / (ms * 1e-3)
    kv_bytes = block_union_bytes(wl, blocks)
    # pooled keys in bf16 (2 bytes an element), as stored
    krep_bytes = krep.numel() * krep.element_size()
    io_bytes = wl.B * wl.Hq * wl.d * (2 + 4)
    step_bytes = kv_bytes + krep_bytes + io_bytes
    gbs = step_bytes / (ms * 1e-3) / 1e9
    log(f"{ms * 1e3:.1f} us/step, {qps:,.0f} queries/s; {step_bytes / 1e6:.1f} MB/step "
        f"= {gbs:,.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of HBM peak); "
        f"pooling {pool_ms * 1e3:.0f} us")
    result = {
        "metric": "block-sparse decode queries/s at L=64K, top-16 blocks of 64 + 64 sinks + "
                  "512 window, GQA 32/8" + (", block choice shared per KV group"
                                            if args.shared_choice else ""),
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "L": wl.L, "Hq": wl.Hq, "Hkv": wl.Hkv,
                   "d": wl.d, "blk": wl.blk, "nsel": wl.nsel, "n_sink": wl.n_sink,
                   "n_win": wl.n_win, "shared_choice": bool(args.shared_choice)},
        "roofline": {"bound": "hbm", "kernel": "block choice + attention (whole step)",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": step_bytes},
        "block_pool_us": round(pool_ms * 1e3, 1),
    }
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle.num_threads()
        t0 = time.perf_counter()
        n = 2
        for b in range(n):
            oracle.block_sparse_decode(wl.q[b:b + 1], wl.k[b:b + 1], wl.v[b:b + 1], wl.blk,
                                       wl.nsel, wl.n_sink, wl.n_win, wl.sm_scale,
                                       shared=args.shared_choice)
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": round(n / dt, 3), "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {wl.B} sequences of block_sparse_64k (full L, all 32 heads, "
                      f"pooling included), fp64 C oracle on {threads} threads, {dt:.2f} s"}
    return result


def run_csa(args, api, dev):
    """Selection over compressed entries: B=32 queries over Lc=32768 entries
    (a 131072-token context at m = 4), k=2048, 128 window entries, H=128,
    c=512: indexer + top-k over the entries, then MQA core attention with
    keys = values = entries over the selection and the window."""
    import torch
    from top_indexer_sparse_amd import workloads
    log("generating csa_decode")
    wl = workloads.csa_decode()
    t = wl.to(dev)
    B, Lc, k, H, c = wl.B, wl.Lc, wl.topk, wl.H, wl.c
    out = torch.empty((B, H, c), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    ws = torch.empty(api.sparse_attn_workspace_bytes(api.SA_OP_CSA_DECODE, B, wl.n_win, Lc, k, H, c),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        api.sparse_attn_csa_decode(t.q_idx, t.w, t.k_idx, None, t.n_comp, k, t.q, t.comp, t.win,
                                   wl.sm_scale, out=out, lse=lse, idx_out=idx, ws=ws,
                                   stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    ms = time_events(step, args.steps, stream)
    qps = B / (ms * 1e-3)
    # algorithmic bytes per query: index keys, index query and weights, the
    # attended entries (selected + window), the core query and the output
    ki = Lc * wl.dI * 2
    qi = wl.HI * wl.dI * 2 + wl.HI * 4
    gather = (k + wl.n_win) * c * 2
    qm, o = H * c * 2, H * c * 4
    per_q = ki + qi + gather + qm + o
    step_frac = per_q * qps / (HBM_PEAK_GBS * 1e9)
    log(f"{ms * 1e3:.1f} us/step, {qps:,.0f} queries/s, whole step {100 * step_frac:.1f}% of HBM peak")
    if args.kernel_only:
        return None
    scores = torch.empty((B, 1, Lc), dtype=torch.float32, device=dev)

    def idx_only():
        api.sparse_attn_indexer_scores(t.q_idx[:, None], t.w[:, None], t.k_idx, scores=scores,
                                       stream=stream)

    idx_only()
    idx_ms = timed_after(step, idx_only, max(5, min(args.steps, 50)), stream)
    idx_bytes = B * (ki + qi)
    idx_gbs = idx_bytes / (idx_ms * 1e-3) / 1e9
    log(f"indexer over the entries {idx_ms * 1e3:.1f} us/launch, {idx_gbs:,.0f} GB/s algorithmic")
    result = {
        "metric": "compressed-entry selection decode queries/s (Lc=32K entries, k=2048, "
                  "128-entry window)",
        "value": round(qps, 1), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "Lc": Lc, "topk": k, "n_win": wl.n_win,
                   "HI": wl.HI, "dI": wl.dI, "H": H, "c": c},
        "hbm_frac_step": round(step_frac, 4), "bytes_per_query": per_q,
        "roofline": {"bound": "hbm", "kernel": "indexer over the entries",
                     "achieved": round(idx_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(idx_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "launch_us": round(idx_ms * 1e3, 2), "bytes_per_launch": idx_bytes},
    }
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle.num_threads()
        # whole sequences, 4 at a time, cycling over the batch until ~10 s
        n, i = 0, 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 10.0:
            sl = slice(i, i + 4)
            oracle.csa_decode(wl.q_idx[sl], wl.w[sl], wl.k_idx[sl], wl.q[sl], wl.comp[sl],
                              wl.win[sl], k, wl.sm_scale)
            n += 4
            i = (i + 4) % B
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": round(n / dt, 3), "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} sequences of csa_decode, 4 at a time cycling over the {B} "
                      f"(all {Lc} entries, all {H} heads each), fp64 oracle, {dt:.2f} s"}
    return result


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_32k",
                    choices=["decode_32k", "decode_128k_fp8", "prefill_16k",
                             "block_sparse_64k", "csa_decode", "prefill_crossover"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--staged", action="store_true",
                    help="prefill_16k: time the three-call path (score tensor, top-k, MLA) "
                         "instead of sparse_attn_prefill")
    ap.add_argument("--fused-select", action="store_true",
                    help="prefill_16k: time the fused select (no score tensor) and the MLA "
                         "instead of sparse_attn_prefill")
    ap.add_argument("--shared-choice", action="store_true",
                    help="block_sparse_64k: one block choice per KV group (sum of its heads' "
                         "block scores)")
    ap.add_argument("--kernel-only", action="store_true",
                    help="only the timed steps (for profiler runs)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="also run 3 plain device copies of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(decode shards by sequence, with no exchange between GPUs). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from top_indexer_sparse_amd import api
    api.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "prefill_16k":
        result = run_prefill(args, api, dev)
    elif args.workload == "block_sparse_64k":
        result = run_block(args, api, dev)
    elif args.workload == "csa_decode":
        result = run_csa(args, api, dev)
    elif args.workload == "prefill_crossover":
        result = run_crossover(args, api, dev)
    else:
        result = run_decode(args, api, dev)
    if result is not None:
        print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
