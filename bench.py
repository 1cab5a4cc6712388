"""Benchmark of the attention step on one MI355X.

Default workload: decode, batch 32, full-attention layer, per-request
context drawn uniformly from [60000, 100000] (seed 1002), page size 1, random
cache rows in ~80 GB of K+V pools, kv_scale 1.  A step is one museattn_attn_step
call (the attention kernel, which also normalises q and k and writes the new
fp8 cache rows, then the combine kernel that merges the split-K partials and
writes the gated output) over that batch with every input already resident in
HBM.

The timed region is one replay of a HIP graph holding the K steps (a decode
loop runs its steps from captured graphs); --eager times K plain calls.

Prints ONE JSON line on stdout (progress goes to stderr):
  value       achieved HBM throughput of the step on the algorithmic K+V bytes
              (256 B per visible key), GB/s
  roofline    the attention kernel alone (the step's dominant kernel), timed
              with HIP events on the stream it runs on, against MI355X's 8 TB/s
  cold_cache_graph_replay  one-step graph replays, each after a 1 GiB read
              flush: median, p10, p90, bootstrap 95% interval of the median,
              and the replay time of a one-kernel graph (launch cost, not
              subtracted)
  gather_probe  the step's K/V row gather alone (full-layer workloads): the
              attention kernel's ceiling on this memory system
  cpu_baseline  the CPU oracle on the same workload, one process per host core,
              and on one thread
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
OPROJ_GEMM_MIN_T = 64   # from this many tokens on the library runs the projection as its LDS-tiled GEMM
OPROJ_HIDDEN = 8192   # the decoder layer's model width (the page's [T, 8192] activations)
PMC_SUMMARY = os.path.join(ROOT, "profiles", "attn_kernel_decode_b32_full_ctx60k-100k_pmc.txt")
ATTN_SOURCE = os.path.join(ROOT, "paged_fp8_kv_amd", "csrc", "attn_splitk.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def hip_elapsed_ms(start, end) -> float:
    """hipEventElapsedTime on the raw handles of two torch events (recorded by
    the library, so torch's own bookkeeping does not know they were recorded)."""
    import ctypes
    global _HIP
    if "_HIP" not in globals():
        _HIP = ctypes.CDLL("libamdhip64.so")
        _HIP.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                             ctypes.c_void_p]
        _HIP.hipEventElapsedTime.restype = ctypes.c_int
    ms = ctypes.c_float()
    st = _HIP.hipEventElapsedTime(ctypes.byref(ms), start.cuda_event, end.cuda_event)
    if st != 0:
        raise RuntimeError(f"hipEventElapsedTime failed with status {st}")
    return ms.value


def kernel_source_hash() -> str:
    with open(ATTN_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(bytes_per_launch_alg):
    """HBM bytes per launch of the attention kernel from the committed PMC
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a copy-kernel calibration), or
    None when the summary is absent, was taken on another kernel source or on
    another workload (its algorithmic bytes per launch differ)."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    vals = {}
    with open(PMC_SUMMARY) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    if vals.get("algorithmic_bytes_per_launch") != str(int(bytes_per_launch_alg)):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# rocprofv3 MFMA counter summaries of the attention kernel, by workload
# (SQ_VALU_MFMA_BUSY_CYCLES over the SIMDs' cycles), committed under profiles/
MFMA_SUMMARIES = {
    "2": "attn_kernel_decode_b32_full_ctx60k-100k_mfma.txt",
    "3f": "attn_kernel_verify_b1_L8_full_ctx80k_mfma.txt",
    "v32f": "attn_kernel_verify_b32_L8_full_ctx60k-100k_mfma_lds.txt",
    "pf1f": "attn_kernel_prefill_b1_L753_full_ctx80k_mfma.txt",
    "pff32": "attn_kernel_prefill_b1_L16384_full_ctx32k_mfma.txt",
}


def read_mfma_busy(cid, attn_flops):
    """The attention kernel's MFMA busy fraction from the workload's committed
    counter summary, or None when there is none, it was taken on another
    kernel source, or its algorithmic FLOPs per dispatch are not this
    workload's (within the summary's 4 printed digits)."""
    name = MFMA_SUMMARIES.get(str(cid))
    if name is None or not os.path.exists(os.path.join(ROOT, "profiles", name)):
        return None
    vals = {}
    with open(os.path.join(ROOT, "profiles", name)) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        busy = float(vals["mfma_busy_fraction"].split()[0])
        if "algorithmic_flop_per_dispatch" in vals:
            alg = float(vals["algorithmic_flop_per_dispatch"].split()[0])
        else:   # "<counted>   (... x 512; algorithmic <flops>)"
            alg = float(vals["mfma_flop_per_dispatch"].split("algorithmic")[1].strip(" )"))
    except (KeyError, ValueError, IndexError):
        return None
    if abs(alg - attn_flops) > 5e-4 * attn_flops:
        return None
    return {"fraction": busy, "from": "profiles/" + name}


def _oracle_job(job, barrier, results, index):
    """One process of the CPU baseline: draws its share of the workload's
    inputs (not timed), waits at the barrier for the other processes, then
    times the oracle (unchanged) on that share with `blas_threads` BLAS
    threads and puts (index, seconds) on the results queue."""
    cid, pool_rows, requests, tokens, blas_threads = job
    from threadpoolctl import threadpool_limits
    import numpy as np
    from oracle import museattn_oracle as O
    from paged_fp8_kv_amd import workloads as W

    with threadpool_limits(blas_threads):
        w = W.config(cid, pool_rows)
        sub = w.subset(requests)
        kp, vp = W.LogicalPool.pair(sub, range(sub.B))
        barrier.wait(timeout=600)
        t0 = time.perf_counter()
        O.attn_step(sub.qkv.float().numpy(), sub.positions, sub.table, kp, vp, B=sub.B, L=sub.L,
                    page_size=sub.page_size, layer_kind=sub.layer_kind, kv_scale=sub.kv_scale,
                    w_q=sub.w_q, w_k=sub.w_k, w_o=sub.w_o, eps=float(np.float32(1e-6)),
                    q_scale=float(np.float32(5.473)), tokens=tokens)
        results.put((index, time.perf_counter() - t0))


def _run_oracle_jobs(jobs):
    """Each job in its own spawned process (fresh interpreters: no GPU state is
    inherited), all released together; returns the per-process seconds."""
    import multiprocessing as mp
    ctx = mp.get_context("spawn")
    barrier, results = ctx.Barrier(len(jobs)), ctx.Queue()
    procs = [ctx.Process(target=_oracle_job, args=(job, barrier, results, i))
             for i, job in enumerate(jobs)]
    for p in procs:
        p.start()
    out = {}
    try:
        for _ in jobs:
            i, sec = results.get(timeout=900)
            out[i] = sec
    finally:
        for p in procs:
            p.join(timeout=60)
            if p.is_alive():
                p.kill()
    return [out[i] for i in range(len(jobs))]


def _step_fraction(w, requests, tokens):
    """The share of the step's work (K+V bytes; attention FLOPs for a prefill
    block) that the oracle does on these requests (and block tokens)."""
    import numpy as np
    if tokens is None:
        return w.subset(requests).kv_bytes / w.kv_bytes
    p = w.positions[tokens].astype(np.int64)
    keys = p + 1 if w.layer_kind == 0 else np.minimum(p + 1, 2048)
    return float(keys.sum()) * 16 * 64 * 4 / w.attn_flops


def cpu_baseline(w, cid, pool_rows, sample_requests: int, sample_tokens: int, max_procs: int):
    """The oracle (as it stands, float64 numpy) on the host cores: a sample of
    the workload's requests (for a prefill block, evenly spaced block tokens
    of request 0) split over one spawned process per core, one BLAS thread
    each, started together after each has drawn its inputs; and the same
    oracle on one thread (one process, one BLAS thread) on a smaller sample.
    Both are scaled to one step by the share of the step's work they did."""
    import numpy as np

    avail = len(os.sched_getaffinity(0))
    procs = max(1, min(max_procs, avail))
    if w.L <= 8:
        req = list(range(min(sample_requests, w.B)))
        groups = [req[i::procs] for i in range(procs) if req[i::procs]]
        jobs = [(cid, pool_rows, g, None, 1) for g in groups]
        one = (cid, pool_rows, req[:1], None, 1)
        what = f"requests 0..{req[-1]} ({len(req)} of {w.B})"
        frac = _step_fraction(w, req, None)
        frac1 = _step_fraction(w, req[:1], None)
    else:
        toks = sorted({int(x) for x in np.linspace(0, w.L - 1, min(sample_tokens, w.L))})
        groups = [toks[i::procs] for i in range(procs) if toks[i::procs]]
        jobs = [(cid, pool_rows, [0], g, 1) for g in groups]
        one = (cid, pool_rows, [0], toks[::max(1, len(toks) // 8)], 1)
        what = f"{len(toks)} evenly spaced block tokens of request 0"
        frac = _step_fraction(w, [0], toks)
        frac1 = _step_fraction(w, [0], one[3])
    log(f"cpu_baseline: {what} over {len(jobs)} processes; one-thread run on a smaller sample")
    wall = max(_run_oracle_jobs(jobs))
    t1 = _run_oracle_jobs([one])[0]
    step_s, step1_s = wall / frac, t1 / frac1
    log(f"cpu_baseline: {len(jobs)} processes {wall:.2f} s -> {step_s:.3f} s/step; "
        f"one thread {t1:.2f} s -> {step1_s:.3f} s/step")
    if w.L <= 8:
        conv, unit = (lambda sec: round(w.kv_bytes / sec / 1e9, 4)), "GB/s"
    else:
        conv, unit = (lambda sec: round(w.attn_flops / sec / 1e12, 6)), "TFLOP/s"
    return {"value": conv(step_s), "unit": unit, "cores": len(jobs), "kind": "oracle",
            "threads_per_process": 1, "host_cores": os.cpu_count(), "available_cores": avail,
            "s_per_step": round(step_s, 4),
            "one_thread": {"value": conv(step1_s), "s_per_step": round(step1_s, 4),
                           "sample_fraction": round(frac1, 5)},
            "sample": f"{what}, {frac * 100:.2f}% of the step's "
                      f"{'K+V bytes' if w.L <= 8 else 'attention FLOPs'}; float64 numpy oracle "
                      f"in {len(jobs)} processes of one BLAS thread each (slowest {wall:.2f} s), "
                      f"scaled to one step"}


TS_SLOTS = 12   # per attention work-group in the instrumented build (device_common.h)
TS_NAMES = ("entry", "plan", "setup", "stream", "partial", "exit")


def phase_report(w, step, ws, G, reps):
    """Per-phase times of the step from the instrumented library (built with
    MUSEATTN_PHASE_TIMES): each attention work-group stamps the GPU's 100 MHz
    real-time counter at entry, when its plan is ready, when its first
    segment's loads and set-up are done, when that segment's key chunks are
    done, when its partials are written and at exit; each combine work-group
    at entry and exit.  All times are relative to the first attention entry;
    medians over `reps` eager steps."""
    import numpy as np
    import torch

    T = w.B * w.L
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    ts_bytes = al((G * TS_SLOTS + 2 * T * 16) * 8)
    region = ws[ws.numel() - ts_bytes:]
    rows = []
    for _ in range(reps):
        region.zero_()
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        v = region.view(torch.int64).cpu().numpy()
        att = v[:G * TS_SLOTS].reshape(G, TS_SLOTS)
        comb = v[G * TS_SLOTS:G * TS_SLOTS + 2 * T * 16].reshape(-1, 2)
        comb = comb[(comb[:, 0] > 0) & (comb[:, 1] > 0)]
        t0 = att[:, 0].min()
        us = lambda x: (x - t0) / 100.0  # noqa: E731  (100 MHz counter -> us)
        act = att[att[:, 6] > 0]
        two = att[att[:, 6] > 1]   # work-groups with a second segment
        r = {"entry_first": 0.0, "entry_last": float(us(att[:, 0].max())),
             "plan_median": float(np.median(act[:, 1] - act[:, 0]) / 100.0),
             "setup_median": float(np.median(act[:, 2] - act[:, 1]) / 100.0),
             "setup_issue_median": float(np.median(act[:, 7] - act[:, 1]) / 100.0),
             "setup_loads_median": float(np.median(act[:, 8] - act[:, 7]) / 100.0),
             "setup_q_median": float(np.median(act[:, 9] - act[:, 8]) / 100.0),
             "setup_barrier_median": float(np.median(act[:, 2] - act[:, 9]) / 100.0),
             "stream_median": float(np.median(act[:, 3] - act[:, 2]) / 100.0),
             "second_segment_setup_median": (float(np.median(two[:, 11] - two[:, 10]) / 100.0)
                                             if len(two) else None),
             "first_segment_setup_same_wgs_median": (float(np.median(two[:, 2] - two[:, 1]) / 100.0)
                                                     if len(two) else None),
             "partial_median": float(np.median(act[:, 4] - act[:, 3]) / 100.0),
             "rest_median": float(np.median(act[:, 5] - act[:, 4]) / 100.0),
             "setup_done_p50": float(np.median(us(act[:, 2]))),
             "setup_done_max": float(us(act[:, 2].max())),
             "attn_exit_p10": float(np.percentile(us(act[:, 5]), 10)),
             "attn_exit_p50": float(np.median(us(act[:, 5]))),
             "attn_exit_p90": float(np.percentile(us(act[:, 5]), 90)),
             "attn_exit_last": float(us(att[:, 5].max())),
             # work-group w runs on XCD w % 8 (round-robin dispatch)
             "attn_exit_by_xcd_median": [float(np.median(us(g[g[:, 6] > 0, 5])))
                                         if (g[:, 6] > 0).any() else 0.0
                                         for g in (att[x::8] for x in range(8))],
             "combine_entry_first": float(us(comb[:, 0].min())),
             "combine_exit_last": float(us(comb[:, 1].max())),
             "active_work_groups": int(len(act)), "combine_work_groups": int(len(comb))}
        crit = act[np.argmax(act[:, 5])]
        r["critical_wg"] = {n: float(us(crit[i])) for i, n in enumerate(TS_NAMES)}
        r["critical_wg"]["segments"] = int(crit[6])
        rows.append(r)
    keys = [k for k in rows[0] if k != "critical_wg" and not k.endswith("work_groups")]
    med = lambda k: (round(float(np.median([r[k] for r in rows])), 2)  # noqa: E731
                     if not isinstance(rows[0][k], list) else
                     [round(float(x), 2) for x in np.median([r[k] for r in rows], axis=0)])
    out = {k: (med(k) if rows[0][k] is not None else None) for k in keys}
    out["active_work_groups"] = rows[0]["active_work_groups"]
    out["combine_work_groups"] = rows[0]["combine_work_groups"]
    mid = sorted(rows, key=lambda r: r["attn_exit_last"])[len(rows) // 2]
    out["critical_wg_of_median_step"] = {k: round(v, 2) for k, v in mid["critical_wg"].items()}
    out["reps"] = reps
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="2",
                    help="workload id (0, 1, 2, 3s, 3f, 4; batch shapes d16s, d16f, d32s, v16s, v16f, v32s, "
                         "v32f; prefill blocks pf1f, pf1s, pf4f, "
                         "pf4s, pff0, pfs32, pff32, pff64)")
    ap.add_argument("--work-groups", type=int, default=0,
                    help="attention work-groups (0 = the library's choice)")
    ap.add_argument("--pool-rows", type=int, default=0,
                    help="override the pool size in rows (0 = the workload's own)")
    ap.add_argument("--cold-reps", type=int, default=200,
                    help="graph replays timed one by one after a 1 GiB cache flush")
    ap.add_argument("--cpu-sample", type=int, default=32, help="requests the oracle times")
    ap.add_argument("--cpu-procs", type=int, default=16,
                    help="most oracle processes (one per host core of the GPU's share)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=96,
                    help="block tokens the oracle times (prefill blocks)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gather-probe", action="store_true",
                    help="skip the row-gather probe (full-layer decode and verify workloads)")
    ap.add_argument("--eager", action="store_true",
                    help="time K eager calls instead of one replay of K captured steps")
    ap.add_argument("--graph-warmup", type=int, default=400,
                    help="untimed steps replayed from the captured graph before the timed "
                         "replay (back-to-back replays take ~10 ms to reach a steady state)")
    ap.add_argument("--oproj", action="store_true",
                    help="the step also runs the decoder layer's output projection "
                         "(bf16 o [8192, 1024]); reported in the 'oproj' field")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="run a 1 GiB device copy first (PMC calibration runs)")
    ap.add_argument("--phases", action="store_true",
                    help="load the instrumented library (per-phase timestamps) and print a "
                         "phase breakdown of the step instead of the benchmark line")
    args = ap.parse_args()
    if args.phases:   # before the package is imported: it reads MUSEATTN_LIB once
        os.environ.setdefault("MUSEATTN_LIB", os.path.join(ROOT, "paged_fp8_kv_amd",
                                                           "libmuseattn_phases.so"))

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the step "
              "shards by request or by key range without kernel changes, but no multi-GPU "
              "run is implemented here.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_fp8_kv_amd as P
    from paged_fp8_kv_amd import workloads as W

    dev = "cuda:0"
    P.lib()
    w = W.config(args.config, args.pool_rows or None)
    log(f"workload {w.name}: B={w.B} L={w.L} keys={int(w.kv_bytes // 256)} "
        f"K+V bytes={w.kv_bytes / 1e6:.1f} MB pool rows={w.num_rows}")
    t0 = time.perf_counter()
    kp, vp = W.build_pools_device(w, dev)
    f = lambda a: torch.from_numpy(a.copy()).to(dev)  # noqa: E731
    d = dict(qkv=w.qkv.to(dev), positions=f(w.positions), table=f(w.table), seq_lens=f(w.seq_lens),
             w_q=f(w.w_q), w_k=f(w.w_k), w_o=f(w.w_o))
    out = torch.empty(w.B, w.L, 1024, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(P.workspace_bytes(w.B, w.L, w.max_seq_len, w.page_size, w.layer_kind,
                                       args.work_groups), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"inputs resident in HBM ({time.perf_counter() - t0:.1f} s)")

    if args.calibration_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        log("calibration copy of 1 GiB done")

    ow = yo = None
    if args.oproj:
        # the decoder layer's output projection after the step (bf16 [8192, 1024] weights)
        ow = W.oproj_weight(w.seed, OPROJ_HIDDEN).to(dev)
        yo = torch.empty(w.T, OPROJ_HIDDEN, dtype=torch.bfloat16, device=dev)

    def step(events=None, oproj_events=None):
        kw = {}
        if args.oproj and events is None:   # attention events are taken on the plain step
            kw = dict(o_weight=ow, y=yo, oproj_events=oproj_events)
        P.attn_step(d["qkv"], d["positions"], d["table"], d["seq_lens"], kp, vp, w.kv_scale,
                    w.page_size, w.layer_kind, out, q_norm_w=d["w_q"], k_norm_w=d["w_k"],
                    o_norm_w=d["w_o"], max_seq_len=w.max_seq_len, workspace=ws,
                    work_groups=args.work_groups, attn_events=events, **kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    if args.phases:
        G = P.work_groups(w.B, w.L, w.max_seq_len, w.layer_kind, args.work_groups)
        rep = phase_report(w, step, ws, G, max(args.steps, 5))
        log("phases (us from the first attention work-group's entry): " + json.dumps(rep))
        print(json.dumps({"phases": rep, "library": os.path.basename(P.LIB_PATH),
                          "config": {"workload": w.name, "B": w.B, "L": w.L,
                                     "layer": "full" if w.layer_kind == 0 else "sliding",
                                     "page_size": w.page_size, "work_groups": G}}), flush=True)
        return

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for pair in evs:        # torch creates the HIP event on its first record
        for e in pair:
            e.record()
    torch.cuda.synchronize()

    def timed_eager():
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(None if args.oproj else evs[i])
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def attn_evented():
        for i in range(args.steps):
            step(evs[i])
        torch.cuda.synchronize()

    mode = "eager"
    if not args.eager:
        # K steps captured into one HIP graph, as a decode loop runs them
        steps_graph = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            step()
        torch.cuda.current_stream().wait_stream(cs)
        torch.cuda.synchronize()
        with torch.cuda.graph(steps_graph):
            for _ in range(args.steps):
                step()
        for _ in range(max(1, -(-args.graph_warmup // args.steps))):
            steps_graph.replay()       # untimed
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        steps_graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        mode = "graph"
    else:
        wall = timed_eager()
    ms_per_step = wall * 1e3 / args.steps
    # the attention kernel's launch duration: HIP events recorded by the library
    # on the kernel's stream around each launch, over K eager steps (event
    # records captured inside a graph do not bracket the kernel on this runtime)
    if mode == "graph" or args.oproj:
        attn_evented()
    attn_ms = [hip_elapsed_ms(s0, e0) for s0, e0 in evs]
    attn_avg_ms = sum(attn_ms) / len(attn_ms)
    log(f"timed {args.steps} steps ({mode}): {ms_per_step * 1e3:.1f} us/step; attention kernel "
        f"avg {attn_avg_ms * 1e3:.1f} us (min {min(attn_ms) * 1e3:.1f})")

    oproj = None
    if args.oproj:
        oevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]
        for pair in oevs:
            for e in pair:
                e.record()
        torch.cuda.synchronize()
        for i in range(args.steps):
            step(oproj_events=oevs[i])
        torch.cuda.synchronize()
        o_ms = [hip_elapsed_ms(s0, e0) for s0, e0 in oevs]
        o_avg = sum(o_ms) / len(o_ms)
        obytes = OPROJ_HIDDEN * 1024 * 2 + w.T * 1024 * 2 + w.T * OPROJ_HIDDEN * 2
        oflops = 2 * w.T * 1024 * OPROJ_HIDDEN
        # the roofline that bounds it: bytes at the HBM peak or products at the
        # bf16 MFMA peak (the same 2.5 PFLOP/s as fp16), whichever takes longer
        mfma_bound = oflops / (MFMA_F16_PEAK_TFLOPS * 1e12) > obytes / (HBM_PEAK_GBS * 1e9)
        if mfma_bound:
            ach, peak, unit = oflops / (o_avg * 1e-3) / 1e12, MFMA_F16_PEAK_TFLOPS, "TFLOP/s"
        else:
            ach, peak, unit = obytes / (o_avg * 1e-3) / 1e9, HBM_PEAK_GBS, "GB/s"
        oproj = {"kernel": ("gemm_kernel (y = out . o^T, LDS-tiled bf16 MFMA GEMM, fp32 sums)"
                            if w.T >= OPROJ_GEMM_MIN_T
                            else "oproj_kernel (y = out . o^T, bf16 MFMA, fp32 sums)"),
                 "hidden": OPROJ_HIDDEN, "tokens": w.T, "bound": "mfma" if mfma_bound else "hbm",
                 "algorithmic_bytes_per_launch": obytes, "algorithmic_flops_per_launch": oflops,
                 "avg_launch_us": round(o_avg * 1e3, 2), "achieved": round(ach, 1), "peak": peak,
                 "unit": unit, "frac": round(ach / peak, 4),
                 "avg_launch_us_from": f"HIP events around each of {args.steps} eager launches"}
        log(f"o-projection avg {o_avg * 1e3:.2f} us ({oproj['achieved']} {unit}, "
            f"{obytes / 1e6:.1f} MB, {oflops / 1e9:.1f} GFLOP)")

    cold = None
    if args.cold_reps > 0:
        # a read of 1 GiB evicts the step's data from the caches without leaving
        # dirty lines behind (a write-flush would add write-back traffic)
        flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            step()
        tiny = torch.zeros(1, device=dev)
        g_tiny = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_tiny):
            tiny.add_(1.0)

        def replay_times(graph):
            out_us = []
            for _ in range(args.cold_reps):
                flush.sum()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                graph.replay()
                e1.record()
                torch.cuda.synchronize()
                out_us.append(e0.elapsed_time(e1) * 1e3)
            return np.sort(np.array(out_us))

        times = replay_times(g)
        tiny_times = replay_times(g_tiny)
        # bootstrap 95% interval of the median (seeded resampling)
        rng = np.random.default_rng(0)
        meds = np.median(rng.choice(times, size=(2000, times.size), replace=True), axis=1)
        med = float(np.median(times))
        cold = {"median_us": round(med, 2),
                "p10_us": round(float(np.percentile(times, 10)), 2),
                "p90_us": round(float(np.percentile(times, 90)), 2),
                "median_ci95_us": [round(float(np.percentile(meds, 2.5)), 2),
                                   round(float(np.percentile(meds, 97.5)), 2)],
                "gbs_at_median": round(w.kv_bytes / (med * 1e-6) / 1e9, 1),
                "reps": int(times.size),
                "trivial_graph_median_us": round(float(np.median(tiny_times)), 2)}
        log(f"graph replay after a 1 GiB flush: median {cold['median_us']} us "
            f"(p10 {cold['p10_us']}, p90 {cold['p90_us']}, 95% CI {cold['median_ci95_us']}); "
            f"a one-kernel graph replays in {cold['trivial_graph_median_us']} us")
        del flush

    kv = w.kv_bytes
    timing_note = f"HIP events around each of {args.steps} eager launches"
    if w.L <= 8:
        # decode and verify read every visible key's 256 bytes once: HBM-bound
        value = kv / (ms_per_step * 1e-3) / 1e9
        unit, peak = "GB/s", HBM_PEAK_GBS
        metric = "us/step and achieved HBM GB/s (% peak), decode-32 full-attn ctx 80K, 1 GPU"
        achieved = kv / (attn_avg_ms * 1e-3) / 1e9
        traffic = read_traffic(kv) if w.L == 1 else None
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": peak,
                    "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic,
                    "kernel": "attn_kernel (q/k norm, cache write, split-K attention)",
                    "algorithmic_bytes_per_launch": kv,
                    "avg_launch_us": round(attn_avg_ms * 1e3, 2), "avg_launch_us_from": timing_note,
                    "mfma_busy": read_mfma_busy(args.config, w.attn_flops)}
    else:
        # a prefill block: 4 * 64 FLOPs per (visible key, token, query head), an
        # fp16 MFMA contraction; each key's bytes are reused by up to L tokens
        fl = w.attn_flops
        value = fl / (ms_per_step * 1e-3) / 1e12
        unit, peak = "TFLOP/s", MFMA_F16_PEAK_TFLOPS
        metric = "us/step and attention TFLOP/s (% of fp16 MFMA peak), prefill block, 1 GPU"
        achieved = fl / (attn_avg_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                    "unit": unit, "frac": round(achieved / peak, 4), "traffic": None,
                    "kernel": "attn_kernel (split-K causal block attention; the new rows are "
                              "written by rows_kernel before it)",
                    "algorithmic_flops_per_launch": fl,
                    "avg_launch_us": round(attn_avg_ms * 1e3, 2), "avg_launch_us_from": timing_note,
                    "mfma_busy": read_mfma_busy(args.config, fl)}

    probe = None
    if w.L <= 8 and w.layer_kind == 0 and not args.no_gather_probe:
        # the step's row gather alone (museattn_gather_probe: every visible
        # key's K and V rows through the table, the attention kernel's
        # concurrency, no arithmetic), timed like the attention kernel
        G = P.work_groups(w.B, w.L, w.max_seq_len, w.layer_kind, args.work_groups)
        chk = torch.empty(G, dtype=torch.int32, device=dev)
        for _ in range(3):
            P.gather_probe(d["table"], d["seq_lens"], kp, vp, w.page_size, w.max_seq_len, chk, G)
        torch.cuda.synchronize()
        pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for e0, e1 in pev:
            e0.record()
            P.gather_probe(d["table"], d["seq_lens"], kp, vp, w.page_size, w.max_seq_len, chk, G)
            e1.record()
        torch.cuda.synchronize()
        p_ms = sum(e0.elapsed_time(e1) for e0, e1 in pev) / len(pev)
        probe = {"kernel": "gather_probe_kernel (the step's K/V rows through the table, "
                           "no arithmetic)",
                 "bytes_per_launch": kv, "avg_launch_us": round(p_ms * 1e3, 2),
                 "gbs": round(kv / (p_ms * 1e-3) / 1e9, 1),
                 "frac_of_peak": round(kv / (p_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                 "attn_kernel_over_probe": round(attn_avg_ms / p_ms, 4),
                 "avg_launch_us_from": f"HIP events around each of {args.steps} eager launches"}
        log(f"gather probe: {probe['avg_launch_us']} us ({probe['gbs']} GB/s); attention kernel "
            f"/ probe = {probe['attn_kernel_over_probe']}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.config, args.pool_rows or None, args.cpu_sample,
                           args.cpu_sample_tokens, args.cpu_procs)

    line = {
        "metric": metric,
        "value": round(value, 2 if w.L > 8 else 1), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2), "timing": mode,
        "graph_warmup_steps": (max(1, -(-args.graph_warmup // args.steps)) * args.steps
                               if mode == "graph" else 0), "pct_peak": round(100 * value / peak, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "kv_dtype": "fp8_e4m3fn", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "L": w.L, "layer": "full" if w.layer_kind == 0
                   else "sliding", "page_size": w.page_size, "kv_scale": w.kv_scale,
                   "ctx_min": int(w.ctx.min()), "ctx_max": int(w.ctx.max()),
                   "ctx_mean": round(float(w.ctx.mean()), 1), "keys": int(kv // 256),
                   "kv_bytes": kv, "attn_flops": w.attn_flops, "pool_rows": w.num_rows,
                   "seed": w.seed,
                   "work_groups": P.work_groups(w.B, w.L, w.max_seq_len, w.layer_kind,
                                                args.work_groups),
                   "step_includes_oproj": bool(args.oproj)},
        "cold_cache_graph_replay": cold,
        "oproj": oproj,
        "roofline": roofline,
        "gather_probe": probe,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
