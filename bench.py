"""Benchmark: paged GQA decode (and prefill) attention on one MI355X.

One step is one pda_decode call (one launch of the split-KV attention kernel,
whose last item per head group merges the splits by log-sum-exp) over the
ragged batch-64 workload: 64 sequences, 32 q / 8 kv heads,
head_dim 128, block_size 16, contexts log-uniform in [128, 32768], 1 % of keys
scaled by 4, paged layout (workload "ragged-b64"; the other named workloads
run the same way, tiled ones as begin_step + step_tile per tile + finalize).  Inputs
are seeded synthetic bf16, resident in HBM before the timed region.

Timing protocol (every workload): the W warm-up steps asked for, then more
warm-up until the GPU runs at its steady rate (at least --min-warmup-ms of
steps, and two consecutive windows of >= 20 ms whose per-step times agree
within 2 %: after an idle period the first tens of milliseconds run up to
20 % slower while the clocks settle); then exactly K steps bracketed by
device synchronisations give `value` and `ms_per_step`; then 5 batches of
>= --batch-ms each (event-timed on the launch stream) give the median and
spread in `steady_state`.  `roofline.achieved` comes from the attention
kernel's own average duration: where the step launches that kernel alone
(pda_decode), the event pair around the K timed steps; where it launches
others too (begin_step, finalize), an event pair around each of its launches
in a further pass over K steps (that figure is also reported for pda_decode,
as `kernel_us_per_launch_event_bracketed`); `roofline.traffic` from the
committed counter summary when the kernel sources still match it.  A
workload whose K/V bytes would sit in the 256 MB last-level cache
(llama3-8b-b16) rotates over enough copies of its pool (>= 7, >= 1 GiB) that
every step reads from HBM.

A prefill workload ("prefill-2048", "prefill-chunk-b16") times one
pda_prefill call per step instead and reports TFLOP/s against the bf16 MFMA
peak (the kernel is bound by the matrix cores, not by HBM); its
`roofline.achieved` uses the event pair around the K timed steps (every
kernel of the step), the per-launch event pairs being reported beside it.  "rope-chunk-b16"
times the rotary step before prefill-chunk-b16's attention: pda_rope over the
chunk's q rows and pda_rope_append_kv of the chunk's new K/V rows into the
cache (HBM-bound).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--blocks-per-split N] [--no-cpu-baseline] [--no-kernel-events]
    python bench.py --copy-calibration [--copy-mib M]   (counter calibration copy)
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0      # MI355X HBM3E peak, GB/s
PEAK_MFMA_BF16_TFS = 2500.0   # MI355X dense bf16 matrix peak, TFLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="ragged-b64",
                    choices=["tiny", "llama3-8b-b16", "ragged-b64", "wide-head-d256", "scratch-b256",
                             "prefill-2048", "prefill-chunk-b16", "rope-chunk-b16"])
    ap.add_argument("--rows-per-wave", type=int, default=0, help="prefill: query rows per wave")
    ap.add_argument("--blocks-per-split", type=int, default=0)
    ap.add_argument("--min-warmup-ms", type=float, default=300.0,
                    help="warm up for at least this long (after the --warmup steps) and until the "
                         "per-step time is steady")
    ap.add_argument("--batch-ms", type=float, default=50.0,
                    help="length of each of the 5 steady-state batches")
    ap.add_argument("--rotate", type=int, default=-1,
                    help="pool copies to rotate over, one per step (-1: automatic, enough copies "
                         "for >= 1 GiB when the pool fits in the last-level cache; 0 or 1: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time the steps without the per-launch attention-kernel events")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (counter calibration)")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--mask-drop", type=float, default=None,
                    help="decode with pda_decode_masked and a seeded random keep-mask dropping "
                         "this fraction of positions (single-tile workloads)")
    ap.add_argument("--decode-via-prefill", action="store_true",
                    help="decode with pda_prefill at q_len 1 (the matrix-core P.V kernel, each kv "
                         "head's G q heads padded to 16 rows) instead of pda_decode (single-tile "
                         "workloads); --blocks-per-split sets its split size")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(w, min_seconds):
    """The fp64 oracle as it stands, on the host cores, over the whole workload
    (repeated until `min_seconds` have passed), in the metric's unit.  The
    small workloads (tiny, llama3-8b-b16) also get a one-thread figure."""
    import oracle
    threads = oracle.host_threads()

    def run(nthreads, seconds):
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.attend_workload(w, threads=nthreads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return el / reps, reps

    per, reps = run(threads, min_seconds)
    res = {"value": w.algorithmic_bytes() / per / 1e12, "unit": "TB/s", "cores": threads,
           "kind": "oracle", "us_per_call": per * 1e6, "cpu_model": cpu_model(),
           "sample": f"whole workload ({w.num_seqs * w.num_q_heads} (sequence, q head) pairs), "
                     f"{reps} repetition(s), fp64 C oracle with OpenMP"}
    if w.name in ("tiny", "llama3-8b-b16") and threads > 1:
        per1, reps1 = run(1, min_seconds / 2)
        res["single_core"] = {"value": w.algorithmic_bytes() / per1 / 1e12, "unit": "TB/s",
                              "us_per_call": per1 * 1e6, "repetitions": reps1}
    return res

def cpu_model():
    """The host CPU's model name (first processor in /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def measure(args, torch, stream, step):
    """Steady-state timing of `step` (one call = one step, enqueued on `stream`).

    1. the --warmup steps asked for;
    2. more warm-up in windows of >= 20 ms (event-timed) until at least
       --min-warmup-ms has passed and two consecutive windows agree within
       2 % per step (at most 5 s);
    3. exactly --steps steps bracketed by device synchronisations (wall
       clock; also an event pair on the stream);
    4. 5 batches of >= --batch-ms each, event-timed.
    Returns a dict of the figures (times in microseconds per step)."""
    sync = torch.cuda.synchronize
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed(n):
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(n):
            step()
        b.record(stream)
        sync()
        return a.elapsed_time(b) * 1e3 / n

    for _ in range(args.warmup):
        step()
    sync()
    t_est = timed(3)
    n_win = max(3, int(np.ceil(20e3 / max(t_est, 1.0))))
    extra, spent_us, prev, converged = 3, 3 * t_est, None, False
    while True:
        t = timed(n_win)
        extra += n_win
        spent_us += n_win * t
        if prev is not None and abs(t - prev) <= 0.02 * prev and spent_us >= args.min_warmup_ms * 1e3:
            converged = True
            break
        if spent_us >= 5e6:
            break
        prev = t
    log(f"warm-up: {args.warmup} + {extra} steps, {spent_us / 1e3:.0f} ms, last window {t:.1f} us/step")

    log(f"timing {args.steps} steps")
    e0, e1 = ev(), ev()
    sync()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    sync()
    wall_us = (time.perf_counter() - t0) * 1e6 / args.steps
    event_us = e0.elapsed_time(e1) * 1e3 / args.steps

    n_b = max(1, int(np.ceil(args.batch_ms * 1e3 / max(t, 1.0))))
    log(f"5 batches of {n_b} steps")
    batches = [timed(n_b) for _ in range(5)]
    med = float(np.median(batches))
    return {"wall_us": wall_us, "event_us": event_us, "warmup_extra_steps": extra,
            "warmup_ms": spent_us / 1e3, "warmup_converged": converged,
            "batch_steps": n_b, "batch_us": batches, "batch_median_us": med,
            "batch_spread_pct": 100.0 * (max(batches) - min(batches)) / med}


def steady_fields(m, per_step_amount, unit, scale):
    """The JSON fields of the warm-up and the 5 steady-state batches."""
    med = m["batch_median_us"]
    return {
        "warmup_extra_steps": m["warmup_extra_steps"],
        "warmup_ms": round(m["warmup_ms"], 1),
        "warmup_converged": m["warmup_converged"],
        "event_us_per_step": round(m["event_us"], 2),
        "steady_state": {"batches": 5, "steps_per_batch": m["batch_steps"],
                         "us_per_step_median": round(med, 2),
                         "us_per_step_min": round(min(m["batch_us"]), 2),
                         "us_per_step_max": round(max(m["batch_us"]), 2),
                         "spread_pct": round(m["batch_spread_pct"], 2),
                         "value_median": round(per_step_amount / (med * 1e-6) / scale, 4),
                         "unit": unit},
    }


# The sources each kernel's code and launch come from (a committed counter
# summary holds for the kernel only while these hash to its recorded value).
KERNEL_SOURCES = {
    "attend_kernel": ["pda_device.h", "pda_internal.h", "pda_attend.hip"],
    "prefill_kernel": ["pda_device.h", "pda_internal.h", "pda_prefill.hip"],
    "rope_kernel": ["pda_device.h", "pda_rope.h", "pda_rope.hip"],
}


def kernel_sources_sha256(kernel="attend_kernel"):
    """Hash of the HIP sources that decide the kernel and its launch."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_gqa_decode_pda_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def cpu_baseline_prefill(w, min_seconds, sample_rows=4096):
    """The fp64 oracle as it stands, on the host cores, over a seeded sample of
    the workload's (sequence, query, q head) rows (repeated until
    `min_seconds` have passed), as TFLOP/s of the sampled rows' own flops."""
    import oracle
    threads = oracle.host_threads()
    S, Q, Hq, D = w.qc.shape
    rng = np.random.Generator(np.random.PCG64(5))
    rows = np.sort(rng.choice(S * Q * Hq, size=min(sample_rows, S * Q * Hq), replace=False))
    keys = w.prefill_keys(True).reshape(-1)[rows // Hq]
    flops = int(keys.sum()) * 4 * D
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.prefill_workload(w, rows=rows, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    per = el / reps
    return {"value": flops / per / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "sample": f"{rows.size} seeded (sequence, query, q head) rows of {S * Q * Hq}, "
                      f"{reps} repetition(s), fp64 C oracle with OpenMP"}


def committed_traffic(workload_name, kernel="attend_kernel"):
    """HBM bytes per attention launch from the committed counter summary for
    this workload, or None when it is missing or the kernel sources changed
    since the counters were taken."""
    import re
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload_name}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text)
    val = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not sha or not val or sha.group(1) != kernel_sources_sha256(kernel):
        return None
    return int(val.group(1))


def copy_calibration(args):
    """A plain device-to-device copy of a known size, for scaling the HBM byte
    counters (run under rocprofv3 --pmc)."""
    import torch
    n = args.copy_mib << 20
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 5}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args)
        return
    import torch

    import workloads
    import paged_gqa_decode_pda_amd as pda

    log(f"generating workload {args.workload}")
    if args.workload == "rope-chunk-b16":
        main_rope(args, workloads.named("prefill-chunk-b16"), torch, pda, torch.device("cuda:0"))
        return
    w = workloads.named(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if w.is_prefill:
        main_prefill(args, w, torch, pda, dev)
        return
    b, c, v = w.stacked_tiles()
    T = len(w.tiles)
    dims = pda.pda_dims(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                        w.tile_capacity)
    q = torch.from_numpy(w.q.view(np.int16)).to(dev)
    pool = torch.from_numpy(w.pool.view(np.int16)).to(dev)
    tables = [torch.from_numpy(b[t]).to(dev) for t in range(T)]
    counts = [torch.from_numpy(c[t]).to(dev) for t in range(T)]
    lastv = [torch.from_numpy(v[t]).to(dev) for t in range(T)]
    bps = args.blocks_per_split
    ws = torch.zeros(pda.pda_workspace_bytes(dims, bps) // 4, dtype=torch.float32, device=dev)
    out = torch.empty(w.num_seqs, w.num_q_heads, w.head_dim, dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()
    S = w.num_seqs

    # Pool copies rotated one per step, so that a pool that fits in the
    # last-level cache (256 MB) is still read from HBM every step.
    pool_bytes = pool.numel() * 2
    ncopy = args.rotate
    if ncopy < 0:
        ncopy = max(7, -(-(1 << 30) // pool_bytes)) if (pool_bytes < (256 << 20) and w.name != "tiny") else 1
    ncopy = max(1, ncopy)
    pools = [pool] + [pool.clone() for _ in range(ncopy - 1)]
    bases = [(p.data_ptr() + 2 * w.k_base, p.data_ptr() + 2 * w.v_base) for p in pools]
    turn = [0]

    def kv():
        kp_, vp_ = bases[turn[0] % ncopy]
        turn[0] += 1
        return kp_, vp_

    if T == 1 and args.mask_drop is not None:
        api = f"pda_decode_masked (keep-mask dropping {args.mask_drop:.0%} of positions)"
        width = int(w.contexts.max()) + 1
        mrng = np.random.default_rng(7)
        kv_mask = torch.from_numpy((mrng.random((S, width)) >= args.mask_drop).astype(np.uint8)).to(dev)

        def step():
            kp, vp = kv()
            pda.pda_decode_masked(dims, q, kp, vp, tables[0], counts[0], lastv[0], w.block_size, S,
                                  w.strides, kv_mask, width, ws, out, bps, stream)
    elif T == 1 and args.decode_via_prefill:
        api = "pda_prefill (q_len 1)"
        pws_n = pda.pda_prefill_workspace_bytes(dims, 1, bps)
        pws = torch.empty(max(1, (pws_n + 3) // 4), dtype=torch.float32, device=dev) if pws_n else None

        def step():
            kp, vp = kv()
            pda.pda_prefill(dims, 1, q, kp, vp, tables[0], counts[0], lastv[0], w.block_size, S,
                            w.strides, True, None, 0, 0, pws, out, bps, 0, stream,
                            workspace_bytes=pws_n)
    elif T == 1:
        api = "pda_decode"

        def step():
            kp, vp = kv()
            pda.pda_decode(dims, q, kp, vp, tables[0], counts[0], lastv[0], w.block_size, S,
                           w.strides, ws, out, bps, stream)
    else:
        api = f"pda_begin_step + {T} x pda_step_tile + pda_finalize"
        state = torch.empty(pda.pda_state_bytes(dims) // 4, dtype=torch.float32, device=dev)
        plan = pda.pda_create(dims, state, ws, bps)

    # Per-launch events around the attention kernel (armed before every call
    # that launches it), created once and recorded once so that they exist.
    launches = T
    n_ev = 0 if args.no_kernel_events else args.steps * launches
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for e in ev_b + ev_a:
        e.record(stream)
    arm_iter = [None]

    def arm():
        if arm_iter[0] is not None:
            i = next(arm_iter[0])
            pda.pda_debug_time_attention(ev_b[i], ev_a[i])

    if T == 1:
        def step_timed():
            arm()
            step()
    else:
        def step_timed():
            kp, vp = kv()
            pda.pda_begin_step(plan, S, stream)
            for t in range(T):
                arm()
                pda.pda_step_tile(plan, q, kp, vp, tables[t], counts[t], lastv[t], w.block_size,
                                  S, w.strides, stream)
            pda.pda_finalize(plan, out, S, stream)
        step = step_timed   # arm() does nothing while no events are armed

    m = measure(args, torch, stream, step)
    if n_ev:
        # K more steps, with every attention launch bracketed by its own event
        # pair (recording them costs a few microseconds per step, so they stay
        # out of the regions above)
        log(f"timing {args.steps} steps with per-launch attention-kernel events")
        arm_iter[0] = iter(range(n_ev))
        for _ in range(args.steps):
            step_timed()
        torch.cuda.synchronize()
        arm_iter[0] = None
    nbytes = w.algorithmic_bytes()
    ms = m["wall_us"] / 1e3
    tbs = nbytes / (ms * 1e-3) / 1e12
    kernel_us = bracketed_us = None
    if n_ev:
        bracketed_us = sum(b.elapsed_time(a) for b, a in zip(ev_b, ev_a)) * 1e3 / n_ev
        kernel_us = bracketed_us
    name = ("prefill_kernel at q_len 1" if args.decode_via_prefill else
            "attend_kernel (paged split-KV attention)")
    how = "average over the timed launches, each bracketed by its own event pair"
    if n_ev and T == 1:
        # the step launches this one kernel and nothing else, so the event
        # pair around the timed region brackets its launches back to back
        # (an event pair around each launch adds a few microseconds to it)
        kernel_us = m["event_us"]
        how = "average over the timed region's back-to-back launches (the step's only kernel)"
    # the step's algorithmic bytes, spread evenly over its attention launches
    bytes_per_launch = nbytes / launches
    if kernel_us:
        achieved_gbs = bytes_per_launch / (kernel_us * 1e-6) / 1e9
        kernel_desc = f"{name}, {how}"
    else:
        achieved_gbs = nbytes / (m["event_us"] * 1e-6) / 1e9
        kernel_desc = f"{api} step (all launches)"
    traffic = committed_traffic(w.name) if (kernel_us and args.mask_drop is None
                                            and not args.decode_via_prefill) else None
    res = {
        "metric": "paged decode attention achieved HBM TB/s (K+V+q+out bytes per call / time)",
        "value": round(tbs, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_call": round(ms * 1e3, 2),
        "pct_of_peak": round(100 * tbs * 1e3 / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "total_tokens": w.total_tokens,
                   "algorithmic_bytes": nbytes, "layout": w.layout, "api": api,
                   "blocks_per_split": bps if args.decode_via_prefill else pda.pda_blocks_per_split(dims, bps),
                   "pool_copies_rotated": ncopy, "parallelism": "single GPU"},
    }
    res.update(steady_fields(m, nbytes, "TB/s", 1e12))
    res["roofline"] = {"bound": "hbm", "kernel": kernel_desc,
                       "achieved": round(achieved_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                       "frac": round(achieved_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                       "algorithmic_bytes_per_launch": int(bytes_per_launch),
                       "kernel_us_per_launch": round(kernel_us, 2) if kernel_us else None,
                       "kernel_us_per_launch_event_bracketed": round(bracketed_us, 2) if bracketed_us else None,
                       "launches_per_step": launches}
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle)")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def main_prefill(args, w, torch, pda, dev):
    """One step = one causal pda_prefill call over the workload's chunks."""
    b, c, v = w.stacked_tiles()
    S, Q, Hq, D = w.qc.shape
    dims = pda.pda_dims(S, Hq, w.num_kv_heads, D, w.block_size, w.tile_capacity)
    qc = torch.from_numpy(w.qc.view(np.int16)).to(dev)
    pool = torch.from_numpy(w.pool.view(np.int16)).to(dev)
    table, count, lastv = (torch.from_numpy(x[0]).to(dev) for x in (b, c, v))
    bps, rpw = args.blocks_per_split, args.rows_per_wave
    nb = pda.pda_prefill_workspace_bytes(dims, Q, bps)
    ws = torch.empty(max(1, (nb + 3) // 4), dtype=torch.float32, device=dev) if nb else None
    out = torch.empty(S, Q, Hq, D, dtype=torch.int16, device=dev)
    kp, vp = pool.data_ptr() + 2 * w.k_base, pool.data_ptr() + 2 * w.v_base
    stream = torch.cuda.current_stream()

    def step():
        pda.pda_prefill(dims, Q, qc, kp, vp, table, count, lastv, w.block_size, S, w.strides,
                        True, None, 0, 0, ws, out, bps, rpw, stream, workspace_bytes=nb)

    n_ev = 0 if args.no_kernel_events else args.steps
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for e in ev_b + ev_a:
        e.record(stream)
    m = measure(args, torch, stream, step)
    ms = m["wall_us"] / 1e3
    kernel_us = bracketed_us = None
    how = "average over the timed launches, each bracketed by its own event pair"
    if n_ev:
        log(f"timing {args.steps} steps with per-launch attention-kernel events")
        for i in range(n_ev):
            pda.pda_debug_time_attention(ev_b[i], ev_a[i])
            step()
        torch.cuda.synchronize()
        bracketed_us = sum(x.elapsed_time(y) for x, y in zip(ev_b, ev_a)) * 1e3 / n_ev
    # The kernel time is the timed region's back-to-back launches (event pair
    # around the region): the prefill kernel, plus the merge kernel when the
    # library splits the KV (conservative then).  Event pairs around each
    # launch time this kernel 10-30 us longer than back-to-back launches run
    # (it re-reads every K/V row from the L2 32 times; the decode kernel,
    # which streams, shows no such gap), so they are reported beside it only.
    kernel_us = m["event_us"]
    how = "average over the timed region's back-to-back launches (every kernel of the step)"
    flops = w.prefill_flops(True)
    tfs = flops / (ms * 1e-3) / 1e12
    achieved = flops / ((kernel_us if kernel_us else ms * 1e3) * 1e-6) / 1e12
    res = {
        "metric": "paged GQA prefill attention achieved TFLOP/s (causal q.K^T and P.V flops / time)",
        "value": round(tfs, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_call": round(ms * 1e3, 2),
        "pct_of_peak": round(100 * tfs / PEAK_MFMA_BF16_TFS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": S, "q_len": Q, "num_q_heads": Hq,
                   "num_kv_heads": w.num_kv_heads, "head_dim": D, "block_size": w.block_size,
                   "total_tokens": w.total_tokens, "causal": True, "algorithmic_flops": flops,
                   "algorithmic_bytes": w.prefill_bytes(), "layout": w.layout, "api": "pda_prefill",
                   "blocks_per_split": bps, "rows_per_wave": rpw, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma",
                     "kernel": f"prefill_kernel (paged MFMA chunk attention), {how}" if kernel_us
                               else "pda_prefill step (all launches)",
                     "achieved": round(achieved, 2), "peak": PEAK_MFMA_BF16_TFS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_MFMA_BF16_TFS, 4),
                     "traffic": committed_traffic(w.name, "prefill_kernel") if kernel_us else None,
                     "algorithmic_flops_per_launch": flops,
                     "kernel_us_per_launch": round(kernel_us, 2) if kernel_us else None,
                     "kernel_us_per_launch_event_bracketed": round(bracketed_us, 2) if bracketed_us else None,
                     "launches_per_step": 1},
    }
    res.update(steady_fields(m, flops, "TFLOP/s", 1e12))
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle, sampled rows)")
        res["cpu_baseline"] = cpu_baseline_prefill(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def main_rope(args, w, torch, pda, dev):
    """One step = pda_rope over the chunk's q rows (into a second buffer) and
    pda_rope_append_kv of one new K row and V row per (chunk token, kv head)
    at the chunk tokens' positions P - q_len + i."""
    import oracle
    S, Q, Hq, D = w.qc.shape
    Hkv, bs = w.num_kv_heads, w.block_size
    T = S * Q
    P = 8192
    ct, st = oracle.rope_tables(P, D)
    pos = (w.contexts[:, None] - Q + np.arange(Q)[None, :]).astype(np.int32).reshape(-1)
    seq = np.repeat(np.arange(S, dtype=np.int32), Q)
    rng = np.random.Generator(np.random.PCG64(9))
    kv = torch.from_numpy(workloads_bits(rng, (2, T, Hkv, D)).view(np.int16)).to(dev)
    qc = torch.from_numpy(w.qc.view(np.int16)).to(dev)
    qo = torch.empty_like(qc)
    pool = torch.from_numpy(w.pool.view(np.int16)).to(dev)
    b, _, _ = w.stacked_tiles()
    table = torch.from_numpy(b[0]).to(dev)
    cd, sd = torch.from_numpy(ct).to(dev), torch.from_numpy(st).to(dev)
    pd, sqd = torch.from_numpy(pos).to(dev), torch.from_numpy(seq).to(dev)
    dims = pda.pda_dims(S, Hq, Hkv, D, bs, w.tile_capacity)
    kp, vp = pool.data_ptr() + 2 * w.k_base, pool.data_ptr() + 2 * w.v_base
    stream = torch.cuda.current_stream()

    def rope_q():
        pda.pda_rope(qc, qo, T, Hq, D, cd, sd, P, pd, stream)

    def step():
        rope_q()
        pda.pda_rope_append_kv(dims, kv[0], kv[1], T, sqd, pd, cd, sd, P, table, kp, vp, w.strides,
                               stream)

    m = measure(args, torch, stream, step)
    ms = m["wall_us"] / 1e3
    # the rope kernel alone (one launch per pda_rope call), events on its stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record(stream)
        rope_q()
        e1.record(stream)
    torch.cuda.synchronize()
    rope_us = sum(e0.elapsed_time(e1) for e0, e1 in evs) * 1e3 / len(evs)
    tbl = 2 * 4 * (D // 2)                       # one cos and one sin row per token
    q_bytes = 2 * T * Hq * D * 2 + T * (tbl + 4)
    kv_bytes = 4 * T * Hkv * D * 2 + T * (tbl + 12)
    nbytes = q_bytes + kv_bytes
    tbs = nbytes / (ms * 1e-3) / 1e12
    achieved = q_bytes / (rope_us * 1e-6) / 1e9
    res = {
        "metric": "rotary embedding (q rows + K/V append into the paged cache) achieved HBM TB/s",
        "value": round(tbs, 4), "unit": "TB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "us_per_call": round(ms * 1e3, 2),
        "pct_of_peak": round(100 * tbs * 1e3 / PEAK_HBM_GBS, 2), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "rope-chunk-b16", "tokens": T, "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": D, "block_size": bs, "max_positions": P,
                   "algorithmic_bytes": nbytes, "api": "pda_rope + pda_rope_append_kv",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "rope_kernel (q rows), average over event-timed launches",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": committed_traffic("rope-chunk-b16", "rope_kernel"),
                     "algorithmic_bytes_per_launch": q_bytes,
                     "kernel_us_per_launch": round(rope_us, 2), "launches_per_step": 2},
    }
    res.update(steady_fields(m, nbytes, "TB/s", 1e12))
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle)")
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.rope(w.qc.reshape(T, Hq, D), ct, st, pos)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        res["cpu_baseline"] = {"value": q_bytes / (el / reps) / 1e12, "unit": "TB/s", "cores": 1,
                               "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": f"q rows of the whole step ({T} tokens x {Hq} heads), "
                                         f"{reps} repetition(s), fp64 C oracle, one thread"}
    print(json.dumps(res), flush=True)


def workloads_bits(rng, shape):
    from workloads import f32_to_bf16_bits
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


if __name__ == "__main__":
    main()
