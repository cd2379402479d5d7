#!/usr/bin/env python3
"""Throughput of the draft-KV ring step on one MI355X.

A step is one pass of the whole ring path for one sequence: the fold-in
(append with RoPE at absolute positions, slot_pos, window mask, noise RoPE
table) and ring_attn (masked GQA attention of the 8 noise queries over the
4096-slot ring, split-K + merge).  By default the fold-in is handed to the
attention launch (ring_begin_step_deferred, then ring_attn: one attention
launch that appends the new rows, writes their slot_pos entries and attends,
then the merge; the masks and noise RoPE table, which that launch does not
read, are rebuilt only when a plain launch or a read needs them);
--step eager gives it a launch of its own (ring_begin_step).  On a ring of
several sequences (batched_seqs) a step is one ring_begin_step_deferred per
sequence, then one ring_attn per layer (--step eager: one
ring_begin_step_batch over all of them, then the ring_attn launches).
Workload: the draft-window decode stream (cap 4096, q_len 8, 32 query / 8 KV
heads x 128, F16), warmed by a 4096-token bulk prefill; synthetic seeded
inputs, already resident in device memory when timing starts.

The timed steps cycle through a pool of independent rings (default 32, about
680 MB) so that every step reads its ring from HBM, not from the 256 MB
Infinity Cache; ``--pool 1`` gives the cache-warm figure.

Prints one JSON line.  ``value`` comes from the timed steps alone.
``roofline`` is for the attention kernel, whose duration comes from HIP events
bound to its own dispatches over an equal segment of the same stream run right
after the timed steps (such events add several microseconds per launch to
back-to-back dispatch, so they are kept out of the timed steps);
``cpu_baseline`` times the CPU oracle on a bounded sample of the same stream.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "ring_attn steps/s + achieved HBM GB/s (% peak), cap=4096, q_len=8, GQA 32/8x128"
RMS_EPS = 1e-6   # epsilon of the K norm of rows projected from features
HBM_PEAK_GBS = 8000.0
WORKLOAD = "decode_stream"


def algorithmic_bytes(w, win: int, kv_total: int) -> dict:
    """Bytes one attention call must move at minimum (per sequence)."""
    kv = (win + w.q_len) * w.kv_row * 2 * 2          # visible K and V rows, F16
    q = w.q_len * w.n_head * w.head_dim * 2          # queries, F16
    noise = 2 * w.q_len * w.kv_row * 2               # noise K and V inputs, F16
    mask = w.q_len * kv_total * 2                    # F16 mask
    out = w.q_len * w.n_head * w.head_dim * 4        # F32 output
    return {"kv": kv, "q": q, "noise": noise, "mask": mask, "out": out,
            "attn_kernel": kv + q + noise + mask, "ring_attn": kv + q + noise + mask + out}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("ring_kernels.hip", "ring_kernels.h", "ring_layout.h"):
        with open(os.path.join(ROOT, "draft_model_kv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_hash: str):
    """HBM bytes per attention launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "ring_attn_decode_stream_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_hash:
        return None
    return t.get("hbm_bytes_per_launch")


def _oracle_steps(w, seconds: float):
    """Steps of the decode stream through the oracle for about `seconds` of
    CPU time: (steps, seconds), inputs generated outside the timed part."""
    import numpy as np
    import oracle.ring_oracle as ro
    import workload as W
    geo = ro.geometry(w.cap, w.q_len, w.head_dim, w.n_head_kv)
    st = ro.RingStep(geo, 1, w.n_head_kv, w.head_dim, w.rope_base)
    stream = W.commit_stream(w, 0)
    p = st.plan(stream[0])
    pos = np.arange(p.start, stream[0])
    st.commit(p, [W.context_rows(w, 0, 0, W.T_K, pos)], [W.context_rows(w, 0, 0, W.T_V, pos)])
    n_steps, t_total = 0, 0.0
    for j in range(1, len(stream)):
        c = stream[j]
        p = st.plan(c)
        pos = np.arange(p.start, c)
        k = W.context_rows(w, 0, 0, W.T_K, pos)
        v = W.context_rows(w, 0, 0, W.T_V, pos)
        q, kn, vn = W.noise_inputs(w, 0, 0, j)
        t0 = time.perf_counter()
        st.commit(p, [k], [v])
        ro.attend(st.caches[0], c, w.cap, q, kn, vn, w.n_head, dtype=np.float32)
        t_total += time.perf_counter() - t0
        n_steps += 1
        if t_total >= seconds and n_steps >= 5:
            break
    return n_steps, t_total


def cpu_baseline(w, seconds: float) -> dict:
    """The oracle (full cache, fp32-accumulated attention) on the host cores,
    with numpy's own thread count and with one thread."""
    avail = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except ImportError:
        threadpool_limits, blas = None, 1
    n, t = _oracle_steps(w, seconds)
    one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            n1, t1 = _oracle_steps(w, seconds / 2)
        one = {"value": n1 / t1, "steps": n1, "seconds": round(t1, 2)}
    return {"value": n / t, "unit": "steps/s", "cores": int(min(blas, avail)), "kind": "oracle",
            "cores_available": avail, "blas_threads": int(blas),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "one_thread": one,
            "sample": f"{n} decode steps of the cap-4096 stream after a 4096-row prefill "
                      f"(store new rows with fp64 RoPE + fp32 attention), {t:.1f} s; the "
                      f"attention's matrix products run on numpy's BLAS threads ({blas}), "
                      f"the rest of the oracle on one"}


def prepare(w, pool: int, total: int, dev, extra0: int = 0, proj: str = "registered",
            workspace: str = "torch"):
    """Rings of workload ``w`` warmed up, and the device-resident inputs of
    ``total`` steps cycled over ``pool`` rings, plus ``extra0`` further steps
    of ring 0 alone (fewer if its stream ends first).  Returns (rings, calls,
    (steps_in, extra), committed, calls0), calls[t] = (handle, [(seq,
    committed, k, v, n)...], [(layer, q, kn, vn)...], weights) and calls0 the
    further steps of ring 0 in the same form."""
    import numpy as np
    import torch
    import workload as W
    import draft_model_kv_amd as R

    streams = [W.commit_stream(w, s_) for s_ in range(w.n_seq)]
    n_warm = W.n_warmup_steps(w)
    n_used0 = -(-total // pool)          # steps ring 0 takes in the cycled calls
    n_dec = min(n_used0 + extra0, len(streams[0]) - n_warm)
    if n_used0 + n_warm > len(streams[0]):
        raise SystemExit(f"need {n_dec} decode steps per ring, stream has {len(streams[0]) - n_warm}")
    rings = [R.Ring(cap=w.cap, q_len=w.q_len, n_head=w.n_head, n_head_kv=w.n_head_kv,
                    head_dim=w.head_dim, n_layer=w.n_layer, n_seq=w.n_seq,
                    rope_base=w.rope_base, device=dev, swa_window=w.swa_window,
                    swa_layers=w.swa_layers, d_model=w.d_model, workspace=workspace)
             for _ in range(pool)]
    s = torch.cuda.current_stream(dev).cuda_stream
    mirror = w.d_model > 0
    if mirror:
        # one copy of the projection weights per ring of the pool, so that a
        # step reads its weights from HBM as it would in a decode where the
        # target model runs between draft steps
        wk, wv, kn = W.projection_weights(w)
        weights = [(torch.from_numpy(wk).to(dev), torch.from_numpy(wv).to(dev),
                    torch.from_numpy(kn).to(dev)) for _ in range(pool)]
        wptrs = [(a.data_ptr(), b.data_ptr(), c.data_ptr(), RMS_EPS) for a, b, c in weights]
        if proj == "registered":
            # each ring keeps its own packed copy in its workspace
            for r, wp in zip(rings, wptrs):
                R.ring_set_kv_weights(r.handle, *wp, s)
            torch.cuda.synchronize(dev)
            weights, wptrs = None, [None] * pool

    def feats(seq, lo, hi):
        return torch.from_numpy(W.fused_features(w, seq, np.arange(lo, hi))).to(dev)

    def rows(seq, lo, hi):
        pos = np.arange(lo, hi)
        k = np.stack([W.context_rows(w, seq, l, W.T_K, pos) for l in range(w.n_layer)])
        v = np.stack([W.context_rows(w, seq, l, W.T_V, pos) for l in range(w.n_layer)])
        return torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev), len(pos)

    # warm-up (prefill): the same rows go to every ring of the pool
    prev = [0] * w.n_seq
    for t in range(n_warm):
        for seq in range(w.n_seq):
            c = streams[seq][t]
            plan, _ = rings[0].plan(seq, c)
            if mirror:
                f = feats(seq, prev[seq], c)
                for r, wp in zip(rings, wptrs):
                    R.ring_mirror_write(r.handle, seq, prev[seq], c - prev[seq], f.data_ptr(), s)
                    if wp is None:
                        R.ring_begin_step_mirror_registered(r.handle, seq, c, s)
                    else:
                        R.ring_begin_step_mirror(r.handle, seq, c, *wp, s)
                torch.cuda.synchronize(dev)
                prev[seq] = c
                del f
                continue
            k, v, n = rows(seq, plan.start, c)
            for r in rings:
                R.ring_begin_step(r.handle, seq, c, k.data_ptr(), v.data_ptr(), n, s)
            torch.cuda.synchronize(dev)
            prev[seq] = c
            del k, v

    steps_in = []
    for j in range(n_dec):
        seqs = []
        for seq in range(w.n_seq):
            c0, c = streams[seq][n_warm + j - 1], streams[seq][n_warm + j]
            if mirror:
                # the features of the newly committed positions (the mirror
                # write is part of the step), no K/V rows
                seqs.append((seq, c, feats(seq, c0, c), c0, c - c0))
                continue
            k, v, n = rows(seq, c0, c)
            seqs.append((seq, c, k, v, n))
        layers = []
        for layer in range(w.n_layer):
            qs, ks, vs = zip(*(W.noise_inputs(w, seq, layer, j) for seq in range(w.n_seq)))
            layers.append((layer, torch.from_numpy(np.stack(qs)).to(dev),
                           torch.from_numpy(np.stack(ks)).to(dev),
                           torch.from_numpy(np.stack(vs)).to(dev)))
        steps_in.append((seqs, layers))
    def call(r_i, j):
        seqs, layers = steps_in[j]
        if mirror:
            sq = [(seq, c, f.data_ptr(), c0, n) for seq, c, f, c0, n in seqs]
        else:
            sq = [(seq, c, k.data_ptr(), v.data_ptr(), n) for seq, c, k, v, n in seqs]
        return (rings[r_i].handle, sq,
                [(layer, q.data_ptr(), kn.data_ptr(), vn.data_ptr()) for layer, q, kn, vn in layers],
                wptrs[r_i] if mirror else None)

    calls = [call(t % pool, t // pool) for t in range(total)]
    calls0 = [call(0, j) for j in range(n_used0, n_dec)]
    committed = [[streams[seq][n_warm + t // pool] for seq in range(w.n_seq)]
                 for t in range(total)]
    extra = weights if mirror else None
    return rings, calls, (steps_in, extra), committed, calls0


# The rocprofv3 runs behind the committed summaries under profiles/, each run
# from /tmp (TMPDIR=/tmp) with REPO the repository root and OUT an output
# directory; `python bench.py --summarize OUT` then writes the summaries.
PROFILE_RUNS = {
    "prof_ktrace": "rocprofv3 --kernel-trace --stats --output-format csv -d OUT/prof_ktrace -o run "
                   "-- python REPO/bench.py --steps 1000 --warmup 100 --no-cpu-baseline "
                   "--floor-launches 0",
    # the floors of the decode stream's attention launch (ring_profile_floor)
    "prof_ktrace_floor": "rocprofv3 --kernel-trace --stats --output-format csv -d "
                         "OUT/prof_ktrace_floor -o run -- python REPO/bench.py --floor "
                         "--floor-launches 400 --warmup 100",
    "bench_floor": "python REPO/bench.py --floor --floor-launches 400 --warmup 100",
    # the step captured in HIP graphs and replayed, against plain launches
    "bench_graph": "python REPO/bench.py --graph --warmup 50",
    "pmc_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/pmc_fetch -o run "
                 "-- python REPO/bench.py --steps 64 --warmup 16 --no-cpu-baseline --floor-launches 0",
    "pmc_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/pmc_write -o run "
                 "-- python REPO/bench.py --steps 64 --warmup 16 --no-cpu-baseline --floor-launches 0",
    "pmc_copy_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/pmc_copy_fetch -o run "
                      "-- python REPO/bench.py --calibrate-copy 1024",
    "pmc_copy_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/pmc_copy_write -o run "
                      "-- python REPO/bench.py --calibrate-copy 1024",
    # the same bench without the profiler (its HIP-event kernel times are
    # compared with the trace; the tracer itself slows event-bound dispatches)
    "bench_plain": "python REPO/bench.py --steps 1000 --warmup 100 --no-cpu-baseline "
                   "--floor-launches 0",
    # rows from the feature mirror: the projection kernel
    "prof_ktrace_mirror": "rocprofv3 --kernel-trace --stats --output-format csv -d "
                          "OUT/prof_ktrace_mirror -o run -- python REPO/bench.py --workload "
                          "mirror_stream --steps 300 --warmup 30 --no-cpu-baseline",
    "pmc_fetch_mirror": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/pmc_fetch_mirror "
                        "-o run -- python REPO/bench.py --workload mirror_stream --steps 32 "
                        "--warmup 8 --no-cpu-baseline",
    "pmc_write_mirror": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/pmc_write_mirror "
                        "-o run -- python REPO/bench.py --workload mirror_stream --steps 32 "
                        "--warmup 8 --no-cpu-baseline",
    "bench_plain_mirror": "python REPO/bench.py --workload mirror_stream --steps 300 --warmup 30 "
                          "--no-cpu-baseline",
}
# the attention on the wider workloads (16 rings; one 32768-slot ring with
# two query blocks per KV head)
WIDE_WORKLOADS = ("batched_seqs", "large_window")
for _wl in WIDE_WORKLOADS:
    PROFILE_RUNS[f"bench_plain_{_wl}"] = (f"python REPO/bench.py --workload {_wl} --steps 200 "
                                          "--warmup 20 --no-cpu-baseline --floor-launches 60")
    PROFILE_RUNS[f"prof_ktrace_{_wl}"] = (f"rocprofv3 --kernel-trace --stats --output-format csv -d "
                                          f"OUT/prof_ktrace_{_wl} -o run -- python REPO/bench.py "
                                          f"--workload {_wl} --steps 200 --warmup 20 --no-cpu-baseline "
                                          "--floor-launches 0")
    for _c in ("fetch", "write"):
        PROFILE_RUNS[f"pmc_{_c}_{_wl}"] = (f"rocprofv3 --pmc {_c.upper()}_SIZE --output-format csv "
                                           f"-d OUT/pmc_{_c}_{_wl} -o run -- python REPO/bench.py "
                                           f"--workload {_wl} --steps 16 --warmup 4 --no-cpu-baseline "
                                           "--floor-launches 0")
# hardware counters of the decode stream's kernels and of the read floor
# on the same grid, one pass per group (at most 8 SQ, 4 TCP, 4 TCC and 2 TA
# counters per pass)
COUNTER_PASSES = {
    "pmc_sq_a": ("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY",
                 "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_VALU",
                 "SQ_ACTIVE_INST_LDS"),
    "pmc_sq_b": ("SQ_INSTS_VMEM_RD", "SQ_INSTS_SALU", "SQ_INSTS_VALU", "SQ_INSTS_LDS",
                 "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_IFETCH", "SQ_ACTIVE_INST_SCA",
                 "SQ_WAIT_INST_LDS"),
    "pmc_tc_a": ("TCP_TCC_READ_REQ", "TCP_TCC_READ_REQ_LATENCY", "TCC_HIT", "TCC_MISS"),
    "pmc_tc_b": ("TCP_PENDING_STALL_CYCLES", "TA_ADDR_STALLED_BY_TC_CYCLES",
                 "TA_DATA_STALLED_BY_TC_CYCLES"),
}
for _run, _ctrs in COUNTER_PASSES.items():
    PROFILE_RUNS[_run] = (f"rocprofv3 --pmc {' '.join(_ctrs)} --output-format csv -d OUT/{_run} "
                          "-o run -- python REPO/bench.py --steps 64 --warmup 16 --no-cpu-baseline "
                          "--floor-launches 64")
CALIBRATE_COPY_MIB = 1024
KERNELS = ("k_ring_attn", "k_ring_step", "k_ring_merge")
KERNELS_MIRROR = ("k_ring_project", "k_ring_step", "k_ring_attn", "k_ring_merge")


def _csv_rows(out_dir: str, run: str, kind: str):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(out_dir, run, "**", f"*{kind}.csv"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *{kind}.csv under {os.path.join(out_dir, run)}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _kib_per_dispatch(out_dir: str, run: str, counter: str, pick, grid=None) -> tuple:
    vals = [float(r["Counter_Value"]) for r in _csv_rows(out_dir, run, "counter_collection")
            if r["Counter_Name"] == counter and pick(r["Kernel_Name"])
            and (grid is None or int(r["Grid_Size"]) == grid)]
    if not vals:
        raise ValueError(f"{run}: no {counter} values for the kernel")
    return sum(vals) / len(vals), len(vals)


def _bench_line(out_dir: str, run: str):
    path = os.path.join(out_dir, run + ".log")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for ln in fh:
            ln = ln.strip()
            if ln.startswith("{") and '"metric"' in ln:
                return json.loads(ln)
    return None


def trace_timeline(out_dir: str, run: str, steps: int) -> dict:
    """Per-dispatch timestamps of the kernel trace: the first `steps`
    consecutive attention dispatches after the clock warm-up's fill kernels
    (the timed steps), each followed by its merge.  Medians in us of the
    attention and merge durations, the gaps between them and the period from
    one attention start to the next."""
    import statistics as stt
    rows = sorted(_csv_rows(out_dir, run, "kernel_trace"), key=lambda r: int(r["Start_Timestamp"]))
    last_fill = max((i for i, r in enumerate(rows) if "Fill" in r["Kernel_Name"]
                     and "rocclr" not in r["Kernel_Name"]), default=-1)
    seq = [r for r in rows[last_fill + 1:] if "k_ring_attn" in r["Kernel_Name"]
           or "k_ring_merge" in r["Kernel_Name"] or "k_ring_step" in r["Kernel_Name"]]
    attn = [i for i, r in enumerate(seq) if "k_ring_attn" in r["Kernel_Name"]][:steps]
    if len(attn) < 3:
        return {}
    t = lambda r, k: int(r[k]) / 1e3  # noqa: E731  ns -> us
    dur_a, dur_m, gap_am, gap_ma, period = [], [], [], [], []
    for j, i in enumerate(attn):
        a = seq[i]
        dur_a.append(t(a, "End_Timestamp") - t(a, "Start_Timestamp"))
        if i + 1 < len(seq) and "k_ring_merge" in seq[i + 1]["Kernel_Name"]:
            m = seq[i + 1]
            dur_m.append(t(m, "End_Timestamp") - t(m, "Start_Timestamp"))
            gap_am.append(t(m, "Start_Timestamp") - t(a, "End_Timestamp"))
            if j + 1 < len(attn):
                gap_ma.append(t(seq[attn[j + 1]], "Start_Timestamp") - t(m, "End_Timestamp"))
        if j + 1 < len(attn):
            period.append(t(seq[attn[j + 1]], "Start_Timestamp") - t(a, "Start_Timestamp"))
    med = lambda v: round(stt.median(v), 3) if v else None  # noqa: E731
    return {"steps": len(attn), "period_us": med(period), "attn_us": med(dur_a),
            "merge_us": med(dur_m), "gap_attn_to_merge_us": med(gap_am),
            "gap_merge_to_next_us": med(gap_ma)}


def summarize_profiles(out_dir: str) -> int:
    """Write profiles/*.md and the traffic JSON from the rocprofv3 CSV output
    of PROFILE_RUNS (and each run's stdout in OUT/<run>.log when present)."""
    khash = kernel_source_hash()
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    wl = "decode_stream (cap 4096, q_len 8, GQA 32/8 x 128, F16, 1 layer, 32-ring pool)"
    cmd = lambda run: PROFILE_RUNS[run]  # noqa: E731

    # kernel trace
    stats = _csv_rows(out_dir, "prof_ktrace", "kernel_stats")
    bl = _bench_line(out_dir, "bench_plain")
    lines = [f"# Kernel trace: k_ring_attn and the ring step kernels, {wl}", "",
             f"Kernel source hash: `{khash}`", "", "Command (cd /tmp; TMPDIR=/tmp):", "",
             f"    {cmd('prof_ktrace')}", "",
             "| kernel | calls | avg us | min us | max us | share of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    trace = {}
    for r in stats:
        name = r["Name"]
        short = next((k for k in KERNELS if k in name), None)
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f}% |")
        if short:
            trace[short] = float(r["AverageNs"]) / 1e3
    tl = trace_timeline(out_dir, "prof_ktrace", 1000)
    if tl:
        lines += ["", f"Timed steps in this trace (median over {tl['steps']} steps, per-dispatch "
                  f"start and end timestamps): one step every {tl['period_us']} us = attention "
                  f"{tl['attn_us']} us + gap {tl['gap_attn_to_merge_us']} us + merge "
                  f"{tl['merge_us']} us + gap {tl['gap_merge_to_next_us']} us to the next "
                  "attention.  The dispatches do not overlap (each duration runs from the "
                  "kernel's start to its end).  The tracer slows the host's submission, so "
                  "here the device waits for the next step (the last gap); without it the "
                  "step is device-bound (below)."]
    if bl:
        ev = {k: v["avg_us"] for k, v in bl.get("kernels", {}).items()}
        lines += ["", "The same bench without the profiler (" + f"`{cmd('bench_plain')}`" + "), "
                  "HIP events bound to the dispatches of its profiled segment: "
                  + ", ".join(f"{k} {v:.2f} us" for k, v in ev.items() if v)
                  + f"; {bl['value']:.0f} steps/s in its timed segment "
                  f"({1e3 * bl['ms_per_step']:.2f} us per step)."]
    with open(os.path.join(prof, "k_ring_attn_decode_stream_kernel_trace.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")

    # HBM traffic from FETCH_SIZE / WRITE_SIZE, scaled by a plain copy
    copy_bytes = CALIBRATE_COPY_MIB << 20
    cf, ncf = _kib_per_dispatch(out_dir, "pmc_copy_fetch", "FETCH_SIZE", lambda n: "copyBuffer" in n)
    cw, ncw = _kib_per_dispatch(out_dir, "pmc_copy_write", "WRITE_SIZE", lambda n: "copyBuffer" in n)
    fetch_scale = copy_bytes / (cf * 1024)
    write_scale = copy_bytes / (cw * 1024)
    rows = {}
    for k in KERNELS:
        f, nf = _kib_per_dispatch(out_dir, "pmc_fetch", "FETCH_SIZE", lambda n, k=k: k in n)
        w, nw = _kib_per_dispatch(out_dir, "pmc_write", "WRITE_SIZE", lambda n, k=k: k in n)
        rows[k] = {"fetch_kib": f, "write_kib": w, "dispatches": min(nf, nw),
                   "hbm_bytes": f * 1024 * fetch_scale + w * 1024 * write_scale}
    import workload as W
    w_ = W.WORKLOADS[WORKLOAD]
    alg = algorithmic_bytes(w_, w_.cap, 0)
    alg_attn = alg["kv"] + alg["q"] + alg["noise"] + w_.q_len * (w_.cap + 2 * w_.q_len) * 2
    t = {"kernel_source_hash": khash, "workload": WORKLOAD,
         "fetch_scale": fetch_scale, "write_scale": write_scale,
         "copy_calibration": {"bytes": copy_bytes, "fetch_kib": cf, "write_kib": cw,
                              "dispatches": [ncf, ncw]},
         "kernels": rows, "hbm_bytes_per_launch": rows["k_ring_attn"]["hbm_bytes"],
         "trace_avg_us": trace.get("k_ring_attn"), "trace_timeline": tl,
         "commands": {k: PROFILE_RUNS[k] for k in ("pmc_fetch", "pmc_write", "pmc_copy_fetch",
                                                  "pmc_copy_write")}}
    with open(os.path.join(prof, "ring_attn_decode_stream_traffic.json"), "w") as fh:
        json.dump(t, fh, indent=1)
        fh.write("\n")
    a = rows["k_ring_attn"]
    lines = [f"# HBM traffic per dispatch: k_ring_attn and the ring step kernels, {wl}", "",
             f"Kernel source hash: `{khash}`", "", "Commands (cd /tmp; TMPDIR=/tmp), one counter per run:", ""]
    lines += [f"    {cmd(r)}" for r in ("pmc_fetch", "pmc_write", "pmc_copy_fetch", "pmc_copy_write")]
    lines += ["", f"Calibration: a plain {CALIBRATE_COPY_MIB} MiB device copy reads FETCH_SIZE "
              f"{cf:.0f} KiB and WRITE_SIZE {cw:.0f} KiB per dispatch, so FETCH_SIZE is scaled by "
              f"{fetch_scale:.3f} and WRITE_SIZE by {write_scale:.3f}.", "",
              "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled HBM MB |",
              "|---|---:|---:|---:|---:|"]
    for k, r in rows.items():
        lines.append(f"| {k} | {r['dispatches']} | {r['fetch_kib']:.1f} | {r['write_kib']:.1f} | "
                     f"{r['hbm_bytes'] / 1e6:.3f} |")
    step = (bl or {}).get("config", {}).get("step", "eager")
    if step == "fused":
        # the bench line's bytes of the fused launch (it also reads the new
        # rows and slot_pos, and writes the rows and their slot_pos entries)
        alg_attn = bl["roofline"]["bytes_per_launch"]
        what = "visible K/V rows, queries, noise rows, the step's new rows, slot_pos"
        wrote = ("split partials, the noise and new rows stored to the ring, the new rows' "
                 "slot_pos entries")
    else:
        what = "visible K/V rows, queries, noise rows, mask"
        wrote = "split partials and the noise rows stored to the ring"
    lines += ["", f"k_ring_attn ({step} step): scaled reads "
              f"{a['fetch_kib'] * 1024 * fetch_scale / 1e6:.3f} MB per launch against "
              f"{alg_attn / 1e6:.3f} MB of algorithmic bytes ({what}); writes "
              f"{a['write_kib'] * 1024 * write_scale / 1e6:.3f} MB ({wrote})."]
    if "k_ring_attn" in trace:
        lines.append(f"Average k_ring_attn duration in the kernel trace: {trace['k_ring_attn']:.2f} us.")
    with open(os.path.join(prof, "k_ring_attn_decode_stream_hbm_traffic.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    written = ["profiles/k_ring_attn_decode_stream_kernel_trace.md",
               "profiles/k_ring_attn_decode_stream_hbm_traffic.md",
               "profiles/ring_attn_decode_stream_traffic.json"]
    if os.path.isdir(os.path.join(out_dir, "prof_ktrace_mirror")):
        written += summarize_mirror(out_dir, khash, fetch_scale, write_scale)
    for wl_name in WIDE_WORKLOADS:
        if os.path.isdir(os.path.join(out_dir, f"prof_ktrace_{wl_name}")):
            written.append(summarize_wide(out_dir, wl_name, khash, fetch_scale, write_scale))
    if os.path.isdir(os.path.join(out_dir, "prof_ktrace_floor")):
        written.append(summarize_floor(out_dir, khash))
    if os.path.exists(os.path.join(out_dir, "bench_graph.log")):
        written.append(summarize_graph(out_dir, khash))
    if all(os.path.isdir(os.path.join(out_dir, r)) for r in COUNTER_PASSES):
        written.append(summarize_counters(out_dir, khash))
    print(json.dumps({"written": written, "kernel_source_hash": khash}))
    return 0


def _json_line(path: str, key: str):
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for ln in fh:
            if ln.strip().startswith("{") and f'"{key}"' in ln:
                return json.loads(ln)
    return None


def floor_table(fl: dict) -> list:
    lines = ["| kind | back to back us | event us |", "|---|---:|---:|"]
    for k, v in fl.items():
        if isinstance(v, dict) and "b2b_us" in v:
            ev = f"{v['event_us']:.2f}" if v.get("event_us") else "-"
            lines.append(f"| {k} | {v['b2b_us']:.2f} | {ev} |")
    return lines


def summarize_counters(out_dir: str, khash: str) -> str:
    """Hardware counters per dispatch of the decode stream's attention and
    merge launches and of the read floors on the attention's grid
    (COUNTER_PASSES), with the ratios they give: where the waves' cycles go."""
    groups = (("k_ring_attn_fused (decode attention)", lambda n: "k_ring_attn_fused" in n),
              ("k_ring_merge<8> (cross-split merge)", lambda n: "k_ring_merge" in n),
              ("k_ring_floor<1> (read floor)", lambda n: "k_ring_floor<1>" in n),
              ("k_ring_floor<2> (read + partials floor)", lambda n: "k_ring_floor<2>" in n))
    vals = {g: {} for g, _ in groups}
    counts = {g: 0 for g, _ in groups}
    for run, ctrs in COUNTER_PASSES.items():
        rows = _csv_rows(out_dir, run, "counter_collection")
        for g, pick in groups:
            per = {}
            for r in rows:
                if pick(r["Kernel_Name"]) and r["Counter_Name"] in ctrs:
                    per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            for c, v in per.items():
                vals[g][c] = sum(v) / len(v)
                counts[g] = max(counts[g], len(v))
    lines = ["# Hardware counters: decode_stream (cap 4096, q_len 8, GQA 32/8 x 128, F16, 1 layer, "
             "32-ring pool)", "", f"Kernel source hash: `{khash}`", "",
             "Commands (cd /tmp; TMPDIR=/tmp), one counter group per run:", ""]
    lines += [f"    {PROFILE_RUNS[r]}" for r in COUNTER_PASSES]
    lines += ["", "Average per dispatch (SQ counters summed over the shader engines; cycle "
              "counts of SQ_WAVE_CYCLES, SQ_WAIT_* and SQ_ACTIVE_INST_* in quad-cycles, "
              "summed over waves).", "",
              "| counter | " + " | ".join(g for g, _ in groups) + " |",
              "|---|" + "---:|" * len(groups)]
    for ctrs in COUNTER_PASSES.values():
        for c in ctrs:
            lines.append(f"| {c} | " + " | ".join(
                f"{vals[g][c]:.4g}" if c in vals[g] else "-" for g, _ in groups) + " |")
    lines += ["", "| derived | " + " | ".join(g for g, _ in groups) + " |",
              "|---|" + "---:|" * len(groups)]

    def ratio(g, a, b, scale=1.0):
        v = vals[g]
        return v[a] / v[b] * scale if v.get(a) is not None and v.get(b) else None

    derived = (
        ("waves", lambda g: vals[g].get("SQ_WAVES")),
        ("cycles per wave (SQ_WAVE_CYCLES x 4 / SQ_WAVES)",
         lambda g: ratio(g, "SQ_WAVE_CYCLES", "SQ_WAVES", 4.0)),
        ("share of wave cycles waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES)",
         lambda g: ratio(g, "SQ_WAIT_ANY", "SQ_WAVE_CYCLES")),
        ("share waiting to issue (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES)",
         lambda g: ratio(g, "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES")),
        ("share issuing vector memory (SQ_ACTIVE_INST_VMEM / SQ_WAVE_CYCLES)",
         lambda g: ratio(g, "SQ_ACTIVE_INST_VMEM", "SQ_WAVE_CYCLES")),
        ("share issuing VALU (SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES)",
         lambda g: ratio(g, "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES")),
        ("vector memory reads per wave", lambda g: ratio(g, "SQ_INSTS_VMEM_RD", "SQ_WAVES")),
        ("scalar ALU instructions per wave", lambda g: ratio(g, "SQ_INSTS_SALU", "SQ_WAVES")),
        ("VALU instructions per wave", lambda g: ratio(g, "SQ_INSTS_VALU", "SQ_WAVES")),
        ("LDS instructions per wave", lambda g: ratio(g, "SQ_INSTS_LDS", "SQ_WAVES")),
        ("instruction fetches per wave", lambda g: ratio(g, "SQ_IFETCH", "SQ_WAVES")),
        ("average L1 -> L2 read latency, cycles (TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ)",
         lambda g: ratio(g, "TCP_TCC_READ_REQ_LATENCY", "TCP_TCC_READ_REQ")),
        ("L2 hit rate (TCC_HIT / (TCC_HIT + TCC_MISS))",
         lambda g: (vals[g]["TCC_HIT"] / (vals[g]["TCC_HIT"] + vals[g]["TCC_MISS"])
                    if vals[g].get("TCC_HIT") is not None and vals[g].get("TCC_MISS") is not None
                    and vals[g]["TCC_HIT"] + vals[g]["TCC_MISS"] > 0 else None)),
    )
    for name, f in derived:
        cells = []
        for g, _ in groups:
            v = f(g)
            cells.append("-" if v is None else (f"{v:.3f}" if v < 10 else f"{v:.4g}"))
        lines.append(f"| {name} | " + " | ".join(cells) + " |")
    lines += ["", "Dispatches averaged per group: " +
              ", ".join(f"{g.split(' ')[0]} {counts[g]}" for g, _ in groups) + "."]
    path = "profiles/k_ring_attn_decode_stream_counters.md"
    with open(os.path.join(ROOT, path), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return path


def summarize_graph(out_dir: str, khash: str) -> str:
    """Graph replay against plain launches (bench.py --graph)."""
    bl = _json_line(os.path.join(out_dir, "bench_graph.log"), "graph")
    g = bl["graph"]
    lines = ["# The decode step as plain launches and as replayed HIP graphs (decode_stream, "
             "cap 4096, 32-ring pool)", "", f"Kernel source hash: `{khash}`", "",
             "Command (cd /tmp; TMPDIR=/tmp):", "", f"    {PROFILE_RUNS['bench_graph']}", "",
             g["what"] + ".  Host: time to submit, per step.  Device: a batch queued behind a "
             "hold launch, HIP events around it, per step (when the batch was not queued in time "
             "the host's pace sets it).", "",
             "| step as | steps per graph | host us per step | device us per step | batch queued |",
             "|---|---:|---:|---:|---|"]
    for k in ("plain", "graph_1", "graph_8"):
        v = g[k]
        lines.append(f"| {'plain launches' if k == 'plain' else 'graph replay'} | "
                     f"{v.get('steps_per_graph', '-')} | {v['host_us']:.2f} | {v['device_us']:.2f} | "
                     f"{'yes' if v['queued_behind_hold'] else 'no'} |")
    p_ = "profiles/ring_step_graph_replay_decode_stream.md"
    with open(os.path.join(ROOT, p_), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return p_


def summarize_floor(out_dir: str, khash: str) -> str:
    """Kernel trace of the floor launches (ring_profile_floor) on the decode
    stream, next to the bench's own floor figures."""
    stats = _csv_rows(out_dir, "prof_ktrace_floor", "kernel_stats")
    bl = None
    path = os.path.join(out_dir, "bench_floor.log")
    if os.path.exists(path):
        with open(path) as fh:
            for ln in fh:
                if ln.strip().startswith("{") and '"floors"' in ln:
                    bl = json.loads(ln)
    names = {"0": "empty", "1": "read", "2": "partials (+ k_ring_merge: two_launch)",
             "3": "last_arriver", "4": "barrier", "6": "hold", "7": "matrix_math",
             "8": "vector_math"}
    lines = ["# Floors of the attention launch: decode_stream (cap 4096, q_len 8, GQA 32/8 x 128, "
             "F16, 1 layer, 32-ring pool)", "", f"Kernel source hash: `{khash}`", "",
             "Command (cd /tmp; TMPDIR=/tmp):", "", f"    {PROFILE_RUNS['prof_ktrace_floor']}", "",
             "Each floor kernel runs on the attention's grid (256 work-groups of 4 waves: 8 KV "
             "heads x 32 splits), work-group order and tiles, with a trivial consumer; "
             "include/ring_kv.h (ring_profile_floor) describes the kinds.", "",
             "| kernel | kind | calls | avg us | min us | max us |", "|---|---|---:|---:|---:|---:|"]
    for r in stats:
        name = r["Name"]
        kind = next((v for k, v in names.items() if f"k_ring_floor<{k}>" in name), "")
        if not kind and "k_ring_merge" not in name:
            continue
        lines.append(f"| `{name}` | {kind or 'merge of the two_launch kind'} | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} |")
    if bl:
        fl = bl["floors"]
        lines += ["", f"The same floors without the profiler (`{PROFILE_RUNS['bench_floor']}`), "
                  f"{fl['launches']} launches each cycled over the pool; per launch, back to back "
                  "(a batch queued behind a hold launch, HIP events around it) and one dispatch "
                  "bound to HIP events:", ""] + floor_table(fl)
        lines.append(f"\nBarrier waits that hit their poll limit: {fl.get('barrier_timeouts')}.")
    p_ = "profiles/k_ring_floor_decode_stream_kernel_trace.md"
    with open(os.path.join(ROOT, p_), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return p_


def projection_segments(out_dir: str, run: str, decode_grid: int) -> dict:
    """Durations of the projection dispatches in a mirror_stream kernel
    trace: the decode-step launches (grid `decode_grid` threads, one per
    step) cut at the bench's segments -- warm-up, timed steps and the
    event-profiled steps cycle the pool's rings (cold weights), the last
    segment runs ring 0 alone (its weights stay in the Infinity Cache) --
    and the prefill's launches.  {name: (dispatches, median us, mean us)}."""
    import statistics as stt
    rows = sorted(_csv_rows(out_dir, run, "kernel_trace"), key=lambda r: int(r["Start_Timestamp"]))
    proj = [r for r in rows if "k_ring_project" in r["Kernel_Name"]]
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3  # noqa: E731
    dec = [dur(r) for r in proj if int(r["Grid_Size_X"]) == decode_grid]
    pre = [dur(r) for r in proj if int(r["Grid_Size_X"]) != decode_grid]
    out = {}
    if pre:
        out["prefill (64-row launches)"] = (len(pre), stt.median(pre), stt.mean(pre))
    cmd = PROFILE_RUNS[run]
    warm = int(re.search(r"--warmup (\d+)", cmd).group(1))
    steps = int(re.search(r"--steps (\d+)", cmd).group(1))
    cuts = (("decode steps: warm-up (pool cycled, cold)", 0, warm),
            ("decode steps: timed (pool cycled, cold)", warm, warm + steps),
            ("decode steps: event-profiled (pool cycled, cold)", warm + steps, warm + 2 * steps),
            ("decode steps: ring 0 alone (its weights in the Infinity Cache)", warm + 2 * steps,
             len(dec)))
    for name, a, b in cuts:
        v = dec[a:b]
        if v:
            out[name] = (len(v), stt.median(v), stt.mean(v))
    return out


def summarize_mirror(out_dir: str, khash: str, fetch_scale: float, write_scale: float):
    """Kernel trace and HBM traffic of the mirror_stream workload (rows from
    the feature mirror through the projection kernel)."""
    import workload as W
    prof = os.path.join(ROOT, "profiles")
    w = W.WORKLOADS["mirror_stream"]
    wl = (f"mirror_stream (cap {w.cap}, {w.n_layer} layers, d_model {w.d_model}, "
          f"GQA {w.n_head}/{w.n_head_kv} x {w.head_dim}, cold weights)")
    stats = _csv_rows(out_dir, "prof_ktrace_mirror", "kernel_stats")
    bl = _bench_line(out_dir, "bench_plain_mirror")
    lines = [f"# Kernel trace: k_ring_project and the ring kernels, {wl}", "",
             f"Kernel source hash: `{khash}`", "", "Command (cd /tmp; TMPDIR=/tmp):", "",
             f"    {PROFILE_RUNS['prof_ktrace_mirror']}", "",
             "| kernel | calls | avg us | min us | max us | share of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    trace = {}
    for r in stats:
        name = r["Name"]
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f}% |")
        short = next((k for k in KERNELS_MIRROR if k in name), None)
        if short and short not in trace:
            trace[short] = float(r["AverageNs"]) / 1e3
    # decode-step projection launches: one 32-row tile (grid = layers x 4
    # half head parts per KV head x d-slices work-groups of 128 threads, in
    # threads); the prefill's 64-row launches have two
    decode_grid = w.n_layer * 4 * w.n_head_kv * (w.d_model // 256) * 128
    seg = projection_segments(out_dir, "prof_ktrace_mirror", decode_grid)
    if seg:
        lines += ["", "k_ring_project per dispatch in this trace (start to end timestamps), "
                  "decode-step launches (one 32-row tile) in the order the bench runs them, "
                  "and the prefill's 64-row launches apart:", "",
                  "| launches | dispatches | median us | mean us |", "|---|---:|---:|---:|"]
        for name, (n, med, mean) in seg.items():
            lines.append(f"| {name} | {n} | {med:.2f} | {mean:.2f} |")
    if bl:
        ev = {k: v["avg_us"] for k, v in bl.get("kernels", {}).items()}
        lines += ["", f"The same bench without the profiler (`{PROFILE_RUNS['bench_plain_mirror']}`), "
                  "HIP events bound to the dispatches of its profiled segment: "
                  + ", ".join(f"{k} {v:.2f} us" for k, v in ev.items() if v)
                  + f"; {bl['value']:.0f} steps/s in its timed segment."]
        if bl.get("floors"):
            lines += ["", "Floors of the projection launch in the same bench run (ring_profile_floor "
                      "kind RING_FLOOR_PROJ_READ: the projection's grid and weight loads with a "
                      "trivial consumer, cycled over the pool's weight copies; ceiling_frac "
                      f"{bl.get('ceiling_frac')}):", ""] + floor_table(bl["floors"])
    with open(os.path.join(prof, "k_ring_project_mirror_stream_kernel_trace.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    rows = {}
    for k, grid in (("k_ring_project", decode_grid), ("k_ring_project (prefill)", 2 * decode_grid)):
        f, nf = _kib_per_dispatch(out_dir, "pmc_fetch_mirror", "FETCH_SIZE",
                                  lambda n: "k_ring_project" in n, grid)
        wv, nw = _kib_per_dispatch(out_dir, "pmc_write_mirror", "WRITE_SIZE",
                                   lambda n: "k_ring_project" in n, grid)
        rows[k] = {"fetch_kib": f, "write_kib": wv, "dispatches": min(nf, nw),
                   "hbm_bytes": f * 1024 * fetch_scale + wv * 1024 * write_scale}
    weights = 2 * w.n_layer * w.kv_row * w.d_model * 2
    p = rows["k_ring_project"]
    lines = [f"# HBM traffic per dispatch: k_ring_project, {wl}", "",
             f"Kernel source hash: `{khash}`", "", "Commands (cd /tmp; TMPDIR=/tmp), one counter per run:", "",
             f"    {PROFILE_RUNS['pmc_fetch_mirror']}", f"    {PROFILE_RUNS['pmc_write_mirror']}", "",
             f"Counters scaled as for the decode-stream summary (FETCH_SIZE x {fetch_scale:.3f}, "
             f"WRITE_SIZE x {write_scale:.3f}, from a plain {CALIBRATE_COPY_MIB} MiB device copy).  "
             "Decode-step launches (one 32-row tile, at most 18 rows) and the prefill's 64-row "
             "launches (two tiles, the weights read once per tile) apart.", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled HBM MB |",
             "|---|---:|---:|---:|---:|"]
    for k, r in rows.items():
        lines.append(f"| {k} | {r['dispatches']} | {r['fetch_kib']:.1f} | {r['write_kib']:.1f} | "
                     f"{r['hbm_bytes'] / 1e6:.3f} |")
    lines += ["", f"k_ring_project in a decode step: {p['fetch_kib'] * 1024 * fetch_scale / 1e6:.3f} MB "
              f"read per launch against {weights / 1e6:.3f} MB of weights (every layer's wk and "
              "wv, read once; the features add under 0.1 MB); writes are the fp32 partial sums of "
              "the 256-dim feature slices."]
    if "k_ring_project" in trace:
        lines.append(f"Average k_ring_project duration in the kernel trace: {trace['k_ring_project']:.2f} us.")
    with open(os.path.join(prof, "k_ring_project_mirror_stream_hbm_traffic.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return ["profiles/k_ring_project_mirror_stream_kernel_trace.md",
            "profiles/k_ring_project_mirror_stream_hbm_traffic.md"]


def summarize_wide(out_dir: str, wl_name: str, khash: str, fetch_scale: float,
                   write_scale: float) -> str:
    """Kernel trace and HBM traffic of k_ring_attn on one of the wider
    workloads, with the bench line's algorithmic bytes per launch."""
    import workload as W
    prof = os.path.join(ROOT, "profiles")
    w = W.WORKLOADS[wl_name]
    wl = (f"{wl_name} ({w.n_seq} x cap {w.cap}, q_len {w.q_len}, GQA {w.n_head}/{w.n_head_kv} x "
          f"{w.head_dim}, {w.n_layer} layer)")
    stats = _csv_rows(out_dir, f"prof_ktrace_{wl_name}", "kernel_stats")
    bl = _bench_line(out_dir, f"bench_plain_{wl_name}")
    lines = [f"# k_ring_attn on {wl}", "", f"Kernel source hash: `{khash}`", "",
             "Commands (cd /tmp; TMPDIR=/tmp):", ""]
    lines += [f"    {PROFILE_RUNS[r]}" for r in (f"prof_ktrace_{wl_name}", f"pmc_fetch_{wl_name}",
                                                 f"pmc_write_{wl_name}", f"bench_plain_{wl_name}")]
    lines += ["", "| kernel | calls | avg us | min us | max us | share of GPU time |",
              "|---|---:|---:|---:|---:|---:|"]
    trace = None
    for r in stats:
        name = r["Name"]
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f}% |")
        if "k_ring_attn" in name and trace is None:
            trace = float(r["AverageNs"]) / 1e3
    f, nf = _kib_per_dispatch(out_dir, f"pmc_fetch_{wl_name}", "FETCH_SIZE", lambda n: "k_ring_attn" in n)
    wv, nw = _kib_per_dispatch(out_dir, f"pmc_write_{wl_name}", "WRITE_SIZE", lambda n: "k_ring_attn" in n)
    lines += ["", f"HBM traffic per k_ring_attn dispatch ({min(nf, nw)} dispatches; counters scaled "
              f"as for the decode-stream summary, FETCH_SIZE x {fetch_scale:.3f}, WRITE_SIZE x "
              f"{write_scale:.3f}): read {f * 1024 * fetch_scale / 1e6:.2f} MB, written "
              f"{wv * 1024 * write_scale / 1e6:.2f} MB."]
    if bl:
        r = bl["roofline"]
        lines.append(
            f"The same bench without the profiler: {bl['value']:.0f} steps/s; k_ring_attn "
            f"{r['avg_launch_us']:.2f} us per launch (HIP events bound to its dispatches) for "
            f"{r['bytes_per_launch'] / 1e6:.2f} MB of algorithmic bytes = {r['achieved']:.0f} GB/s, "
            f"{100 * r['frac']:.1f}% of 8 TB/s; splits: {bl['config']['ring'].split('splits=')[-1]}.")
    if trace:
        lines.append(f"Average k_ring_attn duration in the kernel trace: {trace:.2f} us.")
    if bl and bl.get("floors"):
        lines += ["", "Floors of this launch in the same bench run (ring_profile_floor: the "
                  "attention's grid and tiles with a trivial consumer; "
                  f"ceiling_frac {bl.get('ceiling_frac')}):", ""] + floor_table(bl["floors"])
    path = f"profiles/k_ring_attn_{wl_name}.md"
    with open(os.path.join(ROOT, path), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return path


FLOOR_KINDS = (("empty", 0), ("read", 1), ("read_lockstep", 10), ("partials", 2),
               ("two_launch", 5), ("last_arriver", 3), ("barrier", 4), ("matrix_math", 7),
               ("vector_math", 8))
# rings with 64 queries per KV head (two 32-query blocks): also one read of
# every tile for both blocks, eight waves sharing each tile through LDS
FLOOR_KINDS_TWO_BLOCKS = FLOOR_KINDS + (("shared_tiles", 11),)
# the mirror step's projection launch: its grid with a trivial consumer of
# the registered weights (every pool ring holds its own copy: cold)
FLOOR_KINDS_MIRROR = (("empty", 0), ("proj_read", 9))


def clock_warmup(dev, seconds: float, flush_mib: int) -> int:
    """Keep the GPU busy reading a scratch buffer of `flush_mib` MiB for about
    `seconds` (clocks up).  The buffer is written once and then only read, so
    the Infinity Cache ends up holding its clean lines and nothing of the
    rings, and no write-back of dirty lines is left for the timed steps to
    wait behind.  Returns the number of full reads."""
    import torch
    buf = torch.zeros(flush_mib << 20, dtype=torch.uint8, device=dev).view(torch.int64)
    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(16):
            torch.amax(buf)
            n += 1
        torch.cuda.synchronize(dev)
        if time.perf_counter() - t0 >= seconds:
            break
    del buf
    return n


# Points of a wave's work at which the profiling build reads the clock
# (ring_profile_stamps in include/ring_kv.h), per stamp region.
STAMP_POINTS = {
    "attn": ("entry", "work-group mapped", "first tile's loads issued",
             "queries built, first extra rows staged (past the barrier)",
             "extra key rows attended", "ring tiles attended",
             "waves' blocks exchanged through LDS", "output or partial stored (issued)"),
    "merge": ("entry", "work-group mapped", "partial loads issued", "partials in",
              "past the LDS exchange", None, None, "output stored (issued)"),
    "proj": ("entry", "work-group mapped", "feature and weight loads issued",
             "features staged in LDS", "matrix-core products issued", None, None,
             "slice sums stored (issued)"),
}


def stamp_step_stats(recs: dict, khz: int) -> dict:
    """One stamped step: recs[kernel] = that region's [waves][RING_STAMP_WORDS]
    records (a wave that did not run has entry stamp 0).  Per kernel, per
    point of STAMP_POINTS: the median and the latest wave's microseconds after
    the launch's first wave started (the merge counts from the attention's
    first wave); and where the attention's waves ran (four waves per
    work-group: XCC_ID against the work-group index mod 8, compute units from
    HW_ID's cu, sh and se fields)."""
    import numpy as np
    us = 1000.0 / khz                       # microseconds per clock tick
    out = {}
    a = recs.get("attn")
    valid_a = a[:, 0] != 0 if a is not None else np.zeros(0, dtype=bool)
    t_first = int(a[valid_a, 0].min()) if valid_a.any() else 0
    for name, st in recs.items():
        valid = st[:, 0] != 0
        if not valid.any():
            continue
        base = t_first if name == "merge" and t_first else int(st[valid, 0].min())
        rel = (st[valid, :8].astype(np.int64) - base) * us
        used = [p for p in range(8) if STAMP_POINTS[name][p]]
        out[name] = {"med": [float(np.median(rel[:, p])) for p in used],
                     "max": [float(np.max(rel[:, p])) for p in used]}
    if valid_a.any():
        idx = np.nonzero(valid_a)[0]
        hw, xcc = a[idx, 8].astype(np.int64), a[idx, 9].astype(np.int64)
        block = idx // 4
        # HW_ID: cu_id bits 11:8, sh_id bit 12, se_id bits 15:13
        cu = (xcc << 16) | (hw & 0xFF00)
        _, cnt = np.unique(cu, return_counts=True)
        out["placement"] = {"waves": len(idx), "xcd_is_block_mod_8": float(np.mean(xcc == block % 8)),
                            "cus": len(cnt), "max_waves_per_cu": int(cnt.max())}
    return out


def stamp_summary(steps: list, khz: int) -> dict:
    """The stamped steps' statistics (stamp_step_stats each) summarised:
    medians over steps of each point's median and latest wave."""
    import numpy as np
    out = {"steps": len(steps), "clock_khz": khz,
           "what": "single steps, each queued behind a 14 ms hold launch"}
    for name in ("attn", "merge", "proj"):
        rows = [st[name] for st in steps if name in st]
        if not rows:
            continue
        pts = [p for p in STAMP_POINTS[name] if p]
        med = np.median(np.array([r["med"] for r in rows]), axis=0)
        mx = np.median(np.array([r["max"] for r in rows]), axis=0)
        out[name] = {"points": pts, "median_wave_us": [round(float(x), 3) for x in med],
                     "latest_wave_us": [round(float(x), 3) for x in mx]}
    pl = [st["placement"] for st in steps if "placement" in st]
    if pl:
        out["attn_placement"] = {
            "waves": int(np.median([p["waves"] for p in pl])),
            "xcd_is_block_mod_8": float(np.min([p["xcd_is_block_mod_8"] for p in pl])),
            "compute_units": int(np.median([p["cus"] for p in pl])),
            "max_waves_per_cu": int(np.max([p["max_waves_per_cu"] for p in pl]))}
    return out


def stamps_segment(rings, pool, calls, first, n_steps, run, dev, R) -> dict:
    """Per-wave timestamps (profiling build) of n_steps single steps, each on
    the ring touched longest ago and queued behind a RING_FLOOR_HOLD launch
    (a wave that sleeps about 14 ms), so that its launches dispatch back to
    back as the timed steps' do rather than onto an idle device; summarised
    by stamp_summary."""
    import torch
    regions = (("attn", R.RING_STAMPS_ATTN), ("merge", R.RING_STAMPS_MERGE),
               ("proj", R.RING_STAMPS_PROJ))
    nw = R.RING_STAMP_WAVES
    h0 = rings[0].handle
    for _, reg in regions:
        R.ring_profile_stamps(h0, reg, 0, True)
    steps, khz = [], 0
    s = torch.cuda.current_stream(dev).cuda_stream
    for t in range(first, first + n_steps):
        R.ring_profile_floor(h0, 0, R.RING_FLOOR_HOLD, s)
        run(calls[t:t + 1])
        torch.cuda.synchronize(dev)
        recs = {}
        for name, reg in regions:
            recs[name], khz = R.ring_profile_stamps(h0, reg, nw, True)
        steps.append(stamp_step_stats(recs, khz))
    return stamp_summary(steps, khz)


def stamps_markdown(res: dict, cmd: str) -> str:
    """The stamps mode's JSON as a short markdown summary."""
    lines = [f"# Per-wave timestamps: {res['workload']} ({res['step']} step)", "",
             f"Command: `{cmd}`", "",
             f"Profiling build `libringkv_stamps.so` (`RINGKV_LIB=stamps`): {res['stamps']['steps']} "
             f"single steps, each on the pool ring touched longest ago and queued behind a 14 ms "
             f"hold launch (its launches dispatch back to back, as in the timed steps); clock "
             f"{res['stamps']['clock_khz']} kHz.  Microseconds after the launch's "
             f"first wave started (merge: after the attention's first wave); median over steps "
             f"of the median wave and of the latest wave.  Kernel source hash: "
             f"`{res['kernel_source_hash']}`.", ""]
    for name in ("attn", "merge", "proj"):
        r = res["stamps"].get(name)
        if not r:
            continue
        lines += [f"## {name}", "", "| point | median wave | latest wave |", "|---|---:|---:|"]
        lines += [f"| {p} | {a:.2f} | {b:.2f} |"
                  for p, a, b in zip(r["points"], r["median_wave_us"], r["latest_wave_us"])]
        lines.append("")
    pl = res["stamps"].get("attn_placement")
    if pl:
        lines += ["## attention placement", "",
                  f"{pl['waves']} waves on {pl['compute_units']} compute units (at most "
                  f"{pl['max_waves_per_cu']} waves on one); fraction of waves whose XCC_ID equals "
                  f"their work-group index mod 8: {pl['xcd_is_block_mod_8']:.3f} (lowest over the "
                  f"steps).", ""]
    return "\n".join(lines)


def floor_segment(rings, pool, launches, dev, R, attn_us, step_us, bytes_read, n_layer=1,
                  kinds=FLOOR_KINDS):
    """The ring_profile_floor kinds on layer 0, cycled over the pool (cold).
    Per launch: the device's back-to-back time (HIP events around a batch
    queued behind a RING_FLOOR_HOLD launch, so that the host's submission
    rate does not bound it), and the event-bound duration of one dispatch."""
    import torch
    s = torch.cuda.current_stream(dev).cuda_stream
    fl = R.ring_profile_floor
    out = {"launches": launches, "layer": 0, "kv_bytes_read_per_launch": int(bytes_read)}
    for name, kind in kinds:
        try:
            for t in range(min(pool, launches)):        # one launch per ring first
                fl(rings[t % pool].handle, 0, kind, s)
            torch.cuda.synchronize(dev)
        except R.RingError as e:
            out[name] = {"skipped": str(e)}
            continue
        fl(rings[0].handle, 0, R.RING_FLOOR_HOLD, s)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        th = time.perf_counter()
        for t in range(launches):
            fl(rings[t % pool].handle, 0, kind, s)
        e1.record()
        host_us = (time.perf_counter() - th) / launches * 1e6
        queued = not e0.query()     # the hold still ran when the batch was in
        torch.cuda.synchronize(dev)
        b2b = e0.elapsed_time(e1) * 1e3 / launches
        per_ring = -(-launches // pool) * 2
        for r in rings:
            r.profile_enable(per_ring)
        for t in range(launches):
            fl(rings[t % pool].handle, 0, kind, s)
        torch.cuda.synchronize(dev)
        n_l, ms = 0, 0.0
        for r in rings:
            a_, b_ = r.profile_read(R.RING_KERNEL_FLOOR)
            n_l += a_
            ms += b_
        for r in rings:
            r.profile_enable(0)
        # the two-launch kind times its two dispatches apiece
        ev = 1e3 * ms / launches if n_l else None
        out[name] = {"b2b_us": b2b, "event_us": ev, "host_submit_us": host_us,
                     "queued_behind_hold": bool(queued)}
    out["barrier_timeouts"] = int(sum(R.ring_profile_floor_timeouts(r.handle) for r in rings))
    ceil = {}
    rd = out.get("read", {}).get("event_us")
    if rd and attn_us:
        ceil["attn_kernel"] = rd / attn_us
    tl = out.get("two_launch", {}).get("b2b_us")
    if tl and step_us:
        # layer 0's two-launch floor once per layer of the step
        ceil["step"] = tl * n_layer / step_us
    return out, ceil


GRAPH_PLAIN_STEPS = 400
GRAPH_REPLAYS = 400


def graph_segment(rings, pool, calls, warmup, run, dev, R) -> dict:
    """The step as plain launches against the same step captured in HIP
    graphs (torch.cuda.graph around the C-ABI calls) and replayed unchanged.

    Plain: GRAPH_PLAIN_STEPS steps cycled over the pool.  Graphs: one per
    pool ring holding that ring's next step (so that replays cycle over the
    pool and stay cold), then graphs of 8 steps (8 rings each).  Per step:
    host time to submit, and device time of a batch queued behind a
    RING_FLOOR_HOLD launch (HIP events around the batch)."""
    import torch
    s = torch.cuda.current_stream(dev).cuda_stream

    def timed(submit, n):
        R.ring_profile_floor(rings[0].handle, 0, R.RING_FLOOR_HOLD, s)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        th = time.perf_counter()
        submit()
        host = time.perf_counter() - th
        e1.record()
        queued = not e0.query()
        torch.cuda.synchronize(dev)
        return {"host_us": host / n * 1e6, "device_us": e0.elapsed_time(e1) * 1e3 / n,
                "queued_behind_hold": bool(queued)}

    out = {}
    plain = calls[warmup: warmup + GRAPH_PLAIN_STEPS]
    out["plain"] = timed(lambda: run(plain), len(plain))
    base = warmup + GRAPH_PLAIN_STEPS
    for per in (1, 8):
        graphs = []
        for g0 in range(0, pool, per):
            # the next step of rings g0 .. g0 + per - 1, captured as issued
            step_calls = calls[base + g0: base + g0 + per]
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run(step_calls, s=torch.cuda.current_stream(dev).cuda_stream)
            graphs.append(g)
        base += pool
        for g in graphs:            # first replays (uploads the graphs)
            g.replay()
        torch.cuda.synchronize(dev)
        n_rep = GRAPH_REPLAYS // len(graphs) * len(graphs)

        def replays():
            for i in range(n_rep):
                graphs[i % len(graphs)].replay()
        r_ = timed(replays, n_rep * per)
        r_["steps_per_graph"] = per
        out[f"graph_{per}"] = r_
        del graphs
    out["what"] = ("the fused step (ring_begin_step_deferred + ring_attn: attention launch with "
                   "the fold-in append, then the merge) per step; graphs hold a ring's step "
                   "with its arguments fixed and are replayed unchanged")
    return out


def committed_trace_us(kernel_hash: str):
    """Average duration of the attention kernel in the committed kernel-trace
    summary of the decode stream, if it was taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", "ring_attn_decode_stream_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_hash:
        return None
    return t.get("trace_avg_us")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=WORKLOAD,
                    help="decode_stream (the headline), batched_seqs, large_window, "
                         "long_prompt_wrap or tiny_ring")
    ap.add_argument("--pool", type=int, default=0,
                    help="independent rings cycled through (default: enough to exceed the "
                         "256 MB Infinity Cache; 1 = cache-warm)")
    ap.add_argument("--step", choices=("eager", "fused"), default="fused",
                    help="fused (default): ring_begin_step_deferred, the fold-in append and "
                         "index rebuild run inside the attention launch; eager: "
                         "ring_begin_step's own append launch (rings of several sequences: "
                         "one ring_begin_step_batch call, see --begin); rows from features "
                         "take ring_begin_step_mirror, whatever this says")
    ap.add_argument("--begin", choices=("auto", "per_seq", "batch"), default="auto",
                    help="ring with several sequences: auto takes one ring_begin_step_deferred "
                         "call per sequence for the fused step (rings of up to 16 sequences) "
                         "and one ring_begin_step_batch call for all of them otherwise; "
                         "per_seq one begin call per sequence; batch one "
                         "ring_begin_step_batch call")
    ap.add_argument("--proj", choices=("registered", "caller"), default="registered",
                    help="rows from features: weights registered once per ring "
                         "(ring_set_kv_weights, packed in the projection's load order; "
                         "default) or the caller's weights passed every step")
    ap.add_argument("--workspace", choices=("torch", "library"), default="torch",
                    help="each ring's workspace: a torch tensor (default) or allocated by "
                         "ring_init itself")
    ap.add_argument("--warm-seconds", type=float, default=0.25,
                    help="GPU clock warm-up before the warm-up and timed steps (reads of a "
                         "scratch buffer that also evict the rings from the Infinity Cache)")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="size of that scratch buffer (above the 256 MB Infinity Cache)")
    ap.add_argument("--floor-launches", type=int, default=400,
                    help="launches per ring_profile_floor kind (0: no floor segment)")
    ap.add_argument("--floor", action="store_true",
                    help="only the floor segment (after the same warm-up), one JSON line")
    ap.add_argument("--stamps", type=int, default=0, metavar="STEPS",
                    help="profiling build (libringkv_stamps.so): per-wave timestamps of STEPS "
                         "single steps after the warm-up, printed as JSON")
    ap.add_argument("--stamps-md", default="", metavar="PATH",
                    help="with --stamps: also write the markdown summary to PATH")
    ap.add_argument("--graph", action="store_true",
                    help="only the graph-replay comparison (after the same warm-up), one JSON "
                         "line: the step captured in HIP graphs and replayed, against plain "
                         "launches")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize", metavar="OUT", default="",
                    help="write profiles/ summaries from rocprofv3 output under OUT")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB ten times (scale for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the ring step has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        return 2
    if args.summarize:
        return summarize_profiles(args.summarize)

    import numpy as np
    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 10}), flush=True)
        return 0

    if args.stamps:
        os.environ["RINGKV_LIB"] = "stamps"   # before the package loads its library
    import workload as W
    import draft_model_kv_amd as R

    w = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    geo = R.ring_query_geometry(R.make_config(w.cap, w.q_len, w.n_head, w.n_head_kv,
                                              w.head_dim, w.n_layer, w.n_seq, w.rope_base,
                                              d_model=w.d_model))
    ring_bytes = w.n_seq * w.n_layer * geo.kv_bytes_per_layer
    if w.d_model:
        # each pool member also holds its feature mirror and weight copy
        ring_bytes += w.n_seq * w.cap * w.d_model * 2 + 2 * w.n_layer * w.kv_row * w.d_model * 2
    pool = args.pool or max(1, -(-(512 << 20) // ring_bytes))
    # warm-up, the timed steps, then as many steps again with per-kernel
    # timing events (they slow back-to-back launches, so they stay out of the
    # timed region); ring 0 alone then takes up to min(steps, 1000) more
    # steps for the cache-warm figure
    total = args.warmup + (0 if args.floor else 2 * args.steps)
    if args.stamps:
        total = args.warmup + args.stamps
    if args.graph:
        # plain steps, then one step per pool ring for the captured graphs
        total = args.warmup + GRAPH_PLAIN_STEPS + 8 * pool
    warm_steps = min(args.steps, 1000) if pool > 1 and not (args.floor or args.stamps) else 0
    rings, calls, steps_in, committed, calls0 = prepare(w, pool, total, dev, warm_steps, args.proj,
                                                        args.workspace)
    s = torch.cuda.current_stream(dev).cuda_stream
    out = torch.empty((w.n_seq, w.q_len, w.n_head, w.head_dim), dtype=torch.float32, device=dev)
    mirror = w.d_model > 0
    batched = not mirror and w.n_seq > 1 and (
        args.begin == "batch" or (args.begin == "auto" and (args.step == "eager" or w.n_seq > 16)))
    fused = args.step == "fused" and not mirror and not batched
    step_mode = "mirror" if mirror else "batch" if batched else "fused" if fused else "eager"
    begin = R.ring_begin_step_deferred if fused else R.ring_begin_step
    attn, optr = R.ring_attn, out.data_ptr()
    # the mirror step's feature write is deferred: the projection launch of
    # the step carries it out (one launch fewer per step)
    mwrite, mbegin = R.ring_mirror_write_deferred, R.ring_begin_step_mirror
    mbegin_reg = R.ring_begin_step_mirror_registered
    begin_batch = R.ring_begin_step_batch
    if batched:
        # the batched call's argument lists, built once per call
        calls = [(h, [list(col) for col in zip(*seqs)], layers, wp) for h, seqs, layers, wp in calls]
        calls0 = [(h, [list(col) for col in zip(*seqs)], layers, wp) for h, seqs, layers, wp in calls0]

    def run(seq_calls, s=s):
        for h, seqs, layers, wptr in seq_calls:
            if mirror:
                for seq, c, fp, c0, n in seqs:
                    mwrite(h, seq, c0, n, fp, s)
                    if wptr is None:
                        mbegin_reg(h, seq, c, s)
                    else:
                        mbegin(h, seq, c, *wptr, s)
            elif batched:
                begin_batch(h, *seqs, s)
            else:
                for seq, c, kp, vp, n in seqs:
                    begin(h, seq, c, kp, vp, n, s)
            for layer, qp, knp, vnp in layers:
                attn(h, layer, qp, knp, vnp, optr, s)

    # clocks up and the Infinity Cache evicted, then the warm-up steps (they
    # also warm the host's submission path: run before the clock warm-up,
    # the first timed step took 31-40 us to submit instead of 8-11), then the
    # timed steps: each cycles to the ring touched longest ago (pool x ring
    # bytes >= 512 MB)
    n_fills = clock_warmup(dev, args.warm_seconds, args.flush_mib)
    run(calls[:args.warmup])
    torch.cuda.synchronize(dev)

    if args.graph:
        print(json.dumps({"workload": args.workload, "step": step_mode, "ring_pool": pool,
                          "graph": graph_segment(rings, pool, calls, args.warmup, run, dev, R)}),
              flush=True)
        for r in rings:
            r.close()
        return 0

    if args.stamps:
        res = {"workload": args.workload, "step": step_mode, "ring_pool": pool,
               "ring": rings[0].describe(), "kernel_source_hash": kernel_source_hash(),
               "stamps": stamps_segment(rings, pool, calls, args.warmup, args.stamps, run, dev, R)}
        print(json.dumps(res), flush=True)
        if args.stamps_md:
            with open(args.stamps_md, "w") as f:
                f.write(stamps_markdown(res, "python bench.py " + " ".join(sys.argv[1:])))
        for r in rings:
            r.close()
        return 0

    if args.floor:
        fl, ceil = floor_segment(rings, pool, args.floor_launches, dev, R, None, None,
                                 np.mean([sum(algorithmic_bytes(w, min(c, w.cap), geo.kv_total)["kv"]
                                              for c in cs) for cs in committed]))
        print(json.dumps({"workload": args.workload, "ring": rings[0].describe(), "floors": fl,
                          "ring_pool": pool}), flush=True)
        for r in rings:
            r.close()
        return 0

    t0 = time.perf_counter()
    run(calls[args.warmup:args.warmup + args.steps])
    enqueued = time.perf_counter() - t0
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0

    per_ring = (-(-args.steps // pool) + 1) * max(w.n_seq, w.n_layer)
    for r in rings:
        r.profile_enable(per_ring)
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    run(calls[args.warmup + args.steps: total])
    torch.cuda.synchronize(dev)
    elapsed_prof = time.perf_counter() - t1

    prof = {}
    for kind, name in ((R.RING_KERNEL_STEP, "k_ring_step"), (R.RING_KERNEL_ATTN, "k_ring_attn"),
                       (R.RING_KERNEL_MERGE, "k_ring_merge"), (R.RING_KERNEL_PROJ, "k_ring_project")):
        n_l, ms = 0, 0.0
        for r in rings:
            a, b = r.profile_read(kind)
            n_l += a
            ms += b
        prof[name] = {"launches": n_l, "avg_us": (1e3 * ms / n_l) if n_l else None}
    for r in rings:
        r.profile_enable(0)

    # cache-warm figure: ring 0 alone (its ring stays in the Infinity Cache),
    # continuing its stream after the profiled segment
    mall_warm = None
    if calls0:
        n0 = min(len(calls0) // 4, 20)
        run(calls0[:n0])
        torch.cuda.synchronize(dev)
        tw = time.perf_counter()
        run(calls0[n0:])
        torch.cuda.synchronize(dev)
        tw = time.perf_counter() - tw
        nw = len(calls0) - n0
        mall_warm = {"value": nw / tw, "steps": nw, "ms_per_step": 1e3 * tw / nw,
                     "what": "ring 0 of the pool alone, so that its ring stays in the Infinity Cache"}

    split_desc = rings[0].describe()

    # algorithmic bytes of one attention launch, averaged over the profiled
    # segment (every sequence's visible window at its step)
    seg = committed[args.warmup + args.steps: total]

    def layer_window(c, layer):
        win = min(c, w.cap)
        return min(w.swa_window, win) if (w.swa_layers >> layer) & 1 else win

    def mean_bytes(kind):
        # one launch per (step, layer); each covers every sequence
        return np.mean([sum(algorithmic_bytes(w, layer_window(c, layer), geo.kv_total)[kind]
                            for c in cs) for cs in seg for layer in range(w.n_layer)])

    per_launch = mean_bytes("attn_kernel")
    if fused and prof["k_ring_step"]["launches"]:
        # the library appended the deferred steps at once (a ring whose
        # attention waves stream several tiles each): an eager step
        fused, step_mode = False, "eager"
    fused_extra = 0.0
    if fused and not mirror:
        # the fused launch also reads each new row (K and V, F16) and writes it
        # to the ring, reads slot_pos instead of the mask, and writes the new
        # rows' slot_pos entries
        seg_rows = [sum(n for _, _, _, _, n in steps_in[0][t // pool][0])
                    for t in range(args.warmup + args.steps, total)]
        rows = float(np.mean(seg_rows))
        fused_extra = (rows * w.kv_row * 2 * 2 * 2 + w.n_seq * w.cap * 4
                       - w.n_seq * w.q_len * geo.kv_total * 2 + rows * 4)
        per_launch += fused_extra
    per_call = mean_bytes("ring_attn") + fused_extra
    attn_us = prof["k_ring_attn"]["avg_us"]
    merge_us = prof["k_ring_merge"]["avg_us"] or 0.0
    achieved = per_launch / (attn_us * 1e-6) / 1e9
    khash = kernel_source_hash()
    headline = args.workload == WORKLOAD
    traffic = traffic_from_profiles(khash) if headline else None
    trace_us = committed_trace_us(khash) if headline and fused else None
    ms_per_step = 1e3 * elapsed / args.steps
    roof_attn = {"kernel": "k_ring_attn_fused" if fused else "k_ring_attn", "bound": "hbm",
                 "achieved": achieved,
                 "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                 "traffic": traffic, "bytes_per_launch": int(per_launch),
                 "avg_launch_us": attn_us,
                 "timing": "HIP events bound to each dispatch of a segment like the timed one",
                 "trace_avg_us": trace_us,
                 "frac_trace": (per_launch / (trace_us * 1e-6) / 1e9 / HBM_PEAK_GBS)
                 if trace_us else None}
    roofline = roof_attn
    if mirror:
        # the projection launch of a decode step reads every layer's wk and wv
        # once and the new rows' features (n <= a_step rows of d_model F16),
        # and writes those features into the mirror (the deferred write)
        seg_rows = [sum(n for _, _, _, _, n in steps_in[0][t // pool][0])
                    for t in range(args.warmup + args.steps, total)]
        proj_bytes = (2 * w.n_layer * w.kv_row * w.d_model * 2 +
                      2 * float(np.mean(seg_rows)) * w.d_model * 2)
        proj_us = prof["k_ring_project"]["avg_us"]
        pa = proj_bytes / (proj_us * 1e-6) / 1e9
        roofline = {"kernel": "k_ring_project", "weights": args.proj, "bound": "hbm",
                    "achieved": pa,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": pa / HBM_PEAK_GBS,
                    "traffic": None, "bytes_per_launch": int(proj_bytes),
                    "avg_launch_us": proj_us}
    # the whole step as the timed loop saw it: every attention launch's
    # algorithmic bytes (all layers) per step time
    step_bytes = per_call * w.n_layer
    floors, ceiling = None, None
    if args.floor_launches and mirror:
        floors, _ = floor_segment(rings, pool, args.floor_launches, dev, R, None, None,
                                  2 * w.n_layer * w.kv_row * w.d_model * 2,
                                  kinds=FLOOR_KINDS_MIRROR)
        floors["weight_bytes_per_launch"] = floors.pop("kv_bytes_read_per_launch")
        rd = floors.get("proj_read", {}).get("event_us")
        if rd:
            ceiling = {"proj_kernel": rd / proj_us}
    if args.floor_launches and not mirror:
        two_blocks = w.q_len * (w.n_head // w.n_head_kv) > 32
        floors, ceiling = floor_segment(
            rings, pool, args.floor_launches, dev, R, attn_us, ms_per_step * 1e3,
            np.mean([sum(algorithmic_bytes(w, layer_window(c, 0), geo.kv_total)["kv"] for c in cs)
                     for cs in seg]), w.n_layer,
            kinds=FLOOR_KINDS_TWO_BLOCKS if two_blocks else FLOOR_KINDS)
    for r in rings:
        r.close()
    line = {
        "metric": METRIC if headline else
        f"ring step steps/s + achieved HBM GB/s, workload {args.workload}",
        "value": args.steps / elapsed,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "host_submit_ms_per_step": 1e3 * enqueued / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded normal F16 rows; accepted counts drawn from the "
                "pages' 1422-verification share table)",
        "config": {"workload": args.workload, "step": step_mode, "workspace": args.workspace,
                   **({"proj_weights": args.proj} if mirror else {}),
                   "cap": w.cap, "q_len": w.q_len,
                   "n_head": w.n_head, "n_head_kv": w.n_head_kv, "head_dim": w.head_dim,
                   "n_layer": w.n_layer, "n_seq": w.n_seq, "kv_total": geo.kv_total,
                   "ring_pool": pool,
                   "infinity_cache": "cold" if pool * ring_bytes > (256 << 20) else "warm",
                   "before_timing": f"{n_fills} reads of a {args.flush_mib} MiB scratch buffer "
                                    f"over >= {args.warm_seconds} s (clocks up, the Infinity Cache "
                                    f"left holding its clean lines), then the {args.warmup} warm-up "
                                    f"steps; each timed step takes the ring touched longest ago",
                   "ring": split_desc},
        "roofline": roofline,
        "ring_attn": {"kernels": "k_ring_attn_fused + k_ring_merge" if fused else
                      "k_ring_attn + k_ring_merge",
                      "avg_us": attn_us + merge_us,
                      "calls_per_s": 1e6 / (attn_us + merge_us),
                      "achieved_GBps": per_call / ((attn_us + merge_us) * 1e-6) / 1e9,
                      "frac": per_call / ((attn_us + merge_us) * 1e-6) / 1e9 / HBM_PEAK_GBS},
        "step": {"bytes": int(step_bytes),
                 "achieved_GBps": step_bytes / (ms_per_step * 1e-3) / 1e9,
                 "frac": step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "mall_warm": mall_warm,
        "kernels": prof,
        **({"roofline_attn": roof_attn} if mirror else {}),
        "floors": floors,
        "ceiling_frac": ceiling,
        "profiled_segment_steps_per_s": args.steps / elapsed_prof,
        "kernel_source_hash": khash,
    }
    if not args.no_cpu_baseline and headline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
