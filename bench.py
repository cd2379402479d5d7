#!/usr/bin/env python3
"""Throughput of the draft-KV ring step on one MI355X.

A step is one pass of the whole ring path for one sequence: the fold-in
(append with RoPE at absolute positions, slot_pos, window mask, noise RoPE
table) and ring_attn (masked GQA attention of the 8 noise queries over the
4096-slot ring, split-K + merge).  By default the fold-in is handed to the
attention launch (ring_begin_step_deferred, then ring_attn: one attention
launch that appends, rebuilds the index state and attends, then the merge);
--step eager gives it a launch of its own (ring_begin_step).  On a ring of
several sequences (batched_seqs) a step is one ring_begin_step_batch over all
of them, then one ring_attn per layer.
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


def cpu_baseline(w, seconds: float) -> dict:
    """The oracle (full cache, fp32-accumulated attention) on the host cores."""
    import numpy as np
    import oracle.ring_oracle as ro
    import workload as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    geo = ro.geometry(w.cap, w.q_len, w.head_dim, w.n_head_kv)
    st = ro.RingStep(geo, 1, w.n_head_kv, w.head_dim, w.rope_base)
    stream = W.commit_stream(w, 0)
    p = st.plan(stream[0])
    pos = np.arange(p.start, stream[0])
    st.commit(p, [W.context_rows(w, 0, 0, W.T_K, pos)], [W.context_rows(w, 0, 0, W.T_V, pos)])
    inputs = []
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
    return {"value": n_steps / t_total, "unit": "steps/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n_steps} decode steps of the cap-4096 stream after a 4096-row prefill "
                      f"(store new rows with fp64 RoPE + fp32 attention), {t_total:.1f} s"}


def prepare(w, pool: int, total: int, dev):
    """Rings of workload ``w`` warmed up, and the device-resident inputs of
    ``total`` steps cycled over ``pool`` rings.  Returns (rings, calls, geo,
    committed), calls[t] = (handle, [(seq, committed, k, v, n)...],
    [(layer, q, kn, vn)...])."""
    import numpy as np
    import torch
    import workload as W
    import draft_model_kv_amd as R

    streams = [W.commit_stream(w, s_) for s_ in range(w.n_seq)]
    n_warm = W.n_warmup_steps(w)
    n_dec = -(-total // pool)
    if n_dec + n_warm > len(streams[0]):
        raise SystemExit(f"need {n_dec} decode steps per ring, stream has {len(streams[0]) - n_warm}")
    rings = [R.Ring(cap=w.cap, q_len=w.q_len, n_head=w.n_head, n_head_kv=w.n_head_kv,
                    head_dim=w.head_dim, n_layer=w.n_layer, n_seq=w.n_seq,
                    rope_base=w.rope_base, device=dev, swa_window=w.swa_window,
                    swa_layers=w.swa_layers, d_model=w.d_model) for _ in range(pool)]
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
    calls = []
    for t in range(total):
        r, (seqs, layers) = rings[t % pool], steps_in[t // pool]
        if mirror:
            sq = [(seq, c, f.data_ptr(), c0, n) for seq, c, f, c0, n in seqs]
        else:
            sq = [(seq, c, k.data_ptr(), v.data_ptr(), n) for seq, c, k, v, n in seqs]
        calls.append((r.handle, sq,
                      [(layer, q.data_ptr(), kn.data_ptr(), vn.data_ptr())
                       for layer, q, kn, vn in layers],
                      wptrs[t % pool] if mirror else None))
    committed = [[streams[seq][n_warm + t // pool] for seq in range(w.n_seq)]
                 for t in range(total)]
    extra = weights if mirror else None
    return rings, calls, (steps_in, extra), committed


# The rocprofv3 runs behind the committed summaries under profiles/, each run
# from /tmp (TMPDIR=/tmp) with REPO the repository root and OUT an output
# directory; `python bench.py --summarize OUT` then writes the summaries.
PROFILE_RUNS = {
    "prof_ktrace": "rocprofv3 --kernel-trace --stats --output-format csv -d OUT/prof_ktrace -o run "
                   "-- python REPO/bench.py --steps 1000 --warmup 100 --no-cpu-baseline",
    "pmc_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/pmc_fetch -o run "
                 "-- python REPO/bench.py --steps 64 --warmup 16 --no-cpu-baseline",
    "pmc_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/pmc_write -o run "
                 "-- python REPO/bench.py --steps 64 --warmup 16 --no-cpu-baseline",
    "pmc_copy_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/pmc_copy_fetch -o run "
                      "-- python REPO/bench.py --calibrate-copy 1024",
    "pmc_copy_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/pmc_copy_write -o run "
                      "-- python REPO/bench.py --calibrate-copy 1024",
    # the same bench without the profiler (its HIP-event kernel times are
    # compared with the trace; the tracer itself slows event-bound dispatches)
    "bench_plain": "python REPO/bench.py --steps 1000 --warmup 100 --no-cpu-baseline",
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
                                          "--warmup 20 --no-cpu-baseline")
    PROFILE_RUNS[f"prof_ktrace_{_wl}"] = (f"rocprofv3 --kernel-trace --stats --output-format csv -d "
                                          f"OUT/prof_ktrace_{_wl} -o run -- python REPO/bench.py "
                                          f"--workload {_wl} --steps 200 --warmup 20 --no-cpu-baseline")
    for _c in ("fetch", "write"):
        PROFILE_RUNS[f"pmc_{_c}_{_wl}"] = (f"rocprofv3 --pmc {_c.upper()}_SIZE --output-format csv "
                                           f"-d OUT/pmc_{_c}_{_wl} -o run -- python REPO/bench.py "
                                           f"--workload {_wl} --steps 16 --warmup 4 --no-cpu-baseline")
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
    if bl:
        ev = {k: v["avg_us"] for k, v in bl.get("kernels", {}).items()}
        lines += ["", "The same bench without the profiler (" + f"`{cmd('bench_plain')}`" + "), "
                  "HIP events bound to the dispatches of its profiled segment: "
                  + ", ".join(f"{k} {v:.2f} us" for k, v in ev.items() if v)
                  + f"; {bl['value']:.0f} steps/s in its timed segment."]
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
        # rows and slot_pos and writes the rows and the index state)
        alg_attn = bl["roofline"]["bytes_per_launch"]
        what = ("visible K/V rows, queries, noise rows, the step's new rows, slot_pos; the "
                "index state it rebuilds")
        wrote = "split partials, the noise and new rows stored to the ring, the index state"
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
    print(json.dumps({"written": written, "kernel_source_hash": khash}))
    return 0


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
    if bl:
        ev = {k: v["avg_us"] for k, v in bl.get("kernels", {}).items()}
        lines += ["", f"The same bench without the profiler (`{PROFILE_RUNS['bench_plain_mirror']}`), "
                  "HIP events bound to the dispatches of its profiled segment: "
                  + ", ".join(f"{k} {v:.2f} us" for k, v in ev.items() if v)
                  + f"; {bl['value']:.0f} steps/s in its timed segment."]
    with open(os.path.join(prof, "k_ring_project_mirror_stream_kernel_trace.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    # decode-step projection launches: one 32-row tile (grid = layers x K/V
    # heads x d-slices work-groups of 256 threads); the prefill's 64-row
    # launches have two
    decode_grid = w.n_layer * 2 * w.n_head_kv * (w.d_model // 256) * 256
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
    path = f"profiles/k_ring_attn_{wl_name}.md"
    with open(os.path.join(ROOT, path), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return path


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
                         "ring_begin_step's own append launch.  Rings of several sequences "
                         "take ring_begin_step_batch, rows from features "
                         "ring_begin_step_mirror, whatever this says")
    ap.add_argument("--begin", choices=("auto", "per_seq"), default="auto",
                    help="eager step of a ring with several sequences: auto takes one "
                         "ring_begin_step_batch call for all of them (default), per_seq one "
                         "ring_begin_step call per sequence")
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
    # timed region)
    total = args.warmup + 2 * args.steps
    rings, calls, steps_in, committed = prepare(w, pool, total, dev)
    s = torch.cuda.current_stream(dev).cuda_stream
    out = torch.empty((w.n_seq, w.q_len, w.n_head, w.head_dim), dtype=torch.float32, device=dev)
    mirror = w.d_model > 0
    batched = not mirror and w.n_seq > 1 and args.begin == "auto"
    fused = args.step == "fused" and not mirror and not batched
    step_mode = "mirror" if mirror else "batch" if batched else "fused" if fused else "eager"
    begin = R.ring_begin_step_deferred if fused else R.ring_begin_step
    attn, optr = R.ring_attn, out.data_ptr()
    mwrite, mbegin = R.ring_mirror_write, R.ring_begin_step_mirror
    begin_batch = R.ring_begin_step_batch
    # the batched call's argument lists, per call
    columns = [[list(col) for col in zip(*c[1])] for c in calls] if batched else None

    def run(lo, hi):
        for t in range(lo, hi):
            h, seqs, layers, wptr = calls[t]
            if mirror:
                for seq, c, fp, c0, n in seqs:
                    mwrite(h, seq, c0, n, fp, s)
                    mbegin(h, seq, c, *wptr, s)
            elif batched:
                begin_batch(h, *columns[t], s)
            else:
                for seq, c, kp, vp, n in seqs:
                    begin(h, seq, c, kp, vp, n, s)
            for layer, qp, knp, vnp in layers:
                attn(h, layer, qp, knp, vnp, optr, s)

    run(0, args.warmup)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    run(args.warmup, args.warmup + args.steps)
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0

    per_ring = (-(-args.steps // pool) + 1) * max(w.n_seq, w.n_layer)
    for r in rings:
        r.profile_enable(per_ring)
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    run(args.warmup + args.steps, total)
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

    split_desc = rings[0].describe()
    for r in rings:
        r.close()

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
    if fused and not mirror:
        # the fused launch also reads each new row (K and V, F16) and writes it
        # to the ring, reads slot_pos instead of the mask, and (first layer of
        # a step) writes slot_pos entries, the mask and the noise RoPE table
        seg_rows = [sum(n for _, _, _, _, n in steps_in[0][t // pool][0])
                    for t in range(args.warmup + args.steps, total)]
        rows = float(np.mean(seg_rows))
        per_launch += (rows * w.kv_row * 2 * 2 * 2 + w.n_seq * w.cap * 4
                       - w.n_seq * w.q_len * geo.kv_total * 2
                       + (w.n_seq * (w.q_len * geo.kv_total * 2 + w.q_len * 64 * 2 * 12)
                          + rows * 4) / w.n_layer)
    per_call = mean_bytes("ring_attn")
    attn_us = prof["k_ring_attn"]["avg_us"]
    merge_us = prof["k_ring_merge"]["avg_us"] or 0.0
    achieved = per_launch / (attn_us * 1e-6) / 1e9
    khash = kernel_source_hash()
    traffic = traffic_from_profiles(khash) if args.workload == WORKLOAD else None
    roof_attn = {"kernel": "k_ring_attn_fused" if fused else "k_ring_attn", "bound": "hbm",
                 "achieved": achieved,
                 "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                 "traffic": traffic, "bytes_per_launch": int(per_launch),
                 "avg_launch_us": attn_us}
    roofline = roof_attn
    if mirror:
        # the projection launch of a decode step reads every layer's wk and wv
        # once and the new rows' features (n <= a_step rows of d_model F16)
        seg_rows = [sum(n for _, _, _, _, n in steps_in[0][t // pool][0])
                    for t in range(args.warmup + args.steps, total)]
        proj_bytes = (2 * w.n_layer * w.kv_row * w.d_model * 2 +
                      float(np.mean(seg_rows)) * w.d_model * 2)
        proj_us = prof["k_ring_project"]["avg_us"]
        pa = proj_bytes / (proj_us * 1e-6) / 1e9
        roofline = {"kernel": "k_ring_project", "bound": "hbm", "achieved": pa,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": pa / HBM_PEAK_GBS,
                    "traffic": None, "bytes_per_launch": int(proj_bytes),
                    "avg_launch_us": proj_us}
    line = {
        "metric": METRIC if args.workload == WORKLOAD else
        f"ring step steps/s + achieved HBM GB/s, workload {args.workload}",
        "value": args.steps / elapsed,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded normal F16 rows; accepted counts drawn from the "
                "pages' 1422-verification share table)",
        "config": {"workload": args.workload, "step": step_mode,
                   "cap": w.cap, "q_len": w.q_len,
                   "n_head": w.n_head, "n_head_kv": w.n_head_kv, "head_dim": w.head_dim,
                   "n_layer": w.n_layer, "n_seq": w.n_seq, "kv_total": geo.kv_total,
                   "ring_pool": pool, "infinity_cache": "cold" if pool > 1 or ring_bytes > (256 << 20) else "warm",
                   "ring": split_desc},
        "roofline": roofline,
        "ring_attn": {"kernels": "k_ring_attn + k_ring_merge",
                      "avg_us": attn_us + merge_us,
                      "calls_per_s": 1e6 / (attn_us + merge_us),
                      "achieved_GBps": per_call / ((attn_us + merge_us) * 1e-6) / 1e9},
        "kernels": prof,
        **({"roofline_attn": roof_attn} if mirror else {}),
        "profiled_segment_steps_per_s": args.steps / elapsed_prof,
        "kernel_source_hash": khash,
    }
    if not args.no_cpu_baseline and args.workload == WORKLOAD:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
