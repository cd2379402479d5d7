#!/usr/bin/env python3
"""Throughput of the draft-KV ring step on one MI355X.

A step is one pass of the whole ring path for one sequence: ring_begin_step
(fold-in append with RoPE + slot_pos + window mask) and ring_attn (masked GQA
attention of the 8 noise queries over the 4096-slot ring, split-K + merge).
Workload: the draft-window decode stream (cap 4096, q_len 8, 32 query / 8 KV
heads x 128, F16), warmed by a 4096-token bulk prefill; synthetic seeded
inputs, already resident in device memory when timing starts.

The timed steps cycle through a pool of independent rings (default 32, about
680 MB) so that every step reads its ring from HBM, not from the 256 MB
Infinity Cache; ``--pool 1`` gives the cache-warm figure.

Prints one JSON line.  ``roofline`` is for the attention kernel, whose
duration comes from HIP events bound to its own dispatches during the timed
steps; ``cpu_baseline`` times the CPU oracle on a bounded sample of the same
stream.
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


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--pool", type=int, default=32,
                    help="independent rings cycled through (1 = Infinity-Cache warm)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB ten times (scale for the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the ring step has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        return 2

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

    w = W.WORKLOADS[WORKLOAD]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = W.commit_stream(w, 0)
    pool = max(1, args.pool)
    total = args.warmup + args.steps
    n_dec = -(-total // pool)                       # decode steps per ring
    if n_dec + 1 > len(stream):
        raise SystemExit(f"need {n_dec} decode steps per ring, stream has {len(stream) - 1}")

    # ---- inputs, generated on the host once and made resident on the GPU
    pos0 = np.arange(0, stream[0])
    k0 = torch.from_numpy(W.context_rows(w, 0, 0, W.T_K, pos0)[None]).to(dev)
    v0 = torch.from_numpy(W.context_rows(w, 0, 0, W.T_V, pos0)[None]).to(dev)
    steps_in = []
    for j in range(n_dec):
        c_prev, c = stream[j], stream[j + 1]
        pos = np.arange(c_prev, c)
        q, kn, vn = W.noise_inputs(w, 0, 0, j)
        steps_in.append(dict(
            committed=c, n=len(pos),
            k=torch.from_numpy(W.context_rows(w, 0, 0, W.T_K, pos)[None]).to(dev),
            v=torch.from_numpy(W.context_rows(w, 0, 0, W.T_V, pos)[None]).to(dev),
            q=torch.from_numpy(q[None]).to(dev), kn=torch.from_numpy(kn[None]).to(dev),
            vn=torch.from_numpy(vn[None]).to(dev)))
    out = torch.empty((1, w.q_len, w.n_head, w.head_dim), dtype=torch.float32, device=dev)

    rings = [R.Ring(cap=w.cap, q_len=w.q_len, n_head=w.n_head, n_head_kv=w.n_head_kv,
                    head_dim=w.head_dim, rope_base=w.rope_base, device=dev) for _ in range(pool)]
    s = torch.cuda.current_stream(dev).cuda_stream
    for r in rings:
        R.ring_begin_step(r.handle, 0, stream[0], k0.data_ptr(), v0.data_ptr(), len(pos0), s)
    torch.cuda.synchronize(dev)

    # pointer table of every step, so the loop does no tensor bookkeeping
    calls = []
    for t in range(total):
        r, j = rings[t % pool], t // pool
        x = steps_in[j]
        calls.append((r.handle, x["committed"], x["k"].data_ptr(), x["v"].data_ptr(), x["n"],
                      x["q"].data_ptr(), x["kn"].data_ptr(), x["vn"].data_ptr()))
    begin, attn, optr = R.ring_begin_step, R.ring_attn, out.data_ptr()

    def run(lo, hi):
        for t in range(lo, hi):
            h, c, kp, vp, n, qp, knp, vnp = calls[t]
            begin(h, 0, c, kp, vp, n, s)
            attn(h, 0, qp, knp, vnp, optr, s)

    run(0, args.warmup)
    torch.cuda.synchronize(dev)
    per_ring = -(-args.steps // pool) + 1
    for r in rings:
        r.profile_enable(per_ring)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    run(args.warmup, total)
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0

    prof = {}
    for kind, name in ((R.RING_KERNEL_STEP, "k_ring_step"), (R.RING_KERNEL_ATTN, "k_ring_attn"),
                       (R.RING_KERNEL_MERGE, "k_ring_merge")):
        n_l, ms = 0, 0.0
        for r in rings:
            a, b = r.profile_read(kind)
            n_l += a
            ms += b
        prof[name] = {"launches": n_l, "avg_us": (1e3 * ms / n_l) if n_l else None}

    geo = rings[0].geo
    split_desc = rings[0].describe()
    for r in rings:
        r.close()

    nbytes = algorithmic_bytes(w, w.cap, geo.kv_total)
    attn_us = prof["k_ring_attn"]["avg_us"]
    merge_us = prof["k_ring_merge"]["avg_us"] or 0.0
    achieved = nbytes["attn_kernel"] / (attn_us * 1e-6) / 1e9
    khash = kernel_source_hash()
    traffic = traffic_from_profiles(khash)
    line = {
        "metric": METRIC,
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
        "data": "synthetic (seeded N(0,0.5) F16 rows; accepted counts drawn from the "
                "pages' 1422-verification share table)",
        "config": {"workload": WORKLOAD, "cap": w.cap, "q_len": w.q_len, "n_head": w.n_head,
                   "n_head_kv": w.n_head_kv, "head_dim": w.head_dim, "n_layer": w.n_layer,
                   "n_seq": w.n_seq, "kv_total": geo.kv_total, "ring_pool": pool,
                   "infinity_cache": "cold" if pool > 1 else "warm", "ring": split_desc},
        "roofline": {"kernel": "k_ring_attn", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "bytes_per_launch": nbytes["attn_kernel"],
                     "avg_launch_us": attn_us},
        "ring_attn": {"kernels": "k_ring_attn + k_ring_merge",
                      "avg_us": attn_us + merge_us,
                      "calls_per_s": 1e6 / (attn_us + merge_us),
                      "achieved_GBps": nbytes["ring_attn"] / ((attn_us + merge_us) * 1e-6) / 1e9},
        "kernels": prof,
        "kernel_source_hash": khash,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
