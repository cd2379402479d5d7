"""bench.py's host logic on the CPU: the one-GPU refusal, the algorithmic
bytes its roofline divides by, the counter summary parsing and the rule that
drops stale traffic figures."""

import csv
import json
import os
import subprocess
import sys

import pytest

import bench
import workload as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_algorithmic_bytes_decode_stream():
    """cap 4096, q_len 8, 32/8 heads x 128: visible K and V rows (window plus
    noise block) 4104 x 1024 x 2 B x 2, queries 8 x 32 x 128 x 2 B, noise K and
    V 2 x 8 x 1024 x 2 B, mask 8 x 4128 x 2 B, output 8 x 32 x 128 x 4 B."""
    w = W.WORKLOADS["decode_stream"]
    b = bench.algorithmic_bytes(w, 4096, 4128)
    assert b["kv"] == 16_809_984
    assert b["q"] == 65_536
    assert b["noise"] == 32_768
    assert b["mask"] == 66_048
    assert b["attn_kernel"] == 16_974_336
    assert b["ring_attn"] == 16_974_336 + 131_072


def test_algorithmic_bytes_follow_the_window():
    """A window below cap reads only its own rows; GQA 8 doubles the queries."""
    w = W.WORKLOADS["large_window"]
    small = bench.algorithmic_bytes(w, 1000, 32800)
    full = bench.algorithmic_bytes(w, 32768, 32800)
    assert full["kv"] - small["kv"] == (32768 - 1000) * w.kv_row * 4
    assert small["q"] == 8 * 64 * 128 * 2


def _write_counter_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name",
                                            "Counter_Value"])
        wr.writeheader()
        wr.writerows(rows)


def test_counter_summary_averages_per_dispatch(tmp_path):
    """FETCH_SIZE rows of the kernel (and only of the asked grid size) are
    averaged; other kernels and counters are ignored."""
    _write_counter_csv(str(tmp_path / "pmc" / "run" / "x_counter_collection.csv"), [
        {"Kernel_Name": "ringkv::k_ring_attn<1>", "Grid_Size": 65536,
         "Counter_Name": "FETCH_SIZE", "Counter_Value": 100.0},
        {"Kernel_Name": "ringkv::k_ring_attn<1>", "Grid_Size": 65536,
         "Counter_Name": "FETCH_SIZE", "Counter_Value": 300.0},
        {"Kernel_Name": "ringkv::k_ring_attn<1>", "Grid_Size": 131072,
         "Counter_Name": "FETCH_SIZE", "Counter_Value": 900.0},
        {"Kernel_Name": "ringkv::k_ring_merge<8>", "Grid_Size": 32768,
         "Counter_Name": "FETCH_SIZE", "Counter_Value": 7.0},
        {"Kernel_Name": "ringkv::k_ring_attn<1>", "Grid_Size": 65536,
         "Counter_Name": "WRITE_SIZE", "Counter_Value": 5.0},
    ])
    v, n = bench._kib_per_dispatch(str(tmp_path), "pmc", "FETCH_SIZE",
                                   lambda k: "k_ring_attn" in k, 65536)
    assert (v, n) == (200.0, 2)
    v, n = bench._kib_per_dispatch(str(tmp_path), "pmc", "FETCH_SIZE",
                                   lambda k: "k_ring_attn" in k)
    assert n == 3 and v == pytest.approx(1300.0 / 3)
    with pytest.raises(ValueError):
        bench._kib_per_dispatch(str(tmp_path), "pmc", "FETCH_SIZE",
                                lambda k: "k_ring_project" in k)


def test_traffic_is_dropped_when_the_kernels_changed(tmp_path, monkeypatch):
    """The committed traffic figure counts only for the kernel source it was
    measured on."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "ring_attn_decode_stream_traffic.json").write_text(
        json.dumps({"kernel_source_hash": "abc", "hbm_bytes_per_launch": 123.0}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profiles("abc") == 123.0
    assert bench.traffic_from_profiles("def") is None


def test_bench_line_reader(tmp_path):
    """The summaries take the bench's JSON line from a log that also holds
    other output."""
    (tmp_path / "run.log").write_text("warning: x\n" + json.dumps(
        {"metric": "m", "value": 1.0}) + "\ntrailing\n")
    assert bench._bench_line(str(tmp_path), "run") == {"metric": "m", "value": 1.0}
    assert bench._bench_line(str(tmp_path), "missing") is None


def test_hardware_counter_summary(tmp_path, monkeypatch):
    """The counter summary averages each counter per dispatch of each kernel
    group and derives its ratios from those averages (wait share, cycles per
    wave, L2 hit rate); counters a pass did not collect show as '-'."""
    out = tmp_path / "out"
    for run, ctrs in bench.COUNTER_PASSES.items():
        rows = []
        for k, kname in enumerate(("ringkv::k_ring_attn_fused<1, 4, 1, true>",
                                   "ringkv::k_ring_floor<1>")):
            for disp in range(2):
                for c in ctrs:
                    value = {"SQ_WAVES": 1024.0, "SQ_WAVE_CYCLES": 4000.0 + 1000 * k,
                             "SQ_WAIT_ANY": 2000.0 + 2000 * disp, "TCC_HIT": 30.0,
                             "TCC_MISS": 70.0}.get(c, 1.0)
                    rows.append({"Kernel_Name": kname, "Grid_Size": 65536,
                                 "Counter_Name": c, "Counter_Value": value})
        _write_counter_csv(str(out / run / "x" / "run_counter_collection.csv"), rows)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    path = bench.summarize_counters(str(out), "hash0")
    text = (tmp_path / path).read_text()
    assert "Kernel source hash: `hash0`" in text
    lines = {ln.split(" | ")[0].lstrip("| "): ln for ln in text.splitlines() if ln.startswith("| ")}
    # attention: SQ_WAIT_ANY averages (2000 + 4000) / 2 over 4000 wave cycles
    wait = lines["share of wave cycles waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES)"].split(" | ")
    assert wait[1] == "0.750" and wait[3] == "0.600" and wait[2] == "-"
    cyc = lines["cycles per wave (SQ_WAVE_CYCLES x 4 / SQ_WAVES)"].split(" | ")
    assert cyc[1] == "15.62"
    hit = lines["L2 hit rate (TCC_HIT / (TCC_HIT + TCC_MISS))"].split(" | ")
    assert hit[1] == "0.300"


def _stamp_records(n_waves, entry, points, hw=None, xcc=None):
    """[waves][10] records: stamps entry + points[p] (ticks), HW_ID, XCC_ID."""
    import numpy as np
    r = np.zeros((8192, 10), dtype=np.uint64)
    for w in range(n_waves):
        for p, d in enumerate(points):
            r[w, p] = entry[w] + d if d is not None else 0
        r[w, 8] = 0 if hw is None else hw[w]
        r[w, 9] = 0 if xcc is None else xcc[w]
    return r


def test_stamp_step_statistics():
    """Per-wave stamps of one step (100 MHz clock: 10 ns per tick): the
    attention's points count from its first wave's entry, the merge's from
    the attention's first wave too; the median and the latest wave per point;
    waves that did not run (entry 0) are left out; placement: XCC_ID against
    work-group index mod 8, and compute units told apart by XCC and HW_ID's
    cu/sh/se bits (not its wave and SIMD bits)."""
    import numpy as np
    khz = 100_000
    # 8 waves = 2 work-groups of 4; entries 1000, 1010, ... ticks
    entry = [1000 + 10 * w for w in range(8)]
    pts = [0, 5, 20, 30, 40, 50, 60, 70]
    # work-group 0 on XCD 0, work-group 1 on XCD 1; waves of a group on one
    # compute unit (cu 3 / cu 5), different SIMD and wave ids
    hw = [(3 << 8) | (w & 3) << 4 | w for w in range(4)] + [(5 << 8) | (w & 3) << 4 for w in range(4)]
    xcc = [0] * 4 + [1] * 4
    attn = _stamp_records(8, entry, pts, hw, xcc)
    merge = _stamp_records(2, [1200, 1300], [0, 10, 20, 30, 40, None, None, 90])
    st = bench.stamp_step_stats({"attn": attn, "merge": merge}, khz)
    a = st["attn"]
    # point p of wave w: 10 w + pts[p] ticks after the first entry; median
    # over the 8 waves of 10 w is 35, the latest 70
    assert np.allclose(a["med"], [0.01 * (35 + d) for d in pts])
    assert np.allclose(a["max"], [0.01 * (70 + d) for d in pts])
    # the merge's six points (5 and 6 unused), counted from the attention's
    # first wave: its waves enter 200 and 300 ticks later
    m = st["merge"]
    used = (0, 10, 20, 30, 40, 90)
    assert np.allclose(m["med"], [0.01 * (250 + d) for d in used])
    assert np.allclose(m["max"], [0.01 * (300 + d) for d in used])
    pl = st["placement"]
    assert pl["waves"] == 8 and pl["cus"] == 2 and pl["max_waves_per_cu"] == 4
    assert pl["xcd_is_block_mod_8"] == 1.0
    # a work-group off its XCD shows in the fraction
    attn2 = _stamp_records(8, entry, pts, hw, [0] * 4 + [2] * 4)
    assert bench.stamp_step_stats({"attn": attn2}, khz)["placement"]["xcd_is_block_mod_8"] == 0.5


def test_stamp_summary_takes_medians_over_steps():
    import numpy as np
    khz = 100_000
    steps = []
    for k in range(3):
        a = _stamp_records(4, [0 + 1, 2, 3, 4], [0, 10 * (k + 1), 20, 30, 40, 50, 60, 70])
        steps.append(bench.stamp_step_stats({"attn": a}, khz))
    out = bench.stamp_summary(steps, khz)
    assert out["steps"] == 3 and "merge" not in out
    assert len(out["attn"]["points"]) == 8
    # point 1 is 10 (k + 1) ticks after each wave's entry: median over steps 20
    assert np.isclose(out["attn"]["median_wave_us"][1], 0.01 * (1.5 + 20))
    assert out["attn_placement"]["waves"] == 4
