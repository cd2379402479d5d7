"""The profiling build's per-wave timestamps (ring_profile_stamps), on the GPU.

libringkv_stamps.so is the same sources built with RING_WAVE_STAMPS; the
bench's stamps mode loads it in a process of its own (RINGKV_LIB=stamps) and
reads every wave's clock readings.  Checked here: each stamped kernel records
one entry per wave of its launch, a wave's points come in the order the
kernel passes them, and the product library, built without stamps, refuses
the call with RING_ESTATE and launches nothing.
"""

import json
import os
import subprocess
import sys

import numpy as np
import pytest

import workload as W

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_product_library_refuses_stamps():
    import draft_model_kv_amd as R
    from draft_model_kv_amd import ring as rk
    w = W.WORKLOADS["tiny_ring"]
    ring = R.Ring(cap=w.cap, q_len=w.q_len, n_head=w.n_head, n_head_kv=w.n_head_kv,
                  head_dim=w.head_dim, rope_base=w.rope_base)
    try:
        with pytest.raises(R.RingError) as e:
            R.ring_profile_stamps(ring.handle, R.RING_STAMPS_ATTN, 4)
        assert e.value.code == rk.RING_ESTATE
    finally:
        ring.close()


def _stamps(args):
    print("stamps run:", " ".join(args), flush=True)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                         capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    return json.loads(res.stdout.strip().splitlines()[-1])


@pytest.mark.parametrize("step", ["fused", "eager"])
def test_stamps_of_the_decode_step(step):
    """cap 4096 decode steps: the attention's 1024 waves (32 splits x 8 KV heads
    x 4 waves) and the merge's 512 are all recorded, every wave's points are
    in order, and the merge starts after the attention's last wave ends."""
    res = _stamps(["--stamps", "4", "--warmup", "4", "--pool", "4", "--no-cpu-baseline",
                   "--step", step])
    st = res["stamps"]
    assert st["clock_khz"] > 0
    assert st["attn_placement"]["waves"] == 1024
    for name in ("attn", "merge"):
        med = np.array(st[name]["median_wave_us"])
        late = np.array(st[name]["latest_wave_us"])
        assert len(med) == len([p for p in st[name]["points"]])
        assert (np.diff(med) >= 0).all(), (name, med)
        assert (np.diff(late) >= 0).all(), (name, late)
        assert (late >= med).all()
    assert st["merge"]["median_wave_us"][0] >= st["attn"]["latest_wave_us"][-1]


def test_stamps_of_the_projection():
    """The mirror workload's projection (1280 two-wave work-groups): its points
    in order as well."""
    res = _stamps(["--workload", "mirror_stream", "--stamps", "2", "--warmup", "2",
                   "--pool", "2", "--no-cpu-baseline"])
    med = np.array(res["stamps"]["proj"]["median_wave_us"])
    assert len(med) == 6 and (np.diff(med) >= 0).all(), med
