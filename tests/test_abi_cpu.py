"""The C ABI library on the CPU: it loads, exports the header's functions, and
its pure-host calls (geometry, step planner, validation) match the oracle.
No kernel is launched here."""

import os
import random
import re

import numpy as np
import pytest

import oracle.ring_oracle as ro

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ring_kv.h")

rk = pytest.importorskip("draft_model_kv_amd.ring",
                         reason="libringkv.so not built (python draft_model_kv_amd/build.py)")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(ring_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_exports():
    assert header_functions() == sorted(rk.EXPORTS)


def test_binding_constants_match_the_header():
    """Every RING_* integer constant the header defines has the same value
    in the Python binding (error codes, kernel kinds, floor kinds)."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    defs = dict(re.findall(r"^#define\s+(RING_\w+)\s+\(?(-?\d+)\)?\s*$", text, flags=re.M))
    assert len(defs) >= 20
    for name, value in defs.items():
        if name == "RING_KV_H":
            continue
        assert hasattr(rk, name), name
        assert getattr(rk, name) == int(value), name


def test_library_exports_every_header_function():
    import ctypes
    lib = ctypes.CDLL(rk.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name


def test_stamps_build_exports_every_header_function():
    """The profiling build (per-wave timestamps) is the same ABI."""
    import ctypes
    path = os.path.join(os.path.dirname(rk.LIB_PATH), "libringkv_stamps.so")
    if not os.path.exists(path):
        pytest.skip("libringkv_stamps.so not built")
    lib = ctypes.CDLL(path)
    for name in header_functions():
        assert hasattr(lib, name), name


@pytest.mark.parametrize("cap,q_len,n_head,n_head_kv,n_layer",
                         [(4096, 8, 32, 8, 5), (64, 8, 32, 8, 1), (32768, 8, 64, 8, 1),
                          (1, 1, 8, 8, 1), (100, 3, 16, 4, 2), (23, 8, 32, 8, 1)])
def test_geometry_matches_oracle(cap, q_len, n_head, n_head_kv, n_layer):
    g = rk.ring_query_geometry(rk.make_config(cap, q_len, n_head, n_head_kv, 128, n_layer))
    o = ro.geometry(cap, q_len, 128, n_head_kv)
    assert (g.a_step, g.trash_slot, g.kv_total, g.kv_row) == (o.a_step, o.trash_slot, o.kv_total, o.kv_row)
    assert g.kv_bytes_per_layer * n_layer == ro.ring_bytes(n_layer, o.kv_row, o.kv_total)
    assert g.workspace_bytes >= 2 * g.kv_bytes_per_layer * 0 + g.kv_bytes_per_layer * n_layer


def test_describe_format_has_the_log_fields():
    # the geometry behind the Luce log line of the ring notes (section 11, Test 4)
    g = rk.ring_query_geometry(rk.make_config(4096, 8, 32, 8, 128, 5))
    assert (g.kv_total, g.a_step) == (4128, 18)
    assert round(5 * g.kv_bytes_per_layer / 2**20, 1) == 80.6


@pytest.mark.parametrize("bad", [
    dict(cap=0), dict(q_len=0), dict(q_len=33), dict(head_dim=64), dict(n_head=30),
    dict(n_head_kv=0), dict(n_head=128, n_head_kv=8), dict(n_layer=0), dict(n_seq=0),
    dict(n_seq=65), dict(rope_base=1.0), dict(rope_base=float("inf")),
    dict(swa_window=-1, swa_layers=1), dict(swa_window=16), dict(swa_layers=1),
    dict(swa_window=16, swa_layers=0b10),
])
def test_invalid_config_rejected(bad):
    kw = dict(cap=64, q_len=8, n_head=32, n_head_kv=8, head_dim=128, n_layer=1, n_seq=1,
              rope_base=1e6)
    kw.update(bad)
    with pytest.raises(rk.RingError) as e:
        rk.ring_query_geometry(rk.make_config(**kw))
    assert e.value.code == rk.RING_EINVAL
    assert rk.ring_last_error()


def test_sliding_window_config_accepted():
    """A sliding-window layer set below n_layer is valid and adds one mask."""
    base = rk.ring_query_geometry(rk.make_config(64, n_layer=3))
    g = rk.ring_query_geometry(rk.make_config(64, n_layer=3, swa_window=16, swa_layers=0b101))
    assert (g.a_step, g.trash_slot, g.kv_total) == (base.a_step, base.trash_slot, base.kv_total)
    assert g.workspace_bytes >= base.workspace_bytes + 8 * base.kv_total * 2
    g = rk.ring_query_geometry(rk.make_config(64, n_layer=70, swa_window=1, swa_layers=1 << 63))
    assert g.kv_total == base.kv_total


def test_planner_state_validation():
    cfg = rk.make_config(64)
    for state in [(-1, 0), (10, 11), (200, 100)]:
        with pytest.raises(rk.RingError) as e:
            rk.ring_plan_from_state(cfg, state[0], state[1], 100)
        assert e.value.code == rk.RING_EINVAL
    with pytest.raises(rk.RingError) as e:
        rk.ring_plan_from_state(cfg, 0, 0, -1)
    assert e.value.code == rk.RING_ERANGE
    with pytest.raises(rk.RingError) as e:
        rk.ring_plan_from_state(cfg, 0, 0, 2**31 - 8)
    assert e.value.code == rk.RING_ERANGE


def _compare_stream(cap, q_len, commits):
    cfg = rk.make_config(cap, q_len)
    g = ro.geometry(cap, q_len, 128, 8)
    next_pos, held_lo = 0, 0
    for c in commits:
        lp, ap = rk.ring_plan_from_state(cfg, next_pos, held_lo, c)
        op = ro.plan_step(g, c, next_pos, held_lo)
        assert (lp.win, lp.lo, lp.start, lp.n_new, bool(lp.bulk)) == \
            (op.win, op.lo, op.start, op.n_new, op.bulk), (cap, q_len, c)
        if op.bulk:
            assert ap is None and lp.n_chunks == len(op.chunks)
        else:
            assert list(ap) == op.ap_rows
        next_pos, held_lo = c, op.lo


def test_planner_matches_oracle_random_streams():
    rnd = random.Random(1)
    for cap in list(range(1, 12)) + [64, 100, 4096]:
        for q_len in (1, 2, 8, 16):
            c, commits = 0, []
            for _ in range(80):
                c = max(0, c + rnd.choice([-2 * cap, -3, -1, 0, 1, 2, 3, 5, 8, 9, 19, cap, 3 * cap + 1]))
                commits.append(c)
            _compare_stream(cap, q_len, commits)


def test_planner_on_workload_streams():
    import workload as W
    for name in ("tiny_ring", "decode_stream", "long_prompt_wrap", "batched_seqs"):
        w = W.WORKLOADS[name]
        for seq in range(min(w.n_seq, 4)):
            _compare_stream(w.cap, w.q_len, W.commit_stream(w, seq))


def test_ring_init_without_device_fails_cleanly():
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    with pytest.raises(rk.RingError) as e:
        rk.ring_init(rk.make_config(64))
    assert e.value.code == rk.RING_EDEVICE


@pytest.mark.parametrize("d_model", [-256, 100, 255, 65536 + 256])
def test_invalid_mirror_width_rejected(d_model):
    with pytest.raises(rk.RingError) as e:
        rk.ring_query_geometry(rk.make_config(64, d_model=d_model))
    assert e.value.code == rk.RING_EINVAL


def test_feature_mirror_sizes_the_workspace():
    """A feature mirror adds cap * d_model F16 per sequence, the fp32
    projection scratch (n_layer * d_model / 256 slices of 64 rows x 2 kv_row)
    and room for the registered weights (wk, wv F16 and k_norm fp32)."""
    base = rk.ring_query_geometry(rk.make_config(4096, n_layer=5, n_seq=2))
    g = rk.ring_query_geometry(rk.make_config(4096, n_layer=5, n_seq=2, d_model=2048))
    need = (2 * 4096 * 2048 * 2 + 5 * (2048 // 256) * 64 * 2 * 1024 * 4
            + 5 * 2 * 1024 * 2048 * 2 + 5 * 128 * 4)   # + registered weights, k_norm
    assert need <= g.workspace_bytes - base.workspace_bytes <= need + 1024


def test_mirror_needs_at_most_16_kv_heads():
    rk.ring_query_geometry(rk.make_config(64, n_head=16, n_head_kv=16, d_model=256))
    with pytest.raises(rk.RingError) as e:
        rk.ring_query_geometry(rk.make_config(64, n_head=32, n_head_kv=32, d_model=256))
    assert e.value.code == rk.RING_EINVAL


def _absurd_config():
    """Every size at its limit: 64 sequences x 1024 layers of 2^26-slot rings."""
    return rk.make_config(1 << 26, 8, 32, 8, 128, n_layer=1024, n_seq=64)


def test_absurd_cap_geometry_is_exact():
    """The geometry of the largest accepted ring is computed without overflow:
    2 (K, V) x kv_row x kv_total x 2 B per (sequence, layer)."""
    g = rk.ring_query_geometry(_absurd_config())
    kv_total = ((1 << 26) + 8 + 1 + 31) // 32 * 32
    assert g.kv_total == kv_total
    assert g.kv_bytes_per_layer == 2 * 1024 * kv_total * 2
    assert g.workspace_bytes >= 64 * 1024 * g.kv_bytes_per_layer > 2 ** 53


def _rss_bytes() -> int:
    with open("/proc/self/statm") as f:
        return int(f.read().split()[1]) * os.sysconf("SC_PAGE_SIZE")


def test_absurd_cap_small_workspace_is_enomem_and_leaks_nothing():
    """A caller workspace smaller than the geometry's workspace_bytes is
    refused with RING_ENOMEM before any device call (so this runs without a
    GPU), and the host state of a refused ring_init is released: 5000
    refusals leave the resident set within 4 MiB."""
    cfg = _absurd_config()
    fake = 1 << 20   # 256-byte aligned address, never dereferenced
    with pytest.raises(rk.RingError) as e:
        rk.ring_init(cfg, workspace=fake, workspace_bytes=1 << 30)
    assert e.value.code == rk.RING_ENOMEM
    assert "workspace" in rk.ring_last_error()
    for _ in range(200):   # let allocator pools reach their steady size first
        with pytest.raises(rk.RingError):
            rk.ring_init(cfg, workspace=fake, workspace_bytes=1 << 30)
    before = _rss_bytes()
    for _ in range(5000):
        with pytest.raises(rk.RingError):
            rk.ring_init(cfg, workspace=fake, workspace_bytes=1 << 30)
    assert _rss_bytes() - before < 4 << 20


def test_misaligned_workspace_is_einval():
    with pytest.raises(rk.RingError) as e:
        rk.ring_init(rk.make_config(64), workspace=(1 << 20) + 16, workspace_bytes=1 << 30)
    assert e.value.code == rk.RING_EINVAL
