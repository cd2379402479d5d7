"""HIP ring path against the CPU oracle, element by element (needs the GPU).

Index work (append plan, slot_pos, mask) must be bit-exact; ring K rows within
one F16 ulp of the oracle's rounded RoPE (V exact, empty slots zero);
attention outputs within |gpu - ref| <= 2e-3 + 1e-2 |ref| of the
fp32-accumulated oracle.
"""

import dataclasses
import sys

import numpy as np
import pytest

import workload as W
from tests.harness import Driver, check_close, run_workload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(name="edge", **kw):
    base = dict(name=name, seed=100, cap=64, q_len=8, n_head=32, n_head_kv=8)
    base.update(kw)
    return W.Workload(**base)


def run_steps(d, commits, layers=None, check_rows=True, seq=0):
    layers = range(d.w.n_layer) if layers is None else layers
    stats = []
    for t, c in enumerate(commits):
        d.step(seq, c)
        d.check_index(seq)
        if check_rows:
            for layer in layers:
                d.check_rows(seq, layer)
        for layer in layers:
            stats.append(d.check_attn(layer, d.n_attn))
    return stats


def test_init_state_and_committed_zero():
    d = Driver(small(cap=64))
    d.check_index(0)                 # slot_pos = -1, only the noise visible
    d.check_rows(0, 0)               # every ring row zero
    d.check_attn(0, 0)               # attention with no context at all
    d.close()


def test_single_key_closed_form():
    """q_len = 1, committed = 0: the only visible key is the noise row, out = its V."""
    w = small(cap=40, q_len=1)
    d = Driver(w)
    out, q, kn, vn = d.attn(0, 0)
    for h in range(w.n_head):
        g = h // w.group
        assert np.array_equal(out[0, 0, h], vn[0, 0, g * 128:(g + 1) * 128].astype(np.float32))
    d.close()


def test_tiny_ring_every_step():
    w = W.WORKLOADS["tiny_ring"]
    d = Driver(w)
    stream = W.commit_stream(w, 0)
    say("tiny_ring", len(stream), "steps, cap", w.cap)
    stats = run_steps(d, stream)
    say("tiny_ring worst", max(s["max_ratio"] for s in stats))
    d.close()


@pytest.mark.parametrize("commits", [
    [61, 69, 70, 77],                  # wrap inside one fold-in (slots 61..63, 0..4)
    [128, 129, 136, 192, 200],         # prefill ending at 2 cap, then exact multiples
    [60, 66, 70],                      # committed crosses cap
    [100, 118, 137, 138],              # n_new == a_step (fold-in, no pad), then a_step + 1 (bulk)
    [5, 5, 6, 6],                      # zero-row steps (all pads)
    [200, 150, 151, 300, 290, 291],    # rewinds past what the ring holds
    [50, 40, 45, 20, 64, 70],          # rewinds inside the window
], ids=["wrap_in_fold", "multiple_of_cap", "cross_cap", "a_step_threshold", "zero_rows",
        "rewind_far", "rewind_near"])
def test_edge_streams(commits):
    d = Driver(small(cap=64))
    run_steps(d, commits)
    d.close()


def test_ragged_cap_and_short_block():
    """cap not a multiple of 32, q_len 3 (noise block inside a partial tile)."""
    d = Driver(small(cap=100, q_len=3, n_head=16, n_head_kv=4))
    run_steps(d, [7, 57, 99, 100, 101, 130, 205, 206, 240])
    d.close()


@pytest.mark.parametrize("row_blocks,n_split", [(True, None), (False, None), (True, 1),
                                                (True, 3)],
                         ids=["row_blocks", "one_workgroup", "row_blocks_one_split",
                              "row_blocks_3_splits"])
def test_gqa8_outliers_two_query_blocks(row_blocks, n_split):
    """64 query heads over 8 KV heads: 64 queries per KV head, +-30 outliers;
    the two 32-row query blocks in work-groups of their own (default) or in
    one work-group."""
    w = small(cap=256, n_head=64, sigma=1.0, outlier_p=0.01, seed=104)
    d = Driver(w, n_split=n_split, row_blocks=row_blocks)
    run_steps(d, [300, 301, 305, 313, 330])
    d.close()


@pytest.mark.parametrize("n_split", [2, 3, 7, 16])
@pytest.mark.parametrize("n_head,row_blocks", [(32, None), (64, True), (64, False)],
                         ids=["gqa4", "gqa8_row_blocks", "gqa8_one_workgroup"])
def test_merge_in_launch(n_split, n_head, row_blocks):
    """RING_ATTN_MERGE=kernel: the cross-split merge inside the attention
    launch (waves that stream several tiles, 2..16 splits); the work-group
    that draws the last ticket of its (sequence x KV head, row block) merges
    every split's partial.  Split counts that divide the 128 ring tiles
    evenly and not; 32 or 64 queries per KV head, +-30 outliers; windows
    that wrap the ring end."""
    w = small(cap=4096, n_head=n_head, sigma=1.0, outlier_p=0.01, seed=120 + n_split)
    d = Driver(w, n_split=n_split, row_blocks=row_blocks, merge="kernel")
    run_steps(d, [4000, 4001, 4096, 4100, 4111, 5000, 5003])
    d.close()


def test_floor_kinds_leave_the_ring_as_it_was():
    """Every ring_profile_floor kind (profiling only) on both layers between
    steps: the floors write only the split partials, which every attention
    launch rewrites, and a buffer of their own, so the following steps still
    match the oracle.  Bounded barrier waits all end by their tickets; the
    projection kind needs registered weights; unknown kinds are refused."""
    import torch
    from draft_model_kv_amd import ring as rk
    s = torch.cuda.current_stream().cuda_stream
    d = Driver(small(cap=1024, n_layer=2, seed=150), n_split=4)
    run_steps(d, [900, 901, 909])
    kinds = (rk.RING_FLOOR_EMPTY, rk.RING_FLOOR_READ, rk.RING_FLOOR_READ_LOCKSTEP,
             rk.RING_FLOOR_PARTIALS, rk.RING_FLOOR_TWO_LAUNCH, rk.RING_FLOOR_LAST_ARRIVER,
             rk.RING_FLOOR_BARRIER, rk.RING_FLOOR_MATRIX_MATH, rk.RING_FLOOR_VECTOR_MATH)
    for k in kinds:
        for layer in range(2):
            rk.ring_profile_floor(d.ring.handle, layer, k, s)
    torch.cuda.synchronize()
    assert rk.ring_profile_floor_timeouts(d.ring.handle) == 0
    for kind, code in ((rk.RING_FLOOR_PROJ_READ, rk.RING_ESTATE),
                       (rk.RING_FLOOR_SHARED_TILES, rk.RING_EINVAL), (12, rk.RING_EINVAL),
                       (-1, rk.RING_EINVAL)):
        with pytest.raises(rk.RingError) as e:
            rk.ring_profile_floor(d.ring.handle, 0, kind, s)
        assert e.value.code == code, kind
    with pytest.raises(rk.RingError) as e:
        rk.ring_profile_floor(d.ring.handle, 2, rk.RING_FLOOR_READ, s)
    assert e.value.code == rk.RING_ERANGE
    run_steps(d, [910, 925, 1030, 1031])
    d.close()


def test_shared_tile_floor_leaves_the_ring_as_it_was():
    """The shared-tile floor (64 queries per KV head: two query blocks, eight
    waves per work-group sharing each tile through LDS) between steps of a
    GQA-8 ring whose waves stream several tiles, a ragged split among them;
    the following steps still match the oracle."""
    import torch
    from draft_model_kv_amd import ring as rk
    s = torch.cuda.current_stream().cuda_stream
    d = Driver(small(cap=2000, n_head=64, seed=151), n_split=3)
    run_steps(d, [1900, 1903, 2100])
    for _ in range(3):
        rk.ring_profile_floor(d.ring.handle, 0, rk.RING_FLOOR_SHARED_TILES, s)
    torch.cuda.synchronize()
    run_steps(d, [2101, 2109, 2500])
    d.close()


@pytest.mark.parametrize("n_split", [3, 5])
def test_tile_walk_start_ragged_splits(n_split):
    """Waves that stream several tiles start their split's walk at an
    offset of their own (a multiple of 4 tiles per unit and split, wrapping
    inside the split): splits of 43/42 or 26/24 tiles, so the offset wraps
    at ragged ends, on a full layer and a sliding-window layer whose window
    wraps the ring end (the split's tiles themselves circular)."""
    w = small(cap=4096, n_layer=2, swa_window=1000, swa_layers=0b10, seed=140 + n_split)
    d = Driver(w, n_split=n_split)
    run_steps(d, [4000, 4001, 4096, 4100, 4567, 5003, 8190, 8193])
    d.close()


@pytest.mark.parametrize("row_blocks", [True, False], ids=["row_blocks", "one_workgroup"])
def test_long_noise_block_two_query_blocks(row_blocks):
    """q_len 16 with GQA 4 (m = 64): several rope-table passes, noise rows
    spread over more waves, a ragged cap, two query blocks."""
    w = small(cap=200, q_len=16, n_head=32, seed=110)
    d = Driver(w, row_blocks=row_blocks)
    run_steps(d, [150, 151, 170, 203, 230, 231])
    d.close()


def test_long_noise_block_long_waves():
    """q_len 16 with GQA 4 and one split per KV head: waves stream several
    tiles (the kernel that keeps the next tile in flight) with the noise
    rows of the long block on the same waves."""
    w = small(cap=1000, q_len=16, n_head=32, seed=111)
    d = Driver(w, n_split=1)
    run_steps(d, [600, 601, 617, 990, 1003, 1020])
    d.close()


@pytest.mark.parametrize("q_len,n_head,n_head_kv", [
    (8, 8, 8),      # group 1: one query head per KV head
    (1, 16, 8),     # group 2, a one-row noise block
    (3, 16, 1),     # one KV head for 16 query heads (m = 48, a ragged second block;
                    # one unit, so the work-groups are not pinned to XCDs)
    (13, 24, 8),    # group 3, q_len 13 (m = 39: a ragged second query block)
], ids=["g1_q8", "g2_q1", "g16_q3", "g3_q13"])
@pytest.mark.parametrize("deferred", [False, True], ids=["eager", "fused"])
def test_head_groupings(q_len, n_head, n_head_kv, deferred):
    """Group sizes and noise-block lengths the headline shape does not
    have: every quotient the kernels take by a launch constant (query row
    by group, unit by KV heads, work-group by splits and row blocks) with
    divisors other than the headline's."""
    w = small(cap=160, q_len=q_len, n_head=n_head, n_head_kv=n_head_kv,
              seed=120 + q_len + n_head + n_head_kv)
    d = Driver(w)
    for c in [90, 91, 97, 160, 171, 172]:
        d.step(0, c, deferred=deferred)
        d.check_attn_layers(c)
        d.check_index(0)
        d.check_rows(0, 0)
    d.close()


@pytest.mark.parametrize("cap", [1, 5, 31])
@pytest.mark.parametrize("deferred", [False, True], ids=["eager", "fused"])
def test_degenerate_caps(cap, deferred):
    """Rings smaller than one 32-slot tile and than the noise block (cap 1:
    every step overwrites the one slot; cap 5 and 31: wraps inside every
    fold-in), with rewinds and a bulk step."""
    w = small(name="tiny_caps", cap=cap, seed=160 + cap)
    d = Driver(w)
    commits = [0, 1, 3, 4, 12, 13, 7, 9, 40, 41, 48, 30, 31]
    for c in commits:
        d.step(0, c, deferred=deferred)
        d.check_attn_layers(c)
        d.check_index(0)
        d.check_rows(0, 0)
    d.close()


def test_largest_noise_block_and_sequence_count():
    """q_len 32 with two query heads per KV head (64 queries, the most a KV
    head takes), then 64 sequences (the most a ring holds) in one batched
    append and one attention launch."""
    w = small(cap=96, q_len=32, n_head=16, n_head_kv=8, seed=170)
    d = Driver(w)
    run_steps(d, [40, 41, 60, 97, 130, 131])
    d.close()
    w = small(cap=64, n_seq=64, seed=171)
    d = Driver(w)
    for t, base in enumerate([30, 31, 70, 75]):
        for seq in range(w.n_seq):
            d.step(seq, base + seq % 7 + (seq // 7) * t)
        for seq in (0, 17, 63):
            d.check_index(seq)
            d.check_rows(seq, 0)
        d.check_attn(0, t)
    d.close()


def test_multi_seq_multi_layer():
    w = small(cap=128, n_layer=2, n_seq=3, seed=105)
    d = Driver(w)
    plan = {0: [10, 11, 19, 140], 1: [500, 501, 509, 510], 2: [127, 128, 129, 136]}
    for t in range(4):
        for seq in range(3):
            d.step(seq, plan[seq][t])
            d.check_index(seq)
            for layer in range(2):
                d.check_rows(seq, layer)
        for layer in range(2):
            d.check_attn(layer, t)
    d.close()


@pytest.mark.parametrize("swa,commits", [
    (5, [61, 69, 70, 77, 150, 151]),        # window wraps the ring end
    (1, [3, 4, 12, 64, 65]),                # one visible ring slot at most
    (40, [30, 39, 40, 41, 100, 90, 91]),    # committed below / above the window, rewind
    (64, [60, 66, 70, 200]),                # window == cap: the full layer's slots
    (100, [50, 64, 130]),                   # window > cap
], ids=["wrap", "one", "rewind", "cap", "over_cap"])
def test_sliding_window_layers(swa, commits):
    """Page 1 section 1.4, mask_swa: layers 1 and 2 slide, layer 0 is full."""
    d = Driver(small(cap=64, n_layer=3, swa_window=swa, swa_layers=0b110, seed=107))
    run_steps(d, commits)
    d.close()


def test_sliding_window_ragged_cap_split_counts():
    """cap 100 (a partial last ring tile), q_len 3, windows that start and end
    inside tiles, the window's tiles spread over several splits."""
    for n_split in (1, 3):
        d = Driver(small(cap=100, q_len=3, n_head=16, n_head_kv=4, n_layer=2, swa_window=37,
                         swa_layers=0b10, seed=108), n_split=n_split)
        run_steps(d, [7, 57, 99, 100, 101, 130, 205, 206, 240, 263])
        d.close()


def test_sliding_window_single_noise_row():
    """q_len 1: the causal noise block is the single noise row."""
    d = Driver(small(cap=96, q_len=1, n_layer=2, swa_window=20, swa_layers=0b11, seed=109))
    run_steps(d, [0, 1, 2, 50, 120, 121])
    d.close()


@pytest.mark.parametrize("n_split", [1, 2, 3, 7, 13, 45, 64])
def test_split_counts_agree(n_split):
    """The merge launch's shapes (1, 2, 4 and 16 splits per merge wave; the
    decode workloads' 32 splits take 8); at 45 and 64 splits of a 16-tile
    ring most splits see no ring tile, and some merge waves see only splits
    without a visible key."""
    w = small(cap=512, seed=106)
    d = Driver(w, n_split=n_split)
    run_steps(d, [700, 703, 708], check_rows=False)
    d.close()


@pytest.mark.parametrize("cap,commits", [
    (300, [310, 313, 320, 330]),       # 10 tiles (last ragged): waves of 3, 3, 2 and 2 tiles
    (1000, [200, 204, 990, 1003]),     # window below cap, then across it
], ids=["ragged", "window_grows"])
def test_long_waves(cap, commits):
    """One split per KV head: waves stream three or more tiles, each one's
    successor in flight while it is attended."""
    d = Driver(small(cap=cap, seed=108), n_split=1)
    run_steps(d, commits, check_rows=False)
    d.close()


def test_bulk_chunked_foldin_identical():
    """One bulk step, 1024-row steps and fold-in steps end in the same ring."""
    w = small(cap=1000, seed=107)
    final = 2500
    ways = {"bulk": [final],
            "chunked": list(range(1024, final, 1024)) + [final],
            "fold": list(range(18, final, 18)) + [final]}
    got = {}
    for name, commits in ways.items():
        d = Driver(w)
        for c in commits:
            d.step(0, c)
        d.check_index(0)
        d.check_rows(0, 0)
        k, v = d.ring.rows(0, 0, 0, d.geo.cap)
        got[name] = (d.ring.slot_pos(0), d.ring.mask(0), k.view(np.uint16).copy(),
                     v.view(np.uint16).copy())
        d.close()
    for name in ("chunked", "fold"):
        for a, b in zip(got["bulk"], got[name]):
            assert np.array_equal(a, b), name


def test_error_paths_leave_state_unchanged():
    from draft_model_kv_amd import RingError
    from draft_model_kv_amd.ring import RING_ERANGE, RING_ESTATE, RING_EINVAL
    import torch
    d = Driver(small(cap=64))
    d.step(0, 10)
    before = (d.ring.state(0), d.ring.slot_pos(0).copy(), d.ring.mask(0).copy())
    k = torch.zeros((1, 3, 1024), dtype=torch.float16, device="cuda")
    with pytest.raises(RingError) as e:
        d.ring.begin_step(0, 12, k, k)          # plan says 2 rows
    assert e.value.code == RING_ESTATE
    with pytest.raises(RingError) as e:
        d.ring.begin_step(1, 12, k, k)          # no sequence 1
    assert e.value.code == RING_ERANGE
    q = torch.zeros((1, 8, 32, 128), dtype=torch.float16, device="cuda")
    kn = torch.zeros((1, 8, 1024), dtype=torch.float16, device="cuda")
    with pytest.raises(RingError) as e:
        d.ring.attn(1, q, kn, kn)                # no layer 1
    assert e.value.code == RING_ERANGE
    from draft_model_kv_amd import ring_attn
    out = torch.zeros((1, 8, 32, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(RingError) as e:
        ring_attn(d.ring.handle, 0, q.data_ptr() + 2, kn.data_ptr(), kn.data_ptr(), out.data_ptr())
    assert e.value.code == RING_EINVAL
    after = (d.ring.state(0), d.ring.slot_pos(0), d.ring.mask(0))
    assert before[0] == after[0] and np.array_equal(before[1], after[1]) and np.array_equal(before[2], after[2])
    d.step(0, 12)
    d.check_index(0)
    d.check_attn(0, 0)
    d.close()


# ---------------------------------------------------------------------------
# Full workload sizes, sampled checkpoints (every step runs on the device).
# ---------------------------------------------------------------------------
def _run_workload(name, every, rows_at=(0,), max_steps=None):
    run_workload(name, every, rows_at=rows_at, max_steps=max_steps, say=say)


def test_decode_stream_full():
    _run_workload("decode_stream", every=50, rows_at=(0, 1999))


def test_long_prompt_wrap_full():
    _run_workload("long_prompt_wrap", every=32, rows_at=(511,))


def test_batched_seqs_full():
    _run_workload("batched_seqs", every=16, rows_at=(255,))


def test_large_window_full():
    _run_workload("large_window", every=32, rows_at=(255,))


def test_swa_stream_full():
    _run_workload("swa_stream", every=40, rows_at=(599,))


def test_absurd_cap_library_workspace_is_enomem_and_leaks_nothing():
    """ring_init with no caller workspace and a geometry far beyond the GPU's
    memory (2^54 bytes): the library's hipMalloc fails, the call returns
    RING_ENOMEM, and the device's free memory is what it was before."""
    import torch
    from draft_model_kv_amd import RingError, make_config, ring_init
    from draft_model_kv_amd.ring import RING_ENOMEM
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    cfg = make_config(1 << 26, 8, 32, 8, 128, n_layer=1024, n_seq=64)
    for _ in range(3):
        with pytest.raises(RingError) as e:
            ring_init(cfg)
        assert e.value.code == RING_ENOMEM
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert abs(free1 - free0) < (64 << 20), (free0, free1)
