"""The fused step (ring_begin_step_deferred): a fold-in's rows appended, and
slot_pos, masks and noise RoPE table rebuilt, by the attention launch itself,
against the CPU oracle (needs the GPU).

Same bars as the other parity tests: index state bit-exact, ring K rows
within one F16 ulp (V exact), attention within 2e-3 + 1e-2 |ref|.  Every
check runs after the attention of all layers, so that the fused launches do
the appending; the flush paths (a read, a partial set of layers, two steps in
a row) are tested on their own.
"""

import sys

import numpy as np
import pytest

import workload as W
from tests.harness import Driver, run_workload

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(**kw):
    base = dict(name="fused_edge", seed=300, cap=64, q_len=8, n_head=32, n_head_kv=8)
    base.update(kw)
    return W.Workload(**base)


def run_fused(d, commits, seq=0, rows=True):
    for t, c in enumerate(commits):
        d.step(seq, c, deferred=True)
        d.check_attn_layers(d.n_attn)
        d.check_index(seq)
        if rows:
            for layer in range(d.w.n_layer):
                d.check_rows(seq, layer)


@pytest.mark.parametrize("commits", [
    [40, 41, 47, 59, 64, 70, 77, 78],          # folds, one wrapping the ring end
    [100, 118, 119, 127, 128],                 # n_new == a_step (no pads), then folds
    [50, 40, 45, 20, 64, 70],                  # rewinds inside the window
    [200, 150, 151, 300, 290, 291],            # rewinds that re-append (bulk: immediate)
    [5, 5, 6, 6, 7],                           # zero-row steps
], ids=["fold_wrap", "a_step", "rewind_near", "rewind_far", "zero_rows"])
def test_fused_streams(commits):
    d = Driver(small())
    run_fused(d, commits)
    d.close()


def test_fused_ragged_cap_short_block():
    d = Driver(small(cap=100, q_len=3, n_head=16, n_head_kv=4, seed=301))
    run_fused(d, [7, 20, 57, 60, 99, 100, 101, 105, 130])
    d.close()


@pytest.mark.parametrize("cap,commits", [
    (300, [310, 313, 320, 330]),       # 10 tiles (last ragged): waves of 3, 3, 2 and 2 tiles
    (1000, [200, 204, 990, 1003]),     # window below cap, then across it
], ids=["ragged", "window_grows"])
def test_deferred_on_wide_rings(cap, commits):
    """One split per KV head, so the waves stream three or more tiles: the
    fused launch's long-wave kernel appends and attends the new rows while
    its waves walk several tiles each."""
    d = Driver(small(cap=cap, seed=306), n_split=1)
    run_fused(d, commits, rows=False)
    d.close()


@pytest.mark.parametrize("q_len,n_head", [(8, 32), (16, 32)], ids=["q8", "q16_two_blocks"])
def test_fused_two_tiles_per_wave(q_len, n_head):
    """7 ring tiles (the last ragged) in one split: waves of two tiles, so
    the fused launch keeps the next tile in flight (the deferred steps stay
    fused at this width)."""
    d = Driver(small(cap=200, q_len=q_len, n_head=n_head, seed=307 + q_len), n_split=1)
    run_fused(d, [150, 151, 159, 203, 210, 211, 190, 199])
    d.close()


def test_fused_multi_layer_sliding_window():
    """4 layers, layers 1 and 3 sliding over 16 positions (new rows that fall
    before the window are still appended), full acceptance steps."""
    d = Driver(small(cap=64, n_layer=4, swa_window=16, swa_layers=0b1010, seed=302))
    run_fused(d, [40, 49, 58, 59, 60, 69, 78, 87, 88])
    d.close()


@pytest.mark.parametrize("cap,n_split", [(1024, 4), (1024, 7), (4096, 16)])
def test_fused_merge_in_launch(cap, n_split):
    """RING_ATTN_MERGE=kernel on fused launches whose waves stream two tiles:
    the cross-split merge runs inside the launch (last arriver per sequence
    x KV head)."""
    d = Driver(small(cap=cap, n_layer=2, seed=310 + n_split), n_split=n_split, merge="kernel")
    run_fused(d, [cap - 100, cap - 99, cap - 91, cap + 3, cap + 12, cap + 13, cap + 21])
    d.close()


@pytest.mark.parametrize("row_blocks", [True, False], ids=["row_blocks", "one_workgroup"])
def test_fused_gqa8_outliers(row_blocks):
    """64 queries per KV head: each 32-query block in a work-group of its own
    (both attend the new rows, one stores them), or both blocks in one."""
    d = Driver(small(cap=256, n_head=64, sigma=1.0, outlier_p=0.01, seed=303),
               row_blocks=row_blocks)
    run_fused(d, [300, 301, 309, 318, 330])
    d.close()


def test_fused_multi_seq():
    w = small(cap=128, n_layer=2, n_seq=3, seed=304)
    d = Driver(w)
    plan = {0: [10, 11, 19, 140, 148], 1: [500, 501, 509, 510, 515], 2: [127, 128, 129, 136, 140]}
    for t in range(5):
        for seq in range(3):
            d.step(seq, plan[seq][t], deferred=(t % 2 == 0 or seq != 1))
        d.check_attn_layers(t)
        for seq in range(3):
            d.check_index(seq)
            for layer in range(2):
                d.check_rows(seq, layer)
    d.close()


@pytest.mark.parametrize("n_seq", [16, 17], ids=["sixteen_fused", "seventeen_append_at_once"])
def test_fused_sequence_limit(n_seq):
    """Sixteen sequences fill every per-sequence field of a fused launch
    (lanes 0..15 of its lane-indexed loads); a seventeenth makes the deferred
    steps append at once.  Each sequence
    starts at its own position, some below cap, some past a wrap."""
    w = small(cap=96, n_seq=n_seq, seed=310 + n_seq)
    d = Driver(w)
    starts = [20 + 37 * s for s in range(n_seq)]
    for t, inc in enumerate([0, 1, 7, 3, 9, 2]):
        for s in range(n_seq):
            d.step(s, starts[s] + 5 * t + inc, deferred=True)
        d.check_attn_layers(t)
        for s in range(n_seq):
            d.check_index(s)
            d.check_rows(s, 0)
    d.close()


def test_fused_flush_paths():
    """A read right after the deferred step, attention of one layer of two,
    and two deferred steps in a row: the owed rows go in by the ordinary
    append kernel, and everything still matches."""
    d = Driver(small(n_layer=2, seed=305))
    d.step(0, 40, deferred=True)
    d.check_index(0)                   # flush: rows of both layers appended now
    for layer in range(2):
        d.check_rows(0, layer)
    d.check_attn_layers(0)
    d.step(0, 45, deferred=True)
    out0, q0, kn0, vn0 = d.attn(0, 1)  # layer 0 fused; layer 1 still owed
    from tests.harness import check_close
    check_close(out0[0], d.oracle_attn(0, 0, q0, kn0, vn0), "layer 0 alone")
    d.step(0, 47, deferred=True)       # flushes layer 1 of the previous step
    d.check_attn_layers(2)
    d.check_index(0)
    for layer in range(2):
        d.check_rows(0, layer)
    d.step(0, 49, deferred=True)
    d.step(0, 52, deferred=True)       # nothing ran in between: all owed work flushed
    d.check_attn_layers(3)
    d.check_index(0)
    for layer in range(2):
        d.check_rows(0, layer)
    d.close()


def test_plain_launch_after_fused_rebuilds_index():
    """The fused launch leaves the masks and the noise RoPE table owed; a
    second attention of the same layer and step is a plain launch, which reads
    them, so they are rebuilt first.  Two layers, one sliding-window."""
    w = small(cap=64, n_layer=2, swa_window=12, swa_layers=0b10, seed=320)
    d = Driver(w)
    for t, c in enumerate([40, 41, 49, 58, 70, 60, 61]):
        d.step(0, c, deferred=True)
        d.check_attn_layers(2 * t)       # fused launches append and attend
        d.check_attn_layers(2 * t + 1)   # plain launches on the rebuilt state
        d.check_index(0)
        for layer in range(2):
            d.check_rows(0, layer)
    d.close()


def test_eager_step_after_fused_steps():
    """Fused steps, then an eager step and a mask read in between: the owed
    index state is rebuilt by the eager append itself."""
    d = Driver(small(cap=96, seed=321))
    for c in [50, 51, 59]:
        d.step(0, c, deferred=True)
        d.check_attn_layers(c)
    d.step(0, 62)                        # eager
    d.check_attn(0, 62)
    d.check_index(0)
    d.step(0, 70, deferred=True)
    d.check_attn_layers(70)
    d.check_index(0)
    d.step(0, 71, deferred=True)
    d.check_attn_layers(71)
    d.step(0, 80)                        # eager right after a fused launch
    d.check_attn_layers(80)
    d.check_index(0)
    d.close()


# ---------------------------------------------------------------------------
# Whole workloads through the fused step (the bench's default step), at full
# size: checkpoints every 50 / 32 / 40 steps, at every cap crossing and at
# the last step, each with every layer's output, the index state bit-exact
# and ring rows.
# ---------------------------------------------------------------------------
def test_fused_decode_stream_full():
    """The headline workload: 4096-token bulk prompt, then all 2000 fold-in
    steps deferred into the attention launch."""
    run_workload("decode_stream", every=50, rows_at=(0, 1, 1000), deferred=True, say=say)


def test_fused_long_prompt_wrap_full():
    """5 layers, 32768-token prompt (28672 rows overwritten), all 512 decode
    steps (every 4th commits 8) fused."""
    run_workload("long_prompt_wrap", every=32, rows_at=(0, 255), deferred=True, say=say)


def test_fused_swa_stream_full():
    """4 layers, layers 1 and 3 sliding over 1024 positions (their window
    wraps the ring end as the stream advances), all 600 steps fused."""
    run_workload("swa_stream", every=40, rows_at=(0, 300), deferred=True, say=say)
