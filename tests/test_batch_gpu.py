"""ring_begin_step_batch: the begin steps of several sequences in one call
(fold-ins appended together by one launch of the batched append kernel)
against the CPU oracle, and against ring_begin_step on a twin ring (needs
the GPU).

Same bars as the other parity tests: index state bit-exact, ring K rows
within one F16 ulp of the oracle (V exact), attention within 2e-3 + 1e-2
|ref|; between the batched and the per-sequence call everything is
bit-identical, since both run the same per-row arithmetic.
"""

import sys

import numpy as np
import pytest

import workload as W
from draft_model_kv_amd import RingError
from tests.harness import Driver

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(**kw):
    base = dict(name="batch_edge", seed=400, cap=128, q_len=8, n_head=32, n_head_kv=8)
    base.update(kw)
    return W.Workload(**base)


def check_all(d, seqs=None, rows=True):
    for seq in (range(d.w.n_seq) if seqs is None else seqs):
        d.check_index(seq)
        if rows:
            for layer in range(d.w.n_layer):
                d.check_rows(seq, layer)


def test_batch_streams_twenty_sequences():
    """20 sequences (a launch of 16, then one of 4), starts from below cap to
    many times cap, the workload's accepted-count streams; warm-up bulk plans
    go through the same call."""
    w = small(n_seq=20, n_steps=12, start_lo=20, start_hi=3000,
              forced_starts=((0, 20, 60), (1, 128 - 30, 128 - 5)))
    d = Driver(w)
    streams = [W.commit_stream(w, s) for s in range(w.n_seq)]
    say("batch 20 seqs", len(streams[0]), "steps")
    for t in range(len(streams[0])):
        d.step_batch([(s, streams[s][t]) for s in range(w.n_seq)])
        d.check_attn(0, t)
        check_all(d, rows=(t % 4 == 0 or t == len(streams[0]) - 1))
    d.close()


def test_batch_mixed_plans_in_one_call():
    """Fold-ins, a bulk append, a zero-row step, rewinds (inside the window
    and past it) and a fold-in wrapping the ring end, all in single calls;
    two layers, one of them sliding over 16 positions."""
    w = small(n_seq=6, n_layer=2, swa_window=16, swa_layers=0b10, seed=401)
    d = Driver(w)
    calls = [
        [(0, 40), (1, 300), (2, 5), (3, 127), (4, 1000), (5, 64)],
        [(0, 41), (1, 309), (2, 5), (3, 130), (4, 1017), (5, 70)],
        [(0, 59), (1, 250), (2, 6), (3, 131), (4, 1018), (5, 60)],    # 1, 5: rewinds
        [(0, 200), (1, 251), (2, 14), (3, 128), (4, 900), (5, 61)],   # 0 bulk, 4 far rewind
        [(0, 201), (1, 260), (2, 20), (3, 136), (4, 901), (5, 79)],
    ]
    for t, items in enumerate(calls):
        d.step_batch(items)
        d.check_attn_layers(t)
        check_all(d)
    d.close()


def test_batch_subset_leaves_other_sequences():
    """A call over some sequences only: the others keep their rows, index
    state and plan; per-sequence and batched calls interleave."""
    w = small(n_seq=5, seed=402)
    d = Driver(w)
    d.step_batch([(s, 100 + 37 * s) for s in range(5)])
    for t, (subset, solo) in enumerate([((0, 2, 4), 1), ((3,), 0), ((1, 2), 4)]):
        d.step_batch([(s, d.committed[s] + 1 + s) for s in subset])
        d.step(solo, d.committed[solo] + 3)
        d.check_attn(0, t)
        check_all(d)
    d.close()


def test_batch_flushes_deferred_steps():
    """A sequence with a deferred fold-in still owed is flushed before the
    batched append of its next step."""
    w = small(n_seq=3, n_layer=2, seed=403)
    d = Driver(w)
    d.step_batch([(0, 50), (1, 60), (2, 70)])
    d.step(0, 53, deferred=True)          # owed: both layers and the index state
    d.step(1, 61, deferred=True)
    d.attn(0, 0)                          # layer 0 of sequences 0 and 1 appended by the attention
    d.step_batch([(0, 57), (1, 69), (2, 71)])
    d.check_attn_layers(1)
    check_all(d)
    d.close()


def test_batch_bit_identical_to_per_sequence():
    """Twin rings, the same steps through ring_begin_step_batch and through
    ring_begin_step: rows, slot_pos and masks identical bit for bit."""
    w = small(n_seq=17, n_layer=2, cap=96, seed=404, n_steps=6, start_lo=50, start_hi=900)
    a, b = Driver(w), Driver(w)
    streams = [W.commit_stream(w, s) for s in range(w.n_seq)]
    for t in range(len(streams[0])):
        a.step_batch([(s, streams[s][t]) for s in range(w.n_seq)])
        for s in range(w.n_seq):
            b.step(s, streams[s][t])
        for s in range(w.n_seq):
            assert np.array_equal(a.ring.slot_pos(s), b.ring.slot_pos(s))
            assert np.array_equal(a.ring.mask(s), b.ring.mask(s))
            for layer in range(w.n_layer):
                ka, va = a.ring.rows(s, layer, 0, a.geo.kv_total)
                kb, vb = b.ring.rows(s, layer, 0, b.geo.kv_total)
                assert np.array_equal(ka.view(np.uint16), kb.view(np.uint16)), (t, s, layer)
                assert np.array_equal(va.view(np.uint16), vb.view(np.uint16)), (t, s, layer)
        oa, *_ = a.attn(0, t)
        ob, *_ = b.attn(0, t)
        assert np.array_equal(oa, ob)
    a.close()
    b.close()


def test_batch_rejections_change_nothing():
    """Rejected calls enqueue nothing and leave every sequence's state."""
    import torch
    import draft_model_kv_amd.ring as rk
    w = small(n_seq=4, seed=405)
    d = Driver(w)
    d.step_batch([(s, 40 + s) for s in range(4)])
    before = [d.ring.state(s) for s in range(4)]
    kv = torch.zeros((1, 3, w.kv_row), dtype=torch.float16, device=d.dev)
    h, p = d.ring.handle, kv.data_ptr()
    with pytest.raises(RingError) as e:                       # sequence listed twice
        rk.ring_begin_step_batch(h, [0, 0], [43, 44], [p, p], [p, p], [3, 4])
    assert e.value.code == rk.RING_EINVAL
    with pytest.raises(RingError) as e:                       # n_rows != n_new in entry 1
        rk.ring_begin_step_batch(h, [0, 1], [43, 44], [p, p], [p, p], [3, 2])
    assert e.value.code == rk.RING_ESTATE
    with pytest.raises(RingError) as e:                       # seq out of range
        rk.ring_begin_step_batch(h, [0, 4], [43, 44], [p, p], [p, p], [3, 3])
    assert e.value.code == rk.RING_ERANGE
    with pytest.raises(RingError) as e:                       # NULL rows with n_new > 0
        rk.ring_begin_step_batch(h, [2], [45], [0], [0], [3])
    assert e.value.code == rk.RING_EINVAL
    with pytest.raises(RingError) as e:                       # more entries than sequences
        rk.ring_begin_step_batch(h, [0, 1, 2, 3, 0], [1] * 5, [p] * 5, [p] * 5, [0] * 5)
    assert e.value.code == rk.RING_ERANGE
    rk.ring_begin_step_batch(h, [], [], [], [], [])         # n = 0: nothing to do
    torch.cuda.synchronize(d.dev)
    assert [d.ring.state(s) for s in range(4)] == before
    check_all(d)
    d.check_attn(0, 0)
    d.close()


def test_batch_batched_seqs_workload():
    """The batched-sequences workload (16 rings of cap 4096, starts up to
    131072, two below cap): prefill through the batched call, then 24 decode
    steps, each checked."""
    w = W.WORKLOADS["batched_seqs"]
    d = Driver(w)
    streams = [W.commit_stream(w, s) for s in range(w.n_seq)]
    n_warm = W.n_warmup_steps(w)
    say("batched_seqs", n_warm, "warm-up steps")
    for t in range(n_warm):
        d.step_batch([(s, streams[s][t]) for s in range(w.n_seq)])
    check_all(d, rows=False)
    for j in range(24):
        t = n_warm + j
        d.step_batch([(s, streams[s][t]) for s in range(w.n_seq)])
        if j % 6 == 0 or j == 23:
            d.check_attn(0, j)
            check_all(d, rows=False)
    for s in (0, 1, 7):
        d.check_rows(s, 0)
    d.close()
