"""New rows from fused features: the feature mirror and the K/V projection
on the GPU against the CPU oracle (needs the GPU).

Index work (plan, slot_pos, mask) must be bit-exact; ring K and V rows within
one F16 ulp of the oracle's single rounding of the fp64 projection, norm and
RoPE (the device accumulates the products in fp32); attention outputs within
|gpu - ref| <= 2e-3 + 1e-2 |ref| of the fp32-accumulated oracle.
"""

import sys

import numpy as np
import pytest

import workload as W
from tests.harness import Driver

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(**kw):
    base = dict(name="mirror_edge", seed=200, cap=64, q_len=8, n_head=32, n_head_kv=8,
                n_layer=2, d_model=256)
    base.update(kw)
    return W.Workload(**base)


def run(d, commits, seq=0, rows=True):
    for c in commits:
        d.step(seq, c)
        d.check_index(seq)
        for layer in range(d.w.n_layer):
            if rows:
                d.check_rows(seq, layer)
            d.check_attn(layer, d.n_attn)


@pytest.mark.parametrize("commits", [
    [40, 41, 47, 59, 64, 70, 90, 91],          # fold-ins, wrap inside one fold-in
    [200, 201, 209, 218],                      # bulk of 200 rows (64 + 64 + 64 + 8), then folds
    [50, 40, 45, 20, 64, 70],                  # rewinds inside the window
    [200, 150, 151, 300, 290, 291],            # rewinds past what the ring and mirror hold
    [5, 5, 6, 6],                              # zero-row steps
], ids=["fold_wrap", "bulk_chunks", "rewind_near", "rewind_far", "zero_rows"])
def test_mirror_streams(commits):
    d = Driver(small())
    run(d, commits)
    d.close()


@pytest.mark.parametrize("commits", [
    [40, 41, 47, 59, 64, 70, 90, 91],          # fold-ins: each write carried out by the projection
    [200, 201, 209, 218],                      # a bulk (its write copied first), then folds
    [50, 40, 45, 20, 64, 70],                  # rewinds: writes of other rows than the step's
    [200, 150, 151, 300, 290, 291],
    [5, 5, 6, 6],
], ids=["fold_wrap", "bulk_chunks", "rewind_near", "rewind_far", "zero_rows"])
def test_mirror_streams_deferred_writes(commits):
    """ring_mirror_write_deferred: the step's features are written into the
    mirror by the projection launch when it projects exactly those rows, else
    copied before; the same parity as eager writes."""
    d = Driver(small(seed=205), mirror_deferred=True)
    run(d, commits)
    d.close()


def test_deferred_and_eager_mirror_writes_bit_for_bit():
    """The same stream with deferred and with eager mirror writes (registered
    weights): identical ring rows, attention outputs and mirror contents (the
    next steps project from what the deferred writes left in the mirror)."""
    w = small(d_model=512, seed=206, n_layer=2, cap=100, q_len=3, n_head=16, n_head_kv=4)
    a = Driver(w, registered_weights=True)
    b = Driver(w, registered_weights=True, mirror_deferred=True)
    for t, c in enumerate([70, 71, 75, 76, 90, 140, 141, 150, 60, 61]):
        a.step(0, c)
        b.step(0, c)
        for layer in range(w.n_layer):
            ka, va = a.ring.rows(0, layer, 0, a.geo.cap)
            kb, vb = b.ring.rows(0, layer, 0, b.geo.cap)
            assert np.array_equal(ka.view(np.uint16), kb.view(np.uint16)), (t, layer)
            assert np.array_equal(va.view(np.uint16), vb.view(np.uint16)), (t, layer)
            assert np.array_equal(a.attn(layer, t)[0], b.attn(layer, t)[0]), (t, layer)
        b.check_index(0)
    b.check_attn(0, 200)
    a.close()
    b.close()


@pytest.mark.parametrize("d_model", [512, 768, 2048])
def test_mirror_feature_widths(d_model):
    """Several d-slices per row (2, 3 and 8 slices of 256 feature dims)."""
    d = Driver(small(d_model=d_model, seed=201 + d_model, n_layer=1, cap=100, q_len=3,
                     n_head=16, n_head_kv=4))
    run(d, [70, 71, 75, 140, 141])
    d.close()


def test_mirror_gqa8_outliers():
    d = Driver(small(cap=256, n_head=64, sigma=1.0, outlier_p=0.01, seed=205, d_model=512,
                     n_layer=1))
    run(d, [300, 301, 309, 330])
    d.close()


def test_mirror_errors_leave_state_unchanged():
    from draft_model_kv_amd import ring as rk
    import torch
    d = Driver(small())
    d.step(0, 40)
    before = (d.ring.state(0), d.ring.slot_pos(0).copy(), d.ring.mask(0).copy())
    r = d.ring
    # a position the mirror does not hold
    with pytest.raises(rk.RingError) as e:
        r.begin_step_mirror(0, 43, d.wk_t, d.wv_t, d.kn_t, d.eps)
    assert e.value.code == rk.RING_ESTATE and "mirror" in str(e.value)
    # misaligned weights, negative eps
    with pytest.raises(rk.RingError) as e:
        rk.ring_begin_step_mirror(r.handle, 0, 40, d.wk_t.data_ptr() + 2, d.wv_t.data_ptr(),
                                  d.kn_t.data_ptr(), d.eps)
    assert e.value.code == rk.RING_EINVAL
    with pytest.raises(rk.RingError) as e:
        rk.ring_begin_step_mirror(r.handle, 0, 40, d.wk_t.data_ptr(), d.wv_t.data_ptr(),
                                  d.kn_t.data_ptr(), -1.0)
    assert e.value.code == rk.RING_EINVAL
    with pytest.raises(rk.RingError) as e:
        rk.ring_begin_step_mirror(r.handle, 0, 40, 0, d.wv_t.data_ptr(), d.kn_t.data_ptr(), d.eps)
    assert e.value.code == rk.RING_EINVAL
    with pytest.raises(rk.RingError) as e:
        rk.ring_mirror_write(r.handle, 0, -1, 1, d.wk_t.data_ptr())
    assert e.value.code == rk.RING_ERANGE
    after = (d.ring.state(0), d.ring.slot_pos(0), d.ring.mask(0))
    assert before[0] == after[0]
    assert np.array_equal(before[1], after[1]) and np.array_equal(before[2], after[2])
    # the same step goes through once its features are written
    d.step(0, 43)
    d.check_index(0)
    d.check_attn(0, 0)
    d.close()
    # a ring without a mirror refuses both calls
    plain = rk.Ring(cap=64, device="cuda:0")
    with pytest.raises(rk.RingError) as e:
        rk.ring_mirror_write(plain.handle, 0, 0, 1, d.wk_t.data_ptr())
    assert e.value.code == rk.RING_ESTATE
    plain.close()


def test_mirror_stream_full():
    """The full-size workload: cap 4096, 5 layers, d_model 2048, a 4096-token
    prompt (64 projection launches of 64 rows), then 40 decode steps."""
    w = W.WORKLOADS["mirror_stream"]
    d = Driver(w)
    stream = W.commit_stream(w, 0)[: 1 + 40]
    say("mirror_stream", len(stream), "steps")
    for t, c in enumerate(stream):
        d.step(0, c)
        d.check_index(0)
        if t in (0, 1, 17, len(stream) - 1):
            for layer in range(w.n_layer):
                d.check_rows(0, layer)
        if t % 4 == 0 or t == len(stream) - 1:
            for layer in range(w.n_layer):
                d.check_attn(layer, t)
    d.close()


# ---------------------------------------------------------------------------
# Weights registered once (ring_set_kv_weights): packed in the projection
# kernel's load order, same arithmetic and order of the products.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("commits", [
    [40, 41, 47, 59, 64, 70, 90, 91],
    [200, 201, 209, 218],
    [200, 150, 151, 300, 290, 291],
], ids=["fold_wrap", "bulk_chunks", "rewind_far"])
def test_registered_weights_streams(commits):
    d = Driver(small(seed=210), registered_weights=True)
    run(d, commits)
    d.close()


@pytest.mark.parametrize("d_model,n_head_kv", [(512, 4), (2048, 8), (768, 16)])
def test_registered_equals_caller_weights_bit_for_bit(d_model, n_head_kv):
    """The same stream through the caller's weights and through the
    registered ones: identical ring rows and attention outputs."""
    w = small(d_model=d_model, seed=211 + d_model, n_layer=2, cap=100, q_len=3,
              n_head=2 * n_head_kv, n_head_kv=n_head_kv)
    a, b = Driver(w), Driver(w, registered_weights=True)
    for t, c in enumerate([70, 71, 75, 140, 141]):
        a.step(0, c)
        b.step(0, c)
        for layer in range(w.n_layer):
            # ring slots (the noise rows past cap hold each ring's last noise block)
            ka, va = a.ring.rows(0, layer, 0, a.geo.cap)
            kb, vb = b.ring.rows(0, layer, 0, b.geo.cap)
            assert np.array_equal(ka.view(np.uint16), kb.view(np.uint16)), (t, layer)
            assert np.array_equal(va.view(np.uint16), vb.view(np.uint16)), (t, layer)
            oa = a.attn(layer, t)[0]
            ob = b.attn(layer, t)[0]
            assert np.array_equal(oa, ob), (t, layer)
        a.check_index(0)
        b.check_index(0)
        b.check_attn(0, 100 + t)
    a.close()
    b.close()


def test_registered_weights_needed_for_null():
    from draft_model_kv_amd import ring as rk
    d = Driver(small(seed=212))
    d.write_features(0, np.arange(0, 10))
    with pytest.raises(rk.RingError) as e:
        d.ring.begin_step_mirror(0, 10)          # no weights given, none registered
    assert e.value.code == rk.RING_ESTATE
    with pytest.raises(rk.RingError) as e:
        rk.ring_set_kv_weights(d.ring.handle, d.wk_t.data_ptr() + 2, d.wv_t.data_ptr(),
                               d.kn_t.data_ptr(), d.eps)
    assert e.value.code == rk.RING_EINVAL
    d.close()


def test_projection_floor_kind():
    """ring_profile_floor's projection kind (profiling only): refused until
    weights are registered, then it runs between steps and the stream still
    matches the oracle (it changes no state of the ring)."""
    import torch
    from draft_model_kv_amd import ring as rk
    s = torch.cuda.current_stream().cuda_stream
    d = Driver(small(seed=213))
    with pytest.raises(rk.RingError) as e:
        rk.ring_profile_floor(d.ring.handle, 0, rk.RING_FLOOR_PROJ_READ, s)
    assert e.value.code == rk.RING_ESTATE
    d.close()
    d = Driver(small(seed=213, d_model=2048), registered_weights=True)
    run(d, [40, 41])
    for _ in range(3):
        rk.ring_profile_floor(d.ring.handle, 0, rk.RING_FLOOR_PROJ_READ, s)
    torch.cuda.synchronize()
    run(d, [47, 59, 64])
    d.close()


@pytest.mark.parametrize("deferred", [False, True], ids=["eager_writes", "deferred_writes"])
def test_mirror_stream_full_registered(deferred):
    """The full-size workload through registered weights: 4096-token prompt,
    then 40 decode steps (the bench's mirror step writes its features with
    ring_mirror_write_deferred)."""
    w = W.WORKLOADS["mirror_stream"]
    d = Driver(w, registered_weights=True, mirror_deferred=deferred)
    stream = W.commit_stream(w, 0)[: 1 + 40]
    for t, c in enumerate(stream):
        d.step(0, c)
        d.check_index(0)
        if t in (0, 1, len(stream) - 1):
            for layer in range(w.n_layer):
                d.check_rows(0, layer)
        if t % 8 == 0 or t == len(stream) - 1:
            for layer in range(w.n_layer):
                d.check_attn(layer, t)
    d.close()

