"""ring_attn_noalloc (split partials in the library's static device array)
against ring_attn, through the C ABI (needs the GPU).

Two calls in a row share the static array: first a 4096-slot ring (32
splits, 2.2 MB of partials), then a smaller 512-slot ring (4 splits): the
second must not see the first's leftovers.  Each is compared with ring_attn
on the same ring state (same kernels, so bit for bit) and with the CPU oracle
within the attention tolerance; a deferred (fused) step through
ring_attn_noalloc is checked against the oracle too.  A launch whose partials
exceed the array is refused with RING_EINVAL and changes nothing.
"""

import sys

import numpy as np
import pytest

import workload as W
from tests.harness import Driver, check_close

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _ring(cap, seed, n_seq=1, n_split=None):
    w = W.Workload(name="noalloc", seed=seed, cap=cap, q_len=8, n_head=32, n_head_kv=8,
                   n_seq=n_seq)
    return Driver(w, n_split=n_split)


def _both(d, step):
    """ring_attn_noalloc, then ring_attn, on the same inputs (eager state)."""
    torch = d.torch
    q, kn, vn = d.noise(0, step)
    qt, knt, vnt = (torch.from_numpy(x).to(d.dev) for x in (q, kn, vn))
    c = d.ring.cfg
    shape = (c.n_seq, c.q_len, c.n_head, c.head_dim)
    out_n = torch.full(shape, float("nan"), dtype=torch.float32, device=d.dev)
    d.ring.attn(0, qt, knt, vnt, out=out_n, noalloc=True)
    out_p = d.ring.attn(0, qt, knt, vnt)
    torch.cuda.synchronize(d.dev)
    return out_n.cpu().numpy(), out_p.cpu().numpy(), q, kn, vn


def test_noalloc_matches_ring_attn_two_calls_smaller_second():
    big = _ring(4096, seed=900)
    small = _ring(512, seed=901)
    say("noalloc rings:", big.ring.describe(), "|", small.ring.describe())
    for d, commits in ((big, [4096, 4099, 4107]), (small, [700, 701, 709])):
        for c in commits:
            d.step(0, c)
    # call 1 (large), then call 2 (smaller) through the static array
    for t, d in enumerate((big, small)):
        got_n, got_p, q, kn, vn = _both(d, 10 + t)
        assert np.array_equal(got_n, got_p), "ring_attn_noalloc differs from ring_attn"
        st = check_close(got_n[0], d.oracle_attn(0, 0, q, kn, vn), f"noalloc call {t + 1}")
        say("call", t + 1, "cap", d.w.cap, "worst err/bound", round(st["max_ratio"], 4))
    # and once more in the same order after further steps (the array keeps the
    # last call's contents)
    big.step(0, 4111)
    small.step(0, 712)
    for t, d in enumerate((big, small)):
        got_n, got_p, q, kn, vn = _both(d, 20 + t)
        assert np.array_equal(got_n, got_p)
        check_close(got_n[0], d.oracle_attn(0, 0, q, kn, vn), f"noalloc call {t + 3}")
    big.close()
    small.close()


def test_noalloc_fused_step_against_oracle():
    """A deferred step appended by the attention launch of ring_attn_noalloc."""
    d = _ring(4096, seed=902)
    d.step(0, 4096)
    torch = d.torch
    c = d.ring.cfg
    out = torch.empty((c.n_seq, c.q_len, c.n_head, c.head_dim), dtype=torch.float32,
                      device=d.dev)
    for t, com in enumerate([4097, 4104, 4106, 4114]):
        d.step(0, com, deferred=True)
        q, kn, vn = d.noise(0, t)
        d.ring.attn(0, *(torch.from_numpy(x).to(d.dev) for x in (q, kn, vn)), out=out,
                    noalloc=True)
        torch.cuda.synchronize(d.dev)
        check_close(out.cpu().numpy()[0], d.oracle_attn(0, 0, q, kn, vn), f"fused noalloc {t}")
        d.check_index(0)
        d.check_rows(0, 0)
    d.close()


def test_noalloc_refuses_partials_beyond_the_array():
    """8 sequences x 8 KV heads x 64 splits x 32 rows x 264 B = 34.6 MB > 16 MiB."""
    from draft_model_kv_amd import RingError
    from draft_model_kv_amd.ring import RING_EINVAL
    d = _ring(8192, seed=903, n_seq=8, n_split=64)
    for s in range(8):
        d.step(s, 300 + 997 * s)
    torch = d.torch
    q, kn, vn = d.noise(0, 0)
    qt, knt, vnt = (torch.from_numpy(x).to(d.dev) for x in (q, kn, vn))
    c = d.ring.cfg
    out = torch.zeros((c.n_seq, c.q_len, c.n_head, c.head_dim), dtype=torch.float32,
                      device=d.dev)
    with pytest.raises(RingError) as e:
        d.ring.attn(0, qt, knt, vnt, out=out, noalloc=True)
    assert e.value.code == RING_EINVAL and "static scratch" in str(e.value)
    torch.cuda.synchronize(d.dev)
    assert not out.any(), "a refused call wrote its output"
    got = d.ring.attn(0, qt, knt, vnt).cpu().numpy()
    for s in range(8):
        check_close(got[s], d.oracle_attn(s, 0, q, kn, vn), f"ring_attn seq {s}")
    d.close()
