"""Negative control for the ring-equals-full check (CPU only).

The page's notes on the port (section 2.2, why acceptance fell to 30 %)
describe the broken version that came before the ring: before every
injection it physically removed the cache rows of positions below
pos - window (llama.cpp's seq_rm "roll") and then attended over every row
the cache held, with no -inf window mask; empty and evicted cells were read
as whatever they held.  That is not a mod-cap ring with masks.

This file builds that naive model on purpose (a fixed cache of `cap` cells,
row p in cell p % cap, rows below lo dropped to empty zero cells, attention
over every cell and the noise block with no mask) and checks that the
comparison the ring is held to -- attention equal to the full-cache
oracle's over [lo, committed) plus the noise block, to 1e-12 in fp64 --
tells it apart:
  * it fails on a rewind (rows of positions >= committed stay in their
    cells and are attended) and on a window that is not full yet
    (committed < cap: empty zero cells are attended as keys);
  * it passes on a monotone stream once the window is full, where every
    cell holds a window row and the two models coincide -- so the failures
    above come from the missing mask, not from a check that rejects
    everything.
"""

import math
import random

import numpy as np

import oracle.ring_oracle as ro

D, HK, NH, BASE, Q_LEN = 8, 2, 4, 1e6, 3


class Rows:
    """Row content fixed per (position, epoch): a rewind to c starts a new
    epoch for positions >= c (they will be committed again with other
    tokens), positions below c keep theirs."""

    def __init__(self, seed):
        self.seed = seed
        self.epoch_from = []   # (first position, epoch) in increasing position
        self.n_rewinds = 0

    def rewind(self, c):
        self.n_rewinds += 1
        self.epoch_from = [(p, e) for p, e in self.epoch_from if p < c]
        self.epoch_from.append((c, self.n_rewinds))

    def get(self, positions):
        k = np.empty((len(positions), HK * D), np.float16)
        v = np.empty((len(positions), HK * D), np.float16)
        for j, p in enumerate(positions):
            e = 0
            for p0, e0 in self.epoch_from:
                if p >= p0:
                    e = e0
            rs = np.random.default_rng([self.seed, int(p), e])
            k[j] = rs.normal(size=HK * D)
            v[j] = rs.normal(size=HK * D)
        return k, v


class NaiveRoll:
    """The seq_rm roll: cells [cap] of (position, K rotated, V); -1 = empty.
    Each step injects the positions it has not seen, [max(next, lo),
    committed), at cell p % cap, after dropping the rows below lo; nothing
    else is removed and nothing is masked."""

    def __init__(self, cap):
        self.cap = cap
        self.next = 0
        self.pos = np.full(cap, -1, np.int64)
        self.k = np.zeros((cap, HK * D))
        self.v = np.zeros((cap, HK * D))

    def commit(self, committed, rows):
        lo = committed - min(committed, self.cap)
        drop = (self.pos >= 0) & (self.pos < lo)     # seq_rm(0, pos - window)
        self.pos[drop] = -1
        self.k[drop] = 0.0
        self.v[drop] = 0.0
        positions = np.arange(max(self.next, lo), committed)
        k, v = rows.get(positions)
        k_rot = ro.rope_rows_f16(k, positions, HK, D, BASE).astype(np.float64)
        for j, p in enumerate(positions):
            c = int(p) % self.cap
            self.pos[c], self.k[c], self.v[c] = p, k_rot[j], v[j]
        self.next = committed

    def attend(self, committed, q, kn, vn):
        """Every cell and the noise block, no mask (fp64)."""
        pq = ro.noise_positions(committed, Q_LEN)
        K = np.concatenate([self.k, ro.rope_rows_f16(kn, pq, HK, D, BASE).astype(np.float64)])
        V = np.concatenate([self.v, vn.astype(np.float64)])
        qr = ro.rope(q, pq, BASE)
        out = np.empty((Q_LEN, NH, D))
        for h in range(NH):
            g = h // (NH // HK)
            s = qr[:, h] @ K[:, g * D:(g + 1) * D].T / math.sqrt(D)
            w = np.exp(s - s.max(1, keepdims=True))
            out[:, h] = (w @ V[:, g * D:(g + 1) * D]) / w.sum(1, keepdims=True)
        return out


def _stream(cap, commits, seed):
    """Yield (committed, oracle RingStep, naive model, q, kn, vn) per step,
    both models fed the same rows."""
    rs = np.random.default_rng(seed)
    rows = Rows(seed)
    st = ro.RingStep(ro.geometry(cap, Q_LEN, D, HK), 1, HK, D, BASE)
    naive = NaiveRoll(cap)
    prev = 0
    for c in commits:
        if c < prev:
            rows.rewind(c)
        prev = c
        p = st.plan(c)
        k, v = rows.get(np.arange(p.start, c))
        st.commit(p, [k], [v])
        naive.commit(c, rows)
        q = rs.normal(size=(Q_LEN, NH, D)).astype(np.float16)
        kn = rs.normal(size=(Q_LEN, HK * D)).astype(np.float16)
        vn = rs.normal(size=(Q_LEN, HK * D)).astype(np.float16)
        yield c, st, naive, q, kn, vn


def _worst_gap(cap, commits, seed):
    """|naive - full| (max over elements) at each step of a commit stream."""
    gaps = []
    for c, st, naive, q, kn, vn in _stream(cap, commits, seed):
        full = ro.attend(st.caches[0], c, cap, q, kn, vn, NH)
        gaps.append(float(np.abs(naive.attend(c, q, kn, vn) - full).max()))
    return gaps


# full window, then a rewind of 5 positions: the cells of 35..39 keep their
# rows (rejected drafts) and 27..29 are gone (overwritten by 35..37)
REWIND = [24, 30, 35, 40, 35, 36, 37]
PARTIAL = [1, 3, 4, 7, 12]   # committed < cap = 13 throughout


def test_naive_roll_fails_on_rewind():
    gaps = _worst_gap(8, REWIND, seed=8)
    assert max(gaps[:4]) < 1e-12, gaps             # monotone and full: agrees
    assert min(gaps[4:]) > 1e-3, gaps              # after the rewind: stale rows attended


def test_naive_roll_fails_on_partial_window():
    gaps = _worst_gap(13, PARTIAL, seed=13)
    assert min(gaps) > 1e-3, gaps                  # empty zero cells attended


def test_naive_roll_agrees_on_full_monotone_windows():
    rnd = random.Random(3)
    for cap in (3, 8, 13):
        c, commits = cap, []
        for _ in range(30):
            c += rnd.choice([1, 2, 4, cap, 3 * cap])
            commits.append(c)
        assert max(_worst_gap(cap, commits, seed=cap)) < 1e-12


def test_the_ring_passes_where_the_naive_roll_fails():
    """The same rewind and partial-window streams through the ring model the
    oracle pins (slot_pos + mask over kv_total rows): equal to the full cache."""
    for cap, commits in ((8, REWIND), (13, PARTIAL)):
        geo = ro.geometry(cap, Q_LEN, D, HK)
        for c, st, _, q, kn, vn in _stream(cap, commits, seed=cap):
            full = ro.attend(st.caches[0], c, cap, q, kn, vn, NH)
            K = np.zeros((geo.kv_total, HK * D))
            V = np.zeros((geo.kv_total, HK * D))
            for s in range(cap):
                sp = int(st.slots.slot_pos[s])
                if 0 <= sp < c:
                    K[s], V[s] = st.caches[0].row(sp)
            pq = ro.noise_positions(c, Q_LEN)
            K[cap:cap + Q_LEN] = ro.rope_rows_f16(kn, pq, HK, D, BASE)
            V[cap:cap + Q_LEN] = vn
            bias = st.mask().astype(np.float64)
            qr = ro.rope(q, pq, BASE)
            ring = np.empty_like(full)
            for h in range(NH):
                g = h // (NH // HK)
                s_ = qr[:, h] @ K[:, g * D:(g + 1) * D].T / math.sqrt(D) + bias
                w = np.exp(s_ - s_.max(1, keepdims=True))
                ring[:, h] = (w @ V[:, g * D:(g + 1) * D]) / w.sum(1, keepdims=True)
            assert np.abs(ring - full).max() < 1e-12, (cap, c)
