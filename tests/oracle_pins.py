"""Pins that tie the CPU oracle to the pages and to mathematics.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
something fixed outside the oracle: a value printed on the page
"DFLASH2_RING_PORT.md" (tests/golden), a closed form, an invariant the page
states, or a brute-force evaluation on a tiny input.  They look the oracle up
through the module object ``ro`` at call time, so the mutation test can plant
mistakes in it and check that some pin fails.
"""

from __future__ import annotations

import math
import os
import random

import numpy as np

import oracle.ring_oracle as ro

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split("=")
                out[k] = v
    return out


# --------------------------------------------------------------------------
# Geometry (section 1.1, worked example of section 11 Test 4, formula of 1.7)
# --------------------------------------------------------------------------
def pin_geometry_worked_example():
    g = _golden("luce_ring_log.txt")
    geo = ro.geometry(int(g["cap"]), 8, 128, 8)
    assert geo.kv_total == int(g["kv_total"]), geo
    assert geo.a_step == int(g["a_step"]), geo
    mib = ro.ring_bytes(int(g["layers"]), geo.kv_row, geo.kv_total) / 2.0**20
    assert round(mib, 1) == float(g["f16_cache_mib"]), mib


def pin_geometry_closed_form():
    # kv_total is the smallest multiple of 32 that holds cap ring slots, q_len
    # noise slots and one trash slot; the trash slot sits right after the noise.
    for cap in (1, 2, 23, 24, 31, 64, 100, 4096, 32768):
        for q_len in (1, 2, 7, 8):
            geo = ro.geometry(cap, q_len, 128, 8)
            need = cap + q_len + 1
            assert geo.kv_total % 32 == 0 and need <= geo.kv_total < need + 32, (cap, q_len, geo)
            assert geo.trash_slot == cap + q_len and geo.trash_slot < geo.kv_total
            assert geo.a_step == 2 * q_len + 2
            assert geo.kv_row == 1024


# --------------------------------------------------------------------------
# Append plan and slot map (sections 1.2-1.3)
# --------------------------------------------------------------------------
def _monotone_stream(rnd, cap, n):
    c, out = 0, []
    for _ in range(n):
        c += rnd.choice([0, 1, 1, 2, 3, 5, 8, cap // 2 + 1, cap + 3, 3 * cap])
        out.append(c)
    return out


def pin_plan_monotone_closed_form():
    rnd = random.Random(7)
    for cap in range(1, 10):
        for q_len in (1, 2, 3, 8):
            geo = ro.geometry(cap, q_len, 128, 8)
            st = ro.RingStep(geo, 1, 8, 128, 1e6)
            prev = 0
            for c in _monotone_stream(rnd, cap, 40):
                p = st.plan(c)
                lo = c - min(c, cap)
                assert (p.win, p.lo) == (min(c, cap), lo)
                assert p.start == max(prev, lo) and p.n_new == c - max(prev, lo)
                assert p.bulk == (p.n_new > geo.a_step)
                if p.bulk:
                    pos = [q for a, n in p.chunks for q in range(a, a + n)]
                    assert pos == list(range(p.start, c))
                    assert all(n == ro.BULK_CHUNK for _, n in p.chunks[:-1])
                else:
                    assert len(p.ap_rows) == geo.a_step
                    for i, r in enumerate(p.ap_rows):
                        assert r == ((p.start + i) % cap if i < p.n_new else geo.trash_slot)
                st.slots.apply(p)
                st.next_pos, st.held_lo, st.committed = c, p.lo, c
                # closed form: slot s holds the largest p < c with p = s (mod cap)
                for s in range(cap):
                    want = s + cap * ((c - 1 - s) // cap) if s < min(c, cap) else -1
                    assert st.slots.slot_pos[s] == want, (cap, c, s)
                prev = c


def pin_fold_in_threshold():
    # Bulk only when n_new > a_step: exactly a_step new rows fold in with no pad.
    geo = ro.geometry(64, 8, 128, 8)
    p = ro.plan_step(geo, 100, 100 - geo.a_step, 0)
    assert not p.bulk and p.n_new == geo.a_step and geo.trash_slot not in p.ap_rows
    p = ro.plan_step(geo, 100, 100 - geo.a_step - 1, 0)
    assert p.bulk and p.chunks == [(100 - geo.a_step - 1, geo.a_step + 1)]
    p = ro.plan_step(geo, 100, 100, 36)
    assert p.n_new == 0 and p.ap_rows == [geo.trash_slot] * geo.a_step


def pin_window_held_brute_force():
    """After every step the ring holds the whole window [lo, committed)."""
    rnd = random.Random(11)
    for cap in range(1, 10):
        for q_len in (1, 3, 8):
            geo = ro.geometry(cap, q_len, 128, 8)
            st = ro.RingStep(geo, 1, 8, 128, 1e6)
            held = {}          # slot -> position, by brute force over every write
            c = 0
            for _ in range(60):
                c = max(0, c + rnd.choice([-3 * cap, -cap, -2, -1, 0, 1, 2, 4, cap, 2 * cap + 1]))
                p = st.plan(c)
                for pos in range(p.start, p.committed):
                    held[pos % cap] = pos
                st.slots.apply(p)
                st.next_pos, st.held_lo, st.committed = c, p.lo, c
                lo = c - min(c, cap)
                window = set(range(lo, c))
                in_ring = {q for q in held.values() if lo <= q < c}
                assert in_ring == window, (cap, c, sorted(window - in_ring))
                m = st.mask()
                vis = {int(st.slots.slot_pos[s]) for s in range(cap) if m[0, s] == 0}
                assert vis == window
                assert all(st.slots.slot_pos[s] == held.get(s, -1) for s in range(cap))


def pin_mask_encoding():
    geo = ro.geometry(64, 8, 128, 8)
    for c in (0, 1, 40, 63, 64, 65, 139):
        st = ro.RingStep(geo, 1, 8, 128, 1e6)
        p = st.plan(c)
        st.slots.apply(p)
        st.next_pos, st.held_lo, st.committed = c, p.lo, c
        m = st.mask()
        bits = m.view(np.uint16)
        assert m.shape == (geo.q_len, geo.kv_total)
        assert set(np.unique(bits)) <= {0x0000, 0xFC00}
        assert (bits[:, geo.cap:geo.cap + geo.q_len] == 0).all()
        assert (bits[:, geo.trash_slot:] == 0xFC00).all()
        assert ((bits[0] == 0).sum()) == min(c, geo.cap) + geo.q_len
        assert (bits == bits[0]).all()


# --------------------------------------------------------------------------
# RoPE (absolute positions; rotate-half reading)
# --------------------------------------------------------------------------
def pin_rope_closed_forms():
    d, base = 128, 1e6
    rs = np.random.default_rng(3)
    x = rs.normal(size=(5, d))
    assert np.array_equal(ro.rope(x, np.zeros(5), base), x)           # p = 0 is the identity
    for p in (1, 7, 4097, 131071):
        for i in (0, 1, 17, 63):
            th = p * math.pow(base, -2.0 * i / d)
            e = np.zeros((1, d)); e[0, i] = 1.0
            r = ro.rope(e, np.array([p]), base)[0]
            assert abs(r[i] - math.cos(th)) < 1e-12 and abs(r[i + 64] - math.sin(th)) < 1e-12
            assert np.abs(np.delete(r, [i, i + 64])).max() == 0.0
            e = np.zeros((1, d)); e[0, i + 64] = 1.0
            r = ro.rope(e, np.array([p]), base)[0]
            assert abs(r[i] + math.sin(th)) < 1e-12 and abs(r[i + 64] - math.cos(th)) < 1e-12
    y = ro.rope(x, np.array([3, 70, 5000, 99999, 131072]), base)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def pin_rope_relative():
    """<R_m q, R_n k> depends only on m - n (shift invariance of absolute RoPE)."""
    d, base = 128, 1e6
    rs = np.random.default_rng(5)
    q, k = rs.normal(size=(1, d)), rs.normal(size=(1, d))
    for m, n, shift in ((10, 3, 4096), (70000, 69000, 8192), (5, 5, 123457)):
        a = float((ro.rope(q, [m], base) @ ro.rope(k, [n], base).T)[0, 0])
        b = float((ro.rope(q, [m + shift], base) @ ro.rope(k, [n + shift], base).T)[0, 0])
        c = float((ro.rope(q, [m - n], base) @ k.T)[0, 0])
        assert abs(a - b) < 1e-9 and abs(a - c) < 1e-9


# --------------------------------------------------------------------------
# Attention (plain definition, sections 1.4 / 1.7)
# --------------------------------------------------------------------------
def _cache(n_head_kv=2, d=8, base=1e6):
    return ro.FullCache(n_head_kv * d, n_head_kv, d, base)


def pin_attention_single_key():
    """committed = 0, one noise row: the only visible key, so out = its V."""
    d, hk, nh = 16, 2, 4
    rs = np.random.default_rng(1)
    c = _cache(hk, d)
    q = rs.normal(size=(1, nh, d)).astype(np.float16)
    kn = rs.normal(size=(1, hk * d)).astype(np.float16)
    vn = rs.normal(size=(1, hk * d)).astype(np.float16)
    out = ro.attend(c, 0, 4, q, kn, vn, nh)
    for h in range(nh):
        g = h // (nh // hk)
        assert np.array_equal(out[0, h], vn[0, g * d:(g + 1) * d].astype(np.float64))


def pin_attention_uniform():
    """All keys zero: softmax is uniform, out = mean of the visible V rows."""
    d, hk, nh, cap, q_len = 8, 2, 4, 5, 3
    rs = np.random.default_rng(2)
    c = _cache(hk, d)
    committed = 11
    v = rs.normal(size=(committed, hk * d)).astype(np.float16)
    c.store(np.arange(committed), np.zeros((committed, hk * d), np.float16), v)
    vn = rs.normal(size=(q_len, hk * d)).astype(np.float16)
    q = rs.normal(size=(q_len, nh, d)).astype(np.float16)
    out = ro.attend(c, committed, cap, q, np.zeros((q_len, hk * d), np.float16), vn, nh)
    vis = np.concatenate([v[committed - cap:committed], vn]).astype(np.float64)
    want = vis.sum(0) / (cap + q_len)
    for h in range(nh):
        g = h // (nh // hk)
        assert np.allclose(out[:, h], want[g * d:(g + 1) * d], atol=1e-14)


def pin_attention_two_keys():
    """One context key at p = 0 and one noise key at p = 1, written out by hand."""
    d, hk, nh = 8, 1, 1
    c = _cache(hk, d)
    alpha, beta = 3.0, -2.0
    k0 = np.zeros((1, d), np.float16); k0[0, 0] = alpha
    v0 = np.zeros((1, d), np.float16); v0[0, 1] = 1.0
    c.store(np.array([0]), k0, v0)
    kn = np.zeros((1, d), np.float16); kn[0, 0] = beta
    vn = np.zeros((1, d), np.float16); vn[0, 2] = 1.0
    q = np.zeros((1, 1, d), np.float16); q[0, 0, 0] = 1.0
    out = ro.attend(c, 1, 4, q, kn, vn, nh)[0, 0]
    # The query sits at p = 1: R_1 e_0 = (cos 1) e_0 + (sin 1) e_4 (pair (0, 4)
    # for d = 8, theta_0 = 1).  The context key is unrotated (p = 0), so
    # q.k0 = alpha cos 1.  The noise key is rotated at p = 1 and stored as F16:
    # (f16(beta cos 1), f16(beta sin 1)) on dims (0, 4).
    c1, s1_ = math.cos(1.0), math.sin(1.0)
    kn0 = float(np.float16(beta * c1))
    kn4 = float(np.float16(beta * s1_))
    s0 = alpha * c1 / math.sqrt(d)
    s1 = (c1 * kn0 + s1_ * kn4) / math.sqrt(d)
    w0 = math.exp(s0) / (math.exp(s0) + math.exp(s1))
    assert abs(out[1] - w0) < 1e-14 and abs(out[2] - (1 - w0)) < 1e-14
    assert np.abs(out[[0, 3, 4, 5, 6, 7]]).max() == 0.0


def pin_attention_gqa_map():
    """Query head h reads KV head h // (n_head / n_head_kv)."""
    d, hk, nh, cap, q_len = 4, 4, 8, 6, 2
    rs = np.random.default_rng(4)
    c = _cache(hk, d)
    n = 9
    k = rs.normal(size=(n, hk * d)).astype(np.float16)
    v = np.repeat(np.arange(1, hk + 1, dtype=np.float16), d)[None, :].repeat(n, 0)
    c.store(np.arange(n), k, v)
    out = ro.attend(c, n, cap, rs.normal(size=(q_len, nh, d)).astype(np.float16),
                    rs.normal(size=(q_len, hk * d)).astype(np.float16),
                    v[:q_len], nh)
    for h in range(nh):
        assert np.allclose(out[:, h], h // (nh // hk) + 1, atol=1e-13), h


def _brute_attend(rows_k, rows_v, positions, committed, cap, q, kn, vn, nh, hk, d, base,
                  swa=None):
    """Pure-Python loops: RoPE, scores, softmax, weighted sum (tiny inputs only).

    With ``swa`` (page 1 section 1.4, sliding-window layers) the window is the
    last min(swa, committed, cap) positions and query i sees noise j <= i."""
    def rot(vec, p):
        out = list(vec)
        for i in range(d // 2):
            th = p * base ** (-2.0 * i / d)
            a, b = vec[i], vec[i + d // 2]
            out[i] = a * math.cos(th) - b * math.sin(th)
            out[i + d // 2] = b * math.cos(th) + a * math.sin(th)
        return out
    lo = committed - min(committed, cap, swa if swa is not None else cap)
    keys, vals = [], []
    for p in range(lo, committed):
        j = positions.index(p)
        kr = []
        for g in range(hk):
            kr += [float(np.float16(x)) for x in rot([float(t) for t in rows_k[j][g * d:(g + 1) * d]], p)]
        keys.append(kr)
        vals.append([float(t) for t in rows_v[j]])
    q_len = len(q)
    for i in range(q_len):
        kr = []
        for g in range(hk):
            kr += [float(np.float16(x)) for x in rot([float(t) for t in kn[i][g * d:(g + 1) * d]], committed + i)]
        keys.append(kr)
        vals.append([float(t) for t in vn[i]])
    out = [[[0.0] * d for _ in range(nh)] for _ in range(q_len)]
    grp = nh // hk
    for i in range(q_len):
        for h in range(nh):
            g = h // grp
            qr = rot([float(t) for t in q[i][h]], committed + i)
            n_ctx = len(keys) - q_len
            use = [j for j in range(len(keys))
                   if swa is None or j < n_ctx or j - n_ctx <= i]
            sc = [sum(qr[e] * keys[j][g * d + e] for e in range(d)) / math.sqrt(d) for j in use]
            mx = max(sc)
            w = [math.exp(s - mx) for s in sc]
            tot = sum(w)
            for e in range(d):
                out[i][h][e] = sum(w[t] * vals[j][g * d + e] for t, j in enumerate(use)) / tot
    return np.array(out)


def pin_attention_brute_force():
    d, hk, nh, cap, q_len, base = 4, 2, 4, 5, 2, 1e4
    rs = np.random.default_rng(6)
    rnd = random.Random(6)
    st = ro.RingStep(ro.geometry(cap, q_len, d, hk), 1, hk, d, base)
    all_k, all_v, positions = [], [], []
    c = 0
    for step in range(8):
        c += rnd.choice([1, 2, 3, 7])
        p = st.plan(c)
        k = rs.normal(size=(p.n_new, hk * d)).astype(np.float16)
        v = rs.normal(size=(p.n_new, hk * d)).astype(np.float16)
        st.commit(p, [k], [v])
        for j, pos in enumerate(range(p.start, c)):
            all_k.append(k[j]); all_v.append(v[j]); positions.append(pos)
        q = rs.normal(size=(q_len, nh, d)).astype(np.float16)
        kn = rs.normal(size=(q_len, hk * d)).astype(np.float16)
        vn = rs.normal(size=(q_len, hk * d)).astype(np.float16)
        got = ro.attend(st.caches[0], c, cap, q, kn, vn, nh)
        want = _brute_attend(all_k, all_v, positions, c, cap, q, kn, vn, nh, hk, d, base)
        assert np.abs(got - want).max() < 1e-12, (step, np.abs(got - want).max())


def pin_attention_ring_equals_full():
    """Section 1.7: masked attention over every ring slot equals the full cache.

    The ring view is built slot by slot from slot_pos (section 1.2), with the
    mask (section 1.4) as an additive bias, over all kv_total rows; empty and
    trash slots hold zeros.
    """
    d, hk, nh, base = 8, 2, 4, 1e6
    rs = np.random.default_rng(8)
    rnd = random.Random(8)
    for cap in (3, 8, 13):
        q_len = 3
        geo = ro.geometry(cap, q_len, d, hk)
        st = ro.RingStep(geo, 1, hk, d, base)
        c = 0
        for step in range(25):
            c = max(0, c + rnd.choice([1, 2, 4, cap, -2, 3 * cap]))
            p = st.plan(c)
            pos = np.arange(p.start, c)
            st.commit(p, [rs.normal(size=(p.n_new, hk * d)).astype(np.float16)],
                      [rs.normal(size=(p.n_new, hk * d)).astype(np.float16)])
            q = rs.normal(size=(q_len, nh, d)).astype(np.float16)
            kn = rs.normal(size=(q_len, hk * d)).astype(np.float16)
            vn = rs.normal(size=(q_len, hk * d)).astype(np.float16)
            full = ro.attend(st.caches[0], c, cap, q, kn, vn, nh)
            # ring view
            K = np.zeros((geo.kv_total, hk * d)); V = np.zeros((geo.kv_total, hk * d))
            for s in range(cap):
                sp = int(st.slots.slot_pos[s])
                if sp >= 0 and sp < c:
                    K[s], V[s] = st.caches[0].row(sp)
            pq = ro.noise_positions(c, q_len)
            K[cap:cap + q_len] = ro.rope_rows_f16(kn, pq, hk, d, base)
            V[cap:cap + q_len] = vn
            bias = st.mask().astype(np.float64)
            qr = ro.rope(q, pq, base)
            ring = np.empty_like(full)
            for h in range(nh):
                g = h // (nh // hk)
                s_ = qr[:, h] @ K[:, g * d:(g + 1) * d].T / math.sqrt(d) + bias
                w = np.exp(s_ - s_.max(1, keepdims=True))
                ring[:, h] = (w @ V[:, g * d:(g + 1) * d]) / w.sum(1, keepdims=True)
            assert np.abs(ring - full).max() < 1e-12, (cap, step)


def pin_swa_brute_force():
    """Sliding-window layers (page 1 section 1.4, mask_swa) against pure loops."""
    d, hk, nh, cap, q_len, base = 4, 2, 4, 6, 3, 1e4
    for swa in (1, 2, 5, 9):
        rs = np.random.default_rng(60 + swa)
        rnd = random.Random(60 + swa)
        st = ro.RingStep(ro.geometry(cap, q_len, d, hk), 1, hk, d, base)
        all_k, all_v, positions = [], [], []
        c = 0
        for step in range(7):
            c += rnd.choice([1, 2, 3, 7])
            p = st.plan(c)
            k = rs.normal(size=(p.n_new, hk * d)).astype(np.float16)
            v = rs.normal(size=(p.n_new, hk * d)).astype(np.float16)
            st.commit(p, [k], [v])
            for j, pos in enumerate(range(p.start, c)):
                all_k.append(k[j]); all_v.append(v[j]); positions.append(pos)
            q = rs.normal(size=(q_len, nh, d)).astype(np.float16)
            kn = rs.normal(size=(q_len, hk * d)).astype(np.float16)
            vn = rs.normal(size=(q_len, hk * d)).astype(np.float16)
            got = ro.attend(st.caches[0], c, cap, q, kn, vn, nh, swa_window=swa)
            want = _brute_attend(all_k, all_v, positions, c, cap, q, kn, vn, nh, hk, d, base,
                                 swa=swa)
            assert np.abs(got - want).max() < 1e-12, (swa, step, np.abs(got - want).max())


def pin_swa_ring_equals_window():
    """Section 1.7 for sliding-window layers: masked attention over every ring
    slot with the SWA mask equals the full cache restricted to the last
    min(swa, win) positions with a causal noise block (rewinds included)."""
    d, hk, nh, base = 8, 2, 4, 1e6
    rs = np.random.default_rng(61)
    rnd = random.Random(61)
    for cap, swa in ((3, 2), (8, 5), (13, 13), (13, 40)):
        q_len = 3
        geo = ro.geometry(cap, q_len, d, hk)
        st = ro.RingStep(geo, 1, hk, d, base)
        c = 0
        for step in range(25):
            c = max(0, c + rnd.choice([1, 2, 4, cap, -2, 3 * cap]))
            p = st.plan(c)
            st.commit(p, [rs.normal(size=(p.n_new, hk * d)).astype(np.float16)],
                      [rs.normal(size=(p.n_new, hk * d)).astype(np.float16)])
            q = rs.normal(size=(q_len, nh, d)).astype(np.float16)
            kn = rs.normal(size=(q_len, hk * d)).astype(np.float16)
            vn = rs.normal(size=(q_len, hk * d)).astype(np.float16)
            want = ro.attend(st.caches[0], c, cap, q, kn, vn, nh, swa_window=swa)
            K = np.zeros((geo.kv_total, hk * d)); V = np.zeros((geo.kv_total, hk * d))
            for s_ in range(cap):
                sp = int(st.slots.slot_pos[s_])
                if 0 <= sp < c:
                    K[s_], V[s_] = st.caches[0].row(sp)
            pq = ro.noise_positions(c, q_len)
            K[cap:cap + q_len] = ro.rope_rows_f16(kn, pq, hk, d, base)
            V[cap:cap + q_len] = vn
            bias = st.mask_swa(swa).astype(np.float64)
            qr = ro.rope(q, pq, base)
            ring = np.empty_like(want)
            for h in range(nh):
                g = h // (nh // hk)
                s_ = qr[:, h] @ K[:, g * d:(g + 1) * d].T / math.sqrt(d) + bias
                w = np.exp(s_ - s_.max(1, keepdims=True))
                ring[:, h] = (w @ V[:, g * d:(g + 1) * d]) / w.sum(1, keepdims=True)
            assert np.abs(ring - want).max() < 1e-12, (cap, swa, step)


def pin_swa_invariants():
    """Properties that fix the sliding-window form: the output of noise row i
    does not depend on noise rows j > i nor on positions before the window;
    it does depend on the oldest position inside it; a window of at least
    cap with one noise row is the full-attention result."""
    d, hk, nh, cap, q_len, base = 8, 2, 4, 16, 4, 1e6
    rs = np.random.default_rng(62)
    n = 40
    k = rs.normal(size=(n, hk * d)).astype(np.float16)
    v = rs.normal(size=(n, hk * d)).astype(np.float16)
    q = rs.normal(size=(q_len, nh, d)).astype(np.float16)
    kn = rs.normal(size=(q_len, hk * d)).astype(np.float16)
    vn = rs.normal(size=(q_len, hk * d)).astype(np.float16)

    def run(kk, vv, knn, vnn, swa, ql=q_len):
        c = ro.FullCache(hk * d, hk, d, base)
        c.store(np.arange(n), kk, vv)
        return ro.attend(c, n, cap, q[:ql], knn[:ql], vnn[:ql], nh, swa_window=swa)

    swa = 5
    base_out = run(k, v, kn, vn, swa)
    for i in range(q_len - 1):
        kn2, vn2 = kn.copy(), vn.copy()
        kn2[i + 1:] = rs.normal(size=kn2[i + 1:].shape).astype(np.float16)
        vn2[i + 1:] = rs.normal(size=vn2[i + 1:].shape).astype(np.float16)
        out = run(k, v, kn2, vn2, swa)
        assert np.array_equal(out[: i + 1], base_out[: i + 1]), i
        assert not np.allclose(out[i + 1:], base_out[i + 1:]), i
    k2, v2 = k.copy(), v.copy()
    k2[: n - swa] = 0; v2[: n - swa] = 7
    assert np.array_equal(run(k2, v2, kn, vn, swa), base_out)
    k3, v3 = k.copy(), v.copy()
    v3[n - swa] = 7
    assert not np.allclose(run(k3, v3, kn, vn, swa), base_out)
    c = ro.FullCache(hk * d, hk, d, base)
    c.store(np.arange(n), k, v)
    full = ro.attend(c, n, cap, q[:1], kn[:1], vn[:1], nh)
    assert np.array_equal(run(k, v, kn, vn, cap, ql=1), full)
    assert np.array_equal(run(k, v, kn, vn, 10 * cap, ql=1), full)


def pin_swa_mask_closed_form():
    """mask_swa on monotone streams: ring slot s is visible iff it holds one
    of the last min(swa, committed, cap) positions; noise row i sees noise
    slots cap..cap+i; trash and alignment pad rows never."""
    rnd = random.Random(63)
    for cap, q_len, swa in ((5, 2, 3), (64, 8, 20), (40, 8, 100), (33, 4, 1)):
        g = ro.geometry(cap, q_len, 4, 1)
        for stream in (_monotone_stream(rnd, cap, 30), [0, 1, cap - 1, cap, cap + 1, 5 * cap + 3]):
            st = ro.RingStep(g, 1, 1, 4, 1e6)
            for c in stream:
                p = st.plan(c)
                st.commit(p, [np.zeros((p.n_new, g.kv_row), np.float16)],
                          [np.zeros((p.n_new, g.kv_row), np.float16)])
                m = st.mask_swa(swa).view(np.uint16)
                lo = c - min(swa, c, cap)
                vis = {pos % cap for pos in range(lo, c)}
                for i in range(q_len):
                    row = m[i]
                    assert {int(s_) for s_ in np.flatnonzero(row[:cap] == 0)} == vis, (cap, c, i)
                    assert (row[:cap][row[:cap] != 0] == 0xFC00).all()
                    assert list(row[cap: cap + q_len]) == [0] * (i + 1) + [0xFC00] * (q_len - i - 1)
                    assert (row[cap + q_len:] == 0xFC00).all()


def pin_attention_fp32_mode():
    d, hk, nh, cap, q_len = 128, 8, 32, 64, 8
    rs = np.random.default_rng(9)
    c = ro.FullCache(hk * d, hk, d, 1e6)
    n = 150
    c.store(np.arange(n), (0.5 * rs.normal(size=(n, hk * d))).astype(np.float16),
            (0.5 * rs.normal(size=(n, hk * d))).astype(np.float16))
    args = (c, n, cap, (0.5 * rs.normal(size=(q_len, nh, d))).astype(np.float16),
            (0.5 * rs.normal(size=(q_len, hk * d))).astype(np.float16),
            (0.5 * rs.normal(size=(q_len, hk * d))).astype(np.float16), nh)
    a = ro.attend(*args, dtype=np.float64)
    b = ro.attend(*args, dtype=np.float32)
    assert b.dtype == np.float32 and np.abs(a - b).max() < 1e-5


# --------------------------------------------------------------------------
# New rows' K/V from fused features (the shallow injection named in the test
# log of the ring port page) and the feature mirror
# --------------------------------------------------------------------------
def _one_hot(rows, d_model, cols):
    w = np.zeros((rows, d_model), np.float16)
    w[np.arange(rows), cols] = 1.0
    return w


def pin_project_v_selects_features():
    """V = wv f: rows of wv that pick one feature give that feature exactly;
    a row that adds two features gives their sum rounded once to F16."""
    rs = np.random.default_rng(21)
    n, d_model, hk, d = 5, 40, 2, 8
    f = rs.normal(size=(n, d_model)).astype(np.float16)
    cols = rs.integers(0, d_model, size=hk * d)
    wv = _one_hot(hk * d, d_model, cols)
    wk = (rs.normal(size=(hk * d, d_model)) / 8).astype(np.float16)
    _, v = ro.project_kv(f, wk, wv, np.ones(d), np.arange(n), hk, d, 1e6)
    assert v.dtype == np.float16 and np.array_equal(v, f[:, cols])
    wv2 = wv.copy()
    wv2[0, (cols[0] + 1) % d_model] = 1.0
    _, v2 = ro.project_kv(f, wk, wv2, np.ones(d), np.arange(n), hk, d, 1e6)
    want = (f[:, cols[0]].astype(np.float64) + f[:, (cols[0] + 1) % d_model]).astype(np.float16)
    assert np.array_equal(v2[:, 0], want) and np.array_equal(v2[:, 1:], v[:, 1:])


def pin_project_k_head_rms():
    """With k_norm = 1 every KV head's K has RMS 1 at any position (RoPE keeps
    the norm); the norm is per head, so scaling one head's weights changes
    nothing, and the projection of one head ignores the other's weights."""
    rs = np.random.default_rng(22)
    n, d_model, hk, d = 6, 64, 3, 16
    f = rs.normal(size=(n, d_model)).astype(np.float16)
    wk = (rs.normal(size=(hk * d, d_model)) / 8).astype(np.float16)
    wv = (rs.normal(size=(hk * d, d_model)) / 8).astype(np.float16)
    for pos in (np.arange(n), np.arange(n) + 4093, np.full(n, 131071)):
        k, _ = ro.project_kv(f, wk, wv, np.ones(d), pos, hk, d, 1e6)
        rms = np.sqrt((k.astype(np.float64).reshape(n, hk, d) ** 2).mean(-1))
        assert np.abs(rms - 1.0).max() < 1e-3, rms
    k0, _ = ro.project_kv(f, wk, wv, np.ones(d), np.arange(n), hk, d, 1e6, eps=0.0)
    w2 = wk.copy()
    w2[d:2 * d] *= np.float16(8.0)            # head 1 only, exact power of two
    w2[2 * d:] = (rs.normal(size=(d, d_model)) / 8).astype(np.float16)  # head 2 changed
    k1, _ = ro.project_kv(f, w2, wv, np.ones(d), np.arange(n), hk, d, 1e6, eps=0.0)
    assert np.array_equal(k0[:, :2 * d], k1[:, :2 * d])
    assert not np.array_equal(k0[:, 2 * d:], k1[:, 2 * d:])


def pin_project_k_constant_slice():
    """A head whose pre-norm slice is the constant c normalises to sign(c)
    times k_norm: at p = 0 (RoPE is the identity) K is f16(sign(c) k_norm)."""
    rs = np.random.default_rng(23)
    n, d_model, hk, d = 4, 12, 2, 8
    f = rs.normal(size=(n, d_model)).astype(np.float16)
    f[:, 3] = np.float16(-2.5)
    f[:, 7] = np.float16(0.75)
    wk = np.zeros((hk * d, d_model), np.float16)
    wk[:d, 3] = 1.0      # head 0: every dim reads feature 3
    wk[d:, 7] = 1.0      # head 1: every dim reads feature 7
    knorm = rs.uniform(0.25, 3.0, size=d)
    k, _ = ro.project_kv(f, wk, wk, knorm, np.zeros(n, np.int64), hk, d, 1e6, eps=0.0)
    assert np.array_equal(k[:, :d], np.broadcast_to((-knorm).astype(np.float16), (n, d)))
    assert np.array_equal(k[:, d:], np.broadcast_to(knorm.astype(np.float16), (n, d)))


def pin_project_k_rope_after_norm():
    """Normalised K that is exact in F16 (entries +-1, k_norm powers of two)
    rotated at p is the same as projecting at p: RoPE comes after the norm and
    the weight, at the row's own absolute position, with one rounding."""
    rs = np.random.default_rng(24)
    n, d_model, hk, d = 5, 2 * 16, 2, 16
    f = rs.choice([-1.0, 1.0], size=(n, d_model)).astype(np.float16)
    wk = _one_hot(hk * d, d_model, rs.permutation(d_model)[: hk * d])
    knorm = np.array([1.0, 2.0, 0.5, 4.0] * (d // 4))
    pos = np.array([0, 7, 4096, 70001, 131071])
    k0, _ = ro.project_kv(f, wk, wk, knorm, np.zeros(n, np.int64), hk, d, 1e6, eps=0.0)
    kp, _ = ro.project_kv(f, wk, wk, knorm, pos, hk, d, 1e6, eps=0.0)
    assert np.array_equal(kp, ro.rope_rows_f16(k0, pos, hk, d, 1e6))
    assert not np.array_equal(kp[1:], k0[1:])


def pin_project_scale_invariance():
    """With eps = 0 the K norm ignores a power-of-two scale of the features;
    V scales with it exactly."""
    rs = np.random.default_rng(25)
    n, d_model, hk, d = 7, 48, 2, 8
    f = rs.normal(size=(n, d_model)).astype(np.float16)
    wk = (rs.normal(size=(hk * d, d_model)) / 8).astype(np.float16)
    wv = (rs.normal(size=(hk * d, d_model)) / 8).astype(np.float16)
    knorm = rs.uniform(0.5, 1.5, size=d)
    pos = rs.integers(0, 100000, size=n)
    k1, v1 = ro.project_kv(f, wk, wv, knorm, pos, hk, d, 1e6, eps=0.0)
    k2, v2 = ro.project_kv(f * np.float16(4.0), wk, wv, knorm, pos, hk, d, 1e6, eps=0.0)
    assert np.array_equal(k1, k2)
    assert np.array_equal(v2.astype(np.float64), 4.0 * v1.astype(np.float64))


def pin_feature_mirror_brute_force():
    """The mirror returns, for a position, the features last written for it as
    long as no later write landed in its slot p % cap, and refuses it
    otherwise; over plain streams that is exactly the last cap positions."""
    rs = random.Random(26)
    for cap in (1, 3, 8):
        m = ro.FeatureMirror(cap, 4)
        history = []                  # every (position, features) write, in order
        hi = 0
        for step in range(60):
            rewind = step % 9 == 8 and hi > 2
            if rewind:
                hi -= rs.randint(1, min(hi, cap))        # rewind: rewrite from there
            n = rs.randint(0, 2 * cap)
            pos = np.arange(hi, hi + n)
            feats = np.array([[p, step, p % 7, -p] for p in pos], np.float16).reshape(n, 4)
            m.write(pos, feats)
            history += [(int(p), feats[j]) for j, p in enumerate(pos)]
            hi += n
            written = {p for p, _ in history}
            for p in sorted(written):
                later = [q for q, _ in history if q % cap == p % cap]
                held = later[-1] == p                  # the slot's most recent write
                if held:
                    want = [fv for q, fv in history if q == p][-1]
                    assert np.array_equal(m.read(np.array([p]))[0], want), (cap, step, p)
                else:
                    try:
                        m.read(np.array([p]))
                        raise AssertionError(f"position {p} read after its slot was reused")
                    except KeyError:
                        pass
            if not rewind and n >= cap:
                for p in range(hi - cap, hi):
                    m.read(np.array([p]))


def pin_commit_features_equals_commit():
    """Rows from features through weights that select +-1 features (K exact
    after the norm) equal rows passed directly, over a stream that wraps the
    ring and rewinds: the mirror supplies exactly the positions each plan needs."""
    rs = np.random.default_rng(27)
    cap, q_len, hk, d, nh, d_model = 6, 2, 2, 8, 4, 40
    g = ro.geometry(cap, q_len, d, hk)
    kv_row = hk * d
    wk = _one_hot(kv_row, d_model, np.arange(kv_row))
    wv = _one_hot(kv_row, d_model, np.arange(kv_row) + kv_row)
    a = ro.RingStep(g, 1, hk, d, 1e6)
    b = ro.RingStep(g, 1, hk, d, 1e6)
    mirror = ro.FeatureMirror(cap, d_model)
    feats = {}
    committed = 0
    resupplied = 0
    for step, c in enumerate([4, 5, 9, 10, 12, 11, 7, 8, 15, 16, 19, 30, 31]):
        # the target supplies features of positions past the last step only
        new = np.arange(committed, c) if c > committed else np.arange(0)
        for p in new:
            feats[int(p)] = np.concatenate([rs.choice([-1.0, 1.0], size=kv_row),
                                            rs.normal(size=d_model - kv_row)]).astype(np.float16)
        if new.size:
            mirror.write(new, np.stack([feats[int(p)] for p in new]))
        pa, pb = a.plan(c), b.plan(c)
        assert pa == pb
        pos = np.arange(pa.start, c)
        # a rewind below what the ring holds re-appends window rows whose
        # mirror slots newer positions took: those are supplied again
        for p in pos:
            try:
                mirror.read(np.array([p]))
            except KeyError:
                mirror.write(np.array([p]), feats[int(p)][None])
                resupplied += 1
        rows = np.stack([feats[int(p)] for p in pos]) if pos.size else np.zeros((0, d_model), np.float16)
        a.commit(pa, [rows[:, :kv_row]], [rows[:, kv_row:2 * kv_row]])
        b.commit_features(pb, mirror, [wk], [wv], [np.ones(d)], eps=0.0)
        committed = c
        q = rs.normal(size=(q_len, nh, d)).astype(np.float16)
        kn = rs.normal(size=(q_len, kv_row)).astype(np.float16)
        vn = rs.normal(size=(q_len, kv_row)).astype(np.float16)
        oa = ro.attend(a.caches[0], c, cap, q, kn, vn, nh)
        ob = ro.attend(b.caches[0], c, cap, q, kn, vn, nh)
        assert np.array_equal(oa, ob), step
    assert resupplied > 0      # the stream does reach a rewind past the mirror


ALL_PINS = [
    pin_geometry_worked_example, pin_geometry_closed_form,
    pin_plan_monotone_closed_form, pin_fold_in_threshold,
    pin_window_held_brute_force, pin_mask_encoding,
    pin_rope_closed_forms, pin_rope_relative,
    pin_attention_single_key, pin_attention_uniform, pin_attention_two_keys,
    pin_attention_gqa_map, pin_attention_brute_force,
    pin_swa_brute_force, pin_swa_ring_equals_window, pin_swa_invariants,
    pin_swa_mask_closed_form,
    pin_attention_ring_equals_full, pin_attention_fp32_mode,
    pin_project_v_selects_features, pin_project_k_head_rms, pin_project_k_constant_slice,
    pin_project_k_rope_after_norm, pin_project_scale_invariance,
    pin_feature_mirror_brute_force, pin_commit_features_equals_commit,
]
