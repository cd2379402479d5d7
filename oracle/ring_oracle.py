"""CPU oracle for the DFlash2 draft-KV ring step (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The device path never calls it and shares
no code with it.

Source: page "DFLASH2_RING_PORT.md" (DFlash2 draft KV-ring port to llama.cpp),
section 1 ("what the ring does in Luce"):
  * 1.1  geometry: a_step, trash_slot, kv_total, kv_row; K/V zeroed once.
  * 1.2  slot of position p is p % cap; slot_pos[slot] = p.
  * 1.3  win, lo, start, n_new; bulk append when n_new > a_step, fold-in with
         pad rows to trash_slot otherwise; noise positions committed + i.
  * 1.4  full-attention mask: 0 iff lo <= slot_pos[s] < committed, noise
         block visible both ways, everything else -inf.  Sliding-window
         mask for SWA layers: the window shrinks to
         eff_win = min(swa_window, win) positions ending at committed (the
         same anchor for every noise row) and the noise block is causal
         (noise row i sees noise slots j <= i).
  * 1.6  the legacy path recomputes the whole window every step.
  * 1.7  the ring equals that legacy full-window recompute (absolute RoPE plus
         masks); memory is 2 * n_layer * kv_row * kv_total * 2 bytes.
TL;DR of the same page: absolute RoPE positions, K/V computed for new rows only.

K/V rows from features (the page's notes on the port: Luce keeps a mirror
of the target's features, DraftFeatureMirror, whose capacity is the ring's,
section 1.6, and begin_step computes the new rows' context K/V from it; the
test log's list of refuted hypotheses, item 4, spells the per-layer
computation out as wk/wv @ fused + k_norm + rope, the shallow injection):
  * the mirror holds the fused feature vector of the last cap positions at
    slot p % cap;
  * K = RoPE_p(k_norm(wk @ fused)), V = wv @ fused, k_norm an RMS norm over
    each KV head's head_dim values times a learned head_dim weight.

What the oracle computes is the plain definition the ring is equal to: a
non-ring cache holding every committed position, attended over exactly
[lo, committed) plus the noise block.  Index expectations (slot_pos, mask,
append rows) follow sections 1.2-1.4 written out directly.

Readings where the page is silent (each is listed in the design notes):
  * RoPE is the rotate-half (NeoX) form over the whole head: pairs (i, i+64),
    theta_i = base ** (-2 i / head_dim), angle = p * theta_i, all in fp64.
  * Q and K (context and noise) are rotated, V never; K is rounded to F16
    (round to nearest even) after rotation, as the ring stores F16.
  * scores are q.k / sqrt(head_dim); query head h reads KV head h // group.
  * a rewind (committed below the last step's) drops positions >= committed;
    window rows the ring no longer holds are appended again.
  * bulk appends go in chunks of 1024 rows in ascending position, no pads.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

BULK_CHUNK = 1024
NEG_INF_F16 = np.float16(-np.inf)


# --------------------------------------------------------------------------
# Section 1.1: geometry.
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Geometry:
    cap: int
    q_len: int
    a_step: int
    trash_slot: int
    kv_total: int
    kv_row: int


def align_up(x: int, a: int) -> int:
    return ((x + a - 1) // a) * a


def geometry(cap: int, q_len: int, head_dim: int, n_head_kv: int) -> Geometry:
    """Ring geometry of section 1.1."""
    return Geometry(
        cap=cap,
        q_len=q_len,
        a_step=2 * q_len + 2,
        trash_slot=cap + q_len,
        kv_total=align_up(cap + q_len + 1, 32),
        kv_row=head_dim * n_head_kv,
    )


def ring_bytes(n_layer: int, kv_row: int, kv_total: int) -> int:
    """F16 K plus V ring bytes over all layers (section 1.7 formula)."""
    return 2 * n_layer * kv_row * kv_total * 2


# --------------------------------------------------------------------------
# Section 1.3: window arithmetic and the append plan.
# --------------------------------------------------------------------------
@dataclass
class Plan:
    committed: int
    win: int
    lo: int
    start: int
    n_new: int
    bulk: bool
    # fold-in: a_step destination rows (real slots, then trash_slot pads);
    # bulk: list of (first position, row count) chunks.
    ap_rows: List[int] = field(default_factory=list)
    chunks: List[Tuple[int, int]] = field(default_factory=list)


def plan_step(g: Geometry, committed: int, next_pos: int, held_lo: int) -> Plan:
    """Which rows one begin_step appends, and where.

    ``next_pos`` is the committed count of the previous step and ``held_lo``
    that step's lo (0 before the first step): the ring then holds exactly the
    positions [held_lo, next_pos).
    """
    win = min(committed, g.cap)
    lo = committed - win
    if lo < held_lo:
        # Rewind past what the ring still holds: append the whole window again.
        start = lo
    else:
        start = max(min(next_pos, committed), lo)
    n_new = committed - start
    p = Plan(committed=committed, win=win, lo=lo, start=start, n_new=n_new,
             bulk=n_new > g.a_step)
    if p.bulk:
        first = start
        while first < committed:
            n = min(BULK_CHUNK, committed - first)
            p.chunks.append((first, n))
            first += n
    else:
        p.ap_rows = [(start + i) % g.cap for i in range(n_new)]
        p.ap_rows += [g.trash_slot] * (g.a_step - n_new)
    return p


def noise_positions(committed: int, q_len: int) -> np.ndarray:
    """Absolute positions of the noise block: committed + i."""
    return committed + np.arange(q_len, dtype=np.int64)


# --------------------------------------------------------------------------
# RoPE at absolute positions (TL;DR and section 4 of the page; form = reading).
# --------------------------------------------------------------------------
def rope_inv_freq(head_dim: int, base: float) -> np.ndarray:
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / head_dim)


def rope(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """Rotate the last axis (head_dim) of ``x [n, ..., head_dim]`` at positions [n].

    Pairs (i, i + head_dim/2) turn by angle p * theta_i.  fp64 throughout.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    pos = np.asarray(positions, dtype=np.float64).reshape((-1,) + (1,) * (x.ndim - 1))
    ang = pos * rope_inv_freq(d, base)          # [n, 1.., half]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def rope_rows_f16(rows: np.ndarray, positions: np.ndarray, n_head_kv: int,
                  head_dim: int, base: float) -> np.ndarray:
    """RoPE K rows ``[n, kv_row]`` head by head, then round to F16 (RNE)."""
    n = rows.shape[0]
    r = rope(rows.reshape(n, n_head_kv, head_dim), positions, base)
    return r.reshape(n, n_head_kv * head_dim).astype(np.float16)


# --------------------------------------------------------------------------
# Section 1.6 / 1.7: the full (non-ring) cache the ring is equal to.
# --------------------------------------------------------------------------
class FullCache:
    """Every committed position's RoPE'd K row and V row (F16), by position."""

    BLOCK = 1024

    def __init__(self, kv_row: int, n_head_kv: int, head_dim: int, base: float):
        self.kv_row = kv_row
        self.n_head_kv = n_head_kv
        self.head_dim = head_dim
        self.base = base
        self._k: Dict[int, np.ndarray] = {}
        self._v: Dict[int, np.ndarray] = {}
        self._have: Dict[int, np.ndarray] = {}

    def _block(self, b: int):
        if b not in self._k:
            self._k[b] = np.zeros((self.BLOCK, self.kv_row), np.float16)
            self._v[b] = np.zeros((self.BLOCK, self.kv_row), np.float16)
            self._have[b] = np.zeros(self.BLOCK, bool)
        return self._k[b], self._v[b], self._have[b]

    def store(self, positions: np.ndarray, k_raw: np.ndarray, v_raw: np.ndarray) -> None:
        """Store rows for ``positions``; K gets RoPE at its own position."""
        positions = np.asarray(positions, dtype=np.int64)
        if positions.size == 0:
            return
        k = rope_rows_f16(k_raw, positions, self.n_head_kv, self.head_dim, self.base)
        self.store_rotated(positions, k, v_raw)

    def store_rotated(self, positions: np.ndarray, k: np.ndarray, v_raw: np.ndarray) -> None:
        """Store rows whose K is already rotated (and rounded to F16)."""
        positions = np.asarray(positions, dtype=np.int64)
        if positions.size == 0:
            return
        k = np.asarray(k, dtype=np.float16)
        v = np.asarray(v_raw, dtype=np.float16)
        for b in np.unique(positions // self.BLOCK):
            sel = (positions // self.BLOCK) == b
            kb, vb, hb = self._block(int(b))
            off = positions[sel] - int(b) * self.BLOCK
            kb[off] = k[sel]
            vb[off] = v[sel]
            hb[off] = True

    def rows(self, lo: int, hi: int) -> Tuple[np.ndarray, np.ndarray]:
        """K and V rows of positions [lo, hi); every one must have been stored."""
        ks, vs = [], []
        p = lo
        while p < hi:
            b = p // self.BLOCK
            e = min(hi, (b + 1) * self.BLOCK)
            kb, vb, hb = self._block(b)
            o0, o1 = p - b * self.BLOCK, e - b * self.BLOCK
            if not hb[o0:o1].all():
                missing = p + int(np.argmin(hb[o0:o1]))
                raise KeyError(f"position {missing} was never stored")
            ks.append(kb[o0:o1])
            vs.append(vb[o0:o1])
            p = e
        if not ks:
            z = np.zeros((0, self.kv_row), np.float16)
            return z, z
        return np.concatenate(ks), np.concatenate(vs)

    def row(self, p: int) -> Tuple[np.ndarray, np.ndarray]:
        k, v = self.rows(p, p + 1)
        return k[0], v[0]


def attend(cache: FullCache, committed: int, cap: int, q: np.ndarray,
           k_noise: np.ndarray, v_noise: np.ndarray, n_head: int,
           dtype=np.float64, swa_window: Optional[int] = None) -> np.ndarray:
    """Attention of the noise block over the window [lo, committed) plus noise.

    q: [q_len, n_head, head_dim] F16, pre-RoPE; k_noise, v_noise: [q_len, kv_row]
    F16 (k pre-RoPE).  Returns [q_len, n_head, head_dim] in ``dtype``.  With
    dtype float32 the scores, softmax and weighted sum accumulate in fp32
    (inputs are the same F16 values and fp64 RoPE angles).

    ``swa_window`` selects the sliding-window layer form of section 1.4: the
    window is the last min(swa_window, win) committed positions and noise
    query i attends noise keys j <= i only.
    """
    d = cache.head_dim
    hk = cache.n_head_kv
    group = n_head // hk
    q_len = q.shape[0]
    win = min(committed, cap)
    if swa_window is not None:
        win = min(swa_window, win)
    lo = committed - win
    pq = noise_positions(committed, q_len)

    k_ctx, v_ctx = cache.rows(lo, committed)
    kn = rope_rows_f16(k_noise, pq, hk, d, cache.base)
    keys = np.concatenate([k_ctx, kn]).reshape(-1, hk, d).astype(dtype)
    vals = np.concatenate([v_ctx, np.asarray(v_noise, np.float16)]).reshape(-1, hk, d).astype(dtype)

    qr = rope(q, pq, cache.base).astype(dtype)          # [q_len, n_head, d]
    scale = dtype(1.0 / math.sqrt(d))
    bias = np.zeros((q_len, keys.shape[0]), dtype=dtype)
    if swa_window is not None:
        n_ctx = committed - lo
        later = np.arange(q_len)[None, :] > np.arange(q_len)[:, None]   # key j > query i
        bias[:, n_ctx:] = np.where(later, -np.inf, 0.0)
    out = np.empty((q_len, n_head, d), dtype=dtype)
    for h in range(n_head):
        g = h // group
        s = (qr[:, h, :] @ keys[:, g, :].T) * scale + bias  # [q_len, n_keys]
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        l = w.sum(axis=1, keepdims=True)
        out[:, h, :] = (w @ vals[:, g, :]) / l
    return out


# --------------------------------------------------------------------------
# New rows' K/V from the fused feature vector, and the feature mirror.
# --------------------------------------------------------------------------
RMS_EPS = 1e-6  # epsilon of the per-head RMS norm of K (reading: not on the page)


def project_kv(fused: np.ndarray, wk: np.ndarray, wv: np.ndarray, k_norm: np.ndarray,
               positions: np.ndarray, n_head_kv: int, head_dim: int, base: float,
               eps: float = RMS_EPS) -> Tuple[np.ndarray, np.ndarray]:
    """K and V rows of ``positions`` from their fused feature vectors.

    fused [n, d_model] F16; wk, wv [kv_row, d_model] F16 (output dim first);
    k_norm [head_dim] fp32.  In fp64: k = wk @ f, each KV head's slice scaled
    to unit RMS (eps added to the mean square) and multiplied by k_norm, then
    RoPE at the row's position, then one rounding to F16; v = wv @ f rounded
    to F16.  Returns (K [n, kv_row] F16 rotated, V [n, kv_row] F16).
    """
    n = fused.shape[0]
    f = np.asarray(fused, dtype=np.float64)
    k = f @ np.asarray(wk, dtype=np.float64).T
    v = f @ np.asarray(wv, dtype=np.float64).T
    k = k.reshape(n, n_head_kv, head_dim)
    rms = np.sqrt((k * k).mean(axis=-1, keepdims=True) + eps)
    k = k / rms * np.asarray(k_norm, dtype=np.float64)
    k = rope(k, positions, base).reshape(n, n_head_kv * head_dim)
    return k.astype(np.float16), v.astype(np.float16)


class FeatureMirror:
    """Fused feature vectors of the last ``cap`` positions, slot p % cap."""

    def __init__(self, cap: int, d_model: int):
        self.cap = cap
        self.slots = np.zeros((cap, d_model), np.float16)
        self.slot_pos = np.full(cap, -1, dtype=np.int64)

    def write(self, positions: np.ndarray, features: np.ndarray) -> None:
        for j, p in enumerate(np.asarray(positions, dtype=np.int64)):
            self.slots[p % self.cap] = features[j]
            self.slot_pos[p % self.cap] = p

    def read(self, positions: np.ndarray) -> np.ndarray:
        positions = np.asarray(positions, dtype=np.int64)
        out = np.empty((len(positions), self.slots.shape[1]), np.float16)
        for j, p in enumerate(positions):
            if self.slot_pos[p % self.cap] != p:
                raise KeyError(f"position {p} is not in the mirror")
            out[j] = self.slots[p % self.cap]
        return out


# --------------------------------------------------------------------------
# Sections 1.2 and 1.4: what the ring's index state must be.
# --------------------------------------------------------------------------
class SlotHistory:
    """slot_pos of one sequence, from the append history (section 1.2)."""

    def __init__(self, g: Geometry):
        self.g = g
        self.slot_pos = np.full(g.cap, -1, dtype=np.int32)

    def apply(self, p: Plan) -> None:
        for pos in range(p.start, p.committed):
            self.slot_pos[pos % self.g.cap] = pos


def mask_full(g: Geometry, slot_pos: np.ndarray, committed: int) -> np.ndarray:
    """F16 mask [q_len, kv_total]: 0 where visible, -inf elsewhere (section 1.4)."""
    win = min(committed, g.cap)
    lo = committed - win
    row = np.full(g.kv_total, NEG_INF_F16, dtype=np.float16)
    sp = slot_pos.astype(np.int64)
    row[: g.cap] = np.where((sp >= lo) & (sp < committed), np.float16(0.0), NEG_INF_F16)
    row[g.cap: g.cap + g.q_len] = np.float16(0.0)
    return np.broadcast_to(row, (g.q_len, g.kv_total)).copy()


def mask_swa(g: Geometry, slot_pos: np.ndarray, committed: int, swa_window: int) -> np.ndarray:
    """F16 mask [q_len, kv_total] of a sliding-window layer (section 1.4).

    eff_win = min(swa_window, win) and swa_lo = committed - eff_win: ring slot
    s is visible to every noise row iff swa_lo <= slot_pos[s] < committed;
    noise slot cap + j is visible to noise row i iff j <= i.
    """
    eff_win = min(swa_window, min(committed, g.cap))
    swa_lo = committed - eff_win
    sp = slot_pos.astype(np.int64)
    m = np.full((g.q_len, g.kv_total), NEG_INF_F16, dtype=np.float16)
    m[:, : g.cap] = np.where((sp >= swa_lo) & (sp < committed), np.float16(0.0), NEG_INF_F16)
    for i in range(g.q_len):
        m[i, g.cap: g.cap + i + 1] = np.float16(0.0)
    return m


class RingStep:
    """One sequence's ring state, driven step by step (test harness helper).

    Tracks next_pos / held_lo, the slot history and a full cache per layer.
    ``rows_for(plan)`` says which positions the caller must supply.
    """

    def __init__(self, g: Geometry, n_layer: int, n_head_kv: int, head_dim: int, base: float):
        self.g = g
        self.next_pos = 0
        self.held_lo = 0
        self.slots = SlotHistory(g)
        self.caches = [FullCache(g.kv_row, n_head_kv, head_dim, base) for _ in range(n_layer)]
        self.committed = 0

    def plan(self, committed: int) -> Plan:
        return plan_step(self.g, committed, self.next_pos, self.held_lo)

    def commit(self, p: Plan, k_rows: List[np.ndarray], v_rows: List[np.ndarray]) -> None:
        """Apply a plan with per-layer raw rows for positions [start, committed)."""
        pos = np.arange(p.start, p.committed, dtype=np.int64)
        for layer, cache in enumerate(self.caches):
            cache.store(pos, k_rows[layer], v_rows[layer])
        self._advance(p)

    def commit_features(self, p: Plan, mirror: FeatureMirror, wk: List[np.ndarray],
                        wv: List[np.ndarray], k_norm: List[np.ndarray],
                        eps: float = RMS_EPS) -> None:
        """Apply a plan whose rows come from the mirror's fused features."""
        pos = np.arange(p.start, p.committed, dtype=np.int64)
        if pos.size:
            f = mirror.read(pos)
            for layer, cache in enumerate(self.caches):
                k, v = project_kv(f, wk[layer], wv[layer], k_norm[layer], pos,
                                  cache.n_head_kv, cache.head_dim, cache.base, eps)
                cache.store_rotated(pos, k, v)
        self._advance(p)

    def _advance(self, p: Plan) -> None:
        self.slots.apply(p)
        self.next_pos = p.committed
        self.held_lo = p.lo
        self.committed = p.committed

    def mask(self) -> np.ndarray:
        return mask_full(self.g, self.slots.slot_pos, self.committed)

    def mask_swa(self, swa_window: int) -> np.ndarray:
        return mask_swa(self.g, self.slots.slot_pos, self.committed, swa_window)
