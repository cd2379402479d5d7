"""Drive the HIP ring and the CPU oracle through the same seeded step stream.

Test infrastructure: imports both the binding and the oracle, feeds them the
same ``workload`` inputs and compares them.  Neither side sees the other's
results; only the inputs are shared.
"""

from __future__ import annotations

import bisect
import os
from typing import Dict, List, Optional

import numpy as np

import oracle.ring_oracle as ro
import workload as W
from workload.configs import T_K, T_V

ATOL = 2e-3   # attention output tolerance (absolute part)
RTOL = 1e-2   # attention output tolerance (relative part)


def f16_ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in units in the last place between two F16 arrays (finite)."""
    ia = a.view(np.uint16).astype(np.int32)
    ib = b.view(np.uint16).astype(np.int32)
    # map sign-magnitude to a monotone integer line
    ia = np.where(ia & 0x8000, -(ia & 0x7FFF), ia)
    ib = np.where(ib & 0x8000, -(ib & 0x7FFF), ib)
    return np.abs(ia - ib)


def check_close(got: np.ndarray, ref: np.ndarray, what: str = "",
                abs_bar: bool = True) -> Dict[str, float]:
    """|got - ref| <= ATOL + RTOL |ref| element by element; with ``abs_bar``
    (every workload whose values are N(0, 0.5)) also |got - ref| <= ATOL for
    every element: the stated max-abs bound on its own.  Workloads with +-30
    outliers keep the combined bound only: there outputs reach tens, where
    one F16 step of the inputs is already 2^-6.  Returns error stats, with
    ``abs_ratio`` = max_abs / ATOL and ``max_ratio`` = max of err / bound."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    tol = ATOL + RTOL * np.abs(ref.astype(np.float64))
    bad = err > tol
    stats = {"max_abs": float(err.max()) if err.size else 0.0,
             "max_rel": float((err / np.maximum(np.abs(ref), 1e-30)).max()) if err.size else 0.0,
             "max_ratio": float((err / tol).max()) if err.size else 0.0}
    stats["abs_ratio"] = stats["max_abs"] / ATOL
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; first at "
            f"{tuple(idx)} got {got[tuple(idx)]} ref {ref[tuple(idx)]}; stats {stats}")
    if abs_bar and stats["max_abs"] > ATOL:
        idx = np.unravel_index(int(np.argmax(err)), err.shape)
        raise AssertionError(f"{what}: max abs error {stats['max_abs']:.3g} > {ATOL} at {idx} "
                             f"(got {got[idx]} ref {ref[idx]}); stats {stats}")
    return stats


# Rows projected from features: one F16 ulp of the reference plus this much
# absolute.  The device's fp32 sum of d_model = 2048 products carries an error
# of about sqrt(d_model) 2^-24 |w| |f| (a few 1e-6 after the K norm for the
# synthetic weights); 2^-14 leaves a factor of about 20.
PROJ_ATOL = 2.0 ** -14


def f16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of F16 values at |x| (the subnormal spacing near zero)."""
    a = np.abs(x.astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def check_projected(got: np.ndarray, want: np.ndarray, what: str) -> float:
    """|got - want| <= ulp(want) + PROJ_ATOL element by element (F16 arrays)."""
    g = got.astype(np.float64)
    r = want.astype(np.float64)
    assert np.isfinite(g).all(), f"{what}: non-finite"
    err = np.abs(g - r)
    tol = f16_ulp(want) + PROJ_ATOL
    bad = err > tol
    if bad.any():
        idx = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond one ulp + {PROJ_ATOL}; "
                             f"first at {idx}: {g[idx]} vs {r[idx]}")
    return float((err / tol).max()) if err.size else 0.0


class Epochs:
    """Which generation of row content each position has (rewinds start a new one)."""

    def __init__(self):
        self.starts = [0]
        self.ids = [0]
        self.next_id = 1

    def rewind(self, committed: int) -> None:
        k = bisect.bisect_left(self.starts, committed)
        self.starts, self.ids = self.starts[:k], self.ids[:k]
        if not self.starts or self.starts[-1] != committed:
            self.starts.append(committed)
            self.ids.append(self.next_id)
        else:
            self.ids[-1] = self.next_id
        self.next_id += 1

    def of(self, positions: np.ndarray) -> np.ndarray:
        k = np.searchsorted(np.asarray(self.starts), positions, side="right") - 1
        return np.asarray(self.ids)[k]


class Driver:
    """One ring (all sequences, all layers) and its oracle twin."""

    def __init__(self, w: W.Workload, n_split: Optional[int] = None, device: str = "cuda:0",
                 row_blocks: Optional[bool] = None, registered_weights: bool = False,
                 merge: Optional[str] = None, mirror_deferred: bool = False):
        """n_split: attention splits forced; row_blocks: False puts both
        32-row query blocks of a KV head in one work-group; merge: "kernel"
        merges the splits inside the attention launch where the library
        supports it, instead of in a launch of its own (the library reads
        these settings when the ring is created); registered_weights: rows from
        features go through the weights registered with ring_set_kv_weights
        instead of the caller's; mirror_deferred: features written with
        ring_mirror_write_deferred (kept alive until the next step)."""
        import torch
        from draft_model_kv_amd import Ring
        self.torch = torch
        self.w = w
        self.dev = torch.device(device)
        env = {}
        if n_split is not None:
            env["RING_ATTN_SPLITS"] = str(n_split)
        if row_blocks is not None:
            env["RING_ATTN_ROW_BLOCKS"] = "1" if row_blocks else "0"
        if merge is not None:
            env["RING_ATTN_MERGE"] = merge
        saved = {k: os.environ.get(k) for k in env}
        os.environ.update(env)
        try:
            self.ring = Ring(cap=w.cap, q_len=w.q_len, n_head=w.n_head, n_head_kv=w.n_head_kv,
                             head_dim=w.head_dim, n_layer=w.n_layer, n_seq=w.n_seq,
                             rope_base=w.rope_base, device=self.dev,
                             swa_window=w.swa_window, swa_layers=w.swa_layers,
                             d_model=w.d_model)
        finally:
            for k, v in saved.items():
                if v is None:
                    del os.environ[k]
                else:
                    os.environ[k] = v
        self.geo = ro.geometry(w.cap, w.q_len, w.head_dim, w.n_head_kv)
        self.orc = [ro.RingStep(self.geo, w.n_layer, w.n_head_kv, w.head_dim, w.rope_base)
                    for _ in range(w.n_seq)]
        self.epochs = [Epochs() for _ in range(w.n_seq)]
        self.committed = [0] * w.n_seq
        self.n_attn = 0
        # the max-abs bound on its own for N(0, 0.5) values (not for +-30 outliers)
        self.abs_bar = w.outlier_p == 0.0
        # rows from fused features: the mirror on both sides, and the weights
        self.mirror = w.d_model > 0
        if self.mirror:
            self.eps = ro.RMS_EPS
            self.wk, self.wv, self.kn = W.projection_weights(w)
            self.wk_t = torch.from_numpy(self.wk).to(self.dev)
            self.wv_t = torch.from_numpy(self.wv).to(self.dev)
            self.kn_t = torch.from_numpy(self.kn).to(self.dev)
            self.orc_mirror = [ro.FeatureMirror(w.cap, w.d_model) for _ in range(w.n_seq)]
            self.registered = registered_weights
            self.mirror_deferred = mirror_deferred
            self._keep_feat = []
            if registered_weights:
                self.ring.set_kv_weights(self.wk_t, self.wv_t, self.kn_t, self.eps)
            # (position, epoch) in each mirror slot, as written to both mirrors
            self.mirror_held = [dict() for _ in range(w.n_seq)]

    # ------------------------------------------------------------------ steps
    def rows(self, seq: int, positions: np.ndarray):
        """Raw K and V rows [n_layer, n, kv_row] for positions (their epochs)."""
        w = self.w
        n = len(positions)
        k = np.empty((w.n_layer, n, w.kv_row), np.float16)
        v = np.empty((w.n_layer, n, w.kv_row), np.float16)
        if n == 0:
            return k, v
        ep = self.epochs[seq].of(positions)
        for e in np.unique(ep):
            sel = ep == e
            for layer in range(w.n_layer):
                k[layer, sel] = W.context_rows(w, seq, layer, T_K, positions[sel], int(e))
                v[layer, sel] = W.context_rows(w, seq, layer, T_V, positions[sel], int(e))
        return k, v

    def write_features(self, seq: int, positions: np.ndarray) -> int:
        """Write to both mirrors the features of the positions not held there
        in their current epoch, in contiguous runs; returns rows written."""
        w = self.w
        ep = self.epochs[seq].of(positions) if len(positions) else positions
        held = self.mirror_held[seq]
        need = [int(p) for p, e in zip(positions, ep) if held.get(int(p) % w.cap) != (int(p), int(e))]
        runs, written = [], 0
        for p in need:
            if runs and runs[-1][1] == p:
                runs[-1][1] = p + 1
            else:
                runs.append([p, p + 1])
        for a, b in runs:
            pos = np.arange(a, b, dtype=np.int64)
            pe = self.epochs[seq].of(pos)
            f = np.empty((len(pos), w.d_model), np.float16)
            for e in np.unique(pe):
                sel = pe == e
                f[sel] = W.fused_features(w, seq, pos[sel], int(e))
            ft = self.torch.from_numpy(f).to(self.dev)
            self.ring.mirror_write(seq, a, ft, deferred=self.mirror_deferred)
            if self.mirror_deferred:
                self._keep_feat.append(ft)
            self.orc_mirror[seq].write(pos, f)
            for p, e in zip(pos, pe):
                held[int(p) % w.cap] = (int(p), int(e))
            written += len(pos)
        return written

    def _plan(self, seq: int, committed: int):
        """The step's plan on both sides (they must agree exactly)."""
        if committed < self.committed[seq]:
            self.epochs[seq].rewind(committed)
        lib_plan, lib_ap = self.ring.plan(seq, committed)
        op = self.orc[seq].plan(committed)
        got = (lib_plan.win, lib_plan.lo, lib_plan.start, lib_plan.n_new, bool(lib_plan.bulk))
        want = (op.win, op.lo, op.start, op.n_new, op.bulk)
        assert got == want, f"plan mismatch seq {seq} committed {committed}: {got} != {want}"
        if op.bulk:
            assert lib_plan.n_chunks == len(op.chunks)
        else:
            assert list(lib_ap[: self.geo.a_step]) == op.ap_rows
        return op

    def step_batch(self, items):
        """ring_begin_step_batch over (seq, committed) pairs of distinct
        sequences; the oracle commits each sequence's step."""
        torch = self.torch
        steps, keep, commits = [], {}, []
        for seq, committed in items:
            op = self._plan(seq, committed)
            k, v = self.rows(seq, np.arange(op.start, committed, dtype=np.int64))
            if op.n_new:
                kt = torch.from_numpy(k).to(self.dev)
                vt = torch.from_numpy(v).to(self.dev)
                keep[seq] = (kt, vt)
                steps.append((seq, committed, kt, vt))
            else:
                steps.append((seq, committed, None, None))
            commits.append((seq, committed, op, k, v))
        self.ring.begin_step_batch(steps)
        torch.cuda.synchronize(self.dev)
        for seq, committed, op, k, v in commits:
            self.orc[seq].commit(op, list(k), list(v))
            self.committed[seq] = committed
        return [c[2] for c in commits]

    def step(self, seq: int, committed: int, deferred: bool = False):
        """begin_step on both sides; the plans must agree exactly.  deferred:
        ring_begin_step_deferred (the rows are appended by the attention
        launches; their tensors are kept alive until the next step)."""
        torch = self.torch
        if committed < self.committed[seq]:
            self.epochs[seq].rewind(committed)
        lib_plan, lib_ap = self.ring.plan(seq, committed)
        op = self.orc[seq].plan(committed)
        got = (lib_plan.win, lib_plan.lo, lib_plan.start, lib_plan.n_new, bool(lib_plan.bulk))
        want = (op.win, op.lo, op.start, op.n_new, op.bulk)
        assert got == want, f"plan mismatch seq {seq} committed {committed}: {got} != {want}"
        if op.bulk:
            assert lib_plan.n_chunks == len(op.chunks)
        else:
            assert list(lib_ap[: self.geo.a_step]) == op.ap_rows
        pos = np.arange(op.start, committed, dtype=np.int64)
        if self.mirror:
            self.write_features(seq, pos)
            if self.registered:
                self.ring.begin_step_mirror(seq, committed)
            else:
                self.ring.begin_step_mirror(seq, committed, self.wk_t, self.wv_t, self.kn_t,
                                            self.eps)
            self.orc[seq].commit_features(op, self.orc_mirror[seq], list(self.wk), list(self.wv),
                                          list(self.kn), self.eps)
            if self.mirror_deferred:
                # the deferred rows are in the mirror once the stream has passed the step
                self.torch.cuda.synchronize(self.dev)
                self._keep_feat = []
            self.committed[seq] = committed
            return op
        k, v = self.rows(seq, pos)
        if len(pos):
            kt = torch.from_numpy(k).to(self.dev)
            vt = torch.from_numpy(v).to(self.dev)
            self.ring.begin_step(seq, committed, kt, vt, deferred=deferred)
            self._keep = getattr(self, "_keep", {})
            self._keep[seq] = (kt, vt)
        else:
            self.ring.begin_step(seq, committed, None, None, deferred=deferred)
        self.orc[seq].commit(op, list(k), list(v))
        self.committed[seq] = committed
        return op

    def noise(self, layer: int, step: int):
        w = self.w
        qs, ks, vs = [], [], []
        for seq in range(w.n_seq):
            q, kn, vn = W.noise_inputs(w, seq, layer, step)
            qs.append(q); ks.append(kn); vs.append(vn)
        return np.stack(qs), np.stack(ks), np.stack(vs)

    def attn(self, layer: int, step: int):
        """ring_attn on the device; returns (out, q, k_noise, v_noise) as numpy."""
        torch = self.torch
        q, kn, vn = self.noise(layer, step)
        out = self.ring.attn(layer, torch.from_numpy(q).to(self.dev),
                             torch.from_numpy(kn).to(self.dev),
                             torch.from_numpy(vn).to(self.dev))
        torch.cuda.synchronize(self.dev)
        self.n_attn += 1
        return out.cpu().numpy(), q, kn, vn

    def is_swa(self, layer: int) -> bool:
        return bool((self.w.swa_layers >> layer) & 1)

    def oracle_attn(self, seq: int, layer: int, q, kn, vn, dtype=np.float32):
        w = self.w
        return ro.attend(self.orc[seq].caches[layer], self.committed[seq], w.cap,
                         q[seq], kn[seq], vn[seq], w.n_head, dtype=dtype,
                         swa_window=w.swa_window if self.is_swa(layer) else None)

    # ------------------------------------------------------------ comparisons
    def check_index(self, seq: int):
        """slot_pos and mask bit-exact against the oracle."""
        sp = self.ring.slot_pos(seq)
        want_sp = self.orc[seq].slots.slot_pos
        if not np.array_equal(sp, want_sp):
            bad = np.flatnonzero(sp != want_sp)
            raise AssertionError(f"slot_pos mismatch seq {seq} at slots {bad[:8]}: "
                                 f"{sp[bad[:8]]} != {want_sp[bad[:8]]}")
        m = self.ring.mask(seq)
        want_m = self.orc[seq].mask().view(np.uint16)
        if not np.array_equal(m, want_m):
            bad = np.argwhere(m != want_m)
            raise AssertionError(f"mask mismatch seq {seq} at {bad[:4].tolist()}")
        if self.w.swa_window:
            m = self.ring.mask_swa(seq)
            want_m = self.orc[seq].mask_swa(self.w.swa_window).view(np.uint16)
            if not np.array_equal(m, want_m):
                bad = np.argwhere(m != want_m)
                raise AssertionError(f"sliding-window mask mismatch seq {seq} at {bad[:4].tolist()}")

    def check_rows(self, seq: int, layer: int, max_ulp: int = 1) -> int:
        """Ring rows against the full cache; returns the count of 1-ulp K rows.

        Rows supplied directly: K within one F16 ulp of the oracle's rounding,
        V exact.  Rows projected from features: the device sums the d_model
        exact F16 products in fp32 where the oracle works in fp64, so K (after
        the norm) and V may differ from the oracle's once-rounded value by one
        F16 ulp plus PROJ_ATOL absolute (near zero a F16 ulp is far smaller
        than the fp32 summation error)."""
        g = self.geo
        k, v = self.ring.rows(seq, layer, 0, g.kv_total)
        sp = self.orc[seq].slots.slot_pos
        cache = self.orc[seq].caches[layer]
        filled = np.flatnonzero(sp >= 0)
        empty = np.flatnonzero(sp < 0)
        n_ulp = 0
        if len(filled):
            # rows of positions still held (stale ones after a rewind included)
            want_k = np.empty((len(filled), g.kv_row), np.float16)
            want_v = np.empty((len(filled), g.kv_row), np.float16)
            for j, s in enumerate(filled):
                want_k[j], want_v[j] = cache.row(int(sp[s]))
            if self.mirror:
                for name, got, want in (("K", k[filled], want_k), ("V", v[filled], want_v)):
                    check_projected(got, want, f"{name} rows seq {seq} layer {layer}")
                n_ulp = int((f16_ulp_diff(k[filled], want_k) > 0).sum())
            else:
                d = f16_ulp_diff(k[filled], want_k)
                assert d.max() <= max_ulp, f"K rows differ by {d.max()} ulp (seq {seq} layer {layer})"
                n_ulp = int((d > 0).sum())
                assert np.array_equal(v[filled].view(np.uint16), want_v.view(np.uint16)), \
                    f"V rows differ (seq {seq} layer {layer})"
        assert not k[empty].view(np.uint16).any() and not v[empty].view(np.uint16).any(), \
            "empty ring slots must stay zero"
        tr = g.trash_slot
        assert np.isfinite(k[tr:].astype(np.float32)).all() and np.isfinite(v[tr:].astype(np.float32)).all()
        assert not k[tr].view(np.uint16).any() and not v[tr].view(np.uint16).any(), \
            "trash slot must hold zeros"
        return n_ulp

    def check_noise_rows(self, seq: int, layer: int, kn: np.ndarray, vn: np.ndarray):
        g, w = self.geo, self.w
        k, v = self.ring.rows(seq, layer, g.cap, w.q_len)
        pq = ro.noise_positions(self.committed[seq], w.q_len)
        want = ro.rope_rows_f16(kn[seq], pq, w.n_head_kv, w.head_dim, w.rope_base)
        assert f16_ulp_diff(k, want).max() <= 1
        assert np.array_equal(v.view(np.uint16), vn[seq].view(np.uint16))

    def check_attn_layers(self, step: int, seqs=None) -> Dict[str, float]:
        """Attention of every layer first (so that a deferred step is carried
        out by the attention launches themselves), then every comparison."""
        res = [(layer,) + self.attn(layer, step) for layer in range(self.w.n_layer)]
        worst = {"max_abs": 0.0, "max_rel": 0.0, "max_ratio": 0.0, "abs_ratio": 0.0}
        for layer, out, q, kn, vn in res:
            for seq in (range(self.w.n_seq) if seqs is None else seqs):
                ref = self.oracle_attn(seq, layer, q, kn, vn)
                st = check_close(out[seq], ref, f"attn seq {seq} layer {layer} step {step}",
                                 abs_bar=self.abs_bar)
                self.check_noise_rows(seq, layer, kn, vn)
                for k_ in worst:
                    worst[k_] = max(worst[k_], st[k_])
        return worst

    def check_attn(self, layer: int, step: int, seqs=None, noise_rows: bool = True) -> Dict[str, float]:
        out, q, kn, vn = self.attn(layer, step)
        worst = {"max_abs": 0.0, "max_rel": 0.0, "max_ratio": 0.0, "abs_ratio": 0.0}
        for seq in (range(self.w.n_seq) if seqs is None else seqs):
            ref = self.oracle_attn(seq, layer, q, kn, vn)
            st = check_close(out[seq], ref, f"attn seq {seq} layer {layer} step {step}",
                             abs_bar=self.abs_bar)
            if noise_rows:
                self.check_noise_rows(seq, layer, kn, vn)
            for k_ in worst:
                worst[k_] = max(worst[k_], st[k_])
        return worst

    def close(self):
        self.ring.close()


# ---------------------------------------------------------------------------
# Whole workloads at full size: every step runs on the device, checkpoints are
# compared element by element.
# ---------------------------------------------------------------------------
def checkpoints(n: int, every: int, extra=()) -> set:
    """Steps 0, 1, every `every`-th, the last one and `extra` (of range(n))."""
    pts = set(range(0, n, every)) | {0, 1, n - 1} | set(extra)
    return {p for p in pts if 0 <= p < n}


def run_workload(name: str, every: int, rows_at=(0,), deferred: bool = False,
                 max_steps: Optional[int] = None, say=print) -> float:
    """The named workload through its warm-up and decode steps.

    Checkpoints: every `every`-th step, the first two, the last, and each step
    where a sequence's committed count crosses cap.  At a checkpoint, every
    layer's attention output (and layer 0's noise rows) against the oracle,
    and the index state bit-exact; ring rows of layer 0 at the steps in
    `rows_at` (and of every layer at the last step).  deferred: every decode
    step through ring_begin_step_deferred, so each layer's attention launch
    appends that layer's rows (a checkpoint then runs all layers before any
    comparison, and a step between checkpoints runs them without one).
    Returns the worst err / bound ratio seen."""
    w = W.WORKLOADS[name]
    d = Driver(w)
    streams = [W.commit_stream(w, s) for s in range(w.n_seq)]
    n_warm = W.n_warmup_steps(w)
    say(name, "warm-up", n_warm, "steps", "deferred" if deferred else "eager")
    for t in range(n_warm):
        for seq in range(w.n_seq):
            d.step(seq, streams[seq][t])
    for seq in range(w.n_seq):
        d.check_index(seq)
        for layer in range(w.n_layer):
            d.check_rows(seq, layer)
    n = len(streams[0]) - n_warm if max_steps is None else min(max_steps, len(streams[0]) - n_warm)
    crossings = [t for t in range(n) for seq in range(w.n_seq)
                 if streams[seq][n_warm + t - 1] < w.cap <= streams[seq][n_warm + t]]
    pts = checkpoints(n, every, crossings)
    worst = {"max_ratio": 0.0, "abs_ratio": 0.0}
    for t in range(n):
        for seq in range(w.n_seq):
            d.step(seq, streams[seq][n_warm + t], deferred=deferred)
        if t in pts:
            if deferred:
                st = d.check_attn_layers(t)
            else:
                st = {"max_ratio": 0.0, "abs_ratio": 0.0}
                for layer in range(w.n_layer):
                    s_ = d.check_attn(layer, t, noise_rows=(layer == 0))
                    st = {k: max(st[k], s_[k]) for k in st}
            worst = {k: max(worst[k], st[k]) for k in worst}
            for seq in range(w.n_seq):
                d.check_index(seq)
        else:
            for layer in range(w.n_layer):
                d.attn(layer, t)
        if t in rows_at or t == n - 1:
            for seq in range(min(w.n_seq, 2)):
                for layer in (range(w.n_layer) if t == n - 1 else (0,)):
                    d.check_rows(seq, layer)
    say(name, "steps", n, "checked", len(pts), "worst err/bound", round(worst["max_ratio"], 4),
        "worst abs err/2e-3", round(worst["abs_ratio"], 4))
    d.close()
    return worst["max_ratio"]

