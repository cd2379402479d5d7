"""The five synthetic workloads of the draft-KV ring and their seeded inputs.

Shapes follow the ring geometry of the DFlash2 draft-KV notes (page
"DFLASH2_RING_PORT.md", section 1.1: q_len = 8 noise rows, K/V rows of
head_dim * n_head_kv = 128 * 8 F16 values).  The step stream draws the number
of accepted draft tokens per verification from the share table of the
llama.cpp pull request "speculative : capped recurrent planes for DFlash"
(section "Why the layout matters", 1422 verifications at n-max 7).

All values are generated on the host by ``workload.rng`` and rounded to F16
with round-to-nearest-even.  Nothing here implements the ring method itself:
these are inputs only.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np

from . import rng

# Accepted draft tokens 0..7 and their measured shares in percent (they sum
# to 99.9; the sampler normalises by the sum).
ACCEPT_SHARES = (24.5, 19.5, 15.0, 9.9, 7.7, 5.0, 3.6, 14.7)

# Tensor tags used in the value keys.
T_K, T_V, T_Q, T_KN, T_VN = 1, 2, 3, 4, 5
T_ACC, T_START, T_OUTLIER = 10, 11, 12
T_FEAT, T_WK, T_WV, T_KNORM = 20, 21, 22, 23


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    cap: int
    q_len: int = 8
    n_head: int = 32
    n_head_kv: int = 8
    head_dim: int = 128
    n_layer: int = 1
    n_seq: int = 1
    rope_base: float = 1.0e6
    sigma: float = 0.5
    outlier_p: float = 0.0
    outlier_mag: float = 30.0
    prefill: int = 0            # committed after the warm-up
    prefill_step: int = 0       # 0: one begin_step; else warm-up in steps of this size
    n_steps: int = 0
    full_accept_every: int = 0  # every k-th decode step (k-1, 2k-1, ...) commits q_len
    start_lo: int = 0           # per-seq start drawn from [start_lo, start_hi) when > 0
    start_hi: int = 0
    forced_starts: Tuple[Tuple[int, int, int], ...] = field(default_factory=tuple)
    swa_window: int = 0         # sliding-window layers' window (0: none)
    swa_layers: int = 0         # bit l set: layer l is a sliding-window layer
    d_model: int = 0            # fused feature width (0: rows supplied directly)

    @property
    def kv_row(self) -> int:
        return self.head_dim * self.n_head_kv

    @property
    def group(self) -> int:
        return self.n_head // self.n_head_kv


WORKLOADS: Dict[str, Workload] = {
    "tiny_ring": Workload(
        name="tiny_ring", seed=0, cap=64, prefill=40, n_steps=30),
    "decode_stream": Workload(
        name="decode_stream", seed=1, cap=4096, prefill=4096, n_steps=2000),
    "long_prompt_wrap": Workload(
        name="long_prompt_wrap", seed=2, cap=4096, n_layer=5, prefill=32768,
        prefill_step=1024, n_steps=512, full_accept_every=4),
    "batched_seqs": Workload(
        name="batched_seqs", seed=3, cap=4096, n_seq=16, n_steps=256,
        start_lo=100, start_hi=131072,
        forced_starts=((0, 100, 1000), (1, 4096 - 800, 4096 - 100))),
    "large_window": Workload(
        name="large_window", seed=4, cap=32768, n_head=64, sigma=1.0,
        outlier_p=0.01, prefill=131072, n_steps=256),
    # interleaved full / sliding-window draft layers (layers 1 and 3 slide
    # over the last 1024 positions); the window wraps the ring end
    "swa_stream": Workload(
        name="swa_stream", seed=5, cap=4096, n_layer=4, prefill=4096, n_steps=600,
        swa_window=1024, swa_layers=0b1010),
    # new rows computed from a feature mirror through synthetic projection
    # weights; d_model = 2048 is the hidden size of the DFlash draft that the
    # ring notes convert (6 dense layers, hidden 2048); 5 layers as in the
    # Luce log line of the same notes
    "mirror_stream": Workload(
        name="mirror_stream", seed=6, cap=4096, n_layer=5, prefill=4096, n_steps=600,
        d_model=2048),
}


def _values(w: Workload, keys: np.ndarray, n: int) -> np.ndarray:
    """Seeded N(0, sigma) values (plus optional +-mag outliers), rounded to F16."""
    x = rng.normal(keys, n) * w.sigma
    if w.outlier_p > 0.0:
        okeys = np.asarray(keys, dtype=np.uint64) ^ np.uint64(0x5851F42D4C957F2D)
        u = rng.uniform(okeys, 2 * n)
        hit = u[:, :n] < w.outlier_p
        sign = np.where(u[:, n:] < 0.5, -1.0, 1.0)
        x = np.where(hit, sign * w.outlier_mag, x)
    return x.astype(np.float16)


def context_rows(w: Workload, seq: int, layer: int, tensor: int,
                 positions, epoch: int = 0) -> np.ndarray:
    """Raw (pre-RoPE for K) context rows ``[len(positions), kv_row]`` F16.

    Row content depends only on (seed, seq, layer, tensor, epoch, position),
    so a position appended twice within one epoch gets the same row.
    """
    positions = np.asarray(positions, dtype=np.int64).reshape(-1)
    base = rng.key_of(w.seed, seq, layer, tensor, epoch)
    keys = rng.row_keys(base, positions)
    return _values(w, keys, w.kv_row)


def noise_inputs(w: Workload, seq: int, layer: int, step: int):
    """Noise-block inputs for one (seq, layer, step).

    Returns ``q [q_len, n_head, head_dim]``, ``k_noise [q_len, kv_row]`` (pre
    RoPE) and ``v_noise [q_len, kv_row]``, all F16.
    """
    rows = np.arange(w.q_len, dtype=np.int64)
    q = _values(w, rng.row_keys(rng.key_of(w.seed, seq, layer, T_Q, step), rows),
                w.n_head * w.head_dim).reshape(w.q_len, w.n_head, w.head_dim)
    kn = _values(w, rng.row_keys(rng.key_of(w.seed, seq, layer, T_KN, step), rows), w.kv_row)
    vn = _values(w, rng.row_keys(rng.key_of(w.seed, seq, layer, T_VN, step), rows), w.kv_row)
    return q, kn, vn


def accepted_counts(w: Workload, seq: int, n: int) -> np.ndarray:
    """Accepted draft tokens per step, by inverse CDF of ACCEPT_SHARES."""
    shares = np.asarray(ACCEPT_SHARES, dtype=np.float64)
    cdf = np.cumsum(shares) / shares.sum()
    u = rng.uniform(np.array([rng.key_of(w.seed, seq, T_ACC)], dtype=np.uint64), n)[0]
    return np.minimum(np.searchsorted(cdf, u, side="right"), len(shares) - 1).astype(np.int64)


def start_positions(w: Workload) -> List[int]:
    """Committed count of each sequence after its warm-up."""
    if w.start_hi <= 0:
        return [w.prefill] * w.n_seq
    u = rng.uniform(np.array([rng.key_of(w.seed, T_START)], dtype=np.uint64),
                    4 * w.n_seq)[0]
    forced = {s: (lo, hi) for s, lo, hi in w.forced_starts}
    out: List[int] = []
    j = 0
    for s in range(w.n_seq):
        lo, hi = forced.get(s, (w.start_lo, w.start_hi))
        while True:
            c = lo + int(u[j % len(u)] * (hi - lo))
            j += 1
            if c not in out:
                break
        out.append(c)
    return out


def commit_stream(w: Workload, seq: int) -> List[int]:
    """Committed count at every begin_step of one sequence, warm-up included."""
    start = start_positions(w)[seq]
    stream: List[int] = []
    if w.prefill_step > 0:
        c = 0
        while c < start:
            c = min(start, c + w.prefill_step)
            stream.append(c)
    else:
        stream.append(start)
    acc = accepted_counts(w, seq, w.n_steps)
    c = stream[-1]
    for t in range(w.n_steps):
        if w.full_accept_every and t % w.full_accept_every == w.full_accept_every - 1:
            c += w.q_len
        else:
            c += 1 + int(acc[t])
        stream.append(c)
    return stream


def n_warmup_steps(w: Workload) -> int:
    """Number of warm-up begin_steps at the head of ``commit_stream``."""
    if w.prefill_step > 0:
        return -(-start_positions(w)[0] // w.prefill_step)
    return 1


def fused_features(w: Workload, seq: int, positions, epoch: int = 0) -> np.ndarray:
    """Fused feature vectors ``[len(positions), d_model]`` F16, N(0, 1).

    Like the context rows, a position's features depend only on (seed, seq,
    epoch, position).
    """
    positions = np.asarray(positions, dtype=np.int64).reshape(-1)
    keys = rng.row_keys(rng.key_of(w.seed, seq, T_FEAT, epoch), positions)
    return (rng.normal(keys, w.d_model)).astype(np.float16)


def projection_weights(w: Workload):
    """Synthetic projection weights of every layer.

    ``wk``, ``wv``: F16 ``[n_layer, kv_row, d_model]`` drawn N(0, sigma^2 / d_model)
    so that V = wv f has the workload's sigma for N(0, 1) features;
    ``k_norm``: F32 ``[n_layer, head_dim]`` drawn 1 + 0.1 N(0, 1).
    """
    rows = np.arange(w.kv_row, dtype=np.int64)
    scale = w.sigma / np.sqrt(w.d_model)
    wk = np.empty((w.n_layer, w.kv_row, w.d_model), np.float16)
    wv = np.empty((w.n_layer, w.kv_row, w.d_model), np.float16)
    kn = np.empty((w.n_layer, w.head_dim), np.float32)
    for layer in range(w.n_layer):
        wk[layer] = (rng.normal(rng.row_keys(rng.key_of(w.seed, layer, T_WK), rows), w.d_model)
                     * scale).astype(np.float16)
        wv[layer] = (rng.normal(rng.row_keys(rng.key_of(w.seed, layer, T_WV), rows), w.d_model)
                     * scale).astype(np.float16)
        kn[layer] = (1.0 + 0.1 * rng.normal(np.array([rng.key_of(w.seed, layer, T_KNORM)],
                                                     dtype=np.uint64), w.head_dim)[0])
    return wk, wv, kn
