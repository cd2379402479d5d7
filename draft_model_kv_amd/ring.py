"""ctypes binding of libringkv.so (C ABI in include/ring_kv.h).

The functions keep the C names and do argument marshalling only: every step
of the ring path runs in the library's HIP kernels.  Device buffers are
passed as integer addresses; ``Ring`` wraps them with torch tensors, which
provide device memory and streams and nothing else.

Importing this module fails with ImportError when the library has not been
built (``python -m draft_model_kv_amd.build``); there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

# RINGKV_LIB=stamps loads the profiling build with per-wave timestamps
# (ring_profile_stamps) instead of the product library.
LIB_NAME = "libringkv_stamps.so" if os.environ.get("RINGKV_LIB") == "stamps" else "libringkv.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

RING_OK = 0
RING_EINVAL = -1
RING_ERANGE = -2
RING_ENOMEM = -3
RING_EDEVICE = -4
RING_ESTATE = -5
RING_MAX_SEQ = 64

# Every function the header declares, in header order.
EXPORTS = (
    "ring_query_geometry", "ring_init", "ring_plan_step", "ring_plan_from_state",
    "ring_begin_step", "ring_begin_step_deferred", "ring_begin_step_batch", "ring_mirror_write", "ring_mirror_write_deferred", "ring_set_kv_weights", "ring_begin_step_mirror", "ring_attn", "ring_attn_noalloc",
    "ring_free",
    "ring_last_error", "ring_describe",
    "ring_read_slot_pos", "ring_read_mask", "ring_read_mask_swa", "ring_read_rows",
    "ring_read_state",
    "ring_profile_enable", "ring_profile_read", "ring_profile_floor",
    "ring_profile_floor_timeouts", "ring_profile_stamps",
)
RING_KERNEL_STEP, RING_KERNEL_ATTN, RING_KERNEL_MERGE, RING_KERNEL_PROJ = 0, 1, 2, 3
RING_KERNEL_FLOOR = 4
# kinds of ring_profile_floor
(RING_FLOOR_EMPTY, RING_FLOOR_READ, RING_FLOOR_PARTIALS, RING_FLOOR_LAST_ARRIVER,
 RING_FLOOR_BARRIER, RING_FLOOR_TWO_LAUNCH, RING_FLOOR_HOLD, RING_FLOOR_MATRIX_MATH,
 RING_FLOOR_VECTOR_MATH, RING_FLOOR_PROJ_READ, RING_FLOOR_READ_LOCKSTEP,
 RING_FLOOR_SHARED_TILES) = (0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11)
# regions of ring_profile_stamps and the layout of a wave's record
RING_STAMPS_ATTN, RING_STAMPS_MERGE, RING_STAMPS_PROJ = 0, 1, 2
RING_STAMP_WAVES, RING_STAMP_WORDS = 8192, 10


class RingConfig(ctypes.Structure):
    _fields_ = [("cap", ctypes.c_int32), ("q_len", ctypes.c_int32),
                ("n_head", ctypes.c_int32), ("n_head_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_layer", ctypes.c_int32),
                ("n_seq", ctypes.c_int32), ("rope_base", ctypes.c_float),
                ("swa_window", ctypes.c_int32), ("swa_layers", ctypes.c_uint64),
                ("d_model", ctypes.c_int32)]


class RingKvWeights(ctypes.Structure):
    _fields_ = [("wk", ctypes.c_void_p), ("wv", ctypes.c_void_p), ("k_norm", ctypes.c_void_p),
                ("eps", ctypes.c_float)]


class RingGeometry(ctypes.Structure):
    _fields_ = [("a_step", ctypes.c_int32), ("trash_slot", ctypes.c_int32),
                ("kv_total", ctypes.c_int32), ("kv_row", ctypes.c_int32),
                ("kv_bytes_per_layer", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64)]


class RingPlan(ctypes.Structure):
    _fields_ = [("committed", ctypes.c_int64), ("win", ctypes.c_int64),
                ("lo", ctypes.c_int64), ("start", ctypes.c_int64),
                ("n_new", ctypes.c_int64), ("bulk", ctypes.c_int32),
                ("n_chunks", ctypes.c_int32)]


class RingError(RuntimeError):
    def __init__(self, code: int, fn: str, msg: str):
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python draft_model_kv_amd/build.py); there is no CPU fallback")
    # torch's HIP libraries load their own bundled libamdhip64.so by file name.
    # Loading torch first makes that runtime satisfy this library's
    # libamdhip64.so.7 dependency, so the process has one HIP runtime (two
    # runtimes in one process do not share the device or its memory).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "ring_query_geometry": [ctypes.POINTER(RingConfig), ctypes.POINTER(RingGeometry)],
        "ring_init": [ctypes.POINTER(RingConfig), P, SZ, P, ctypes.POINTER(P)],
        "ring_plan_step": [P, I32, I64, ctypes.POINTER(RingPlan), P],
        "ring_plan_from_state": [ctypes.POINTER(RingConfig), I64, I64, I64,
                                 ctypes.POINTER(RingPlan), P],
        "ring_begin_step": [P, I32, I64, P, P, I64, P],
        "ring_begin_step_deferred": [P, I32, I64, P, P, I64, P],
        "ring_begin_step_batch": [P, I32, P, P, P, P, P, P],
        "ring_mirror_write": [P, I32, I64, I64, P, P],
        "ring_mirror_write_deferred": [P, I32, I64, I64, P, P],
        "ring_set_kv_weights": [P, ctypes.POINTER(RingKvWeights), P],
        "ring_begin_step_mirror": [P, I32, I64, ctypes.POINTER(RingKvWeights), P],
        "ring_attn": [P, I32, P, P, P, P, P],
        "ring_attn_noalloc": [P, I32, P, P, P, P, P],
        "ring_free": [P],
        "ring_last_error": [],
        "ring_describe": [P, ctypes.c_char_p, SZ],
        "ring_read_slot_pos": [P, I32, P],
        "ring_read_mask": [P, I32, P],
        "ring_read_mask_swa": [P, I32, P],
        "ring_read_rows": [P, I32, I32, I32, I32, P, P],
        "ring_read_state": [P, I32, ctypes.POINTER(I64), ctypes.POINTER(I64)],
        "ring_profile_enable": [P, I32],
        "ring_profile_read": [P, I32, ctypes.POINTER(I32), ctypes.POINTER(ctypes.c_double)],
        "ring_profile_floor": [P, I32, I32, P],
        "ring_profile_floor_timeouts": [P, ctypes.POINTER(ctypes.c_uint32)],
        "ring_profile_stamps": [P, I32, P, I32, I32, ctypes.POINTER(I32)],
    }
    for name in EXPORTS:
        fn = getattr(lib, name)
        fn.argtypes = sig[name]
        fn.restype = ctypes.c_char_p if name == "ring_last_error" else ctypes.c_int
    return lib


_lib = _load()


def _check(code: int, fn: str) -> None:
    if code != RING_OK:
        raise RingError(code, fn, _lib.ring_last_error().decode())


def ring_last_error() -> str:
    return _lib.ring_last_error().decode()


def make_config(cap, q_len=8, n_head=32, n_head_kv=8, head_dim=128, n_layer=1,
                n_seq=1, rope_base=1.0e6, swa_window=0, swa_layers=0, d_model=0) -> RingConfig:
    return RingConfig(cap, q_len, n_head, n_head_kv, head_dim, n_layer, n_seq, rope_base,
                      swa_window, swa_layers, d_model)


def ring_query_geometry(cfg: RingConfig) -> RingGeometry:
    g = RingGeometry()
    _check(_lib.ring_query_geometry(ctypes.byref(cfg), ctypes.byref(g)), "ring_query_geometry")
    return g


def ring_init(cfg: RingConfig, workspace: int = 0, workspace_bytes: int = 0,
              stream: int = 0) -> int:
    h = ctypes.c_void_p()
    _check(_lib.ring_init(ctypes.byref(cfg), workspace or None, workspace_bytes,
                          stream or None, ctypes.byref(h)), "ring_init")
    return h.value


def _plan_out(plan: RingPlan, ap: np.ndarray):
    return plan, (ap.copy() if not plan.bulk else None)


def ring_plan_step(handle: int, seq: int, committed: int, a_step: int = 64):
    plan = RingPlan()
    ap = np.zeros(max(a_step, 66), dtype=np.int32)
    _check(_lib.ring_plan_step(handle, seq, committed, ctypes.byref(plan),
                               ap.ctypes.data), "ring_plan_step")
    return _plan_out(plan, ap)


def ring_plan_from_state(cfg: RingConfig, next_pos: int, held_lo: int, committed: int):
    plan = RingPlan()
    ap = np.zeros(2 * cfg.q_len + 2, dtype=np.int32)
    _check(_lib.ring_plan_from_state(ctypes.byref(cfg), next_pos, held_lo, committed,
                                     ctypes.byref(plan), ap.ctypes.data),
           "ring_plan_from_state")
    return _plan_out(plan, ap)


def ring_begin_step(handle: int, seq: int, committed: int, k_new: int, v_new: int,
                    n_rows: int, stream: int = 0) -> None:
    _check(_lib.ring_begin_step(handle, seq, committed, k_new or None, v_new or None,
                                n_rows, stream or None), "ring_begin_step")


def ring_begin_step_deferred(handle: int, seq: int, committed: int, k_new: int, v_new: int,
                             n_rows: int, stream: int = 0) -> None:
    _check(_lib.ring_begin_step_deferred(handle, seq, committed, k_new or None, v_new or None,
                                         n_rows, stream or None), "ring_begin_step_deferred")


def ring_begin_step_batch(handle: int, seqs, committed, k_new, v_new, n_rows,
                          stream: int = 0) -> None:
    """seqs, committed, k_new, v_new (device addresses), n_rows: sequences of
    equal length n, one entry per sequence."""
    n = len(seqs)
    if not (len(committed) == len(k_new) == len(v_new) == len(n_rows) == n):
        raise ValueError("ring_begin_step_batch: argument lists differ in length")
    a_seq = (ctypes.c_int32 * max(n, 1))(*seqs)
    a_com = (ctypes.c_int64 * max(n, 1))(*committed)
    a_k = (ctypes.c_void_p * max(n, 1))(*[p or None for p in k_new])
    a_v = (ctypes.c_void_p * max(n, 1))(*[p or None for p in v_new])
    a_n = (ctypes.c_int64 * max(n, 1))(*n_rows)
    _check(_lib.ring_begin_step_batch(handle, n, a_seq, a_com, a_k, a_v, a_n, stream or None),
           "ring_begin_step_batch")


def ring_mirror_write_deferred(handle: int, seq: int, pos0: int, n: int, features: int,
                               stream: int = 0) -> None:
    _check(_lib.ring_mirror_write_deferred(handle, seq, pos0, n, features or None, stream or None),
           "ring_mirror_write_deferred")


def ring_mirror_write(handle: int, seq: int, pos0: int, n: int, features: int,
                      stream: int = 0) -> None:
    _check(_lib.ring_mirror_write(handle, seq, pos0, n, features or None, stream or None),
           "ring_mirror_write")


def ring_set_kv_weights(handle: int, wk: int, wv: int, k_norm: int, eps: float,
                        stream: int = 0) -> None:
    w = RingKvWeights(wk or None, wv or None, k_norm or None, eps)
    _check(_lib.ring_set_kv_weights(handle, ctypes.byref(w), stream or None), "ring_set_kv_weights")


def ring_begin_step_mirror(handle: int, seq: int, committed: int, wk: int, wv: int, k_norm: int,
                           eps: float, stream: int = 0) -> None:
    w = RingKvWeights(wk or None, wv or None, k_norm or None, eps)
    _check(_lib.ring_begin_step_mirror(handle, seq, committed, ctypes.byref(w), stream or None),
           "ring_begin_step_mirror")


def ring_begin_step_mirror_registered(handle: int, seq: int, committed: int,
                                      stream: int = 0) -> None:
    """ring_begin_step_mirror with w == NULL: the weights of ring_set_kv_weights."""
    _check(_lib.ring_begin_step_mirror(handle, seq, committed, None, stream or None),
           "ring_begin_step_mirror")


def ring_attn(handle: int, layer: int, q: int, k_noise: int, v_noise: int, out: int,
              stream: int = 0) -> None:
    _check(_lib.ring_attn(handle, layer, q or None, k_noise or None, v_noise or None,
                          out or None, stream or None), "ring_attn")


def ring_attn_noalloc(handle: int, layer: int, q: int, k_noise: int, v_noise: int, out: int,
                      stream: int = 0) -> None:
    _check(_lib.ring_attn_noalloc(handle, layer, q or None, k_noise or None, v_noise or None,
                                  out or None, stream or None), "ring_attn_noalloc")


def ring_free(handle: int) -> None:
    _check(_lib.ring_free(handle), "ring_free")


def ring_describe(handle: int) -> str:
    buf = ctypes.create_string_buffer(256)
    _check(_lib.ring_describe(handle, buf, 256), "ring_describe")
    return buf.value.decode()


def ring_read_slot_pos(handle: int, seq: int, cap: int) -> np.ndarray:
    out = np.empty(cap, dtype=np.int32)
    _check(_lib.ring_read_slot_pos(handle, seq, out.ctypes.data), "ring_read_slot_pos")
    return out


def ring_read_mask(handle: int, seq: int, q_len: int, kv_total: int) -> np.ndarray:
    out = np.empty((q_len, kv_total), dtype=np.uint16)
    _check(_lib.ring_read_mask(handle, seq, out.ctypes.data), "ring_read_mask")
    return out


def ring_read_mask_swa(handle: int, seq: int, q_len: int, kv_total: int) -> np.ndarray:
    out = np.empty((q_len, kv_total), dtype=np.uint16)
    _check(_lib.ring_read_mask_swa(handle, seq, out.ctypes.data), "ring_read_mask_swa")
    return out


def ring_read_rows(handle: int, seq: int, layer: int, slot0: int, n: int,
                   kv_row: int) -> Tuple[np.ndarray, np.ndarray]:
    k = np.empty((n, kv_row), dtype=np.uint16)
    v = np.empty((n, kv_row), dtype=np.uint16)
    _check(_lib.ring_read_rows(handle, seq, layer, slot0, n, k.ctypes.data, v.ctypes.data),
           "ring_read_rows")
    return k.view(np.float16), v.view(np.float16)


def ring_read_state(handle: int, seq: int) -> Tuple[int, int]:
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.ring_read_state(handle, seq, ctypes.byref(a), ctypes.byref(b)),
           "ring_read_state")
    return a.value, b.value


def ring_profile_enable(handle: int, max_launches: int) -> None:
    _check(_lib.ring_profile_enable(handle, max_launches), "ring_profile_enable")


def ring_profile_read(handle: int, kernel: int) -> Tuple[int, float]:
    n, ms = ctypes.c_int32(), ctypes.c_double()
    _check(_lib.ring_profile_read(handle, kernel, ctypes.byref(n), ctypes.byref(ms)),
           "ring_profile_read")
    return n.value, ms.value


def ring_profile_floor(handle: int, layer: int, kind: int, stream: int = 0) -> None:
    _check(_lib.ring_profile_floor(handle, layer, kind, stream or None), "ring_profile_floor")


def ring_profile_floor_timeouts(handle: int) -> int:
    n = ctypes.c_uint32()
    _check(_lib.ring_profile_floor_timeouts(handle, ctypes.byref(n)), "ring_profile_floor_timeouts")
    return n.value


def ring_profile_stamps(handle: int, region: int, max_waves: int, clear: bool = True
                        ) -> Tuple[np.ndarray, int]:
    """Per-wave stamps of `region` (profiling build only): a uint64 array
    [max_waves][RING_STAMP_WORDS] and the clock's rate in kHz."""
    out = np.zeros((max_waves, RING_STAMP_WORDS), dtype=np.uint64)
    khz = ctypes.c_int32()
    _check(_lib.ring_profile_stamps(handle, region, out.ctypes.data if max_waves else None,
                                    max_waves, int(clear), ctypes.byref(khz)),
           "ring_profile_stamps")
    return out, khz.value


class Ring:
    """One ring on the current GPU, its workspace a torch uint8 tensor.

    Tensors passed in must be contiguous CUDA (HIP) tensors of the documented
    dtype and shape; they are handed to the library by address on torch's
    current stream.
    """

    def __init__(self, cap, q_len=8, n_head=32, n_head_kv=8, head_dim=128, n_layer=1,
                 n_seq=1, rope_base=1.0e6, device=None, swa_window=0, swa_layers=0, d_model=0,
                 workspace: str = "torch"):
        """workspace: "torch" (a torch uint8 tensor, the default) or
        "library" (ring_init allocates it, ring_free releases it)."""
        import torch
        self._torch = torch
        self.cfg = make_config(cap, q_len, n_head, n_head_kv, head_dim, n_layer, n_seq, rope_base,
                               swa_window, swa_layers, d_model)
        self.geo = ring_query_geometry(self.cfg)
        self.device = torch.device(device or "cuda")
        if workspace == "library":
            with torch.cuda.device(self.device):
                self.workspace = None
                self.handle = ring_init(self.cfg, 0, 0, self._stream())
        elif workspace == "torch":
            self.workspace = torch.empty(self.geo.workspace_bytes + 256, dtype=torch.uint8,
                                         device=self.device)
            base = self.workspace.data_ptr()
            off = (-base) % 256
            self.handle = ring_init(self.cfg, base + off, self.geo.workspace_bytes, self._stream())
        else:
            raise ValueError(f"workspace {workspace!r}: 'torch' or 'library'")
        self.a_step = self.geo.a_step

    def _stream(self) -> int:
        return self._torch.cuda.current_stream(self.device).cuda_stream

    def _ptr(self, t, dtype, shape, name):
        torch = self._torch
        if t is None:
            return 0
        if t.dtype != dtype or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError(f"{name}: need a contiguous {dtype} CUDA tensor")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
        return t.data_ptr()

    def plan(self, seq: int, committed: int):
        return ring_plan_step(self.handle, seq, committed, self.a_step)

    def begin_step(self, seq: int, committed: int, k_new, v_new, deferred: bool = False) -> None:
        """deferred: the rows are appended by the next attention of each layer
        (k_new / v_new must then stay alive until those have run)."""
        torch = self._torch
        c = self.cfg
        n = 0 if k_new is None else k_new.shape[1]
        shape = (c.n_layer, n, self.geo.kv_row)
        fn = ring_begin_step_deferred if deferred else ring_begin_step
        fn(self.handle, seq, committed,
           self._ptr(k_new, torch.float16, shape, "k_new"),
           self._ptr(v_new, torch.float16, shape, "v_new"), n, self._stream())

    def begin_step_batch(self, steps) -> None:
        """steps: (seq, committed, k_new, v_new) per sequence, as begin_step."""
        torch = self._torch
        c = self.cfg
        seqs, com, kp, vp, ns = [], [], [], [], []
        for seq, committed, k_new, v_new in steps:
            n = 0 if k_new is None else k_new.shape[1]
            shape = (c.n_layer, n, self.geo.kv_row)
            seqs.append(seq)
            com.append(committed)
            kp.append(self._ptr(k_new, torch.float16, shape, "k_new"))
            vp.append(self._ptr(v_new, torch.float16, shape, "v_new"))
            ns.append(n)
        ring_begin_step_batch(self.handle, seqs, com, kp, vp, ns, self._stream())

    def mirror_write(self, seq: int, pos0: int, features, deferred: bool = False) -> None:
        """features: F16 [n, d_model] of positions [pos0, pos0 + n).  deferred:
        ring_mirror_write_deferred (the tensor must stay alive and unchanged
        until the next begin_step_mirror of the sequence)."""
        torch = self._torch
        n = features.shape[0]
        fn = ring_mirror_write_deferred if deferred else ring_mirror_write
        fn(self.handle, seq, pos0, n,
           self._ptr(features, torch.float16, (n, self.cfg.d_model), "features"),
           self._stream())

    def set_kv_weights(self, wk, wv, k_norm, eps: float) -> None:
        """Register the projection weights (shapes as for begin_step_mirror)."""
        torch = self._torch
        c = self.cfg
        wshape = (c.n_layer, self.geo.kv_row, c.d_model)
        ring_set_kv_weights(self.handle, self._ptr(wk, torch.float16, wshape, "wk"),
                            self._ptr(wv, torch.float16, wshape, "wv"),
                            self._ptr(k_norm, torch.float32, (c.n_layer, c.head_dim), "k_norm"),
                            eps, self._stream())

    def begin_step_mirror(self, seq: int, committed: int, wk=None, wv=None, k_norm=None,
                          eps: float = 0.0) -> None:
        """wk, wv: F16 [n_layer, kv_row, d_model]; k_norm: F32 [n_layer, head_dim].
        All None: the weights registered with set_kv_weights."""
        torch = self._torch
        c = self.cfg
        if wk is None and wv is None and k_norm is None:
            ring_begin_step_mirror_registered(self.handle, seq, committed, self._stream())
            return
        wshape = (c.n_layer, self.geo.kv_row, c.d_model)
        ring_begin_step_mirror(self.handle, seq, committed,
                               self._ptr(wk, torch.float16, wshape, "wk"),
                               self._ptr(wv, torch.float16, wshape, "wv"),
                               self._ptr(k_norm, torch.float32, (c.n_layer, c.head_dim), "k_norm"),
                               eps, self._stream())

    def attn(self, layer: int, q, k_noise, v_noise, out=None, noalloc: bool = False):
        """ring_attn (noalloc: ring_attn_noalloc, split partials in the
        library's static array; `out` must then be given, so that the call
        allocates nothing)."""
        torch = self._torch
        c = self.cfg
        if out is None:
            if noalloc:
                raise ValueError("ring_attn_noalloc writes into a given `out`")
            out = torch.empty((c.n_seq, c.q_len, c.n_head, c.head_dim), dtype=torch.float32,
                              device=self.device)
        (ring_attn_noalloc if noalloc else ring_attn)(self.handle, layer,
                  self._ptr(q, torch.float16, (c.n_seq, c.q_len, c.n_head, c.head_dim), "q"),
                  self._ptr(k_noise, torch.float16, (c.n_seq, c.q_len, self.geo.kv_row), "k_noise"),
                  self._ptr(v_noise, torch.float16, (c.n_seq, c.q_len, self.geo.kv_row), "v_noise"),
                  self._ptr(out, torch.float32, (c.n_seq, c.q_len, c.n_head, c.head_dim), "out"),
                  self._stream())
        return out

    def slot_pos(self, seq: int) -> np.ndarray:
        return ring_read_slot_pos(self.handle, seq, self.cfg.cap)

    def mask(self, seq: int) -> np.ndarray:
        return ring_read_mask(self.handle, seq, self.cfg.q_len, self.geo.kv_total)

    def mask_swa(self, seq: int) -> np.ndarray:
        return ring_read_mask_swa(self.handle, seq, self.cfg.q_len, self.geo.kv_total)

    def rows(self, seq: int, layer: int, slot0: int, n: int):
        return ring_read_rows(self.handle, seq, layer, slot0, n, self.geo.kv_row)

    def state(self, seq: int):
        return ring_read_state(self.handle, seq)

    def describe(self) -> str:
        return ring_describe(self.handle)

    def profile_enable(self, max_launches: int) -> None:
        ring_profile_enable(self.handle, max_launches)

    def floor(self, layer: int, kind: int) -> None:
        """One profiling-only floor launch of `layer` (RING_FLOOR_*)."""
        ring_profile_floor(self.handle, layer, kind, self._stream())

    def profile_read(self, kernel: int) -> Tuple[int, float]:
        return ring_profile_read(self.handle, kernel)

    def close(self) -> None:
        if getattr(self, "handle", None):
            ring_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
