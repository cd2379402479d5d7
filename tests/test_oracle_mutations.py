"""Plant plausible mistakes in the CPU oracle and check that the pins see them.

Each mutation rewrites one oracle function from its source with a single
textual change (a dropped term, a flipped sign, a wrong index or bound) and
runs every pin against the mutated module.  At least one pin must fail.
Everything here runs on the CPU; the oracle module is restored afterwards.
"""

import inspect
import textwrap

import pytest

import oracle.ring_oracle as ro
from tests import oracle_pins as P

MUTATIONS = [
    # (function, original text, mistaken text)
    ("geometry", "align_up(cap + q_len + 1, 32)", "align_up(cap + q_len, 32)"),
    ("geometry", "2 * q_len + 2", "2 * q_len + 1"),
    ("geometry", "trash_slot=cap + q_len", "trash_slot=cap + q_len - 1"),
    ("ring_bytes", "2 * n_layer * kv_row * kv_total * 2", "n_layer * kv_row * kv_total * 2"),
    ("plan_step", "bulk=n_new > g.a_step", "bulk=n_new >= g.a_step"),
    ("plan_step", "start = max(min(next_pos, committed), lo)", "start = min(next_pos, committed)"),
    ("plan_step", "if lo < held_lo:", "if False:"),
    ("plan_step", "[g.trash_slot] * (g.a_step - n_new)", "[g.cap] * (g.a_step - n_new)"),
    ("plan_step", "(start + i) % g.cap", "(start + i + 1) % g.cap"),
    ("rope", "a * c - b * s", "a * c + b * s"),
    ("rope", "b * c + a * s", "b * c - a * s"),
    ("rope", "a, b = x[..., :half], x[..., half:]", "a, b = x[..., 0::2], x[..., 1::2]"),
    ("rope_inv_freq", "-2.0 * i / head_dim", "-1.0 * i / head_dim"),
    ("rope_rows_f16", ".astype(np.float16)", ".astype(np.float64)"),
    ("attend", "scale = dtype(1.0 / math.sqrt(d))", "scale = dtype(1.0)"),
    ("attend", "g = h // group", "g = h % hk"),
    ("attend", "lo = committed - win", "lo = committed - win + 1"),
    ("attend", "kn = rope_rows_f16(k_noise, pq, hk, d, cache.base)",
     "kn = np.asarray(k_noise, np.float16)"),
    ("attend", "qr = rope(q, pq, cache.base).astype(dtype)",
     "qr = rope(q, pq + 1, cache.base).astype(dtype)"),
    ("attend", "w = np.exp(s - m)", "w = np.exp(s - m) + 1e-9"),
    ("attend", "vals = np.concatenate([v_ctx, np.asarray(v_noise, np.float16)])",
     "vals = np.concatenate([k_ctx, np.asarray(v_noise, np.float16)])"),
    ("mask_full", "(sp >= lo) & (sp < committed)", "(sp > lo) & (sp < committed)"),
    ("mask_full", "(sp >= lo) & (sp < committed)", "(sp >= lo) & (sp <= committed)"),
    ("mask_full", "row[g.cap: g.cap + g.q_len] = np.float16(0.0)",
     "row[g.cap: g.cap + g.q_len - 1] = np.float16(0.0)"),
    ("mask_full", "row[g.cap: g.cap + g.q_len] = np.float16(0.0)",
     "row[g.cap: g.cap + g.q_len + 1] = np.float16(0.0)"),
    ("SlotHistory.apply", "self.slot_pos[pos % self.g.cap] = pos",
     "self.slot_pos[(pos + 1) % self.g.cap] = pos"),
    ("noise_positions", "committed + np.arange(q_len, dtype=np.int64)",
     "committed + 1 + np.arange(q_len, dtype=np.int64)"),
    # sliding-window layers (page 1 section 1.4, mask_swa)
    ("attend", "win = min(swa_window, win)", "win = min(swa_window, cap)"),
    ("attend", "win = min(swa_window, win)", "win = min(swa_window + 1, win)"),
    ("attend", "bias[:, n_ctx:] = np.where(later, -np.inf, 0.0)", "bias[:, n_ctx:] = 0.0"),
    ("attend", "later = np.arange(q_len)[None, :] > np.arange(q_len)[:, None]",
     "later = np.arange(q_len)[None, :] < np.arange(q_len)[:, None]"),
    ("mask_swa", "(sp >= swa_lo) & (sp < committed)", "(sp > swa_lo) & (sp < committed)"),
    ("mask_swa", "eff_win = min(swa_window, min(committed, g.cap))",
     "eff_win = min(swa_window - 1, min(committed, g.cap))"),
    ("mask_swa", "m[i, g.cap: g.cap + i + 1] = np.float16(0.0)",
     "m[i, g.cap: g.cap + i] = np.float16(0.0)"),
    ("mask_swa", "m[i, g.cap: g.cap + i + 1] = np.float16(0.0)",
     "m[i, g.cap: g.cap + g.q_len] = np.float16(0.0)"),
    # new rows' K/V from fused features, and the feature mirror
    ("project_kv", "k = k / rms * np.asarray(k_norm, dtype=np.float64)",
     "k = k * np.asarray(k_norm, dtype=np.float64)"),
    ("project_kv", "k = k / rms * np.asarray(k_norm, dtype=np.float64)", "k = k / rms"),
    ("project_kv", "(k * k).mean(axis=-1, keepdims=True)", "(k * k).sum(axis=-1, keepdims=True)"),
    ("project_kv", "(k * k).mean(axis=-1, keepdims=True)",
     "(k * k).mean(axis=(-1, -2), keepdims=True)"),
    ("project_kv", "k = rope(k, positions, base)", "k = rope(k, positions + 1, base)"),
    ("project_kv", "k = rope(k, positions, base).reshape(n, n_head_kv * head_dim)",
     "k = k.reshape(n, n_head_kv * head_dim)"),
    ("project_kv", "v = f @ np.asarray(wv, dtype=np.float64).T",
     "v = f @ np.asarray(wk, dtype=np.float64).T"),
    ("FeatureMirror.write", "self.slots[p % self.cap] = features[j]",
     "self.slots[(p + 1) % self.cap] = features[j]"),
    ("FeatureMirror.read", "if self.slot_pos[p % self.cap] != p:", "if False:"),
    ("RingStep.commit_features", "f = mirror.read(pos)", "f = mirror.read(pos[::-1])"),
]


def _patch(fname, old, new):
    """Return (target, attr, original) after replacing ro.<fname> with a mutant."""
    if "." in fname:
        cls_name, meth = fname.split(".")
        target = getattr(ro, cls_name)
        orig = target.__dict__[meth]
    else:
        target, meth = ro, fname
        orig = getattr(ro, fname)
    src = textwrap.dedent(inspect.getsource(orig))
    assert old in src, (fname, old)
    ns = dict(ro.__dict__)
    exec(compile(src.replace(old, new, 1), f"<mutant {fname}>", "exec"), ns)
    setattr(target, meth, ns[meth])
    return target, meth, orig


@pytest.mark.parametrize("fname,old,new", MUTATIONS,
                         ids=[f"{m[0]}:{i}" for i, m in enumerate(MUTATIONS)])
def test_mutation_is_caught(fname, old, new):
    target, meth, orig = _patch(fname, old, new)
    caught = []
    try:
        for pin in P.ALL_PINS:
            try:
                pin()
            except (AssertionError, KeyError, ValueError, IndexError):
                caught.append(pin.__name__)
    finally:
        setattr(target, meth, orig)
    assert caught, f"no pin caught mutation {fname}: {old!r} -> {new!r}"


def test_unmutated_oracle_passes_all_pins():
    for pin in P.ALL_PINS:
        pin()
