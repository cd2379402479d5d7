"""The split partials are stored as F16 outputs normalised by their own
softmax sums, with fp32 (max, sum) pairs (k_ring_attn / k_ring_merge).  This
CPU emulation bounds what that rounding costs against the output tolerance
(|err| <= 2e-3 + 1e-2 |ref|), on the value distributions of the workloads
with and without +-30 outliers: exact fp64 attention against the same
attention split over key ranges, each split's output rounded to F16 (RNE),
merged in fp32 with weights 2^(m_t - M) l_t."""

import numpy as np
import pytest


def f16(x):
    return x.astype(np.float16).astype(np.float32)


def bf16(x):
    """Round to 8 significant bits (bfloat16), nearest-even."""
    b = x.astype(np.float32).view(np.uint32)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def emulate(n_keys, n_q, n_split, sigma, outlier_p, seed, d=128, rounding=f16):
    rng = np.random.default_rng(seed)

    def draw(shape):
        x = rng.normal(0.0, sigma, shape)
        if outlier_p:
            hit = rng.random(shape) < outlier_p
            x[hit] = np.where(rng.random(hit.sum()) < 0.5, -30.0, 30.0)
        return x.astype(np.float16).astype(np.float64)

    q, k, v = draw((n_q, d)), draw((n_keys, d)), draw((n_keys, d))
    s = q @ k.T / np.sqrt(d)
    p = np.exp(s - s.max(1, keepdims=True))
    ref = (p @ v) / p.sum(1, keepdims=True)
    per = -(-n_keys // n_split)
    parts = []
    for t in range(n_split):
        st = s[:, t * per:(t + 1) * per]
        mt = st.max(1, keepdims=True)
        pt = np.exp(st - mt)
        lt = pt.sum(1, keepdims=True)
        ot = (pt @ v[t * per:(t + 1) * per]) / lt
        parts.append((np.float32(np.log2(np.e)) * mt.astype(np.float32), lt.astype(np.float32),
                      rounding(ot)))
    big_m = np.max([m for m, _, _ in parts], axis=0)
    num = np.zeros((n_q, d), np.float32)
    den = np.zeros((n_q, 1), np.float32)
    for m, l, o in parts:
        a = np.exp2(m - big_m).astype(np.float32) * l
        num += a * o
        den += a
    err = np.abs(num / den - ref)
    return float((err / (2e-3 + 1e-2 * np.abs(ref))).max()), float(err.max())


@pytest.mark.parametrize("n_keys,n_q,n_split,sigma,outlier_p,bound", [
    (4096, 32, 32, 0.5, 0.0, 0.02),     # decode stream
    (4096, 32, 4, 0.5, 0.0, 0.02),      # a ring of the batched sequences
    (8192, 64, 16, 1.0, 0.01, 0.3),     # the large window's values (+-30 outliers)
])
def test_f16_normalised_partials_within_tolerance(n_keys, n_q, n_split, sigma, outlier_p, bound):
    ratio, max_abs = emulate(n_keys, n_q, n_split, sigma, outlier_p, seed=n_keys + n_split)
    assert ratio < bound, (ratio, max_abs)
    if outlier_p == 0.0:
        assert max_abs < 2e-4      # far inside the 2e-3 absolute bar


def test_emulation_catches_a_coarser_rounding():
    """Negative control: the same emulation with the partials rounded to 8
    significant bits (bfloat16) fails the outlier bound above."""
    ratio, _ = emulate(8192, 64, 16, 1.0, 0.01, seed=8192 + 16, rounding=bf16)
    assert ratio > 0.3, ratio
