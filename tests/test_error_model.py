"""The per-element rounding model that bounds the matrix-core path in the GPU
parity tests (tests/helpers.py: mfma_query, weight_sigma), checked on the CPU
against an emulation of that path's arithmetic: the query times
fp32(scale * log2 e) in fp32, rounded to F16; scores in log2 units; F16
softmax weights taken against a running maximum that may lag the row maximum
by up to 2^8 (the lazy rescale); the row sum over the same F16 weights; all
else exact.  The model must cover every emulated error within SIGMA_Z of its
standard deviations, must not be loose (RMS of the normalised errors near the
expected ~0.7), and a dropped cell must break it."""

import math

import numpy as np
import pytest

from oracle.attention import masked_attention
from oracle.kvcache import f16_round
from tests.helpers import SIGMA_FLOOR, SIGMA_Z, mfma_query, weight_sigma

LN2 = math.log(2.0)


def problem(rng, T, n, H, HK, D, needle=0.0):
    """T queries over n cells of one stream; query t sees cells 0..n_t-1 with
    n_t spread over [1, n]."""
    q = rng.standard_normal((T, H * D)).astype(np.float32)
    k = f16_round(rng.standard_normal((1, n, HK * D)))
    v = f16_round(rng.standard_normal((1, n, HK * D)))
    if needle:
        k[0, n // 2] = f16_round(k[0, n // 2] * needle)
    lens = np.unique(np.linspace(1, n, T).astype(int))
    lens = np.resize(lens, T)
    mask = np.where(np.arange(n)[None, :] < lens[:, None], 0.0, -np.inf)
    return q, k, v, mask, lens


def emulate(q, k, v, mask, H, HK, D, rng, drop=None):
    """The matrix-core path's arithmetic over the same inputs; drop[t] = a
    visible cell left out of row t (all heads), -1 for none."""
    T = q.shape[0]
    g = H // HK
    c32 = np.float32(np.float32(1.0) / np.sqrt(np.float32(D)) * np.float32(1.4426950408889634))
    out = np.zeros((T, H * D))
    K = k[0].astype(np.float64)
    V = v[0].astype(np.float64)
    for t in range(T):
        vis = np.isfinite(mask[t])
        if drop is not None and drop[t] >= 0:
            vis[drop[t]] = False
        idx = np.nonzero(vis)[0]
        for h in range(H):
            kh = K[idx, (h // g) * D:(h // g + 1) * D]
            vh = V[idx, (h // g) * D:(h // g + 1) * D]
            qt = (q[t, h * D:(h + 1) * D] * c32).astype(np.float16).astype(np.float64)
            s = kh @ qt                                   # log2 units
            m = s.max() - rng.uniform(0.0, 8.0)           # running maximum lagging by < 2^8
            p = np.exp2(s - m).astype(np.float16).astype(np.float64)
            out[t, h * D:(h + 1) * D] = (p @ vh) / p.sum()
    return out


def model(q, k, v, mask, H, HK, D):
    T = q.shape[0]
    qt = mfma_query(q, D)
    args = (k, v, np.zeros(T, dtype=int), mask, H, HK, LN2)
    return masked_attention(qt, *args), weight_sigma(qt, *args)


CASES = [   # T, n, H, HK, D, needle
    (24, 300, 2, 1, 128, 0.0),
    (16, 3000, 2, 1, 128, 0.0),
    (24, 200, 4, 2, 64, 0.0),
    (32, 120, 2, 1, 16, 0.0),
    (16, 400, 2, 1, 128, 6.0),     # one dominant key in the middle of every row that reaches it
]


@pytest.mark.parametrize("T,n,H,HK,D,needle", CASES)
def test_model_covers_emulated_roundings(T, n, H, HK, D, needle):
    rng = np.random.default_rng(7 + n + D)
    q, k, v, mask, _ = problem(rng, T, n, H, HK, D, needle)
    alt, sig = model(q, k, v, mask, H, HK, D)
    zs = []
    for rep in range(3):
        err = np.abs(emulate(q, k, v, mask, H, HK, D, rng) - alt)
        assert (err <= SIGMA_Z * sig + SIGMA_FLOOR).all(), (err / np.maximum(sig, 1e-30)).max()
        live = sig > 1e-6
        zs.append(err[live] / sig[live])
    z = np.concatenate(zs)
    # not loose: F16 rounding of values spread over their binade has ~0.73 of
    # the RMS the model assumes
    assert 0.4 < math.sqrt((z * z).mean()) < 1.0, math.sqrt((z * z).mean())


def test_f16_query_rounding_is_a_separate_term():
    """The query rounding moves outputs by about as much as the weight
    roundings do: measured against the fp32-query oracle, the emulated errors
    are ~1.4x larger in units of the weight model's sigma than against alt,
    which accounts for the query rounding exactly."""
    rng = np.random.default_rng(3)
    T, n, H, HK, D = 16, 3000, 2, 1, 128
    q, k, v, mask, _ = problem(rng, T, n, H, HK, D)
    exact = masked_attention(q, k, v, np.zeros(T, dtype=int), mask, H, HK, 1.0 / math.sqrt(D))
    alt, sig = model(q, k, v, mask, H, HK, D)
    e = emulate(q, k, v, mask, H, HK, D, rng)
    live = sig > 1e-6
    rms = [math.sqrt(((np.abs(e - r)[live] / sig[live]) ** 2).mean()) for r in (exact, alt)]
    assert rms[0] > 1.25 * rms[1], rms


@pytest.mark.parametrize("n", [64, 700, 3000])
def test_dropped_cell_breaks_the_model(n):
    """Leaving out one visible cell of median weight in every row with at
    least 16 visible cells puts every such row outside the bound."""
    rng = np.random.default_rng(n)
    T, H, HK, D = 12, 2, 1, 128
    q, k, v, mask, lens = problem(rng, T, n, H, HK, D)
    alt, sig = model(q, k, v, mask, H, HK, D)
    drop = []
    for t in range(T):
        s = (q[t, :D].astype(np.float64) @ k[0, :lens[t], :D].astype(np.float64).T)
        drop.append(int(np.argsort(s)[lens[t] // 2]) if lens[t] >= 16 else -1)
    err = np.abs(emulate(q, k, v, mask, H, HK, D, rng, drop=drop) - alt)
    beyond = (err > SIGMA_Z * sig + SIGMA_FLOOR).any(axis=1)
    rows = lens >= 16
    assert rows.any() and beyond[rows].all(), list(zip(lens[rows], beyond[rows]))
