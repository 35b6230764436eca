"""Pins of the oracle's FP8 W8A8 comparator: per-row E4M3 quantization and the
grouped FP8 GEMM.

The pages compare QUADS against FP8 rollout (arXiv abstract on the mlsanity
page; blog post, section "What it buys") without saying how the FP8 engine
scales; the oracle reads it as per-token activation scales and per-output-
channel weight scales, s = amax/448, E4M3 elements rounded to nearest even
with saturation.  These tests pin that reading against an independent exact
brute force (Fractions, exhaustive nearest search), closed forms and
invariants."""
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import brute


def _e4m3_points():
    vals = sorted(set(brute.E4M3.values()))
    pts = []
    for a, b in zip(vals, vals[1:]):
        m = np.float32(float((a + b) / 2))
        pts += [float(a), float(m), float(np.nextafter(m, np.float32(0))),
                float(np.nextafter(m, np.float32(1e9)))]
    pts += [448.0, 455.0, 463.99, 464.0, 500.0, 1e30, 2.0 ** -10, 2.0 ** -11 * 1.5,
            1e-40]
    return pts


def test_fp8_encode_vs_exhaustive_nearest(orc):
    for p in _e4m3_points():
        p32 = np.float32(p)
        ref = brute.e4m3_nearest(Fr(float(p32)))
        assert orc.fp8_encode(float(p32)) == ref, p
        assert orc.fp8_encode(float(-p32)) == 0x80 | ref, p


def test_fp8_encode_landmarks(orc):
    assert orc.fp8_encode(448.0) == 0x7E
    assert orc.fp8_encode(1e6) == 0x7E          # saturates, never NaN
    assert orc.fp8_encode(-1e6) == 0xFE
    assert orc.fp8_encode(1.0) == 0x38
    assert orc.fp8_encode(0.0) == 0x00
    assert orc.fp8_encode(-0.0) == 0x80          # sign kept
    assert orc.fp8_encode(-2.0 ** -11) == 0x80   # rounds to zero, sign kept
    assert orc.fp8_encode(2.0 ** -10 * 1.01) == 0x01  # above half the smallest subnormal


@pytest.mark.parametrize("amax,s", [(448.0, 1.0), (0.0, 0.0), (896.0, 2.0),
                                    (448.0 * 2.0 ** -20, 2.0 ** -20), (7.0, 0.015625)])
def test_fp8_row_scale_closed_form(orc, amax, s):
    assert orc.fp8_row_scale(amax) == s


def test_fp8_row_scale_vs_exact(orc):
    rng = np.random.default_rng(1)
    for a in np.exp(rng.uniform(-30, 30, 400)).astype(np.float32):
        ref = brute.rn32(brute.rn64(Fr(float(a)) / 448))
        assert Fr(float(np.float32(orc.fp8_row_scale(float(a))))) == ref


def _rows(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((6, 48)) * np.exp(rng.uniform(-4, 4, (6, 1)))).astype(np.float32)
    x[1] = 0.0                                  # all-zero row
    x[2, 5] = 1e4                               # one outlier: the rest go subnormal
    x[3, :8] = -1e-30                           # negatives that round to zero
    x[4] = np.float32(448.0) * np.arange(48, dtype=np.float32) / 47  # scale exactly 1
    return x


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fp8_quantize_rows_vs_brute(orc, seed):
    x = _rows(seed)
    codes, scales = orc.fp8_quantize_rows(x)
    bc, bs = brute.fp8_quantize_rows([[Fr(float(v)) for v in row] for row in x])
    assert codes.tolist() == bc
    assert [Fr(float(s)) for s in scales] == bs


def test_fp8_quantize_rows_invariants(orc):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 256)) * 3).astype(np.float32)
    x[7] = 0.0
    codes, scales = orc.fp8_quantize_rows(x)
    assert scales[7] == 0.0 and not codes[7].any()
    dec = np.vectorize(orc.e4m3_value)(codes & 0x7F) * np.where(codes & 0x80, -1.0, 1.0)
    for i in range(64):
        if i == 7:
            continue
        j = int(np.argmax(np.abs(x[i])))
        assert codes[i, j] & 0x7F == 0x7E           # the row max lands on 448
        assert np.all(np.sign(dec[i]) * np.sign(x[i]) >= 0)
        # error within half an E4M3 spacing at the scaled value (plus FP32 slop)
        v = np.abs(x[i].astype(np.float64)) / scales[i]
        e = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
        half = 2.0 ** (e - 4)
        assert np.all(np.abs(v - np.abs(dec[i])) <= half * (1 + 1e-6) + 1e-9)


def _fp8_weights(orc, rng, G, N, K):
    ws = rng.standard_normal((G, N, K)).astype(np.float32) * 0.05
    parts = [orc.fp8_quantize_rows(ws[g]) for g in range(G)]
    return (np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))


def test_fp8_gemm_vs_brute_tiny(orc):
    rng = np.random.default_rng(5)
    K, N = 16, 3
    x = rng.standard_normal((4, K)).astype(np.float32)
    ac, as_ = orc.fp8_quantize_rows(x)
    wc, wsc = _fp8_weights(orc, rng, 2, N, K)
    offsets = np.array([0, 3, 5], np.int32)
    gather = np.array([2, 0, 3, 1, 1], np.int32)
    y = orc.fp8_grouped_gemm(N, K, offsets, gather, (ac, as_), (wc, wsc))
    ref = brute.fp8_gemm(ac.tolist(), [Fr(float(s)) for s in as_],
                         [(wc[g].tolist(), [Fr(float(s)) for s in wsc[g]]) for g in range(2)],
                         offsets.tolist(), gather.tolist(), N)
    assert [[Fr(float(v)) for v in row] for row in y] == ref


def test_fp8_gemm_vs_integer_matmul(orc):
    rng = np.random.default_rng(6)
    G, N, K, src = 3, 8, 128, 10
    x = (rng.standard_normal((src, K)) * 4).astype(np.float32)
    ac, as_ = orc.fp8_quantize_rows(x)
    wc, wsc = _fp8_weights(orc, rng, G, N, K)
    offsets = np.array([0, 4, 4, 11], np.int32)     # includes an empty group
    gather = rng.integers(0, src, 11).astype(np.int32)
    y = orc.fp8_grouped_gemm(N, K, offsets, gather, (ac, as_), (wc, wsc))

    def img(c):  # exact integer image value * 2^9 by table lookup
        t = np.array([float(brute.fp8_value(b) * 512) if (b & 0x7F) != 0x7F else 0.0
                      for b in range(256)])
        return t[c].astype(np.int64)

    ai, wi = img(ac), img(wc)
    for g in range(G):
        for j in range(offsets[g], offsets[g + 1]):
            acc = wi[g] @ ai[gather[j]]                # exact int64
            ref = (as_[gather[j]].astype(np.float64) * wsc[g].astype(np.float64)
                   * acc.astype(np.float64) * 2.0 ** -18)
            np.testing.assert_allclose(y[j], ref.astype(np.float32), rtol=2e-7, atol=0)
    # the sampled form agrees with the full one
    rows = np.array([0, 3, 10, 7], np.int64)
    cols = np.array([1, 7, 0, 5], np.int64)
    s = orc.fp8_grouped_gemm_sample(N, K, offsets, gather, (ac, as_), (wc, wsc), rows, cols)
    assert np.array_equal(s, y[rows, cols])


def test_fp8_gemm_planted_mistakes_fail(orc):
    """A transposed weight or a dropped row scale changes the result."""
    rng = np.random.default_rng(7)
    K, N = 32, 32
    x = rng.standard_normal((32, K)).astype(np.float32) * np.exp(rng.uniform(-2, 2, (32, 1)))
    ac, as_ = orc.fp8_quantize_rows(x.astype(np.float32))
    wc, wsc = _fp8_weights(orc, rng, 1, N, K)
    off = np.array([0, 32], np.int32)
    y = orc.fp8_grouped_gemm(N, K, off, None, (ac, as_), (wc, wsc))
    yt = orc.fp8_grouped_gemm(N, K, off, None, (ac, as_), (wc.transpose(0, 2, 1).copy(), wsc))
    y1 = orc.fp8_grouped_gemm(N, K, off, None, (ac, np.ones_like(as_)), (wc, wsc))
    assert not np.allclose(y, yt) and not np.allclose(y, y1)
