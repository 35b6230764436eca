"""Pins of the oracle's quantizer and RAC stages: the hand-derived worked
example, an exact rational brute force on small tensors, closed-form
lossless cases, idempotence, the RAC error guarantee and the selection rule.

RAC: QUADS blog post, section "Two fixes, on two different sides" (top ~50%
of activation channels by quantization error get a second, residual FP4
pass); activation quantization is online: QUADS arXiv abstract (mlsanity
page, "Abstract (arXiv)")."""
import os
from fractions import Fraction as Fr

import numpy as np
import pytest

from nvfp4_w4a4_moe_quant_amd import datagen
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.txt")


def _golden():
    out = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        out[key] = vals
    return out


def test_worked_example(orc):
    g = _golden()
    x = np.array([[float(v) for v in g["x"]]], np.float32)
    d = orc.quantize_rac(x, n_select=16)
    hexes = lambda a: [f"{int(b):02X}" for b in np.ravel(a)]
    assert d["s_t"] == float(g["tensor_scale"][0])
    assert hexes(d["scales"]) == g["scales"]
    assert hexes(d["codes"]) == g["codes"]
    assert [int(v) for v in d["score"]] == [int(v) for v in g["score"]]
    assert [int(v) for v in d["selected"]] == [int(v) for v in g["selected"]]
    assert [int(v) for v in d["active"]] == [int(v) for v in g["active"]]
    assert d["s_tr"] == float(g["residual_tensor_scale"][0]) == d["s_t"]
    assert d["amax_r"] == 256.0
    assert hexes(d["res_scales"]) == g["residual_scales"]
    assert hexes(d["res_codes"]) == g["residual_codes"]
    rec = orc.dequantize(d["codes"], d["scales"], d["s_t"]).astype(np.float64) + \
        orc.dequantize(d["res_codes"], d["res_scales"], d["s_tr"])
    assert list(x[0].astype(np.float64) - rec[0]) == [float(v) for v in g["rac_error"]]


def _unpack(codes):
    lo = codes & 15
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


def _brute_inputs(seed, rows, K):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, K)).astype(np.float32)
    x[:, rng.integers(0, K)] *= 37.0                 # an outlier channel
    x[0, :16] = 0.0                                  # an all-zero block
    x[1, 16:32] *= np.float32(1e-5)                  # subnormal block scales
    x[2, 3] = np.float32(5.0 * np.abs(x).max())      # a saturating block
    return x


@pytest.mark.parametrize("seed,rows,K", [(10, 4, 64), (11, 3, 48), (12, 5, 32)])
def test_quantize_and_rac_vs_brute(orc, seed, rows, K):
    x = _brute_inputs(seed, rows, K)
    xf = [[Fr(float(v)) for v in row] for row in x]
    codes, scales, s_t = brute.quantize(xf)
    d = orc.quantize_rac(x, n_select=K // 2)
    assert Fr(d["s_t"]) == s_t
    assert np.array_equal(d["scales"], np.array(scales, np.uint8))
    assert np.array_equal(_unpack(d["codes"]), np.array(codes, np.uint8))
    e = brute.errors(xf, codes, scales, s_t)
    score, chmax = brute.channel_scores(e, s_t)
    assert [int(v) for v in d["score"]] == score
    assert [Fr(float(v)) for v in d["chmax"]] == chmax
    sel = brute.select(score, K // 2)
    assert [int(v) for v in d["selected"]] == sel
    amax_r = max([chmax[k] for k in sel], default=Fr(0))
    assert Fr(d["amax_r"]) == amax_r
    r = [[e[i][k] if k in sel else Fr(0) for k in range(K)] for i in range(rows)]
    assert max((abs(v) for row in r for v in row), default=Fr(0)) == amax_r
    rc, rs, rt = brute.quantize(r, s_t=s_t)      # the residual pass uses the main s_t
    assert Fr(d["s_tr"]) == rt == s_t
    assert np.array_equal(d["res_scales"], np.array(rs, np.uint8))
    assert np.array_equal(_unpack(d["res_codes"]), np.array(rc, np.uint8))


def test_lossless_power_of_two_case(orc):
    """x = g * s_b * s_t with g on the grid, every block reaching 6, s_b any
    normal E4M3 value and s_t a power of two: q is exact, deq(q(x)) = x,
    e = 0, every score is 0, the selection is the lowest K/2 indices and the
    residual is zero."""
    rng = np.random.default_rng(5)
    rows, K = 8, 64
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)
    g = grid[rng.integers(0, 8, (rows, K))] * rng.choice([-1, 1], (rows, K))
    g[:, ::16] = 6.0                              # every block reaches 6
    sb_codes = rng.integers(0x08, 0x7F, (rows, K // 16))
    sb_codes[0, 0] = 0x7E                         # one block at 448 -> amax = 2688 s_t
    sb = np.array([[orc.e4m3_value(int(c)) for c in r] for r in sb_codes], np.float32)
    s_t = np.float32(2.0 ** -3)
    x = (g * np.repeat(sb, 16, axis=1) * s_t).astype(np.float32)
    d = orc.quantize_rac(x, n_select=K // 2)
    assert d["s_t"] == s_t
    assert np.array_equal(d["scales"], sb_codes.astype(np.uint8))
    deq = orc.dequantize(d["codes"], d["scales"], d["s_t"])
    assert np.array_equal(deq, x)
    assert not d["score"].any() and not d["chmax"].any()
    assert list(d["selected"]) == list(range(K // 2))
    assert not d["res_codes"].any() and not d["res_scales"].any()
    assert d["amax_r"] == 0.0 and d["s_tr"] == d["s_t"]


def test_all_zero_input(orc):
    x = np.zeros((5, 32), np.float32)
    d = orc.quantize_rac(x, n_select=16)
    assert d["s_t"] == 0.0 and not d["codes"].any() and not d["scales"].any()
    assert list(d["selected"]) == list(range(16)) and d["s_tr"] == 0.0


@pytest.mark.parametrize("wid", [1, 2])
def test_idempotence(orc, wid):
    w = datagen.WORKLOADS[wid]
    x = datagen.activations(w)
    codes, scales, s_t = orc.quantize(x)
    deq = orc.dequantize(codes, scales, s_t)
    # (ii) with scales recomputed: a fixed point when every block scale is normal
    assert (scales[np.any(x.reshape(x.shape[0], -1, 16) != 0, axis=2)] >= 0x08).all()
    c2, s2, t2 = orc.quantize(deq)
    assert t2 <= s_t
    assert np.array_equal(orc.dequantize(c2, s2, t2), deq)


def test_idempotence_fixed_scales(orc):
    """(i) With the scales held fixed, q(deq(q(x))) = q(x): deq values lie on
    grid * S_b, and re-dividing by S_b lands on the same grid point."""
    w = datagen.WORKLOADS[1]
    x = datagen.activations(w)
    amax = float(np.abs(x).max())
    codes, scales, s_t = orc.quantize(x, amax=amax)
    deq = orc.dequantize(codes, scales, s_t)
    c2, s2, t2 = orc.quantize(deq, amax=amax)
    assert t2 == s_t and np.array_equal(s2, scales) and np.array_equal(c2, codes)


@pytest.mark.parametrize("wid", [1, 2])
def test_rac_never_worse_than_naive(orc, wid):
    w = datagen.WORKLOADS[wid]
    x = datagen.activations(w).astype(np.float64)
    d = orc.quantize_rac(x.astype(np.float32), n_select=x.shape[1] // 2)
    naive = orc.dequantize(d["codes"], d["scales"], d["s_t"]).astype(np.float64)
    rac = naive + orc.dequantize(d["res_codes"], d["res_scales"], d["s_tr"])
    en, er = np.abs(x - naive), np.abs(x - rac)
    # unselected channels keep exactly the naive error
    uns = d["mask"] == 0
    assert np.array_equal(er[:, uns], en[:, uns])
    # selected: |r - deq(q(r))| <= |r| up to FP32 rounding of the dequantized value
    slack = 1e-6 * np.abs(x) + 1e-30
    assert (er <= en + slack).all()
    assert np.linalg.norm(x - rac) < np.linalg.norm(x - naive)
    # the outlier channels carry the largest errors and are selected
    assert d["mask"][datagen.outlier_channels(w)].all()


def test_selection_edge_counts(orc):
    rng = np.random.default_rng(6)
    score = rng.integers(0, 5, 64).astype(np.int64)     # many ties
    chmax = rng.uniform(0, 1, 64).astype(np.float32)
    for n in [0, 1, 31, 32, 63, 64]:
        sel, mask, active, amax_r = orc.rac_select(score, chmax, n)
        want = brute.select([int(v) for v in score], n)
        assert list(sel) == want and mask.sum() == n
        assert list(active) == [int(mask[16 * b:16 * b + 16].any()) for b in range(4)]
        assert amax_r == (float(chmax[want].max()) if n else 0.0)


def test_score_bound(orc):
    """q = floor(|e| 2^(8-Es)) stays below 2^17 on the workloads (so the
    clamp never acts and the score is the plain sum of squares)."""
    for wid in [1, 2]:
        x = datagen.activations(datagen.WORKLOADS[wid])
        codes, scales, s_t = orc.quantize(x)
        _, chmax = orc.channel_stats(x, codes, scales, s_t)
        sh = orc.score_shift(s_t)
        assert float(chmax.max()) * 2.0 ** sh < 2 ** 17
        assert float(chmax.max()) <= 448.0 * s_t * 1.0001
