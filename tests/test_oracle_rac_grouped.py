"""Pins of the oracle's per-expert RAC (each expert group's rows form their
own tensor for the tensor scale, channel statistics, selection and residual;
QUADS blog post, section "Two fixes, on two different sides", leaves the
granularity open) and of the grouped GEMM with per-group activation and
residual tensor scales."""
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import brute


def _x(seed, rows, K):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, K)).astype(np.float32)
    x[:, rng.integers(0, K, 2)] *= 30.0
    return x


def test_one_group_is_the_per_tensor_path(orc):
    x = _x(1, 40, 64)
    d = orc.quantize_rac_grouped(x, np.array([0, 40], np.int32), None, 32)
    p = orc.quantize_rac(x, 32)
    for k in ("codes", "scales", "res_codes", "res_scales"):
        assert np.array_equal(d[k], p[k]), k
    assert np.array_equal(d["score"][0], p["score"]) and np.array_equal(d["chmax"][0], p["chmax"])
    assert np.array_equal(d["selected"][0], p["selected"]) and np.array_equal(d["active"][0], p["active"])
    assert d["s_t"][0] == np.float32(p["s_t"]) and d["s_tr"][0] == np.float32(p["s_tr"])


def _brute_group(sub, n_sel):
    xf = [[Fr(float(v)) for v in row] for row in sub]
    codes, scales, s_t = brute.quantize(xf)
    e = brute.errors(xf, codes, scales, s_t)
    score, chmax = brute.channel_scores(e, s_t)
    sel = brute.select(score, n_sel)
    r = [[e[i][k] if k in sel else Fr(0) for k in range(len(sub[0]))] for i in range(len(sub))]
    rc, rs, s_tr = brute.quantize(r, s_t=s_t)        # the residual pass uses the group's s_t
    return dict(codes=codes, scales=scales, s_t=s_t, score=score, chmax=chmax, sel=sel,
                res_codes=rc, res_scales=rs, s_tr=s_tr)


def _unpack(c):
    return np.stack([c & 15, c >> 4], -1).reshape(c.shape[0], -1)


def test_groups_with_gather_vs_brute(orc):
    K, src = 32, 12
    x = _x(2, src, K)
    offsets = np.array([0, 5, 5, 9, 14], np.int32)   # group 1 is empty
    gather = np.random.default_rng(3).integers(0, src, 14).astype(np.int32)
    n_sel = 12
    d = orc.quantize_rac_grouped(x, offsets, gather, n_sel)
    for g in range(4):
        j0, j1 = offsets[g], offsets[g + 1]
        if j1 == j0:  # empty group: zero scales, the lowest-index selection
            assert d["s_t"][g] == 0 and d["s_tr"][g] == 0
            assert d["selected"][g].tolist() == list(range(n_sel))
            assert not d["score"][g].any()
            continue
        b = _brute_group(x[gather[j0:j1]], n_sel)
        assert Fr(float(d["s_t"][g])) == b["s_t"]
        assert _unpack(d["codes"][j0:j1]).tolist() == b["codes"]
        assert d["scales"][j0:j1].tolist() == b["scales"]
        assert d["score"][g].tolist() == b["score"]
        assert [Fr(float(v)) for v in d["chmax"][g]] == b["chmax"]
        assert d["selected"][g].tolist() == b["sel"]
        assert Fr(float(d["s_tr"][g])) == b["s_tr"] == b["s_t"]
        assert _unpack(d["res_codes"][j0:j1]).tolist() == b["res_codes"]
        assert d["res_scales"][j0:j1].tolist() == b["res_scales"]


def test_grouped_gemm_per_group_scales(orc):
    """Per-group activation/residual scales: each group's rows equal the
    exact brute-force GEMM with that group's scales."""
    K, N, src = 32, 4, 10
    x = _x(4, src, K)
    offsets = np.array([0, 3, 3, 8], np.int32)
    gather = np.random.default_rng(5).integers(0, src, 8).astype(np.int32)
    d = orc.quantize_rac_grouped(x, offsets, gather, 16)
    rng = np.random.default_rng(6)
    ws = [orc.quantize((rng.standard_normal((N, K)) * 0.05).astype(np.float32)) for _ in range(3)]
    w = (np.stack([q[0] for q in ws]), np.stack([q[1] for q in ws]),
         np.array([q[2] for q in ws], np.float32))
    # rows are already in grouped order: the GEMM runs without a gather
    y = orc.grouped_gemm(N, K, offsets, None, (d["codes"], d["scales"], d["s_t"]),
                         (d["res_codes"], d["res_scales"], d["s_tr"]), w)
    unp = lambda c: _unpack(c).tolist()
    for g in (0, 2):
        j0, j1 = offsets[g], offsets[g + 1]
        a = (unp(d["codes"][j0:j1]), d["scales"][j0:j1].tolist(), Fr(float(d["s_t"][g])))
        r = (unp(d["res_codes"][j0:j1]), d["res_scales"][j0:j1].tolist(), Fr(float(d["s_tr"][g])))
        wg = [(unp(w[0][g]), w[1][g].tolist(), Fr(float(w[2][g])))]
        ref = brute.gemm(a, r, wg, [0, j1 - j0], None, N)
        got = [[Fr(float(v)) for v in row] for row in y[j0:j1]]
        assert got == [[brute.rn32(v) for v in row] for row in ref]
    # a scalar scale and a constant per-group array agree
    c = np.full(3, d["s_t"][0], np.float32)
    y1 = orc.grouped_gemm(N, K, offsets, None, (d["codes"], d["scales"], float(d["s_t"][0])), None, w)
    y2 = orc.grouped_gemm(N, K, offsets, None, (d["codes"], d["scales"], c), None, w)
    assert np.array_equal(y1, y2)
