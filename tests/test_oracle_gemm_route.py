"""Pins of the oracle's grouped W4A4 GEMM (with and without the RAC residual
pass), its MoE routing and the SiLU*mul step.

GEMM: 4-bit by 4-bit GEMMs on NVFP4 operands (QUADS arXiv abstract, mlsanity
page "Abstract (arXiv)"); the residual pass adds to an unchanged main pass
(QUADS blog post, section "Two fixes, on two different sides").
Routing and SiLU*mul belong to the MoE FFN layer the workloads describe."""
from fractions import Fraction as Fr

import numpy as np
import pytest

from nvfp4_w4a4_moe_quant_amd import datagen
from oracle import brute


def _unpack(codes):
    return np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], -1)


def _q(orc, x):
    c, s, t = orc.quantize(x)
    return c, s, t


def _wq(orc, ws):
    parts = [orc.quantize(w) for w in ws]
    return (np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]),
            np.array([p[2] for p in parts], np.float32))


def _tiny_case(orc, seed, rac=True, gather=True):
    rng = np.random.default_rng(seed)
    K, N, src = 32, 5, 4
    x = rng.standard_normal((src, K)).astype(np.float32)
    x[:, 7] *= 25
    d = orc.quantize_rac(x, n_select=K // 2)
    a = (d["codes"], d["scales"], d["s_t"])
    r = (d["res_codes"], d["res_scales"], d["s_tr"]) if rac else None
    ws = [rng.standard_normal((N, K)).astype(np.float32) * 0.02 for _ in range(3)]
    w = _wq(orc, ws)
    offsets = np.array([0, 3, 3, 6], np.int32)          # group 1 is empty
    g = np.array([2, 0, 3, 1, 1, 0], np.int32) if gather else None
    if not gather:
        offsets = np.array([0, 2, 2, 4], np.int32)
    return K, N, a, r, w, offsets, g


@pytest.mark.parametrize("seed,rac,gather", [(20, True, True), (21, False, True),
                                             (22, True, False)])
def test_gemm_vs_fraction_bruteforce(orc, seed, rac, gather):
    K, N, a, r, w, offsets, g = _tiny_case(orc, seed, rac, gather)
    out = orc.grouped_gemm(N, K, offsets, g, a, r, w)
    ub = lambda op: (_unpack(op[0]).tolist(), op[1].tolist(), Fr(op[2]))
    wb = [(_unpack(w[0][e]).tolist(), w[1][e].tolist(), Fr(float(w[2][e])))
          for e in range(w[0].shape[0])]
    exact = brute.gemm(ub(a), None if r is None else ub(r), wb,
                       [int(v) for v in offsets], None if g is None else list(g), N)
    for j in range(out.shape[0]):
        for n in range(N):
            assert Fr(float(out[j, n])) == brute.rn32(exact[j][n]), (j, n)


def test_gemm_sample_equals_full_and_main_pass_intact(orc):
    K, N, a, r, w, offsets, g = _tiny_case(orc, 23)
    full, ms, rs = orc.grouped_gemm(N, K, offsets, g, a, r, w, want_sums=True)
    naive, ms0, _ = orc.grouped_gemm(N, K, offsets, g, a, None, w, want_sums=True)
    assert np.array_equal(ms, ms0)             # main accumulator unchanged by RAC
    rows = np.repeat(np.arange(full.shape[0]), N)
    cols = np.tile(np.arange(N), full.shape[0])
    smp = orc.grouped_gemm_sample(N, K, offsets, g, a, r, w, rows, cols)
    assert np.array_equal(smp, full.ravel())
    # naive output is exactly the main sum scaled
    wt = w[2][[0, 0, 0, 2, 2, 2]]
    ref = (np.float64(a[2]) * ms0 * 2.0 ** -20 * wt[:, None]).astype(np.float32)
    assert np.array_equal(naive, ref)


def test_gemm_lossless_equals_float64_matmul(orc):
    """Operands exactly representable (grid * power-of-two scales): the GEMM
    output equals the plain float64 matmul of the original matrices."""
    rng = np.random.default_rng(24)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])

    def exact_matrix(rows, K, st_exp):
        g = grid[rng.integers(0, 8, (rows, K))] * rng.choice([-1, 1], (rows, K))
        g[:, ::16] = 6.0
        sb = 2.0 ** rng.integers(-4, 5, (rows, K // 16))
        sb[0, 0] = 448.0
        return (g * np.repeat(sb, 16, axis=1) * 2.0 ** st_exp).astype(np.float32)

    A = exact_matrix(6, 64, -2)
    W = exact_matrix(7, 64, -9)
    a = _q(orc, A)
    w = _wq(orc, [W])
    assert np.array_equal(orc.dequantize(*a), A)
    out = orc.grouped_gemm(7, 64, np.array([0, 6], np.int32), None, a, None, w)
    ref = A.astype(np.float64) @ W.astype(np.float64).T
    assert np.array_equal(out, ref.astype(np.float32))


def test_route_vs_sort(orc):
    rng = np.random.default_rng(25)
    T, E, k = 50, 12, 3
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[0] = 0.5                                      # all tied
    logits[1, [2, 5]] = 9.0                              # a tie at the top
    logits[:, 11] = -np.inf                              # an expert never chosen
    d = orc.route(logits, k)
    counts = np.zeros(E, np.int64)
    for t in range(T):
        want = sorted(range(E), key=lambda e: (-logits[t, e], e))[:k]
        assert list(d["topk_ids"][t]) == want
        counts[want] += 1
        p = np.exp(logits[t].astype(np.float64) - logits[t].max())
        p /= p.sum()
        np.testing.assert_allclose(d["topk_weights"][t], p[want], rtol=1e-6)
    assert list(d["topk_ids"][0]) == [0, 1, 2]
    assert list(d["topk_ids"][1][:2]) == [2, 5]
    assert list(np.diff(d["offsets"])) == list(counts) and counts[11] == 0
    assert d["offsets"][-1] == T * k
    # gather: expert-major, tokens ascending; row_of inverts it
    for e in range(E):
        seg = d["gather"][d["offsets"][e]:d["offsets"][e + 1]]
        assert list(seg) == [t for t in range(T) if e in d["topk_ids"][t]]
    for t in range(T):
        for s in range(k):
            j = d["row_of"][t, s]
            assert d["gather"][j] == t
            e = d["topk_ids"][t, s]
            assert d["offsets"][e] <= j < d["offsets"][e + 1]


def test_zipf_routing_has_empty_experts(orc):
    w = datagen.small_moe(40, T=512, E=32, topk=4, H=64, I=32, routing="zipf",
                          n_empty=3)
    d = orc.route(datagen.router_logits(w), w.topk)
    counts = np.diff(d["offsets"])
    assert (counts == 0).sum() == 3 and counts.sum() == 512 * 4


def test_silu_mul(orc):
    rng = np.random.default_rng(26)
    y = (rng.standard_normal((7, 10)) * 3).astype(np.float32)
    h, amax = orc.silu_mul(y, 5)
    for i in range(7):
        for j in range(5):
            g, u = float(y[i, j]), float(y[i, 5 + j])
            v = g / (1.0 + np.exp(-g)) * u
            want = brute.rnbf16(Fr(v))
            got = np.array([int(h[i, j]) << 16], np.uint32).view(np.float32)[0]
            # double evaluation of silu: equal to rounding the double value
            assert Fr(float(got)) == want
    hf = (h.astype(np.uint32) << 16).view(np.float32)
    assert amax == np.abs(hf).max()
