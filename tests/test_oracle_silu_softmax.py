"""Pins of the oracle's SiLU*mul and routing-softmax weights against
references that share nothing with it: Python ``decimal`` at 50 significant
digits (a correctly rounded exp), exact rational rounding from
``oracle/brute.py``, and closed forms.

Each pin is also run on deliberately wrong variants (exp with the wrong sign,
gate and up halves swapped, SiLU replaced by the identity or by the bare
sigmoid, top-k weights renormalized, the softmax's max shift dropped) to show
that it rejects them.

Sources: the SiLU*mul epilogue is the MoE FFN's activation (h = silu(gate) * up,
silu(g) = g / (1 + e^-g), rounded once to bf16, gate in the first half of the
fused output); the routing weights are the softmax of the router logits at the
chosen experts, not renormalized."""
from decimal import Decimal, getcontext
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import brute

getcontext().prec = 50


def _silu_dec(g: float) -> Decimal:
    d = Decimal(float(g))
    return d / (1 + (-d).exp())


def _bf16_value(bits) -> Fr:
    f = np.array([int(bits) << 16], np.uint32).view(np.float32)[0]
    return Fr(float(f))


def _near_bf16_tie(v: Fr) -> bool:
    """True when v lies within 2^-40 (relative) of a bf16 rounding midpoint;
    there a double evaluation may legitimately round the other way."""
    if v == 0:
        return False
    a = abs(v)
    q = brute.rnbf16(a)
    # quantum of the bf16 grid around a (8 significant bits)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fr(2) ** e > a:
        e -= 1
    while Fr(2) ** (e + 1) <= a:
        e += 1
    quantum = Fr(2) ** (max(e, -126) - 7)
    mid_dist = abs(abs(a - q) - quantum / 2)
    return mid_dist <= a * Fr(1, 2 ** 40)


def silu_pin(y, I, h):
    """Checks h (bf16 bits [rows, I]) against bf16(silu(gate) * up) of y
    (float32 [rows, 2I], gate in columns [0, I)), computed in decimal and
    rounded exactly.  Returns (mismatches, skipped near-tie elements)."""
    bad = skipped = 0
    rows = y.shape[0]
    for i in range(rows):
        for j in range(I):
            g, u = float(y[i, j]), float(y[i, I + j])
            v = Fr(_silu_dec(g) * Decimal(u))
            if _near_bf16_tie(v):
                skipped += 1
                continue
            if _bf16_value(h[i, j]) != brute.rnbf16(v):
                bad += 1
    return bad, skipped


def _silu_inputs():
    rng = np.random.default_rng(2024)
    I = 16
    y = (rng.standard_normal((6, 2 * I)) * 4).astype(np.float32)
    # specials in the gate half: zero, tiny, large of both signs, +-1
    y[0, :8] = [0.0, 1e-30, -1e-30, 30.0, -30.0, 80.0, -80.0, 1.0]
    y[1, :4] = [-1.0, 0.5, -0.5, 1e-8]
    y[2, I:I + 4] = [1.0, -1.0, 0.0, 1e6]      # up half
    return y, I


def _variant(y, I, fn):
    rows = y.shape[0]
    h = np.zeros((rows, I), np.uint16)
    for i in range(rows):
        for j in range(I):
            v = fn(float(y[i, j]), float(y[i, I + j]))
            f = np.float32(float(brute.rnbf16(Fr(v)))) if np.isfinite(v) else np.float32(v)
            h[i, j] = np.array([f], np.float32).view(np.uint32)[0] >> 16
    return h


def test_silu_mul_against_decimal(orc):
    y, I = _silu_inputs()
    h, amax = orc.silu_mul(y, I)
    bad, skipped = silu_pin(y, I, h)
    assert bad == 0 and skipped <= 1
    hf = (h.astype(np.uint32) << 16).view(np.float32)
    assert amax == np.abs(hf).max()


@pytest.mark.parametrize("name,fn", [
    ("exp sign flipped", lambda g, u: g / (1.0 + np.exp(min(g, 700.0))) * u),
    ("gate and up swapped", lambda g, u: u / (1.0 + np.exp(-max(min(u, 700.0), -700.0))) * g),
    ("identity instead of silu", lambda g, u: g * u),
    ("sigmoid without the gate factor", lambda g, u: u / (1.0 + np.exp(-max(g, -700.0)))),
])
def test_silu_pin_rejects_planted_mistakes(name, fn):
    y, I = _silu_inputs()
    bad, _ = silu_pin(y, I, _variant(y, I, fn))
    assert bad > 0, name


def test_silu_closed_forms(orc):
    """silu(0) = 0 for any up; for large g, silu(g) = g to within e^-g (so
    bf16(silu(g) * 1) = bf16(g)); for very negative g the product underflows
    to zero; and silu(g) - silu(-g) = g exactly, checked through bf16 with
    u = 1 (each side within half a bf16 ulp)."""
    g = np.array([0.0, 0.0, 40.0, 20.5, -120.0, 1.5, -1.5, 3.25, -3.25], np.float32)
    u = np.array([5.0, -7.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0], np.float32)
    y = np.concatenate([g[:, None], u[:, None]], axis=1)
    h, _ = orc.silu_mul(y, 1)
    v = (h[:, 0].astype(np.uint32) << 16).view(np.float32)
    assert v[0] == 0.0 and v[1] == 0.0
    assert v[2] == 40.0 and v[3] == 20.5
    assert v[4] == 0.0
    for a, b, gg in [(5, 6, 1.5), (7, 8, 3.25)]:
        ulp = lambda t: 2.0 ** (np.floor(np.log2(abs(t))) - 7)
        assert abs((float(v[a]) - float(v[b])) - gg) <= (ulp(v[a]) + ulp(v[b])) / 2


def test_silu_mul_gate_up_layout(orc):
    """Gate in columns [0, I), up in [I, 2I): with up = 1, h = bf16(silu(gate));
    with gate = 30 (silu within 1e-12 of 30), h = bf16(30 * up)."""
    I = 4
    gate = np.array([[0.5, -2.0, 3.0, 8.0]], np.float32)
    up = np.array([[1.0, 1.0, 1.0, 1.0]], np.float32)
    h, _ = orc.silu_mul(np.concatenate([gate, up], 1), I)
    for j in range(I):
        assert _bf16_value(h[0, j]) == brute.rnbf16(Fr(_silu_dec(float(gate[0, j]))))
    gate = np.full((1, I), 30.0, np.float32)
    up = np.array([[0.25, -3.0, 7.0, 0.0]], np.float32)
    h, _ = orc.silu_mul(np.concatenate([gate, up], 1), I)
    for j in range(I):
        assert _bf16_value(h[0, j]) == brute.rnbf16(Fr(30 * float(up[0, j])))


# ------------------------------------------------------------ routing softmax

def _softmax_dec(row):
    """Full softmax of one logit row in decimal (finite logits)."""
    d = [Decimal(float(v)) for v in row]
    m = max(d)
    ex = [(v - m).exp() for v in d]
    s = sum(ex)
    return [e / s for e in ex]


def softmax_pin(logits, ids, wts):
    """Every chosen weight must be within one FP32 ulp of the decimal softmax
    probability of its expert over all E logits.  Returns the mismatches."""
    bad = 0
    for t in range(logits.shape[0]):
        p = _softmax_dec(logits[t])
        for s in range(ids.shape[1]):
            want = Fr(p[int(ids[t, s])])
            got = Fr(float(wts[t, s])) if np.isfinite(wts[t, s]) else None
            # one FP32 ulp of the weight, at least the smallest subnormal
            ulp = max(brute.rn32(want) * Fr(1, 2 ** 23), Fr(1, 2 ** 149))
            if got is None or abs(got - want) > ulp:
                bad += 1
    return bad


def _logits():
    rng = np.random.default_rng(77)
    lg = rng.standard_normal((12, 8)).astype(np.float32) * 2
    lg[0] = 0.25                              # all equal: 1/8 each
    lg[1] = [500.0, 499.0, 498.0, 10.0, 0.0, -3.0, 1.0, 2.0]   # overflow without the shift
    lg[2] = [-400.0, -401.0, -399.5, -402.0, -398.0, -410.0, -405.0, -400.5]
    return lg


def test_route_softmax_weights_against_decimal(orc):
    lg = _logits()
    for k in (1, 3, 8):
        d = orc.route(lg, k)
        assert softmax_pin(lg, d["topk_ids"], d["topk_weights"]) == 0
    d = orc.route(lg, 8)
    w = d["topk_weights"].astype(np.float64)
    assert np.all(w[0] == 0.125)
    # all E experts chosen: the weights sum to 1 within 8 FP32 roundings
    assert np.all(np.abs(w.sum(1) - 1.0) <= 8 * 2.0 ** -24)
    # ratios follow exp(l_i - l_j) (two FP32 roundings of each weight)
    for t in range(lg.shape[0]):
        for a, b in [(0, 1), (1, 2), (0, 7)]:
            ia, ib = d["topk_ids"][t, a], d["topk_ids"][t, b]
            if min(w[t, a], w[t, b]) < 2.0 ** -126:
                continue                      # underflowed in FP32: no ratio to check
            want = (Decimal(float(lg[t, ia])) - Decimal(float(lg[t, ib]))).exp()
            got = Decimal(float(w[t, a])) / Decimal(float(w[t, b]))
            assert abs(got / want - 1) <= Decimal(2) ** -22
    # not renormalized: with k < E the chosen weights sum to less than 1
    d3 = orc.route(lg, 3)
    sums = d3["topk_weights"].astype(np.float64).sum(1)
    assert np.all(np.delete(sums, [0, 1]) < 1.0 - 1e-3) and abs(sums[0] - 0.375) < 1e-7


def _planted_route_weights(lg, ids, mode):
    w = np.zeros(ids.shape, np.float32)
    for t in range(lg.shape[0]):
        l = lg[t].astype(np.float64)
        with np.errstate(over="ignore", invalid="ignore"):
            if mode == "renormalized":
                e = np.exp(l - l.max())
                w[t] = e[ids[t]] / e[ids[t]].sum()
            elif mode == "softmin":
                e = np.exp(-(l - l.min()))
                w[t] = e[ids[t]] / e.sum()
            elif mode == "no max shift":
                e = np.exp(l.astype(np.float32))
                w[t] = e[ids[t]] / e.sum()
    return w


@pytest.mark.parametrize("mode", ["renormalized", "softmin", "no max shift"])
def test_softmax_pin_rejects_planted_mistakes(orc, mode):
    lg = _logits()
    d = orc.route(lg, 3)
    assert softmax_pin(lg, d["topk_ids"], _planted_route_weights(lg, d["topk_ids"], mode)) > 0
