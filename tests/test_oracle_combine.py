"""Pins of the oracle's MoE combine (weighted sum of each token's expert
outputs in slot order, FP32 rounding per operation, optional bf16 output):
the rational brute force with explicit rounding, exact cases, the gather
special case and the FP32 error bound against a float64 sum."""
from fractions import Fraction as Fr

import numpy as np

from nvfp4_w4a4_moe_quant_amd import datagen as D
from oracle import brute


def _case(seed, T=5, k=3, H=24, E=6):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    return logits, rng.standard_normal((T * k, H)).astype(np.float32) * 3.0


def test_combine_vs_brute(orc):
    logits, y = _case(1)
    rt = orc.route(logits, 3)
    f, b = orc.moe_combine(y, rt["row_of"], rt["topk_weights"])
    yf = [[Fr(float(v)) for v in row] for row in y]
    wf = [[Fr(float(v)) for v in row] for row in rt["topk_weights"]]
    bf, bb = brute.moe_combine(yf, rt["row_of"].tolist(), wf)
    assert [[Fr(float(v)) for v in row] for row in f] == bf
    got_b = D.bf16_to_f32(b).astype(np.float64)
    assert [[Fr(float(v)) for v in row] for row in got_b] == bb


def test_combine_exact_cases(orc):
    """Power-of-two weights and small integer outputs sum exactly; k = 1 with
    weight 1 is a gather by row_of."""
    rng = np.random.default_rng(2)
    T, k, H = 7, 4, 16
    y = rng.integers(-50, 50, (T * k, H)).astype(np.float32)
    row_of = rng.permutation(T * k).astype(np.int32).reshape(T, k)
    w = np.array([[0.5, 0.25, 0.125, 0.0625]] * T, np.float32)
    f, _ = orc.moe_combine(y, row_of, w)
    ref = (w[:, :, None].astype(np.float64) * y[row_of].astype(np.float64)).sum(1)
    assert np.array_equal(f.astype(np.float64), ref)
    f1, _ = orc.moe_combine(y, row_of[:, :1], np.ones((T, 1), np.float32))
    assert np.array_equal(f1, y[row_of[:, 0]])


def test_combine_error_bound(orc):
    logits, y = _case(3, T=64, k=8, H=256, E=32)
    rt = orc.route(logits, 8)
    f, _ = orc.moe_combine(y, rt["row_of"], rt["topk_weights"])
    w = rt["topk_weights"].astype(np.float64)
    terms = w[:, :, None] * y[rt["row_of"]].astype(np.float64)
    ref = terms.sum(1)
    bound = 9 * 2.0 ** -24 * np.abs(terms).sum(1)
    assert np.all(np.abs(f - ref) <= bound + 1e-30)
    # the slot order is part of the definition: a reversed order differs somewhere
    fr, _ = orc.moe_combine(y, rt["row_of"][:, ::-1].copy(), rt["topk_weights"][:, ::-1].copy())
    assert not np.array_equal(f, fr)
