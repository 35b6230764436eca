"""Pins of the oracle's trainer-side weight fake-quantization (quantize then
dequantize with the rollout's own NVFP4 path; QUADS blog post, section "Two
fixes, on two different sides": Asymmetric QAT fake-quantizes weights only;
arXiv abstract on the mlsanity page: weights align through a shared
quantization-dequantization path).  Checked against the exact rational brute
force, the exact product rounded once, lossless inputs and the error bound."""
from fractions import Fraction as Fr

import numpy as np
import pytest

from nvfp4_w4a4_moe_quant_amd import datagen as D
from oracle import brute


def _bf16_value(bits):
    return D.bf16_to_f32(np.asarray(bits, np.uint16)).astype(np.float64)


def _cases():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((6, 64)).astype(np.float32) * 0.02
    x[0, :16] = 0.0                         # zero block
    x[1, 16:32] *= 1e-4                     # subnormal block scale
    x[2, 7] = 3.0                           # tensor amax from one weight
    x[3] = np.float32(0.0)                  # zero row
    yield x
    yield (rng.standard_normal((3, 32)) * 50).astype(np.float32)


@pytest.mark.parametrize("idx", [0, 1])
def test_qdq_vs_brute(orc, idx):
    x = list(_cases())[idx]
    f, b, s_t = orc.qdq(x)
    bf, bb, bs = brute.qdq([[Fr(float(v)) for v in row] for row in x])
    assert Fr(float(np.float32(s_t))) == bs
    assert [[Fr(float(v)) for v in row] for row in f] == bf
    assert [[Fr(float(v)) for v in row] for row in _bf16_value(b)] == bb


def test_qdq_is_exact_product_rounded_once(orc):
    rng = np.random.default_rng(12)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    codes, scales, s_t = orc.quantize(x)
    f, _, _ = orc.qdq(x)
    st = Fr(float(np.float32(s_t)))
    unpacked = np.stack([codes & 15, codes >> 4], -1).reshape(8, 128)
    for r in range(8):
        for k in range(0, 128, 7):
            exact = brute.value(int(unpacked[r, k])) * brute.E4M3[int(scales[r, k // 16])] * st
            assert Fr(float(f[r, k])) == brute.rn32(exact)


def test_qdq_lossless_inputs(orc):
    """x = g * s_b * s_t with s_t a power of two and each block reaching 6 s_b
    s_t: quantize-dequantize returns x exactly (FP32 and bf16)."""
    rng = np.random.default_rng(13)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    e4m3 = np.array([448.0, 1.0, 1.125, 1.25, 2.0, 3.5, 0.5, 0.0625])
    s_t = 2.0 ** -10
    x = np.zeros((4, 128))
    for r in range(4):
        for b in range(8):
            sb = e4m3[(r + b) % 8]
            g = grid[rng.integers(0, 8, 16)] * rng.choice([-1, 1], 16)
            g[0] = 6.0
            x[r, 16 * b:16 * b + 16] = g * sb * s_t
    # block (0, 0) has s_b = 448 and holds 6 * 448 * s_t: s_t is exactly 2^-10
    x = x.astype(np.float32)
    f, b, st = orc.qdq(x)
    assert st == s_t
    assert np.array_equal(f, x)
    assert np.array_equal(_bf16_value(b), x.astype(np.float64))   # values have <= 8 bits


def test_qdq_error_bound(orc):
    """|qdq(x) - x| is at most half an E2M1 step of the block (times S_b), and
    the bf16 output is the FP32 output rounded to nearest even."""
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    f, b, s_t = orc.qdq(x)
    codes, scales, _ = orc.quantize(x)
    Sb = np.vectorize(orc.e4m3_value)(scales).astype(np.float64) * s_t
    step = np.repeat(Sb, 16, axis=1) * 2.0           # largest E2M1 gap is 2
    assert np.all(np.abs(f.astype(np.float64) - x) <= step / 2 * (1 + 1e-6) + 1e-30)
    ref = np.array([brute.rnbf16(Fr(float(v))) for v in f.ravel()[:2000]], dtype=object)
    got = [Fr(float(v)) for v in _bf16_value(b).ravel()[:2000]]
    assert list(ref) == got
