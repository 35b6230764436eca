"""Pins of the oracle's number formats against closed forms and exhaustive
brute force (E2M1 grid: QUADS blog post, section "The failure mode" -- eight
magnitude levels per sign; E4M3 scales per 16 elements and the FP32 tensor
scale amax/(6*448) are the NVFP4 layout this library implements)."""
from fractions import Fraction as Fr

import numpy as np
import pytest

from oracle import brute


def test_e2m1_decode_is_the_grid(orc):
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    vals = [orc.e2m1_value(c) for c in range(16)]
    assert vals[:8] == grid
    assert vals[8:] == [-g for g in grid]
    # eight distinct magnitudes per sign
    assert len(set(abs(v) for v in vals)) == 8


@pytest.mark.parametrize("byte", range(256))
def test_e4m3_decode_closed_form(orc, byte):
    v = orc.e4m3_value(byte)
    s, e, m = byte >> 7, (byte >> 3) & 15, byte & 7
    if e == 15 and m == 7:
        assert np.isnan(v)
        return
    ref = brute.E4M3[byte & 0x7F]
    assert Fr(abs(v)) == ref and (v < 0) == (s == 1 and ref != 0)


def test_e4m3_landmarks(orc):
    assert orc.e4m3_value(0x7E) == 448.0
    assert orc.e4m3_value(0x38) == 1.0
    assert orc.e4m3_value(0x78) == 256.0
    assert orc.e4m3_value(0x01) == 2.0 ** -9
    assert orc.e4m3_value(0x08) == 2.0 ** -6


def _e4m3_probe_points():
    vals = sorted(set(brute.E4M3.values()))
    pts = []
    for a, b in zip(vals, vals[1:]):
        mid = (a + b) / 2
        m = np.float32(float(mid))
        pts += [float(a), float(b), float(m),
                float(np.nextafter(m, np.float32(0))),
                float(np.nextafter(m, np.float32(1e9)))]
    pts += [448.0, 449.0, 463.9, 464.0, 465.0, 479.0, 480.0, 1e6, 2.0 ** -10,
            2.0 ** -10 * 1.0000001, 2.0 ** -11, 1e-30, 0.0]
    rng = np.random.default_rng(0)
    pts += list(np.exp(rng.uniform(np.log(2.0 ** -12), np.log(600.0), 3000))
                .astype(np.float32).astype(float))
    return pts


def test_e4m3_encode_vs_exhaustive_nearest(orc):
    for p in _e4m3_probe_points():
        p32 = float(np.float32(p))
        assert orc.e4m3_encode(p32) == brute.e4m3_nearest(Fr(p32)), p32


def test_e2m1_encode_tie_table(orc):
    # every tie point resolves to the even grid index
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for t, idx in ties.items():
        assert orc.e2m1_encode(t) == idx
        assert orc.e2m1_encode(-t) == (0 if idx == 0 else 8 | idx)
    assert orc.e2m1_encode(-0.0) == 0 and orc.e2m1_encode(-0.1) == 0
    assert orc.e2m1_encode(7.0) == 7 and orc.e2m1_encode(-1e30) == 15


def test_e2m1_encode_vs_exhaustive_nearest(orc):
    rng = np.random.default_rng(1)
    pts = list(rng.uniform(-8, 8, 4000).astype(np.float32))
    for t in [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]:
        m = np.float32(t)
        pts += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(9))]
    for v in pts:
        v = float(v)
        idx = brute.e2m1_nearest(abs(Fr(v)))
        want = (8 | idx) if (v < 0 and idx) else idx
        assert orc.e2m1_encode(v) == want, v


def test_tensor_scale_correct_rounding(orc):
    rng = np.random.default_rng(2)
    for a in list(rng.exponential(10.0, 500).astype(np.float32)) + [2688.0, 1.0, 0.0]:
        a = float(np.float32(a))
        assert Fr(orc.tensor_scale(a)) == brute.rn32(Fr(a) / 2688)


def test_block_scale_rho_correct_rounding(orc):
    rng = np.random.default_rng(3)
    for _ in range(2000):
        st = float(np.float32(rng.exponential(0.01)))
        ab = float(np.float32(rng.uniform(0, 2688 * st)))
        rho = brute.rn32(Fr(ab) / (6 * Fr(st)))
        assert orc.block_scale_code(ab, st) == brute.e4m3_nearest(rho)


def test_bf16_rne_vs_brute(orc):
    rng = np.random.default_rng(4)
    pts = list(rng.standard_normal(2000) * 10.0 ** rng.integers(-6, 6, 2000))
    # exact ties between bf16 neighbours
    pts += [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(2.0 + 2.0 ** -7), 2.0 ** -130]
    for v in pts:
        want = brute.rnbf16(Fr(v))
        bits = orc.bf16_rne(float(v))
        got = np.array([bits << 16], np.uint32).view(np.float32)[0]
        assert Fr(float(got)) == want, v
