"""Exact rational brute force for tiny inputs -- TEST INFRASTRUCTURE ONLY.

A second, independent formulation of the NVFP4 + RAC definitions, used to
pin the C oracle: every value is a ``fractions.Fraction`` and every IEEE
rounding step is an explicit round-to-nearest-even onto the target format
(``rn``).  Nearest-value searches enumerate the representable values
instead of using exponent arithmetic, and sums are exact.  Pure Python,
so only for small shapes.
"""
from __future__ import annotations

from fractions import Fraction as Fr
import math

TWO = Fr(2)


def rn(q: Fr, p: int, emin: int) -> Fr:
    """Round q to the nearest binary float with p significant bits and minimum
    normal exponent emin (gradual underflow below it); ties to even."""
    if q == 0:
        return Fr(0)
    s = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while TWO ** e > a:
        e -= 1
    while TWO ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = TWO ** (e - (p - 1))
    m = a / quantum
    n = math.floor(m)
    frac = m - n
    if frac > Fr(1, 2) or (frac == Fr(1, 2) and n % 2 == 1):
        n += 1
    return s * n * quantum


def rn32(q: Fr) -> Fr:
    return rn(q, 24, -126)


def rn64(q: Fr) -> Fr:
    return rn(q, 53, -1022)


def rnbf16(q: Fr) -> Fr:
    return rn(q, 8, -126)


# --- formats, enumerated from their definitions ----------------------------
E2M1 = [Fr(0), Fr(1, 2), Fr(1), Fr(3, 2), Fr(2), Fr(3), Fr(4), Fr(6)]


def e4m3_table():
    """byte -> value for all finite non-negative OCP E4M3 bytes (0..0x7E)."""
    out = {}
    for b in range(0x7F):
        e, m = b >> 3, b & 7
        if e == 0:
            out[b] = Fr(m, 8) * TWO ** (1 - 7)
        else:
            out[b] = (1 + Fr(m, 8)) * TWO ** (e - 7)
    return out


E4M3 = e4m3_table()


def e4m3_nearest(rho: Fr) -> int:
    """Nearest E4M3 byte by exhaustive search, ties to the even byte,
    saturating at 448."""
    if rho >= 448:
        return 0x7E
    best, bd = None, None
    for b, v in E4M3.items():
        d = abs(v - rho)
        if bd is None or d < bd or (d == bd and b % 2 == 0):
            best, bd = b, d
    return best


def e2m1_nearest(a: Fr) -> int:
    """Nearest grid index by exhaustive search, ties to the even index."""
    if a > 6:
        return 7
    best, bd = None, None
    for i, g in enumerate(E2M1):
        d = abs(g - a)
        if bd is None or d < bd or (d == bd and i % 2 == 0):
            best, bd = i, d
    return best


# --- quantizer ---------------------------------------------------------------
def quantize(x, amax=None, s_t=None):
    """x: list of rows of Fractions (FP32 values).  Returns (codes, scale bytes,
    s_t) with codes as a list of rows of 4-bit ints (unpacked).  s_t, when
    given, is the tensor scale to use (the residual pass uses the main pass's);
    otherwise s_t = RN32(amax / 2688) with amax = max|x| by default."""
    rows, K = len(x), len(x[0])
    if s_t is None:
        if amax is None:
            amax = max((abs(v) for row in x for v in row), default=Fr(0))
        s_t = rn32(Fr(amax) / 2688)
    s_t = Fr(s_t)
    codes, scales = [], []
    for row in x:
        crow, srow = [], []
        for b in range(K // 16):
            blk = row[16 * b:16 * b + 16]
            amax_b = max(abs(v) for v in blk)
            if s_t == 0:
                sc = 0
            else:
                rho = rn32(amax_b / (6 * s_t))  # one correct rounding
                sc = e4m3_nearest(rho)
            sb = E4M3[sc]
            Sb = rn32(sb * s_t)
            rb = rn32(1 / Sb) if Sb > 0 else Fr(0)
            for v in blk:
                q = rn32(v * rb)
                idx = e2m1_nearest(abs(q))
                crow.append((8 | idx) if (q < 0 and idx != 0) else idx)
            srow.append(sc)
        codes.append(crow)
        scales.append(srow)
    return codes, scales, s_t


def value(code: int) -> Fr:
    g = E2M1[code & 7]
    return -g if code & 8 else g


def dequant(code: int, sc: int, s_t: Fr) -> Fr:
    return rn32(rn32(value(code) * E4M3[sc]) * s_t)


def errors(x, codes, scales, s_t):
    return [[rn32(x[r][k] - dequant(codes[r][k], scales[r][k // 16], s_t))
             for k in range(len(x[0]))] for r in range(len(x))]


def channel_scores(e, s_t):
    """score[k] = sum_r floor(|e| * 2^(8 - Es))^2 with q clamped to 2^17-1,
    Es the exponent of s_t written as f * 2^Es, f in [1/2, 1)."""
    if s_t == 0:
        es = 0
    else:
        es = 0
        while TWO ** es <= s_t:
            es += 1
        while TWO ** (es - 1) > s_t:
            es -= 1
    shift = 8 - es
    K = len(e[0])
    score = []
    for k in range(K):
        acc = 0
        for r in range(len(e)):
            q = min(math.floor(abs(e[r][k]) * TWO ** shift), 2 ** 17 - 1)
            acc += q * q
        score.append(acc)
    chmax = [max(abs(e[r][k]) for r in range(len(e))) for k in range(K)]
    return score, chmax


def select(score, n_sel):
    order = sorted(range(len(score)), key=lambda k: (-score[k], k))
    return sorted(order[:n_sel])


def gemm(a, r, w, offsets, gather, N):
    """Exact Y as Fractions.  a/r = (codes rows, scale rows, s_t) unpacked
    lists; w = list over groups of (codes rows [N], scale rows [N], s_t)."""
    total = offsets[-1]
    out = []
    for j in range(total):
        g = max(i for i in range(len(offsets) - 1) if offsets[i] <= j)
        src = gather[j] if gather is not None else j
        wc, wsc, wts = w[g]
        row = []
        for n in range(N):
            def dot(op):
                c, s, _ = op
                return sum(value(c[src][k]) * E4M3[s[src][k // 16]] *
                           value(wc[n][k]) * E4M3[wsc[n][k // 16]]
                           for k in range(len(wc[n])))
            y = a[2] * dot(a)
            if r is not None:
                y += r[2] * dot(r)
            row.append(wts * y)
        out.append(row)
    return out


# --- FP8 W8A8 comparator -------------------------------------------------------
def fp8_quantize_rows(x):
    """Per-row E4M3 quantization: s = RN32(RN64(amax / 448)), r = RN32(RN64(1/s)),
    code = sign(x) | nearest E4M3 of |RN32(x r)| (ties to the even byte,
    saturating).  x: list of rows of Fractions; returns (code rows, scales)."""
    codes, scales = [], []
    for row in x:
        amax = max((abs(v) for v in row), default=Fr(0))
        s = rn32(rn64(Fr(amax) / 448))
        r = rn32(rn64(1 / s)) if s > 0 else Fr(0)
        crow = []
        for v in row:
            q = rn32(v * r)
            crow.append((0x80 if v < 0 else 0) | e4m3_nearest(abs(q)))
        codes.append(crow)
        scales.append(s)
    return codes, scales


def fp8_value(b: int) -> Fr:
    v = E4M3[b & 0x7F]
    return -v if b & 0x80 else v


def fp8_gemm(a_codes, a_scales, w, offsets, gather, N):
    """Exact RN32 of s_a * s_w * sum_k A W as Fractions; w = list over groups of
    (code rows [N], scales [N])."""
    out = []
    for j in range(offsets[-1]):
        g = max(i for i in range(len(offsets) - 1) if offsets[i] <= j)
        src = gather[j] if gather is not None else j
        wc, wsc = w[g]
        row = []
        for n in range(N):
            acc = sum(fp8_value(a_codes[src][k]) * fp8_value(wc[n][k])
                      for k in range(len(wc[n])))
            row.append(rn32(a_scales[src] * wsc[n] * acc))
        out.append(row)
    return out


# --- trainer-side weight fake-quant --------------------------------------------
def qdq(x, amax=None):
    """Quantize then dequantize with exact rationals: (FP32 values as
    Fractions, bf16 values as Fractions, s_t).  FP32 value = RN32(g s_b s_t)
    formed as RN32(RN32(g s_b) s_t); bf16 value = RNbf16 of the FP32 value."""
    codes, scales, s_t = quantize(x, amax)
    f = [[dequant(codes[r][k], scales[r][k // 16], s_t) for k in range(len(x[0]))]
         for r in range(len(x))]
    b = [[rnbf16(v) for v in row] for row in f]
    return f, b, s_t


# --- MoE combine -----------------------------------------------------------------
def moe_combine(y, row_of, w):
    """Exact rationals with explicit FP32 rounding of every product and sum,
    slot order: returns (FP32 rows, bf16 rows) as Fractions."""
    f, b = [], []
    for t in range(len(row_of)):
        row_f = []
        for h in range(len(y[0])):
            acc = Fr(0)
            for s in range(len(row_of[t])):
                acc = rn32(acc + rn32(w[t][s] * y[row_of[t][s]][h]))
            row_f.append(acc)
        f.append(row_f)
        b.append([rnbf16(v) for v in row_f])
    return f, b
