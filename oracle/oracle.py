"""Python face of the CPU oracle (oracle.c) -- TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
module.  It loads ``liboracle.so`` (compiled from oracle.c with gcc, strict
IEEE: -O2 -fno-fast-math -ffp-contract=off) and wraps each function with
NumPy marshalling.  No arithmetic of the method happens in this file.

Parity status: every function is pinned by the CPU tests in
``tests/test_oracle_*.py`` (closed forms, brute force, the worked example,
invariants, and for the SiLU*mul step and the routing weights a 50-digit
``decimal`` evaluation of exp).  The GPU's SiLU uses the hardware exp, so H
is compared with the oracle within one bf16 ulp.

``build_sanitized()`` compiles the same source with AddressSanitizer and
UndefinedBehaviorSanitizer; setting NVFP4RAC_ORACLE_LIB to its path (with
libasan preloaded) makes ``lib()`` load that build instead.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
          "-shared", "-fPIC", "-std=c11"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized() -> str:
    """Compile oracle.c with ASan + UBSan (abort on the first report) into
    liboracle_san.so next to it; returns the path."""
    path = os.path.join(_HERE, "liboracle_san.so")
    flags = [f for f in CFLAGS if f != "-O2"] + [
        "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
        "-fno-sanitize-recover=all"]
    tmp = path + f".tmp{os.getpid()}"
    subprocess.run(["gcc", *flags, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, path)
    return path


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_F = ctypes.c_float

_SIGS = {
    "or_e2m1_value": (ctypes.c_double, [ctypes.c_int]),
    "or_e4m3_value": (ctypes.c_double, [ctypes.c_int]),
    "or_e4m3_encode": (ctypes.c_int, [_F]),
    "or_e2m1_encode": (ctypes.c_int, [_F]),
    "or_tensor_scale": (_F, [_F]),
    "or_block_scale_code": (ctypes.c_int, [_F, _F]),
    "or_dequant": (_F, [ctypes.c_int, ctypes.c_int, _F]),
    "or_score_shift": (ctypes.c_int, [_F]),
    "or_score_term": (_I64, [_F, ctypes.c_int]),
    "or_quantize": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "or_dequantize": (None, [_P, _P, _F, _I64, _I64, _P]),
    "or_channel_stats": (None, [_P, _I64, _I64, _I64, _P, _P, _F, _P, _P]),
    "or_rac_select": (None, [_P, _P, _I64, _I64, _P, _P, _P, _P]),
    "or_rac_residual": (None, [_P, _I64, _I64, _I64, _P, _P, _F, _P, _P, _P, _P, _P]),
    "or_grouped_gemm": (None, [_I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _F,
                               _P, _P, _F, _P, _P, _P, _P, _P, _P, _P, _P]),
    "or_grouped_gemm_sample": (None, [_I64, _I64, _I64, _P, _P, _P, _P, _F,
                                      _P, _P, _F, _P, _P, _P, _I64, _P, _P, _P, _P, _P]),
    "or_quantize_rac_grouped": (None, [_P, _I64, _P, _I64, _P, _I64, _P, _P, _P, _P, _P, _P,
                                       _P, _P, _P, _P]),
    "or_bf16_rne": (ctypes.c_uint16, [ctypes.c_double]),
    "or_silu_mul": (None, [_P, _I64, _I64, _P, _P]),
    "or_route": (None, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "or_qdq": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, _P]),
    "or_moe_combine": (None, [_P, _P, _P, _I64, _I64, _I64, _P, _P]),
    "or_fp8_row_scale": (_F, [_F]),
    "or_fp8_encode": (ctypes.c_int, [_F]),
    "or_fp8_quantize_rows": (None, [_P, _I64, _I64, _I64, _P, _P]),
    "or_fp8_grouped_gemm": (None, [_I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "or_fp8_grouped_gemm_sample": (None, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P,
                                          _I64, _P, _P, _P]),
}


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("NVFP4RAC_ORACLE_LIB")
        if not path:
            path = build()
        l = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ scalars
def e2m1_value(code: int) -> float:
    return lib().or_e2m1_value(code)


def e4m3_value(byte: int) -> float:
    return lib().or_e4m3_value(byte)


def e4m3_encode(rho: float) -> int:
    return lib().or_e4m3_encode(rho)


def e2m1_encode(v: float) -> int:
    return lib().or_e2m1_encode(v)


def tensor_scale(amax: float) -> float:
    return lib().or_tensor_scale(amax)


def block_scale_code(amax_b: float, s_t: float) -> int:
    return lib().or_block_scale_code(amax_b, s_t)


def score_shift(s_t: float) -> int:
    return lib().or_score_shift(s_t)


def bf16_rne(v: float) -> int:
    return lib().or_bf16_rne(v)


# ------------------------------------------------------------ tensor ops
def quantize(x, amax=None):
    """x: float32 [rows, K] -> (codes u8 [rows, K/2], scales u8 [rows, K/16], s_t)."""
    x = _c(x, np.float32)
    rows, K = x.shape
    codes = np.zeros((rows, K // 2), np.uint8)
    scales = np.zeros((rows, K // 16), np.uint8)
    ts = np.zeros(1, np.float32)
    am = None if amax is None else np.array([amax], np.float32)
    rc = lib().or_quantize(_p(x), rows, K, K, _p(am), _p(codes), _p(scales), _p(ts))
    if rc:
        raise ValueError("K must be a multiple of 16")
    return codes, scales, float(ts[0])


def dequantize(codes, scales, s_t):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    rows, K = codes.shape[0], codes.shape[1] * 2
    out = np.zeros((rows, K), np.float32)
    lib().or_dequantize(_p(codes), _p(scales), s_t, rows, K, _p(out))
    return out


def channel_stats(x, codes, scales, s_t):
    x = _c(x, np.float32)
    rows, K = x.shape
    score = np.zeros(K, np.int64)
    chmax = np.zeros(K, np.float32)
    lib().or_channel_stats(_p(x), rows, K, K, _p(_c(codes, np.uint8)),
                           _p(_c(scales, np.uint8)), s_t, _p(score), _p(chmax))
    return score, chmax


def rac_select(score, chmax, n_select):
    score = _c(score, np.int64)
    chmax = _c(chmax, np.float32)
    K = score.shape[0]
    sel = np.zeros(max(n_select, 0), np.int32)
    mask = np.zeros(K, np.uint8)
    active = np.zeros(K // 16, np.uint8)
    am = np.zeros(1, np.float32)
    lib().or_rac_select(_p(score), _p(chmax), K, n_select, _p(sel), _p(mask),
                        _p(active), _p(am))
    return sel, mask, active, float(am[0])


def rac_residual(x, codes, scales, s_t, mask):
    """-> (res_codes, res_scales, s_tr (the residual's tensor scale, = s_t),
    r float32)."""
    x = _c(x, np.float32)
    rows, K = x.shape
    rc = np.zeros((rows, K // 2), np.uint8)
    rs = np.zeros((rows, K // 16), np.uint8)
    ts = np.zeros(1, np.float32)
    r = np.zeros((rows, K), np.float32)
    lib().or_rac_residual(_p(x), rows, K, K, _p(_c(codes, np.uint8)),
                          _p(_c(scales, np.uint8)), s_t, _p(_c(mask, np.uint8)),
                          _p(rc), _p(rs), _p(ts), _p(r))
    return rc, rs, float(ts[0]), r


def _ts(v):
    """A tensor scale: a float (per tensor) or an array [G] (per group)."""
    if np.ndim(v) == 0:
        return float(v), None
    return 0.0, _c(v, np.float32)


def grouped_gemm(N, K, offsets, gather, a, r, w, *, want_sums=False):
    """a = (codes, scales, s_t) of A [src_rows, K]; r likewise or None;
    w = (codes [G, N, K/2], scales [G, N, K/16], s_t[G]).  The activation and
    residual tensor scales are floats, or arrays [G] for per-group scales.
    offsets: int32 [G+1]; gather: int32 [total_rows] or None."""
    offsets = _c(offsets, np.int32)
    G = offsets.shape[0] - 1
    total = int(offsets[-1])
    src_rows = a[0].shape[0]
    gather = None if gather is None else _c(gather, np.int32)
    wc, ws, wt = _c(w[0], np.uint8), _c(w[1], np.uint8), _c(w[2], np.float32)
    assert wc.shape == (G, N, K // 2) and ws.shape == (G, N, K // 16)
    out = np.zeros((total, N), np.float32)
    ms = np.zeros((total, N), np.int64) if want_sums else None
    rsum = np.zeros((total, N), np.int64) if want_sums else None
    rc_ = None if r is None else _c(r[0], np.uint8)
    rs_ = None if r is None else _c(r[1], np.uint8)
    at, atg = _ts(a[2])
    rt, rtg = (0.0, None) if r is None else _ts(r[2])
    lib().or_grouped_gemm(G, N, K, total, src_rows, _p(offsets), _p(gather),
                          _p(_c(a[0], np.uint8)), _p(_c(a[1], np.uint8)), at,
                          _p(rc_), _p(rs_), rt, _p(wc), _p(ws), _p(wt),
                          _p(out), _p(ms), _p(rsum), _p(atg), _p(rtg))
    return (out, ms, rsum) if want_sums else out


def grouped_gemm_sample(N, K, offsets, gather, a, r, w, rows, cols):
    offsets = _c(offsets, np.int32)
    G = offsets.shape[0] - 1
    gather = None if gather is None else _c(gather, np.int32)
    rows = _c(rows, np.int64)
    cols = _c(cols, np.int64)
    out = np.zeros(rows.shape[0], np.float32)
    rc_ = None if r is None else _c(r[0], np.uint8)
    rs_ = None if r is None else _c(r[1], np.uint8)
    at, atg = _ts(a[2])
    rt, rtg = (0.0, None) if r is None else _ts(r[2])
    lib().or_grouped_gemm_sample(G, N, K, _p(offsets), _p(gather),
                                 _p(_c(a[0], np.uint8)), _p(_c(a[1], np.uint8)), at,
                                 _p(rc_), _p(rs_), rt, _p(_c(w[0], np.uint8)),
                                 _p(_c(w[1], np.uint8)), _p(_c(w[2], np.float32)),
                                 rows.shape[0], _p(rows), _p(cols), _p(out), _p(atg), _p(rtg))
    return out


def silu_mul(y, I):
    """y float32 [rows, 2I] (gate first) -> (h bf16 bits u16 [rows, I], max|h|)."""
    y = _c(y, np.float32)
    rows = y.shape[0]
    h = np.zeros((rows, I), np.uint16)
    am = np.zeros(1, np.float32)
    lib().or_silu_mul(_p(y), rows, I, _p(h), _p(am))
    return h, float(am[0])


def route(logits, k):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.zeros((T, k), np.int32)
    wts = np.zeros((T, k), np.float32)
    off = np.zeros(E + 1, np.int32)
    gather = np.zeros(T * k, np.int32)
    row_of = np.zeros((T, k), np.int32)
    lib().or_route(_p(logits), T, E, k, _p(ids), _p(wts), _p(off), _p(gather),
                   _p(row_of))
    return dict(topk_ids=ids, topk_weights=wts, offsets=off, gather=gather,
                row_of=row_of)


def moe_combine(y, row_of, weights):
    """y float32 [rows, H] (grouped order); row_of int32 [T, k]; weights
    float32 [T, k] -> (FP32 [T, H], bf16 bits u16 [T, H])."""
    y = _c(y, np.float32)
    row_of = _c(row_of, np.int32)
    weights = _c(weights, np.float32)
    T, k = row_of.shape
    H = y.shape[1]
    f = np.zeros((T, H), np.float32)
    b = np.zeros((T, H), np.uint16)
    lib().or_moe_combine(_p(y), _p(row_of), _p(weights), T, k, H, _p(f), _p(b))
    return f, b


# ------------------------------------ trainer-side weight fake-quant
def qdq(x, amax=None):
    """x float32 [rows, K] -> (FP32 fake-quant [rows, K], bf16 bits u16
    [rows, K], s_t): the rollout's NVFP4 quantize then dequantize."""
    x = _c(x, np.float32)
    rows, K = x.shape
    f = np.zeros((rows, K), np.float32)
    b = np.zeros((rows, K), np.uint16)
    ts = np.zeros(1, np.float32)
    am = None if amax is None else np.array([amax], np.float32)
    if lib().or_qdq(_p(x), rows, K, _p(am), _p(f), _p(b), _p(ts)):
        raise ValueError("K must be a multiple of 16")
    return f, b, float(ts[0])


# ------------------------------------------------- FP8 W8A8 comparator
def fp8_row_scale(amax: float) -> float:
    return lib().or_fp8_row_scale(amax)


def fp8_encode(v: float) -> int:
    return lib().or_fp8_encode(v)


def fp8_quantize_rows(x):
    """x float32 [rows, K] -> (codes u8 [rows, K] E4M3, scales float32 [rows])."""
    x = _c(x, np.float32)
    rows, K = x.shape
    codes = np.zeros((rows, K), np.uint8)
    scales = np.zeros(rows, np.float32)
    lib().or_fp8_quantize_rows(_p(x), rows, K, K, _p(codes), _p(scales))
    return codes, scales


def fp8_grouped_gemm(N, K, offsets, gather, a, w):
    """a = (codes [src_rows, K], scales [src_rows]); w = (codes [G, N, K],
    scales [G, N]); offsets int32 [G+1]; gather int32 [total_rows] or None."""
    offsets = _c(offsets, np.int32)
    G = offsets.shape[0] - 1
    total = int(offsets[-1])
    gather = None if gather is None else _c(gather, np.int32)
    wc, ws = _c(w[0], np.uint8), _c(w[1], np.float32)
    assert wc.shape == (G, N, K) and ws.shape == (G, N)
    out = np.zeros((total, N), np.float32)
    lib().or_fp8_grouped_gemm(G, N, K, total, _p(offsets), _p(gather),
                              _p(_c(a[0], np.uint8)), _p(_c(a[1], np.float32)),
                              _p(wc), _p(ws), _p(out))
    return out


def fp8_grouped_gemm_sample(N, K, offsets, gather, a, w, rows, cols):
    offsets = _c(offsets, np.int32)
    G = offsets.shape[0] - 1
    gather = None if gather is None else _c(gather, np.int32)
    rows = _c(rows, np.int64)
    cols = _c(cols, np.int64)
    out = np.zeros(rows.shape[0], np.float32)
    lib().or_fp8_grouped_gemm_sample(G, N, K, _p(offsets), _p(gather),
                                     _p(_c(a[0], np.uint8)), _p(_c(a[1], np.float32)),
                                     _p(_c(w[0], np.uint8)), _p(_c(w[1], np.float32)),
                                     rows.shape[0], _p(rows), _p(cols), _p(out))
    return out


def quantize_rac_grouped(x, offsets, gather, n_select):
    """Per-expert RAC: each group's rows (x[gather[j]] or x[j] for grouped row
    j) form their own tensor.  n_select None quantizes only.  Returns a dict
    of grouped-order codes/scales/residual and per-group arrays."""
    x = _c(x, np.float32)
    K = x.shape[1]
    offsets = _c(offsets, np.int32)
    G = offsets.shape[0] - 1
    rows = int(offsets[-1])
    gather = None if gather is None else _c(gather, np.int32)
    rac = n_select is not None
    ns = n_select if rac else 0
    d = dict(codes=np.zeros((rows, K // 2), np.uint8), scales=np.zeros((rows, K // 16), np.uint8),
             s_t=np.zeros(G, np.float32))
    if rac:
        d.update(score=np.zeros((G, K), np.int64), chmax=np.zeros((G, K), np.float32),
                 selected=np.zeros((G, ns), np.int32), active=np.zeros((G, K // 16), np.uint8),
                 res_codes=np.zeros((rows, K // 2), np.uint8),
                 res_scales=np.zeros((rows, K // 16), np.uint8), s_tr=np.zeros(G, np.float32))
    lib().or_quantize_rac_grouped(
        _p(x), K, _p(offsets), G, _p(gather), ns, _p(d["codes"]), _p(d["scales"]),
        _p(d["s_t"]), _p(d.get("score")), _p(d.get("chmax")), _p(d.get("selected")),
        _p(d.get("active")), _p(d.get("res_codes")), _p(d.get("res_scales")), _p(d.get("s_tr")))
    return d


# ------------------------------------------------------------- composites
def quantize_rac(x, n_select, amax=None):
    """Quantize + RAC for one GEMM input; returns a dict of every stage."""
    codes, scales, s_t = quantize(x, amax)
    score, chmax = channel_stats(x, codes, scales, s_t)
    sel, mask, active, amax_r = rac_select(score, chmax, n_select)
    rc, rs, s_tr, r = rac_residual(x, codes, scales, s_t, mask)
    return dict(codes=codes, scales=scales, s_t=s_t, score=score, chmax=chmax,
                selected=sel, mask=mask, active=active, s_tr=s_tr, amax_r=amax_r,
                res_codes=rc, res_scales=rs, r=r)
