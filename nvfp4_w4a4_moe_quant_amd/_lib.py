"""ctypes binding of libnvfp4rac (the C ABI in include/nvfp4rac.h).

Argument marshalling only: tensors are passed as device pointers, outputs and
workspaces are allocated with torch on the tensors' device, and each call is
enqueued on torch's current HIP stream.  Every computation happens in the
library's HIP kernels; there is no CPU fallback -- importing this module
without the built library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4rac.so")

NVFP4_IN_F32, NVFP4_IN_BF16 = 0, 1
NVFP4_EPI_F32, NVFP4_EPI_SILU_MUL_BF16, NVFP4_EPI_BF16 = 0, 1, 2
NVFP4_GEMM_SKIP_INACTIVE_BLOCKS = 1
NVFP4_GEMM_PER_GROUP_SCALES = 2

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t


class GemmArgs(ctypes.Structure):
    """Mirror of w4a4_gemm_args_t."""
    _fields_ = [
        ("num_groups", _I64), ("N", _I64), ("K", _I64), ("total_rows", _I64),
        ("group_offsets", _P), ("gather_rows", _P),
        ("a_codes", _P), ("a_scales", _P), ("a_tscale", _P),
        ("r_codes", _P), ("r_scales", _P), ("r_tscale", _P),
        ("kblock_active", _P),
        ("w_codes", _P), ("w_scales", _P), ("w_tscale", _P),
        ("epilogue", _I64), ("out", _P), ("out_amax", _P), ("flags", _I64),
        ("out_y", _P),
    ]


class Fp8GemmArgs(ctypes.Structure):
    """Mirror of fp8_gemm_args_t."""
    _fields_ = [
        ("num_groups", _I64), ("N", _I64), ("K", _I64), ("total_rows", _I64),
        ("group_offsets", _P), ("gather_rows", _P),
        ("a_codes", _P), ("a_scales", _P), ("w_codes", _P), ("w_scales", _P),
        ("epilogue", _I64), ("out", _P),
    ]


_SIGS = {
    "nvfp4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "nvfp4_quantize_workspace_size": (_SZ, [_I64, _I64]),
    "nvfp4_quantize": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, _P, _P,
                                      _P, _P, _P, _SZ, _P]),
    "rac_select_residual_workspace_size": (_SZ, [_I64, _I64]),
    "rac_select_residual": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, _P,
                                           _P, _P, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_route_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "moe_route": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "w4a4_grouped_gemm_rac_workspace_size": (_SZ, [ctypes.POINTER(GemmArgs)]),
    "w4a4_grouped_gemm_rac": (ctypes.c_int, [ctypes.POINTER(GemmArgs), _P, _SZ, _P]),
    "moe_combine": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, ctypes.c_int, _P, _P]),
    "nvfp4_quantize_grouped_workspace_size": (_SZ, [_I64, _I64]),
    "nvfp4_quantize_grouped": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _P, _I64, _I64, _P,
                                              _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "rac_select_residual_grouped_workspace_size": (_SZ, [_I64, _I64]),
    "rac_select_residual_grouped": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _P, _I64, _I64,
                                                   _P, _P, _P, _P, _P, _I64, _P, _P, _P, _P, _P,
                                                   _P, _SZ, _P]),
    "nvfp4_qdq_workspace_size": (_SZ, [_I64, _I64]),
    "nvfp4_qdq": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _P, ctypes.c_int, _P, _P,
                                 _P, _SZ, _P]),
    "nvfp4_dequantize": (ctypes.c_int, [_P, _P, _P, _I64, _I64, ctypes.c_int, _P, _P]),
    "fp8_quantize_rows": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _P, _P, _P]),
    "fp8_grouped_gemm": (ctypes.c_int, [ctypes.POINTER(Fp8GemmArgs), _P]),
    "nvfp4_check_groups": (ctypes.c_int, [_P, _I64, _I64, _P, _I64]),
    "nvfp4_quantize_rac_static": (ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, _P,
                                                 _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P]),
}
EXPORTS = tuple(_SIGS)


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -m nvfp4_w4a4_moe_quant_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


class NVFP4Error(RuntimeError):
    pass


def _check(status: int):
    if status != 0:
        raise NVFP4Error(f"status {status}: {lib().nvfp4_status_string(status).decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ws(nbytes: int, dev) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=dev)


def _dtype_code(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return NVFP4_IN_BF16
    if x.dtype == torch.float32:
        return NVFP4_IN_F32
    raise TypeError(f"unsupported dtype {x.dtype}")


class NVFP4(NamedTuple):
    codes: torch.Tensor    # uint8 [rows, K/2]
    scales: torch.Tensor   # uint8 [rows, K/16]
    tscale: torch.Tensor   # float32 [1]


class QuantOut(NamedTuple):
    q: NVFP4
    channel_score: Optional[torch.Tensor]  # int64 [K]
    channel_max: Optional[torch.Tensor]    # float32 [K]


class RacOut(NamedTuple):
    r: NVFP4
    selected: torch.Tensor       # int32 [n_select]
    kblock_active: torch.Tensor  # uint8 [K/16]


class RouteOut(NamedTuple):
    topk_ids: torch.Tensor
    topk_weights: torch.Tensor
    expert_offsets: torch.Tensor
    gather_rows: torch.Tensor
    row_of: torch.Tensor


def nvfp4_quantize(x: torch.Tensor, *, amax_in: Optional[torch.Tensor] = None,
                   stats: bool = False, channel_max: bool = True) -> QuantOut:
    """NVFP4-quantize a 2-D bf16/fp32 device tensor (row stride honoured).
    stats: the RAC channel scores; channel_max (with stats): also max|e| per
    channel, which the selection does not need."""
    assert x.dim() == 2 and x.stride(1) == 1
    rows, K = x.shape
    dev = x.device
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((rows, K // 16), dtype=torch.uint8, device=dev)
    ts = torch.empty(1, dtype=torch.float32, device=dev)
    score = torch.empty(K, dtype=torch.int64, device=dev) if stats else None
    chmax = torch.empty(K, dtype=torch.float32, device=dev) if stats and channel_max else None
    L = lib()
    ws = _ws(L.nvfp4_quantize_workspace_size(rows, K), dev)
    _check(L.nvfp4_quantize(_ptr(x), _dtype_code(x), rows, K, x.stride(0), _ptr(amax_in),
                            _ptr(codes), _ptr(scales), _ptr(ts), _ptr(score), _ptr(chmax),
                            _ptr(ws), ws.numel(), _stream(dev)))
    return QuantOut(NVFP4(codes, scales, ts), score, chmax)


def rac_select_residual(x: torch.Tensor, qo: QuantOut, n_select: int) -> RacOut:
    assert qo.channel_score is not None, "quantize with stats=True first"
    rows, K = x.shape
    dev = x.device
    q = qo.q
    sel = torch.empty(max(n_select, 1), dtype=torch.int32, device=dev)[:n_select]
    kact = torch.empty(K // 16, dtype=torch.uint8, device=dev)
    rc = torch.empty((rows, K // 2), dtype=torch.uint8, device=dev)
    rs = torch.empty((rows, K // 16), dtype=torch.uint8, device=dev)
    rts = torch.empty(1, dtype=torch.float32, device=dev)
    L = lib()
    ws = _ws(L.rac_select_residual_workspace_size(rows, K), dev)
    _check(L.rac_select_residual(_ptr(x), _dtype_code(x), rows, K, x.stride(0), _ptr(q.codes),
                                 _ptr(q.scales), _ptr(q.tscale), _ptr(qo.channel_score),
                                 _ptr(qo.channel_max), n_select, _ptr(sel), _ptr(kact),
                                 _ptr(rc), _ptr(rs), _ptr(rts), _ptr(ws), ws.numel(),
                                 _stream(dev)))
    return RacOut(NVFP4(rc, rs, rts), sel, kact)


def nvfp4_quantize_rac_static(x: torch.Tensor, n_select: int, *,
                              amax_in: Optional[torch.Tensor] = None, channel_max: bool = True):
    """nvfp4_quantize (with statistics) + rac_select_residual in one call that
    takes no workspace (the library's per-device scratch).  Returns
    (QuantOut, RacOut)."""
    assert x.dim() == 2 and x.stride(1) == 1
    rows, K = x.shape
    dev = x.device
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((rows, K // 16), dtype=torch.uint8, device=dev)
    ts = torch.empty(1, dtype=torch.float32, device=dev)
    score = torch.empty(K, dtype=torch.int64, device=dev)
    chmax = torch.empty(K, dtype=torch.float32, device=dev) if channel_max else None
    sel = torch.empty(max(n_select, 1), dtype=torch.int32, device=dev)[:n_select]
    kact = torch.empty(K // 16, dtype=torch.uint8, device=dev)
    rc = torch.empty((rows, K // 2), dtype=torch.uint8, device=dev)
    rs = torch.empty((rows, K // 16), dtype=torch.uint8, device=dev)
    rts = torch.empty(1, dtype=torch.float32, device=dev)
    _check(lib().nvfp4_quantize_rac_static(
        _ptr(x), _dtype_code(x), rows, K, x.stride(0), _ptr(amax_in), _ptr(codes), _ptr(scales),
        _ptr(ts), _ptr(score), _ptr(chmax), n_select, _ptr(sel), _ptr(kact), _ptr(rc), _ptr(rs),
        _ptr(rts), _stream(dev)))
    return (QuantOut(NVFP4(codes, scales, ts), score, chmax),
            RacOut(NVFP4(rc, rs, rts), sel, kact))


def nvfp4_quantize_grouped(x: torch.Tensor, group_offsets: torch.Tensor, total_rows: int, *,
                           gather_rows: Optional[torch.Tensor] = None,
                           stats: bool = False, channel_max: bool = True) -> QuantOut:
    """Per-expert quantization: each group's rows (x[gather[j]] or x[j]) as
    their own tensor.  Returns grouped-order codes/scales, tscale [G] and, with
    stats, score [G, K] and channel max [G, K]."""
    assert x.dim() == 2 and x.stride(1) == 1
    K = x.shape[1]
    G = group_offsets.numel() - 1
    dev = x.device
    codes = torch.empty((total_rows, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((total_rows, K // 16), dtype=torch.uint8, device=dev)
    ts = torch.empty(G, dtype=torch.float32, device=dev)
    score = torch.empty((G, K), dtype=torch.int64, device=dev) if stats else None
    chmax = (torch.empty((G, K), dtype=torch.float32, device=dev) if stats and channel_max
             else None)
    L = lib()
    ws = _ws(L.nvfp4_quantize_grouped_workspace_size(G, K), dev)
    _check(L.nvfp4_quantize_grouped(_ptr(x), _dtype_code(x), K, x.stride(0), _ptr(group_offsets),
                                    G, total_rows, _ptr(gather_rows), _ptr(codes), _ptr(scales),
                                    _ptr(ts), _ptr(score), _ptr(chmax), _ptr(ws), ws.numel(),
                                    _stream(dev)))
    return QuantOut(NVFP4(codes, scales, ts), score, chmax)


def rac_select_residual_grouped(x: torch.Tensor, qo: QuantOut, group_offsets: torch.Tensor,
                                total_rows: int, n_select: int, *,
                                gather_rows: Optional[torch.Tensor] = None) -> RacOut:
    """Per-expert RAC: selection, masks and residual per group."""
    K = x.shape[1]
    G = group_offsets.numel() - 1
    dev = x.device
    sel = torch.empty((G, max(n_select, 1)), dtype=torch.int32, device=dev)
    kact = torch.empty((G, K // 16), dtype=torch.uint8, device=dev)
    rc = torch.empty((total_rows, K // 2), dtype=torch.uint8, device=dev)
    rs = torch.empty((total_rows, K // 16), dtype=torch.uint8, device=dev)
    rts = torch.empty(G, dtype=torch.float32, device=dev)
    L = lib()
    ws = _ws(L.rac_select_residual_grouped_workspace_size(G, K), dev)
    _check(L.rac_select_residual_grouped(
        _ptr(x), _dtype_code(x), K, x.stride(0), _ptr(group_offsets), G, total_rows,
        _ptr(gather_rows), _ptr(qo.q.scales), _ptr(qo.q.tscale), _ptr(qo.channel_score),
        _ptr(qo.channel_max), n_select, _ptr(sel), _ptr(kact), _ptr(rc), _ptr(rs), _ptr(rts),
        _ptr(ws), ws.numel(), _stream(dev)))
    return RacOut(NVFP4(rc, rs, rts), sel[:, :n_select], kact)


def moe_route(logits: torch.Tensor, k: int) -> RouteOut:
    assert logits.dtype == torch.float32 and logits.is_contiguous()
    T, E = logits.shape
    dev = logits.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    gather = torch.empty(T * k, dtype=torch.int32, device=dev)
    row_of = torch.empty((T, k), dtype=torch.int32, device=dev)
    L = lib()
    ws = _ws(L.moe_route_workspace_size(T, E, k), dev)
    _check(L.moe_route(_ptr(logits), T, E, k, _ptr(ids), _ptr(wts), _ptr(off), _ptr(gather),
                       _ptr(row_of), _ptr(ws), ws.numel(), _stream(dev)))
    return RouteOut(ids, wts, off, gather, row_of)


def w4a4_grouped_gemm_rac(a: NVFP4, w: NVFP4, group_offsets: torch.Tensor, *, N: int, K: int,
                          total_rows: int, gather_rows: Optional[torch.Tensor] = None,
                          r: Optional[NVFP4] = None,
                          kblock_active: Optional[torch.Tensor] = None,
                          epilogue: int = NVFP4_EPI_F32,
                          out: Optional[torch.Tensor] = None,
                          out_amax: Optional[torch.Tensor] = None,
                          skip_inactive: bool = False,
                          per_group_scales: bool = False,
                          out_y: Optional[torch.Tensor] = None,
                          validate: bool = False) -> torch.Tensor:
    """w: codes [G, N, K/2], scales [G, N, K/16], tscale [G].  With the SiLU*mul
    epilogue, out_y (float32 [total_rows, N]) also receives the FP32 gate/up
    values before the SiLU.  validate=True checks the offsets and gather
    indices on the host first (check_groups; synchronizes)."""
    dev = a.codes.device
    G = group_offsets.numel() - 1
    if validate:
        check_groups(group_offsets, total_rows, gather_rows, a.codes.shape[0])
    if out is None:
        if epilogue == NVFP4_EPI_F32:
            out = torch.empty((total_rows, N), dtype=torch.float32, device=dev)
        else:
            out = torch.empty((total_rows, N // 2), dtype=torch.bfloat16, device=dev)
    args = GemmArgs(
        num_groups=G, N=N, K=K, total_rows=total_rows,
        group_offsets=_ptr(group_offsets), gather_rows=_ptr(gather_rows),
        a_codes=_ptr(a.codes), a_scales=_ptr(a.scales), a_tscale=_ptr(a.tscale),
        r_codes=_ptr(r.codes if r else None), r_scales=_ptr(r.scales if r else None),
        r_tscale=_ptr(r.tscale if r else None), kblock_active=_ptr(kblock_active),
        w_codes=_ptr(w.codes), w_scales=_ptr(w.scales), w_tscale=_ptr(w.tscale),
        epilogue=epilogue, out=_ptr(out), out_amax=_ptr(out_amax),
        flags=(NVFP4_GEMM_SKIP_INACTIVE_BLOCKS if skip_inactive else 0) |
              (NVFP4_GEMM_PER_GROUP_SCALES if per_group_scales else 0),
        out_y=_ptr(out_y))
    L = lib()
    nbytes = L.w4a4_grouped_gemm_rac_workspace_size(ctypes.byref(args))
    ws = _ws(nbytes, dev) if nbytes else None
    _check(L.w4a4_grouped_gemm_rac(ctypes.byref(args), _ptr(ws), 0 if ws is None else ws.numel(),
                                   _stream(dev)))
    return out


def check_groups(group_offsets: torch.Tensor, total_rows: int,
                 gather_rows: Optional[torch.Tensor] = None, src_rows: int = 0) -> None:
    """Checks the grouped GEMM's offsets and gather indices on host copies
    (nvfp4_check_groups); raises NVFP4Error on a violation.  Synchronizes with
    the device to copy the arrays."""
    import numpy as np
    offs = np.ascontiguousarray(group_offsets.cpu().numpy(), np.int32)
    gat = None if gather_rows is None else \
        np.ascontiguousarray(gather_rows.cpu().numpy(), np.int32)
    if gat is not None and gat.size < total_rows:
        raise NVFP4Error(f"gather_rows has {gat.size} entries, total_rows is {total_rows}")
    _check(lib().nvfp4_check_groups(
        offs.ctypes.data_as(ctypes.c_void_p), offs.size - 1, total_rows,
        None if gat is None else gat.ctypes.data_as(ctypes.c_void_p), src_rows))


def moe_combine(y: torch.Tensor, row_of: torch.Tensor, topk_weights: torch.Tensor, *,
                out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """Token-order output [T, H] from the grouped expert outputs y [rows, H]."""
    T, k = row_of.shape
    H = y.shape[1]
    dev = y.device
    out = torch.empty((T, H), dtype=out_dtype, device=dev)
    _check(lib().moe_combine(_ptr(y), _ptr(row_of), _ptr(topk_weights), T, k, H,
                             _dtype_code(out), _ptr(out), _stream(dev)))
    return out


# ------------------------------------ trainer-side weight fake-quant
def nvfp4_qdq(x: torch.Tensor, *, out_dtype: torch.dtype = torch.bfloat16,
              amax_in: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The rollout's NVFP4 quantize-dequantize of a 2-D bf16/fp32 tensor,
    returned as bf16 or FP32 [rows, K]."""
    assert x.dim() == 2 and x.stride(1) == 1
    rows, K = x.shape
    dev = x.device
    out = torch.empty((rows, K), dtype=out_dtype, device=dev)
    ts = torch.empty(1, dtype=torch.float32, device=dev)
    L = lib()
    ws = _ws(L.nvfp4_qdq_workspace_size(rows, K), dev)
    _check(L.nvfp4_qdq(_ptr(x), _dtype_code(x), rows, K, x.stride(0), _ptr(amax_in),
                       _dtype_code(out), _ptr(out), _ptr(ts), _ptr(ws), ws.numel(),
                       _stream(dev)))
    return out


def nvfp4_dequantize(q: NVFP4, *, out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Dequantized values of an NVFP4 tensor (codes [rows, K/2])."""
    rows, K = q.codes.shape[0], q.codes.shape[1] * 2
    dev = q.codes.device
    out = torch.empty((rows, K), dtype=out_dtype, device=dev)
    _check(lib().nvfp4_dequantize(_ptr(q.codes), _ptr(q.scales), _ptr(q.tscale), rows, K,
                                  _dtype_code(out), _ptr(out), _stream(dev)))
    return out


# ------------------------------------------------- FP8 W8A8 comparator
class FP8(NamedTuple):
    codes: torch.Tensor    # uint8 [rows, K] (E4M3), or [G, N, K] for weights
    scales: torch.Tensor   # float32 [rows], or [G, N]


def fp8_quantize_rows(x: torch.Tensor, out: Optional[FP8] = None) -> FP8:
    """Per-row E4M3 quantization of x [rows, K] (bf16 or FP32)."""
    assert x.dim() == 2 and x.is_contiguous()
    rows, K = x.shape
    dev = x.device
    if out is None:
        out = FP8(torch.empty((rows, K), dtype=torch.uint8, device=dev),
                  torch.empty(rows, dtype=torch.float32, device=dev))
    _check(lib().fp8_quantize_rows(_ptr(x), _dtype_code(x), rows, K, _ptr(out.codes),
                                   _ptr(out.scales), _stream(dev)))
    return out


def fp8_grouped_gemm(a: FP8, w: FP8, group_offsets: torch.Tensor, *, N: int, K: int,
                     total_rows: int, gather_rows: Optional[torch.Tensor] = None,
                     epilogue: int = NVFP4_EPI_F32,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """w: codes [G, N, K], scales [G, N].  epilogue F32, SILU_MUL_BF16 or BF16."""
    dev = a.codes.device
    G = group_offsets.numel() - 1
    if out is None:
        if epilogue == NVFP4_EPI_F32:
            out = torch.empty((total_rows, N), dtype=torch.float32, device=dev)
        elif epilogue == NVFP4_EPI_BF16:
            out = torch.empty((total_rows, N), dtype=torch.bfloat16, device=dev)
        else:
            out = torch.empty((total_rows, N // 2), dtype=torch.bfloat16, device=dev)
    args = Fp8GemmArgs(
        num_groups=G, N=N, K=K, total_rows=total_rows,
        group_offsets=_ptr(group_offsets), gather_rows=_ptr(gather_rows),
        a_codes=_ptr(a.codes), a_scales=_ptr(a.scales),
        w_codes=_ptr(w.codes), w_scales=_ptr(w.scales),
        epilogue=epilogue, out=_ptr(out))
    _check(lib().fp8_grouped_gemm(ctypes.byref(args), _stream(dev)))
    return out
