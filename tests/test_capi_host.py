"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/nvfp4rac.h declares, and rejects invalid arguments
with the documented status before enqueuing any work."""
import ctypes
import os
import re

import pytest

from nvfp4_w4a4_moe_quant_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "nvfp4rac.h")
OK, ENULL, ESHAPE, EDTYPE, EALIGN, EWS, EHIP = range(7)


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return L.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(L.EXPORTS)
    for n in names:
        assert hasattr(lib, n)


def test_missing_library_raises():
    with pytest.raises(RuntimeError):
        L.load("/nonexistent/libnvfp4rac.so")


def test_status_strings(lib):
    for s in range(7):
        assert lib.nvfp4_status_string(s)
    assert b"unknown" in lib.nvfp4_status_string(99)


FAKE = ctypes.c_void_p(0x100000)      # 16-byte aligned, never dereferenced
FAKE_MIS = ctypes.c_void_p(0x100004)  # misaligned
FAKE_MIS2 = ctypes.c_void_p(0x100002)  # misaligned even for 4-byte elements


def _q(lib, x=FAKE, dtype=1, rows=4, K=32, ldx=32, codes=FAKE, scales=FAKE, ts=FAKE,
       score=None, chmax=None, ws=FAKE, wsb=1 << 20, amax=None):
    return lib.nvfp4_quantize(x, dtype, rows, K, ldx, amax, codes, scales, ts, score, chmax,
                              ws, wsb, None)


def test_quantize_validation(lib):
    assert _q(lib, x=None) == ENULL
    assert _q(lib, codes=None) == ENULL
    assert _q(lib, chmax=FAKE) == ENULL            # chmax without score
    assert _q(lib, score=FAKE, chmax=FAKE_MIS2) == EALIGN
    assert _q(lib, score=FAKE_MIS) == EALIGN       # int64 scores: 8-byte aligned
    assert _q(lib, dtype=7) == EDTYPE
    assert _q(lib, K=24, ldx=32) == ESHAPE          # K % 16
    assert _q(lib, rows=-1) == ESHAPE
    assert _q(lib, ldx=16) == ESHAPE                # ldx < K
    assert _q(lib, ldx=40, K=32) == EALIGN          # ldx % 16
    assert _q(lib, x=FAKE_MIS) == EALIGN
    assert _q(lib, ws=None) == EWS
    assert _q(lib, wsb=16) == EWS


def test_rac_validation(lib):
    def call(**kw):
        a = dict(x=FAKE, dtype=1, rows=4, K=32, ldx=32, codes=FAKE, scales=FAKE, ts=FAKE,
                 score=FAKE, chmax=FAKE, nsel=16, sel=FAKE, kact=FAKE, rc=FAKE, rs=FAKE,
                 rts=FAKE, ws=FAKE, wsb=1 << 20)
        a.update(kw)
        return lib.rac_select_residual(a["x"], a["dtype"], a["rows"], a["K"], a["ldx"],
                                       a["codes"], a["scales"], a["ts"], a["score"], a["chmax"],
                                       a["nsel"], a["sel"], a["kact"], a["rc"], a["rs"],
                                       a["rts"], a["ws"], a["wsb"], None)
    assert call(score=None) == ENULL
    assert call(nsel=33) == ESHAPE
    assert call(nsel=-1) == ESHAPE
    assert call(K=16 * 1024 * 2, ldx=16 * 1024 * 2) == ESHAPE
    assert call(sel=None) == ENULL
    assert call(rc=FAKE_MIS) == EALIGN
    assert call(scales=None) == ENULL
    assert call(ws=None) == EWS
    assert call(wsb=64) == EWS


def test_static_quant_rac_validation(lib):
    """nvfp4_quantize_rac_static rejects bad arguments before touching the
    device (no scratch lookup, nothing enqueued)."""
    def call(**kw):
        a = dict(x=FAKE, dtype=1, rows=4, K=32, ldx=32, amax=None, codes=FAKE, scales=FAKE,
                 ts=FAKE, score=FAKE, chmax=FAKE, nsel=16, sel=FAKE, kact=FAKE, rc=FAKE, rs=FAKE,
                 rts=FAKE)
        a.update(kw)
        return lib.nvfp4_quantize_rac_static(
            a["x"], a["dtype"], a["rows"], a["K"], a["ldx"], a["amax"], a["codes"], a["scales"],
            a["ts"], a["score"], a["chmax"], a["nsel"], a["sel"], a["kact"], a["rc"], a["rs"],
            a["rts"], None)
    assert call(K=16384 + 16, ldx=16384 + 16) == ESHAPE   # beyond the scratch's limit
    assert call(nsel=33) == ESHAPE
    assert call(chmax=FAKE_MIS2) == EALIGN  # channel_max may be NULL, not misaligned
    assert call(score=None) == ENULL
    assert call(score=None, chmax=None) == ENULL
    assert call(sel=None) == ENULL
    assert call(rc=None) == ENULL
    assert call(x=None) == ENULL
    assert call(dtype=9) == EDTYPE
    assert call(K=24, ldx=32) == ESHAPE
    assert call(codes=FAKE_MIS) == EALIGN
    assert call(rc=FAKE_MIS) == EALIGN


def test_route_validation(lib):
    def call(T=8, E=16, k=2, ws=FAKE, wsb=1 << 20, ids=FAKE):
        return lib.moe_route(FAKE, T, E, k, ids, None, FAKE, FAKE, FAKE, ws, wsb, None)
    assert call(ids=None) == ENULL
    assert lib.moe_route(None, 8, 16, 2, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                         None) == ENULL            # logits needed when T > 0
    assert lib.moe_route(None, 0, 16, 2, None, None, None, None, None, FAKE, 1 << 20,
                         None) == ENULL            # expert_offsets needed even when T == 0
    assert call(k=0) == ESHAPE
    assert call(k=17, E=32) == ESHAPE
    assert call(E=2000) == ESHAPE
    assert call(k=5, E=4) == ESHAPE
    assert call(ws=None) == EWS


def test_gemm_validation(lib):
    def call(**kw):
        a = L.GemmArgs(num_groups=2, N=256, K=256, total_rows=10, group_offsets=FAKE,
                       a_codes=FAKE, a_scales=FAKE, a_tscale=FAKE, w_codes=FAKE,
                       w_scales=FAKE, w_tscale=FAKE, epilogue=0, out=FAKE)
        for k, v in kw.items():
            setattr(a, k, v)
        return lib.w4a4_grouped_gemm_rac(ctypes.byref(a), None, 0, None)
    assert lib.w4a4_grouped_gemm_rac(None, None, 0, None) == ENULL
    assert call(out=None) == ENULL
    assert call(out=None, total_rows=0) == OK       # empty problem: nothing enqueued
    assert call(r_codes=FAKE) == ENULL              # residual codes without scales
    assert call(epilogue=5) == EDTYPE
    assert call(epilogue=2) == EDTYPE               # plain bf16: the FP8 GEMM's only
    assert call(K=200) == ESHAPE                    # K % 128
    assert call(N=96) == ESHAPE                     # N % 128
    assert call(num_groups=0) == ESHAPE
    assert call(a_codes=FAKE_MIS) == EALIGN
    assert call(out=FAKE_MIS) == EALIGN             # every tensor 16-byte aligned
    assert call(kblock_active=ctypes.c_void_p(0x100004), r_codes=FAKE, r_scales=FAKE,
                r_tscale=FAKE) == EALIGN
    assert call(epilogue=1, out_y=ctypes.c_void_p(0x100002)) == EALIGN   # FP32 side output


def test_check_groups(lib):
    """nvfp4_check_groups on host arrays: each rule, and the binding's raise."""
    import numpy as np

    def chk(offs, total, gather=None, src=0):
        o = np.ascontiguousarray(offs, np.int32)
        g = None if gather is None else np.ascontiguousarray(gather, np.int32)
        return lib.nvfp4_check_groups(o.ctypes.data_as(ctypes.c_void_p), o.size - 1, total,
                                      None if g is None else g.ctypes.data_as(ctypes.c_void_p),
                                      src)
    assert chk([0, 3, 3, 7], 7) == OK
    assert chk([0, 3, 3, 7], 7, [0, 1, 2, 4, 4, 3, 0], 5) == OK
    assert chk([0, 3, 3, 7], 7, [0, 1, 2, 5, 4, 3, 0], 5) == ESHAPE   # index == src_rows
    assert chk([0, 3, 3, 7], 7, [0, 1, -1, 4, 4, 3, 0], 5) == ESHAPE  # negative index
    assert chk([0, 4, 3, 7], 7) == ESHAPE            # decreasing
    assert chk([1, 3, 3, 7], 7) == ESHAPE            # does not start at 0
    assert chk([0, 3, 3, 6], 7) == ESHAPE            # does not end at total_rows
    assert chk([0], 0) == ESHAPE                     # no group
    assert lib.nvfp4_check_groups(None, 1, 0, None, 0) == ENULL
    import torch
    with pytest.raises(L.NVFP4Error):
        L.check_groups(torch.tensor([0, 2, 1], dtype=torch.int32), 1)
    with pytest.raises(L.NVFP4Error):
        L.check_groups(torch.tensor([0, 2], dtype=torch.int32), 2,
                       torch.tensor([0, 9], dtype=torch.int32), src_rows=4)
    L.check_groups(torch.tensor([0, 2], dtype=torch.int32), 2,
                   torch.tensor([0, 3], dtype=torch.int32), src_rows=4)


def test_fp8_validation(lib):
    def q(x=FAKE, dt=1, rows=4, K=32, codes=FAKE, sc=FAKE):
        return lib.fp8_quantize_rows(x, dt, rows, K, codes, sc, None)
    assert q(x=None) == ENULL
    assert q(sc=None) == ENULL
    assert q(dt=3) == EDTYPE
    assert q(K=24) == ESHAPE                        # K % 16
    assert q(rows=-1) == ESHAPE
    assert q(x=FAKE_MIS) == EALIGN
    assert q(sc=ctypes.c_void_p(0x100002)) == EALIGN
    assert q(rows=0, x=None) == OK                  # empty: nothing enqueued

    def g(**kw):
        a = L.Fp8GemmArgs(num_groups=2, N=256, K=256, total_rows=10, group_offsets=FAKE,
                          a_codes=FAKE, a_scales=FAKE, w_codes=FAKE, w_scales=FAKE,
                          epilogue=0, out=FAKE)
        for k, v in kw.items():
            setattr(a, k, v)
        return lib.fp8_grouped_gemm(ctypes.byref(a), None)
    assert lib.fp8_grouped_gemm(None, None) == ENULL
    assert g(out=None) == ENULL
    assert g(w_scales=None) == ENULL
    assert g(out=None, total_rows=0) == OK
    assert g(epilogue=5) == EDTYPE
    assert g(epilogue=3) == EDTYPE
    assert g(epilogue=2, out=None, total_rows=0) == OK   # plain bf16 output: accepted
    assert g(K=192) == ESHAPE                       # K % 128
    assert g(N=96) == ESHAPE                        # N % 128
    assert g(num_groups=0) == ESHAPE
    assert g(a_codes=FAKE_MIS) == EALIGN
    assert g(a_scales=ctypes.c_void_p(0x100002)) == EALIGN


def test_qdq_validation(lib):
    def q(x=FAKE, dt=1, rows=4, K=32, ldx=32, od=1, out=FAKE, ts=FAKE, ws=FAKE, wsb=1 << 20,
          amax=None):
        return lib.nvfp4_qdq(x, dt, rows, K, ldx, amax, od, out, ts, ws, wsb, None)
    assert q(out=None) == ENULL
    assert q(ts=None) == ENULL
    assert q(od=4) == EDTYPE
    assert q(K=24, ldx=32) == ESHAPE
    assert q(out=FAKE_MIS) == EALIGN
    assert q(ws=None) == EWS

    def d(codes=FAKE, sc=FAKE, ts=FAKE, rows=4, K=32, od=0, out=FAKE):
        return lib.nvfp4_dequantize(codes, sc, ts, rows, K, od, out, None)
    assert d(codes=None) == ENULL
    assert d(ts=None) == ENULL
    assert d(od=3) == EDTYPE
    assert d(K=24) == ESHAPE
    assert d(rows=-1) == ESHAPE
    assert d(codes=FAKE_MIS) == EALIGN
    assert d(rows=0, codes=None) == OK


def test_combine_validation(lib):
    def c(y=FAKE, ro=FAKE, w=FAKE, T=4, k=2, H=32, od=1, out=FAKE):
        return lib.moe_combine(y, ro, w, T, k, H, od, out, None)
    assert c(y=None) == ENULL
    assert c(w=None) == ENULL
    assert c(od=2) == EDTYPE
    assert c(H=20) == ESHAPE                        # H % 8
    assert c(k=0) == ESHAPE
    assert c(k=17) == ESHAPE
    assert c(out=FAKE_MIS) == EALIGN
    assert c(T=0, y=None) == OK


def test_grouped_rac_validation(lib):
    def q(x=FAKE, dt=1, K=32, ldx=32, off=FAKE, G=2, rows=8, codes=FAKE, ts=FAKE, ws=FAKE,
          wsb=1 << 20, score=None, chmax=None):
        return lib.nvfp4_quantize_grouped(x, dt, K, ldx, off, G, rows, None, codes, FAKE, ts,
                                          score, chmax, ws, wsb, None)
    assert q(off=None) == ENULL
    assert q(ts=None) == ENULL
    assert q(G=0) == ESHAPE
    assert q(G=70000) == ESHAPE
    assert q(K=24, ldx=32) == ESHAPE
    assert q(dt=5) == EDTYPE
    assert q(x=FAKE_MIS) == EALIGN
    assert q(ws=None) == EWS
    assert q(chmax=FAKE) == ENULL                   # channel_max needs channel_score
    assert q(score=FAKE, chmax=FAKE_MIS2) == EALIGN

    def r(nsel=16, K=32, sel=FAKE, ws=FAKE, wsb=1 << 20, kact=FAKE):
        return lib.rac_select_residual_grouped(FAKE, 1, K, K, FAKE, 2, 8, None, FAKE, FAKE, FAKE,
                                               FAKE, nsel, sel, kact, FAKE, FAKE, FAKE, ws, wsb,
                                               None)
    assert r(nsel=33) == ESHAPE
    assert r(sel=None) == ENULL
    assert r(kact=None) == ENULL
    assert r(K=32768) == ESHAPE
    assert r(ws=None) == EWS
    assert r(wsb=16) == EWS
