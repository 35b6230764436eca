"""Helpers shared by the GPU parity tests (device upload, exact and
tolerance comparisons, and the quantize + RAC parity check)."""
import sys

import numpy as np
import torch

from nvfp4_w4a4_moe_quant_amd import _lib as L
from nvfp4_w4a4_moe_quant_amd import datagen as D

DEV = "cuda:0"
REL_F = 1e-5


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(x, dtype):
    x = np.ascontiguousarray(x, np.float32)
    if dtype == "bf16":
        return torch.from_numpy(D.bf16_bits(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(x).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def eq(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    bad = np.flatnonzero(a.ravel() != b.ravel())
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:8]}: " \
                          f"gpu {a.ravel()[bad[:8]]} oracle {b.ravel()[bad[:8]]}"


def rel_frob(gpu, ref):
    ref = np.asarray(ref, np.float64)
    d = np.linalg.norm(np.asarray(gpu, np.float64) - ref)
    n = np.linalg.norm(ref)
    return d / n if n else d


def bf16_ulp_ok(h_gpu_bits, h_ref_bits):
    a = D.bf16_to_f32(np.asarray(h_gpu_bits, np.uint16)).astype(np.float64)
    b = D.bf16_to_f32(np.asarray(h_ref_bits, np.uint16)).astype(np.float64)
    ulp = np.maximum(np.abs(b), 2.0 ** -126) * 2.0 ** -7
    return np.abs(a - b) <= ulp * 1.0001


def check_quant_rac(orc, x, dtype, n_select, amax=None, ldx_pad=0):
    """Quantize + RAC on the GPU and the oracle; everything bit-exact."""
    rows, K = x.shape
    if ldx_pad:
        big = np.zeros((rows, K + ldx_pad), np.float32)
        big[:, :K] = x
        xd = to_dev(big, dtype)[:, :K]
    else:
        xd = to_dev(x, dtype)
    am = None if amax is None else torch.tensor([amax], dtype=torch.float32, device=DEV)
    qo = L.nvfp4_quantize(xd, amax_in=am, stats=True)
    rac = L.rac_select_residual(xd, qo, n_select)
    d = orc.quantize_rac(x, n_select, amax=amax)
    eq(host(qo.q.tscale)[0], np.float32(d["s_t"]), "tensor scale")
    eq(host(qo.q.scales), d["scales"], "block scales")
    eq(host(qo.q.codes), d["codes"], "codes")
    eq(host(qo.channel_score), d["score"], "channel score")
    eq(host(qo.channel_max), d["chmax"], "channel max")
    eq(host(rac.selected), d["selected"], "selected")
    eq(host(rac.kblock_active), d["active"], "kblock_active")
    eq(host(rac.r.tscale)[0], np.float32(d["s_tr"]), "residual tensor scale")
    eq(host(rac.r.scales), d["res_scales"], "residual scales")
    eq(host(rac.r.codes), d["res_codes"], "residual codes")
    # the statistics without the channel maximum (the kernel variant the
    # pipeline runs): the same scores, codes, selection and residual
    qn = L.nvfp4_quantize(xd, amax_in=am, stats=True, channel_max=False)
    assert qn.channel_max is None
    rn = L.rac_select_residual(xd, qn, n_select)
    eq(host(qn.q.codes), d["codes"], "codes (no channel max)")
    eq(host(qn.q.scales), d["scales"], "block scales (no channel max)")
    eq(host(qn.channel_score), d["score"], "channel score (no channel max)")
    eq(host(rn.selected), d["selected"], "selected (no channel max)")
    eq(host(rn.r.codes), d["res_codes"], "residual codes (no channel max)")
    return qo, rac, d
