"""The allocation-free entry point nvfp4_quantize_rac_static (scratch in the
library's per-device array) against the workspace-taking nvfp4_quantize +
rac_select_residual: every output bit-exact, on two calls in a row, the second
with a smaller input (the scratch keeps the first call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

from nvfp4_w4a4_moe_quant_amd import _lib as L
from nvfp4_w4a4_moe_quant_amd import datagen as D
from gpu_util import DEV, eq, host, say, to_dev

pytestmark = pytest.mark.gpu


def _x(seed, rows, K):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 25.0
    return D.bf16_to_f32(D.bf16_bits(x))


def _compare(x, n_sel, amax=None):
    xd = to_dev(x, "bf16")
    am = None if amax is None else torch.tensor([amax], dtype=torch.float32, device=DEV)
    qs, rs = L.nvfp4_quantize_rac_static(xd, n_sel, amax_in=am)
    torch.cuda.synchronize()
    qo = L.nvfp4_quantize(xd, amax_in=am, stats=True)
    ro = L.rac_select_residual(xd, qo, n_sel)
    for name, a, b in [("codes", qs.q.codes, qo.q.codes), ("scales", qs.q.scales, qo.q.scales),
                       ("tensor scale", qs.q.tscale, qo.q.tscale),
                       ("channel score", qs.channel_score, qo.channel_score),
                       ("channel max", qs.channel_max, qo.channel_max),
                       ("selected", rs.selected, ro.selected),
                       ("kblock_active", rs.kblock_active, ro.kblock_active),
                       ("residual codes", rs.r.codes, ro.r.codes),
                       ("residual scales", rs.r.scales, ro.r.scales),
                       ("residual tensor scale", rs.r.tscale, ro.r.tscale)]:
        eq(host(a), host(b), name)
    # channel_max NULL: the same results without the diagnostic maximum
    qn, rn = L.nvfp4_quantize_rac_static(xd, n_sel, amax_in=am, channel_max=False)
    torch.cuda.synchronize()
    assert qn.channel_max is None
    for name, a, b in [("codes", qn.q.codes, qo.q.codes),
                       ("channel score", qn.channel_score, qo.channel_score),
                       ("selected", rn.selected, ro.selected),
                       ("residual codes", rn.r.codes, ro.r.codes),
                       ("residual scales", rn.r.scales, ro.r.scales)]:
        eq(host(a), host(b), name + " (no channel max)")


def test_static_quant_rac_two_calls():
    say("no-alloc quantize+RAC: 4096 x 2048, then 96 x 512")
    _compare(_x(1, 4096, 2048), 1024)
    _compare(_x(2, 96, 512), 256)


def test_static_quant_rac_amax_in_and_max_k():
    say("no-alloc quantize+RAC: amax_in, K = 16384, then a smaller input")
    x = _x(3, 40, 16384)
    _compare(x, 8192, amax=float(np.abs(x).max()))
    _compare(_x(4, 17, 64), 32)


def test_static_quant_rac_rejects_k_beyond_limit():
    say("no-alloc quantize+RAC: K above the scratch limit")
    x = torch.zeros((2, 16384 + 16), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(L.NVFP4Error):
        L.nvfp4_quantize_rac_static(x, 8)
