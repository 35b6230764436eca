"""GPU parity of the trainer-side weight fake-quantization (nvfp4_qdq) and of
nvfp4_dequantize, through the C ABI, against the CPU oracle; and the shared
quantization-dequantization path itself: the trainer's fake-quantized weight
equals, bit for bit, what the rollout dequantizes from its own quantized copy
of the same weight (QUADS blog post, section "Two fixes, on two different
sides"; arXiv abstract on the mlsanity page).  All comparisons are exact."""
import numpy as np
import pytest
import torch

from nvfp4_w4a4_moe_quant_amd import _lib as L
from nvfp4_w4a4_moe_quant_amd import datagen as D
from nvfp4_w4a4_moe_quant_amd import pipeline as P

pytestmark = pytest.mark.gpu
from gpu_util import DEV, eq, host, say, to_dev


def _weights(rows, K, dtype, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((rows, K)) * 0.02).astype(np.float32)
    w[:, rng.integers(0, K, 2)] *= 20.0
    if rows > 3:
        w[0, :16] = 0.0                      # zero block
        w[1, 16:32] *= 1e-5                  # subnormal block scale
        w[2] = 0.0                           # zero row
    if dtype == "bf16":
        w = D.bf16_to_f32(D.bf16_bits(w))
    return w


def _bits16(t):
    return host(t.view(torch.int16)).view(np.uint16)


@pytest.mark.parametrize("rows,K,dtype", [(1536, 2048, "bf16"), (2048, 768, "bf16"),
                                          (256, 256, "f32"), (3, 48, "f32"),
                                          (37, 4112, "bf16")])
def test_qdq_parity(orc, rows, K, dtype):
    say(f"qdq {rows}x{K} {dtype}")
    w = _weights(rows, K, dtype, rows + K)
    f_ref, b_ref, _ = orc.qdq(w)
    wd = to_dev(w, dtype)
    eq(host(L.nvfp4_qdq(wd, out_dtype=torch.float32)), f_ref, "qdq fp32")
    eq(_bits16(L.nvfp4_qdq(wd, out_dtype=torch.bfloat16)), b_ref, "qdq bf16")


def test_qdq_amax_in(orc):
    say("qdq with amax_in")
    w = _weights(64, 512, "f32", 5)
    amax = float(np.abs(w).max()) * 3.0
    f_ref, b_ref, _ = orc.qdq(w, amax=amax)
    am = torch.tensor([amax], dtype=torch.float32, device=DEV)
    eq(host(L.nvfp4_qdq(to_dev(w, "f32"), out_dtype=torch.float32, amax_in=am)), f_ref,
       "qdq fp32 amax_in")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_trainer_weight_equals_rollout_dequant(orc, dtype):
    """qdq(W) == dequantize(quantize(W)) on the GPU, and both equal the oracle."""
    say(f"shared qdq path {dtype}")
    w = _weights(768, 2048, dtype, 9)
    wd = to_dev(w, dtype)
    q = L.nvfp4_quantize(wd).q
    for od in (torch.float32, torch.bfloat16):
        a = L.nvfp4_qdq(wd, out_dtype=od)
        b = L.nvfp4_dequantize(q, out_dtype=od)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16) if od == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if od == torch.bfloat16 else b.view(torch.int32))
    codes, scales, s_t = orc.quantize(w)
    eq(host(L.nvfp4_dequantize(L.NVFP4(torch.from_numpy(codes).to(DEV),
                                       torch.from_numpy(scales).to(DEV),
                                       torch.tensor([s_t], dtype=torch.float32, device=DEV)))),
       orc.dequantize(codes, scales, s_t), "dequantize of oracle codes")


def test_fake_quant_autograd_straight_through(orc):
    say("fake-quant autograd")
    w = _weights(128, 256, "bf16", 3)
    wd = to_dev(w, "bf16").requires_grad_(True)
    y = P.NVFP4WeightFakeQuant.apply(wd)
    _, b_ref, _ = orc.qdq(w)
    eq(_bits16(y.detach()), b_ref, "fake-quant forward")
    g = torch.randn_like(y)
    (y * g).sum().backward()
    torch.cuda.synchronize()
    assert torch.equal(wd.grad, g)
