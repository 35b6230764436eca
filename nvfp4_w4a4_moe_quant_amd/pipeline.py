"""The rollout hot path as a sequence of C-ABI calls (no arithmetic here).

Dense linear (one GEMM input):
    nvfp4_quantize(X, stats) -> rac_select_residual -> w4a4_grouped_gemm_rac
MoE FFN layer (QUADS rollout: online NVFP4 activations + RAC on every GEMM
input, 4-bit by 4-bit expert GEMMs; arXiv abstract on the mlsanity page and the
blog post's section "Two fixes, on two different sides"):
    moe_route(logits)
    nvfp4_quantize(X, stats) -> rac_select_residual(X)
    w4a4_grouped_gemm_rac(gate/up, gather = routed rows, epilogue SiLU*mul -> H
                          bf16 and max|H|)
    nvfp4_quantize(H, amax_in = max|H|, stats) -> rac_select_residual(H)
    w4a4_grouped_gemm_rac(down) -> Y (FP32, rows in expert order)
    moe_combine(Y, row_of, routing weights) -> token-order output (moe_block)
GraphedMoEBlock captures the whole block once as a HIP graph for fixed
shapes (decode), so a step replays every kernel with no host work per launch.
Weights are quantized once, per expert and projection, by the same
nvfp4_quantize (every engine quantizes the synchronized weights the same way:
blog post, section "The failure mode").
"""
from __future__ import annotations

from typing import Dict, Iterable, NamedTuple, Optional, Tuple

import torch

from . import _lib as L


class QuantWeights(NamedTuple):
    w: L.NVFP4          # codes [G, N, K/2], scales [G, N, K/16], tscale [G]
    N: int
    K: int


def quantize_weights(mats: Iterable[Tuple[int, torch.Tensor]], G: int, N: int, K: int,
                     device) -> QuantWeights:
    """mats yields (group index, W_g [N, K] on any device); each W_g becomes one
    NVFP4 tensor with its own tensor scale."""
    codes = torch.empty((G, N, K // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((G, N, K // 16), dtype=torch.uint8, device=device)
    ts = torch.empty(G, dtype=torch.float32, device=device)
    for g, wg in mats:
        wg = wg.to(device, non_blocking=True)
        q = L.nvfp4_quantize(wg).q
        codes[g].copy_(q.codes)
        scales[g].copy_(q.scales)
        ts[g:g + 1].copy_(q.tscale)
    return QuantWeights(L.NVFP4(codes, scales, ts), N, K)


class GemmInput(NamedTuple):
    qo: L.QuantOut
    rac: Optional[L.RacOut]
    skip_inactive: bool = False
    per_group: bool = False  # per-expert tensor scales (quantize_input_grouped)


# Below this selected fraction of channels, many 16-blocks are likely to hold
# no selected channel, and the GEMM skips their residual MFMAs; above it the
# branch-free residual pass is faster (an inactive block's residual is zero).
SKIP_BELOW_FRACTION = 1.0 / 8


def quantize_input(x: torch.Tensor, n_select: Optional[int],
                   amax_in: Optional[torch.Tensor] = None) -> GemmInput:
    """Online quantization of a GEMM input; n_select None turns RAC off."""
    qo = L.nvfp4_quantize(x, amax_in=amax_in, stats=n_select is not None, channel_max=False)
    rac = L.rac_select_residual(x, qo, n_select) if n_select is not None else None
    skip = n_select is not None and n_select <= SKIP_BELOW_FRACTION * x.shape[1]
    return GemmInput(qo, rac, skip)


def quantize_input_grouped(x: torch.Tensor, offsets: torch.Tensor, total_rows: int,
                           n_select: Optional[int],
                           gather: Optional[torch.Tensor] = None) -> GemmInput:
    """Per-expert RAC: each expert's rows (gathered from x when gather is
    given) are quantized and compensated as their own tensor; the GEMM then
    runs on grouped rows without a gather."""
    qo = L.nvfp4_quantize_grouped(x, offsets, total_rows, gather_rows=gather,
                                  stats=n_select is not None, channel_max=False)
    rac = (L.rac_select_residual_grouped(x, qo, offsets, total_rows, n_select, gather_rows=gather)
           if n_select is not None else None)
    skip = n_select is not None and n_select <= SKIP_BELOW_FRACTION * x.shape[1]
    return GemmInput(qo, rac, skip, True)


def gemm(inp: GemmInput, wq: QuantWeights, offsets: torch.Tensor, total_rows: int, *,
         gather: Optional[torch.Tensor] = None, epilogue: int = L.NVFP4_EPI_F32,
         out_amax: Optional[torch.Tensor] = None) -> torch.Tensor:
    return L.w4a4_grouped_gemm_rac(
        inp.qo.q, wq.w, offsets, N=wq.N, K=wq.K, total_rows=total_rows, gather_rows=gather,
        r=inp.rac.r if inp.rac else None,
        kblock_active=inp.rac.kblock_active if inp.rac else None,
        epilogue=epilogue, out_amax=out_amax, skip_inactive=inp.skip_inactive,
        per_group_scales=inp.per_group)


def dense_forward(x: torch.Tensor, wq: QuantWeights, n_select: Optional[int],
                  offsets: Optional[torch.Tensor] = None) -> Dict:
    """offsets: the one-group offsets [0, rows] (int32, on the device); made
    here when not given (a host-to-device copy, so a graph capture passes
    its own)."""
    rows = x.shape[0]
    if offsets is None:
        offsets = torch.tensor([0, rows], dtype=torch.int32, device=x.device)
    inp = quantize_input(x, n_select)
    y = gemm(inp, wq, offsets, rows)
    return dict(x_in=inp, y=y, offsets=offsets)


def moe_forward(x: torch.Tensor, logits: torch.Tensor, wgu: QuantWeights, wd: QuantWeights,
                topk: int, n_sel_x: Optional[int], n_sel_h: Optional[int],
                per_expert: bool = False) -> Dict:
    """per_expert: RAC (and the activation tensor scales) per expert group
    instead of per GEMM-input tensor; the gate/up input is then quantized per
    expert from the gathered token rows."""
    T = x.shape[0]
    rt = L.moe_route(logits, topk)
    rows = T * topk
    amax_h = torch.zeros(1, dtype=torch.float32, device=x.device)
    if per_expert:
        x_in = quantize_input_grouped(x, rt.expert_offsets, rows, n_sel_x, gather=rt.gather_rows)
        h = gemm(x_in, wgu, rt.expert_offsets, rows, epilogue=L.NVFP4_EPI_SILU_MUL_BF16,
                 out_amax=amax_h)
        h_in = quantize_input_grouped(h, rt.expert_offsets, rows, n_sel_h)
    else:
        x_in = quantize_input(x, n_sel_x)
        h = gemm(x_in, wgu, rt.expert_offsets, rows, gather=rt.gather_rows,
                 epilogue=L.NVFP4_EPI_SILU_MUL_BF16, out_amax=amax_h)
        h_in = quantize_input(h, n_sel_h, amax_in=amax_h)
    y = gemm(h_in, wd, rt.expert_offsets, rows)
    return dict(route=rt, x_in=x_in, h=h, amax_h=amax_h, h_in=h_in, y=y)


def moe_block(x: torch.Tensor, logits: torch.Tensor, wgu: QuantWeights, wd: QuantWeights,
              topk: int, n_sel_x: Optional[int], n_sel_h: Optional[int],
              out_dtype: torch.dtype = torch.bfloat16) -> Dict:
    """The full MoE FFN block: moe_forward, then the weighted combine."""
    d = moe_forward(x, logits, wgu, wd, topk, n_sel_x, n_sel_h)
    d["out"] = L.moe_combine(d["y"], d["route"].row_of, d["route"].topk_weights,
                             out_dtype=out_dtype)
    return d


class GraphedMoEBlock:
    """moe_block captured once as a HIP graph (torch.cuda.CUDAGraph) for fixed
    T, H, E.  The graph reads its inputs from two static buffers: its own, or
    the caller's x [T, H] and logits [T, E] when given (a producer that writes
    the next step's inputs there lets a call replay with no copy).  A call
    copies inputs that live elsewhere into those buffers and replays; the
    returned tensor is the graph's static output, overwritten by the next
    call.  Every kernel of the block only reads device memory the graph owns,
    the static inputs or the caller's weights, and nothing in it is a memset
    node."""

    def __init__(self, wgu: QuantWeights, wd: QuantWeights, topk: int, n_sel_x: Optional[int],
                 n_sel_h: Optional[int], T: int, E: int, x_dtype: torch.dtype, device,
                 out_dtype: torch.dtype = torch.bfloat16, warmup: int = 2,
                 x: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None):
        if x is not None:
            assert x.shape == (T, wgu.K) and x.dtype == x_dtype and x.is_contiguous()
        if logits is not None:
            assert logits.shape == (T, E) and logits.dtype == torch.float32
            assert logits.is_contiguous()
        self.x = x if x is not None else torch.zeros((T, wgu.K), dtype=x_dtype, device=device)
        self.logits = (logits if logits is not None
                       else torch.zeros((T, E), dtype=torch.float32, device=device))
        args = (wgu, wd, topk, n_sel_x, n_sel_h, out_dtype)
        side = torch.cuda.Stream(device)
        side.wait_stream(torch.cuda.current_stream(device))
        with torch.cuda.stream(side):
            for _ in range(warmup):
                moe_block(self.x, self.logits, *args)
        torch.cuda.current_stream(device).wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.out = moe_block(self.x, self.logits, *args)["out"]

    def __call__(self, x: Optional[torch.Tensor] = None,
                 logits: Optional[torch.Tensor] = None) -> torch.Tensor:
        if x is not None and x.data_ptr() != self.x.data_ptr():
            self.x.copy_(x)
        if logits is not None and logits.data_ptr() != self.logits.data_ptr():
            self.logits.copy_(logits)
        self.graph.replay()
        return self.out


class GraphedDense:
    """dense_forward captured once as a HIP graph for fixed [rows, K] (the
    decode shape): a call copies x into the static input and replays every
    kernel of quantize + RAC + GEMM with no host work per launch."""

    def __init__(self, wq: QuantWeights, n_select: Optional[int], rows: int,
                 x_dtype: torch.dtype, device, warmup: int = 2):
        self.x = torch.zeros((rows, wq.K), dtype=x_dtype, device=device)
        self.offsets = torch.tensor([0, rows], dtype=torch.int32, device=device)
        side = torch.cuda.Stream(device)
        side.wait_stream(torch.cuda.current_stream(device))
        with torch.cuda.stream(side):
            for _ in range(warmup):
                dense_forward(self.x, wq, n_select, self.offsets)
        torch.cuda.current_stream(device).wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.y = dense_forward(self.x, wq, n_select, self.offsets)["y"]

    def __call__(self, x: torch.Tensor) -> torch.Tensor:
        self.x.copy_(x)
        self.graph.replay()
        return self.y


class NVFP4WeightFakeQuant(torch.autograd.Function):
    """Trainer-side Asymmetric QAT for one weight matrix: the forward pass
    uses the rollout's NVFP4 quantize-dequantize of W (nvfp4_qdq, bf16 out),
    the backward pass hands the gradient to W unchanged (straight-through).
    Activations stay unquantized (QUADS blog post, section "Two fixes, on two
    different sides")."""

    @staticmethod
    def forward(ctx, w: torch.Tensor) -> torch.Tensor:
        return L.nvfp4_qdq(w.detach().contiguous(), out_dtype=w.dtype)

    @staticmethod
    def backward(ctx, grad: torch.Tensor) -> torch.Tensor:
        return grad
