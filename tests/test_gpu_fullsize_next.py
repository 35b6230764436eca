"""GPU parity of the comparator and follow-on rows at the MoE FFN workload's
full size (128 experts, top-8, 4096 tokens, hidden 2048, intermediate 768),
in the launch configuration the benchmark times: the FP8 W8A8 comparator,
per-expert RAC, the weighted combine and the trainer-side fake-quant.

Bit-exact where the result is integer or byte data; GEMM outputs on sampled
(row, column) pairs that the oracle computes one by one (largest, median,
smallest and random experts, first and last rows).  No oracle input comes
from the GPU: the combine runs on seeded expert outputs."""
import numpy as np
import pytest
import torch

from nvfp4_w4a4_moe_quant_amd import _lib as L
from nvfp4_w4a4_moe_quant_amd import datagen as D
from nvfp4_w4a4_moe_quant_amd import pipeline as P
from gpu_util import DEV, REL_F, bf16_ulp_ok, eq, host, rel_frob, say, to_dev
from test_gpu_fullsize import _sample_experts, _sample_points

pytestmark = pytest.mark.gpu
W = D.WORKLOADS[3]


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _fp8_value_table(orc):
    t = np.array([orc.e4m3_value(b & 0x7F) for b in range(256)], np.float64)
    t[[0x7F, 0xFF]] = 0.0
    return np.where(np.arange(256) & 0x80, -t, t)


def test_full_fp8_comparator(orc):
    """X per-row E4M3 in full; the gate/up FP8 GEMM with gather and SiLU*mul
    on samples, within the FP8 instruction's bound (test_gpu_fp8)."""
    w = W
    say(f"full fp8 comparator {w.name}")
    x, lg = D.activations(w), D.router_logits(w)
    rt_ref = orc.route(lg, w.topk)
    offs = rt_ref["offsets"]
    experts = _sample_experts(offs, 401)
    xq = L.fp8_quantize_rows(to_dev(x, "bf16"))
    ac, as_ = orc.fp8_quantize_rows(x)
    eq(host(xq.codes), ac, "X fp8 codes")
    eq(host(xq.scales), as_, "X row scales")
    # weights: every expert quantized on the GPU as the benchmark does
    wc = torch.empty((w.E, 2 * w.I, w.H), dtype=torch.uint8, device=DEV)
    ws = torch.empty((w.E, 2 * w.I), dtype=torch.float32, device=DEV)
    ref = {}
    for e, m in D.expert_weights(w, "gate_up"):
        L.fp8_quantize_rows(to_dev(m, "bf16"), out=L.FP8(wc[e], ws[e]))
        if e in experts:
            ref[e] = orc.fp8_quantize_rows(D.bf16_to_f32(D.bf16_bits(m)))
    for e in experts:
        eq(host(wc[e]), ref[e][0], f"weight codes e{e}")
    rt = L.moe_route(_t(lg), w.topk)
    h = L.fp8_grouped_gemm(xq, L.FP8(wc, ws), rt.expert_offsets, N=2 * w.I, K=w.H,
                           total_rows=w.T * w.topk, gather_rows=rt.gather_rows,
                           epilogue=L.NVFP4_EPI_SILU_MUL_BF16)
    h_gpu = D.bf16_to_f32(host(h.view(torch.int16)).view(np.uint16)).astype(np.float64)
    val = _fp8_value_table(orc)
    rows, cols = _sample_points(offs, experts, w.I, 402)
    bad = 0
    for e in experts:
        sel = (rows >= offs[e]) & (rows < offs[e + 1])
        rr, cc = rows[sel], cols[sel]
        g_rows = rt_ref["gather"][offs[e]:offs[e + 1]].astype(np.int32)
        off1 = np.array([0, len(g_rows)], np.int32)
        wst = (ref[e][0][None], ref[e][1][None])
        loc = rr - offs[e]
        gate = orc.fp8_grouped_gemm_sample(2 * w.I, w.H, off1, g_rows, (ac, as_), wst, loc, cc)
        up = orc.fp8_grouped_gemm_sample(2 * w.I, w.H, off1, g_rows, (ac, as_), wst, loc,
                                         cc + w.I)
        h_ref, _ = orc.silu_mul(np.stack([gate, up], axis=1).astype(np.float32), 1)
        hr = D.bf16_to_f32(h_ref[:, 0]).astype(np.float64)
        for i, (j, c) in enumerate(zip(g_rows[loc], cc)):
            bnd = []
            for n in (c, c + w.I):
                p = np.abs(val[ac[j]] * val[ref[e][0][n]])
                gm = p.reshape(-1, 8).max(-1)
                ex = np.floor(np.log2(np.where(gm > 0, gm, 1.0)))
                t = (np.where(gm > 0, 7.0 * np.exp2(ex - 13), 0.0).sum()
                     + (w.H / 64 + 4) * 2.0 ** -24 * p.sum())
                bnd.append(float(as_[j]) * float(ref[e][1][n]) * t)
            g, u = float(gate[i]), float(up[i])
            tol = (max(abs(hr[i]), 2.0 ** -126) * 2.0 ** -7 + 1.1 * abs(u) * (bnd[0] + 2e-7 * abs(g))
                   + abs(g / (1 + np.exp(-g))) * (bnd[1] + 2e-7 * abs(u)))
            bad += abs(h_gpu[rr[i], cc[i]] - hr[i]) > tol * 1.0001
    say(f"  fp8 H samples beyond the bound: {bad}/{rows.size}")
    assert bad == 0


def test_full_per_expert_rac(orc):
    """Per-expert quantize + RAC of the routed X (32768 x 2048) in full, and
    the gate/up GEMM with per-group scales on samples."""
    w = W
    rows_total = w.T * w.topk
    say(f"full per-expert rac {w.name}")
    x, lg = D.activations(w), D.router_logits(w)
    rt_ref = orc.route(lg, w.topk)
    offs = rt_ref["offsets"]
    rt = L.moe_route(_t(lg), w.topk)
    inp = P.quantize_input_grouped(to_dev(x, "bf16"), rt.expert_offsets, rows_total,
                                   w.n_select_x, gather=rt.gather_rows)
    d = orc.quantize_rac_grouped(x, offs, rt_ref["gather"], w.n_select_x)
    eq(host(inp.qo.q.tscale), d["s_t"], "tensor scales")
    eq(host(inp.qo.q.codes), d["codes"], "codes")
    eq(host(inp.qo.q.scales), d["scales"], "scales")
    eq(host(inp.rac.selected), d["selected"], "selected")
    eq(host(inp.rac.r.tscale), d["s_tr"], "residual tensor scales")
    eq(host(inp.rac.r.codes), d["res_codes"], "residual codes")
    eq(host(inp.rac.r.scales), d["res_scales"], "residual scales")
    experts = _sample_experts(offs, 403)
    wq = P.quantize_weights(((e, to_dev(m, "bf16")) for e, m in D.expert_weights(w, "gate_up")),
                            w.E, 2 * w.I, w.H, DEV)
    y = P.gemm(inp, wq, rt.expert_offsets, rows_total)   # F32 epilogue: raw gate/up outputs
    y_gpu = host(y)
    rows, cols = _sample_points(offs, experts, 2 * w.I, 404)
    got, want = [], []
    for e, m in D.expert_weights(w, "gate_up", experts):
        c, s, t = orc.quantize(m)
        sel = (rows >= offs[e]) & (rows < offs[e + 1])
        rr, cc = rows[sel], cols[sel]
        j0, j1 = int(offs[e]), int(offs[e + 1])
        a = (d["codes"][j0:j1], d["scales"][j0:j1], float(d["s_t"][e]))
        r = (d["res_codes"][j0:j1], d["res_scales"][j0:j1], float(d["s_tr"][e]))
        want.append(orc.grouped_gemm_sample(2 * w.I, w.H, np.array([0, j1 - j0], np.int32), None,
                                            a, r, (c[None], s[None], np.array([t], np.float32)),
                                            rr - j0, cc))
        got.append(y_gpu[rr, cc])
    err = rel_frob(np.concatenate(got), np.concatenate(want))
    say(f"  per-expert gate/up samples rel frob {err:.3e}")
    assert err <= REL_F


def test_full_combine(orc):
    w = W
    say(f"full combine {w.name}")
    lg = D.router_logits(w)
    rt_ref = orc.route(lg, w.topk)
    y = (np.random.default_rng(405).standard_normal((w.T * w.topk, w.H)) * 0.1).astype(np.float32)
    f_ref, b_ref = orc.moe_combine(y, rt_ref["row_of"], rt_ref["topk_weights"])
    out = L.moe_combine(_t(y), _t(rt_ref["row_of"]), _t(rt_ref["topk_weights"]),
                        out_dtype=torch.bfloat16)
    eq(host(out.view(torch.int16)).view(np.uint16), b_ref, "combine bf16")


def test_full_trainer_qdq(orc):
    w = W
    say(f"full trainer fake-quant {w.name}")
    for e, m in D.expert_weights(w, "gate_up", [0, 63, 127]):
        f_ref, b_ref, _ = orc.qdq(D.bf16_to_f32(D.bf16_bits(m)))
        out = L.nvfp4_qdq(to_dev(m, "bf16"), out_dtype=torch.bfloat16)
        eq(host(out.view(torch.int16)).view(np.uint16), b_ref, f"qdq expert {e}")
