"""Benchmark of the NVFP4 W4A4 + RAC rollout hot path on one MI355X.

One step = one pass of the whole path over one batch of seeded synthetic
input already resident in HBM:
  MoE workloads:  moe_route -> nvfp4_quantize(X)+rac_select_residual(X) ->
                  gate/up grouped GEMM (RAC fused, SiLU*mul epilogue, max|H|)
                  -> nvfp4_quantize(H)+rac_select_residual(H) -> down grouped
                  GEMM (RAC fused)
  dense workloads: nvfp4_quantize(X)+rac_select_residual(X) -> W4A4 GEMM
Weights are quantized once before timing (offline, as in rollout).

Comparators (timed after the main measurement, same inputs, same weights):
the same path with RAC off (naive NVFP4 W4A4), and an FP8 (E4M3) W8A8 step
with per-row activation and per-channel weight scales -- the format the pages
compare QUADS's rollout throughput against.

Prints one JSON line.  `value` is the algorithmic GEMM TFLOP/s of the whole
step (main + residual passes of every GEMM, residual counted over the active
K-blocks only) divided by the step time; `roofline` covers the dominant
kernel (the gate/up grouped GEMM, or the dense GEMM) timed with HIP events on
the launch stream; `cpu_baseline` times the CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2516.6   # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_FP8_TFLOPS = 5033.2   # MI355X dense fp8 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=5,
                    help="1-5 (default 5: the large MoE FFN layer, E=256, H=7168, I=2048, "
                         "8192 tokens, the largest workload that fits one GPU)")
    ap.add_argument("--no-rac", action="store_true", help="naive W4A4 (RAC off)")
    ap.add_argument("--cpu-baseline", type=int, default=1)
    ap.add_argument("--comparators", type=int, default=1,
                    help="also time RAC-off NVFP4 and FP8 W8A8 steps")
    ap.add_argument("--extras", type=int, default=1,
                    help="MoE workloads: also time the full block (weighted combine), a "
                         "16-token decode call eager vs HIP-graph replay, and the trainer-side "
                         "weight fake-quant; dense workloads: the step eager vs HIP-graph replay")
    ap.add_argument("--fp8-library-reference", type=int, default=1,
                    help="also time the vendor FP8 GEMM (hipBLASLt through torch._scaled_mm, "
                         "row/column scales, bf16 out) on the dense shape of each GEMM: a "
                         "reference point for what an FP8 GEMM reaches on this chip, not a "
                         "part of the path")
    ap.add_argument("--cpu-sample-experts", type=int, default=0,
                    help="experts in the oracle's GEMM sample (0: as many as fit about "
                         "0.6 TFLOP of work: the largest, median and smallest non-empty "
                         "experts, then seeded random ones)")
    ap.add_argument("--decode-leg", type=int, default=1,
                    help="MoE workloads: also time the decode-shaped dense GEMM "
                         "(16x4096x4096, NVFP4 + RAC) against HBM and the launch floor")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path runs on a single MI355X "
              "(no sharding or collectives); rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from nvfp4_w4a4_moe_quant_amd import _lib as L
    from nvfp4_w4a4_moe_quant_amd import datagen as D
    from nvfp4_w4a4_moe_quant_amd import pipeline as P

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = D.WORKLOADS[args.workload]

    def to_dev(a, dtype):
        if dtype == "bf16":
            return torch.from_numpy(D.bf16_bits(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    t_setup = time.time()
    x_np = D.activations(w)
    x = to_dev(x_np, w.x_dtype)
    rac = not args.no_rac
    nsx = w.n_select_x if rac else None
    cmp_ = bool(args.comparators)

    def fp8_buf(G, N, K):
        return L.FP8(torch.empty((G, N, K), dtype=torch.uint8, device=dev),
                     torch.empty((G, N), dtype=torch.float32, device=dev)) if cmp_ else None

    def tee(gen, dtype, f8):
        """Upload each weight matrix once; FP8-quantize it for the comparator
        while the NVFP4 quantizer takes it."""
        for e, m in gen:
            t = to_dev(m, dtype)
            if f8 is not None:
                L.fp8_quantize_rows(t, out=L.FP8(f8.codes[e], f8.scales[e]))
            yield e, t

    if w.kind == "moe":
        lg_np = D.router_logits(w)
        lg = torch.from_numpy(lg_np).to(dev)
        f8_gu, f8_d = fp8_buf(w.E, 2 * w.I, w.H), fp8_buf(w.E, w.H, w.I)
        wgu = P.quantize_weights(tee(D.expert_weights(w, "gate_up"), "bf16", f8_gu),
                                 w.E, 2 * w.I, w.H, dev)
        wd = P.quantize_weights(tee(D.expert_weights(w, "down"), "bf16", f8_d),
                                w.E, w.H, w.I, dev)
        nsh = w.n_select_h if rac else None
        rows = w.T * w.topk
        amax_h = torch.zeros(1, dtype=torch.float32, device=dev)
    else:
        f8_w = fp8_buf(1, w.N, w.K)
        wq = P.quantize_weights(tee([(0, D.dense_weight(w))], w.x_dtype, f8_w), 1, w.N, w.K, dev)
        offs = torch.tensor([0, w.rows], dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    t_setup = time.time() - t_setup

    NEV = 6 if w.kind == "moe" else 3

    def step(ev, nsx=nsx, nsh=nsh if w.kind == "moe" else None):
        if w.kind == "moe":
            amax_h.zero_()  # SiLU*mul epilogue max-combines into it
            ev[0].record()
            rt = L.moe_route(lg, w.topk)
            ev[1].record()
            x_in = P.quantize_input(x, nsx)
            ev[2].record()
            h = P.gemm(x_in, wgu, rt.expert_offsets, rows, gather=rt.gather_rows,
                       epilogue=L.NVFP4_EPI_SILU_MUL_BF16, out_amax=amax_h)
            ev[3].record()
            h_in = P.quantize_input(h, nsh, amax_in=amax_h)
            ev[4].record()
            y = P.gemm(h_in, wd, rt.expert_offsets, rows)
            ev[5].record()
            return x_in, h_in, y, rt
        ev[0].record()
        x_in = P.quantize_input(x, nsx)
        ev[1].record()
        y = P.gemm(x_in, wq, offs, w.rows)
        ev[2].record()
        return x_in, None, y, None

    def step_pe(ev):
        """Per-expert RAC: each expert's gathered rows quantized and
        compensated as their own tensor, GEMMs with per-group scales."""
        amax_h.zero_()
        ev[0].record()
        rt = L.moe_route(lg, w.topk)
        ev[1].record()
        x_in = P.quantize_input_grouped(x, rt.expert_offsets, rows, nsx, gather=rt.gather_rows)
        ev[2].record()
        h = P.gemm(x_in, wgu, rt.expert_offsets, rows, epilogue=L.NVFP4_EPI_SILU_MUL_BF16,
                   out_amax=amax_h)
        ev[3].record()
        h_in = P.quantize_input_grouped(h, rt.expert_offsets, rows, nsh)
        ev[4].record()
        y = P.gemm(h_in, wd, rt.expert_offsets, rows)
        ev[5].record()
        return y

    def step_fp8(ev):
        """FP8 W8A8 comparator: the same routing, per-row E4M3 activations."""
        if w.kind == "moe":
            ev[0].record()
            rt = L.moe_route(lg, w.topk)
            ev[1].record()
            xq = L.fp8_quantize_rows(x)
            ev[2].record()
            h = L.fp8_grouped_gemm(xq, f8_gu, rt.expert_offsets, N=2 * w.I, K=w.H,
                                   total_rows=rows, gather_rows=rt.gather_rows,
                                   epilogue=L.NVFP4_EPI_SILU_MUL_BF16)
            ev[3].record()
            hq = L.fp8_quantize_rows(h)
            ev[4].record()
            y = L.fp8_grouped_gemm(hq, f8_d, rt.expert_offsets, N=w.H, K=w.I, total_rows=rows)
            ev[5].record()
            return y
        ev[0].record()
        xq = L.fp8_quantize_rows(x)
        ev[1].record()
        y = L.fp8_grouped_gemm(xq, f8_w, offs, N=w.N, K=w.K, total_rows=w.rows)
        ev[2].record()
        return y

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(NEV)]

    def timed(fn):
        """W untimed steps, then K steps between synchronizations; returns the
        last step's outputs, ms per step and the per-step events."""
        for _ in range(args.warmup):
            o = fn(mk())
        torch.cuda.synchronize()
        evs = [mk() for _ in range(args.steps)]
        t0 = time.perf_counter()
        for i in range(args.steps):
            o = fn(evs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return o, (t1 - t0) * 1e3 / args.steps, evs

    out, ms_step, evs = timed(step)

    def seg(i, evs=evs):  # mean ms of segment i over the timed steps
        return float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs]))

    x_in, h_in, y, rt = out
    bx = int(x_in.rac.kblock_active.sum().item()) if rac else 0
    res = {}
    if w.kind == "moe":
        bh = int(h_in.rac.kblock_active.sum().item()) if rac else 0
        N_gu, K_gu, N_d, K_d = 2 * w.I, w.H, w.H, w.I
        f_gu = 2.0 * rows * N_gu * (K_gu + 16 * bx)
        f_d = 2.0 * rows * N_d * (K_d + 16 * bh)
        t_route, t_qx, t_gu, t_qh, t_d = (seg(i) for i in range(5))
        flops = f_gu + f_d
        dom = dict(name="w4a4_grouped_gemm_rac gate/up (SiLU*mul epilogue)", flops=f_gu, ms=t_gu)
        qx_bytes = w.T * w.H * 2 + 2 * (w.T * w.H // 2 + w.T * w.H // 16) if rac else \
            w.T * w.H * 2 + w.T * w.H // 2 + w.T * w.H // 16
        qh_bytes = rows * w.I * 2 + (2 if rac else 1) * (rows * w.I // 2 + rows * w.I // 16)
        res.update(
            route_us=t_route * 1e3,
            quant_x=dict(us=t_qx * 1e3, bytes=qx_bytes, gbs=qx_bytes / t_qx / 1e6,
                         frac_hbm=qx_bytes / t_qx / 1e6 / PEAK_HBM_GBS),
            gemm_gate_up=dict(us=t_gu * 1e3, tflops=f_gu / t_gu / 1e9,
                              frac_mfma=f_gu / t_gu / 1e9 / PEAK_F16_TFLOPS,
                              active_kblocks=bx, kblocks=K_gu // 16),
            quant_h=dict(us=t_qh * 1e3, bytes=qh_bytes, gbs=qh_bytes / t_qh / 1e6,
                         frac_hbm=qh_bytes / t_qh / 1e6 / PEAK_HBM_GBS),
            gemm_down=dict(us=t_d * 1e3, tflops=f_d / t_d / 1e9,
                           frac_mfma=f_d / t_d / 1e9 / PEAK_F16_TFLOPS,
                           active_kblocks=bh, kblocks=K_d // 16))
        cnt = np.diff(rt.expert_offsets.cpu().numpy())
        # quantize + RAC of X with cold caches (X is otherwise read from the
        # Infinity Cache after the first step)
        t_qx_cold = cold_ms(lambda: P.quantize_input(x, nsx), dev)
        res["quant_x_cold_cache"] = dict(
            us=t_qx_cold * 1e3, gbs=qx_bytes / t_qx_cold / 1e6,
            frac_hbm=qx_bytes / t_qx_cold / 1e6 / PEAK_HBM_GBS,
            note="512 MiB written before every call, so X comes from HBM")
        res["rows_per_expert"] = dict(min=int(cnt.min()), median=float(np.median(cnt)),
                                      max=int(cnt.max()), empty=int((cnt == 0).sum()))
        cfg = dict(workload=w.name, tokens=w.T, experts=w.E, topk=w.topk, hidden=w.H,
                   intermediate=w.I, gemm_rows=rows, rac=rac, n_select_x=nsx, n_select_h=nsh)
    else:
        f = 2.0 * w.rows * w.N * (w.K + 16 * bx)
        t_q, t_g = seg(0), seg(1)
        flops = f
        # bytes the GEMM must move: W codes + scales, A and R codes + scales,
        # FP32 output (the decode shape is bound by streaming W from HBM)
        nv = lambda r, k: r * k // 2 + r * k // 16
        g_bytes = nv(w.N, w.K) + (2 if rac else 1) * nv(w.rows, w.K) + 4 * w.rows * w.N
        # the eager step is bound by host launch work at this size, so the
        # GEMM's own duration is taken from a graph of back-to-back launches
        t_gk = dense_gemm_replay_ms(P, x_in, wq, offs, w.rows)
        dom = dict(name="w4a4_grouped_gemm_rac dense", flops=f, ms=t_gk, bytes=g_bytes)
        q_bytes = w.rows * w.K * (2 if w.x_dtype == "bf16" else 4) + \
            (2 if rac else 1) * nv(w.rows, w.K)
        res.update(quant_x=dict(us=t_q * 1e3, bytes=q_bytes, gbs=q_bytes / t_q / 1e6),
                   gemm=dict(us=t_g * 1e3, tflops=f / t_g / 1e9, bytes=g_bytes,
                             gbs=g_bytes / t_g / 1e6,
                             frac_hbm=g_bytes / t_g / 1e6 / PEAK_HBM_GBS),
                   gemm_back_to_back=dict(us=t_gk * 1e3, gbs=g_bytes / t_gk / 1e6,
                                          frac_hbm=g_bytes / t_gk / 1e6 / PEAK_HBM_GBS))
        t_cold = cold_ms(lambda: P.gemm(x_in, wq, offs, w.rows), dev)
        res["gemm_cold_cache"] = dict(us=t_cold * 1e3, gbs=g_bytes / t_cold / 1e6,
                                      frac_hbm=g_bytes / t_cold / 1e6 / PEAK_HBM_GBS,
                                      note="512 MiB written between launches, so W comes "
                                           "from HBM, not the 256 MB Infinity Cache")
        cfg = dict(workload=w.name, rows=w.rows, K=w.K, N=w.N, rac=rac, n_select_x=nsx)

    value = flops / (ms_step * 1e-3) / 1e12
    if cmp_:
        res["comparators"] = comparators(w, timed, step, step_fp8, seg, ms_step, rac, NEV,
                                         step_pe if w.kind == "moe" else None)
        if args.fp8_library_reference:
            lib = library_fp8_reference(w, dev)
            f8 = res["comparators"]["fp8_w8a8"]
            ours = ([f8.get("gemm_gate_up_us"), f8.get("gemm_down_us")] if w.kind == "moe"
                    else [f8.get("gemm_us")])
            libs = [v.get("us") for v in lib.values()]
            if None not in ours and None not in libs:
                # the FP8 step with the library's dense GEMM times in place of
                # this library's grouped FP8 GEMMs (no grouping, no gather)
                est = f8["ms_per_step"] + (sum(libs) - sum(ours)) * 1e-3
                lib["ours_over_library"] = [round(a / b, 3) for a, b in zip(ours, libs)]
                lib["fp8_step_ms_with_library_gemms"] = round(est, 4)
                lib["nvfp4_rac_step_over_that"] = round(ms_step / est, 4)
            res["comparators"]["fp8_dense_library_reference"] = lib
    if args.extras and w.kind == "moe":
        res.update(moe_extras(w, dev, x, lg, wgu, wd, nsx, nsh, timed, step, ms_step, NEV))
    if args.extras and w.kind == "dense":
        res["graph"] = dense_graph(w, dev, x, wq, nsx, flops)
    if args.decode_leg and w.kind == "moe":
        res["decode_gemm"] = decode_leg(dev, rac)
    if "bytes" in dom:  # HBM-bound (decode shape): GB/s on the bytes the GEMM must move
        ach = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": dom["name"], "achieved": round(ach, 3),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                    "traffic": measured_traffic(f"gemm_{w.name}")}
    else:
        ach = dom["flops"] / (dom["ms"] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": dom["name"], "achieved": round(ach, 3),
                    "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / PEAK_F16_TFLOPS, 4),
                    "traffic": measured_traffic(f"gemm_gate_up_{w.name}")}
    line = {
        "metric": "NVFP4 W4A4+RAC MoE grouped GEMM TFLOP/s (whole step, algorithmic flops)",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded; bf16 activations, N(0,0.02) weights pre-quantized to NVFP4)",
        "config": cfg,
        "roofline": roofline,
        "breakdown": res,
        "setup_s": round(t_setup, 1),
    }
    if args.cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, x_np, args.cpu_sample_experts, rac)
    print(json.dumps(line), flush=True)


def comparators(w, timed, step, step_fp8, seg, ms_step, rac, nev, step_pe=None):
    """RAC-off NVFP4 and FP8 W8A8 steps on the same inputs and weights."""
    out = {}
    if rac:
        _, ms_naive, ev_n = timed(lambda ev: step(ev, None, None))
        gi = 2 if w.kind == "moe" else 1
        out["nvfp4_rac_off"] = dict(ms_per_step=round(ms_naive, 4),
                                    gemm_first_us=round(seg(gi, ev_n) * 1e3, 2),
                                    rac_step_overhead=round(ms_step / ms_naive - 1.0, 4))
        if step_pe is not None:
            _, ms_pe, ev_p = timed(step_pe)
            out["nvfp4_rac_per_expert"] = dict(
                ms_per_step=round(ms_pe, 4),
                stages_us=[round(seg(i, ev_p) * 1e3, 2) for i in range(nev - 1)],
                stages=["route", "quantize+RAC X per expert (gathered)", "gate/up GEMM",
                        "quantize+RAC H per expert", "down GEMM"])
    _, ms_f8, ev_f = timed(step_fp8)
    if w.kind == "moe":
        rows = w.T * w.topk
        f_gu, f_d = 2.0 * rows * 2 * w.I * w.H, 2.0 * rows * w.H * w.I
        t = [seg(i, ev_f) for i in range(nev - 1)]
        out["fp8_w8a8"] = dict(
            ms_per_step=round(ms_f8, 4), route_us=round(t[0] * 1e3, 2),
            quant_x_us=round(t[1] * 1e3, 2), gemm_gate_up_us=round(t[2] * 1e3, 2),
            gemm_gate_up_tflops=round(f_gu / t[2] / 1e9, 1),
            gemm_gate_up_frac_fp8_mfma=round(f_gu / t[2] / 1e9 / PEAK_FP8_TFLOPS, 4),
            quant_h_us=round(t[3] * 1e3, 2), gemm_down_us=round(t[4] * 1e3, 2),
            gemm_down_tflops=round(f_d / t[4] / 1e9, 1),
            nvfp4_rac_step_over_fp8_step=round(ms_step / ms_f8, 4))
    else:
        f = 2.0 * w.rows * w.N * w.K
        t = [seg(i, ev_f) for i in range(nev - 1)]
        out["fp8_w8a8"] = dict(ms_per_step=round(ms_f8, 4), quant_x_us=round(t[0] * 1e3, 2),
                               gemm_us=round(t[1] * 1e3, 2),
                               gemm_tflops=round(f / t[1] / 1e9, 1),
                               nvfp4_rac_step_over_fp8_step=round(ms_step / ms_f8, 4))
    return out


def moe_extras(w, dev, x, lg, wgu, wd, nsx, nsh, timed, step, ms_step, nev):
    """Full MoE block (with the weighted combine), decode latency eager vs
    HIP-graph replay, and the trainer-side weight fake-quant."""
    import torch

    from nvfp4_w4a4_moe_quant_amd import _lib as L
    from nvfp4_w4a4_moe_quant_amd import pipeline as P

    out = {}
    # full block: the step plus the combine (bf16 out), and the combine alone
    def block_step(ev):
        x_in, h_in, y, rt = step(ev)
        o = L.moe_combine(y, rt.row_of, rt.topk_weights, out_dtype=torch.bfloat16)
        ev[nev - 1].record()
        return y, rt, o
    (y, rt, _), ms_block, _ = timed(block_step)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for _ in range(3):
        L.moe_combine(y, rt.row_of, rt.topk_weights, out_dtype=torch.bfloat16)
    ev[0].record()
    for _ in range(20):
        L.moe_combine(y, rt.row_of, rt.topk_weights, out_dtype=torch.bfloat16)
    ev[1].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) / 20 * 1e3
    rows = w.T * w.topk
    cbytes = rows * w.H * 4 + w.T * w.topk * 8 + w.T * w.H * 2
    out["moe_block"] = dict(ms_per_step_with_combine=round(ms_block, 4),
                            combine_us=round(us, 2), combine_bytes=cbytes,
                            combine_gbs=round(cbytes / us / 1e3, 1),
                            combine_frac_hbm=round(cbytes / us / 1e3 / PEAK_HBM_GBS, 4))
    # decode: 16 tokens through the same layer, one call at a time
    Td = 16
    xd, lgd = x[:Td].contiguous(), lg[:Td].contiguous()
    args = (wgu, wd, w.topk, w.H // 2 if nsx else None, w.I // 2 if nsh else None)
    # the graph reads the step's inputs where the caller keeps them (no copy);
    # fed from other buffers it copies them in first
    g = P.GraphedMoEBlock(*args, T=Td, E=w.E, x_dtype=x.dtype, device=dev, x=xd, logits=lgd)
    xo, lgo = xd.clone(), lgd.clone()
    modes = dict(eager=lambda: P.moe_block(xd, lgd, *args), graph=lambda: g(),
                 graph_cp=lambda: g(xo, lgo))
    for fn in modes.values():
        for _ in range(3):
            fn()
    torch.cuda.synchronize()
    # the modes alternate in blocks of 10 calls (the weight streaming of a
    # call varies by several percent over time); medians of the blocks
    per = {k: [] for k in modes}
    for _ in range(6):
        for k, fn in modes.items():
            t0 = time.perf_counter()
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
            per[k].append((time.perf_counter() - t0) / 10 * 1e6)
    eager_us, graph_us, graph_cp_us = (float(np.median(per[k])) for k in modes)
    out["decode_graph"] = dict(tokens=Td, eager_us_per_call=round(eager_us, 1),
                               graph_us_per_call=round(graph_us, 1),
                               speedup=round(eager_us / graph_us, 3),
                               graph_with_input_copies_us=round(graph_cp_us, 1))
    out["decode_gemms"] = decode_moe_gemms(w, P, L, xd, lgd, args)
    # a larger decode batch: 256 tokens, 8 routed rows per expert on average
    Tb = 256
    xb, lgb = x[:Tb].contiguous(), lg[:Tb].contiguous()
    gb = P.GraphedMoEBlock(*args, T=Tb, E=w.E, x_dtype=x.dtype, device=dev, x=xb, logits=lgb)
    modes_b = dict(eager=lambda: P.moe_block(xb, lgb, *args), graph=lambda: gb())
    for fn in modes_b.values():
        for _ in range(2):
            fn()
    torch.cuda.synchronize()
    per_b = {k: [] for k in modes_b}
    for _ in range(3):
        for k, fn in modes_b.items():
            t0 = time.perf_counter()
            for _ in range(5):
                fn()
            torch.cuda.synchronize()
            per_b[k].append((time.perf_counter() - t0) / 5 * 1e6)
    out["decode_graph_256"] = dict(tokens=Tb,
                                   eager_us_per_call=round(float(np.median(per_b["eager"])), 1),
                                   graph_us_per_call=round(float(np.median(per_b["graph"])), 1))
    del gb
    # trainer-side fake-quant of the gate/up weight bank (bf16 -> bf16)
    wb = (torch.randn((w.E * 2 * w.I, w.H), device=dev) * 0.02).to(torch.bfloat16)
    for _ in range(2):
        L.nvfp4_qdq(wb, out_dtype=torch.bfloat16)
    ev[0].record()
    for _ in range(5):
        L.nvfp4_qdq(wb, out_dtype=torch.bfloat16)
    ev[1].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) / 5 * 1e3
    qbytes = wb.numel() * 4
    out["trainer_qdq"] = dict(shape=list(wb.shape), us=round(us, 1), bytes=qbytes,
                              gbs=round(qbytes / us / 1e3, 1),
                              frac_hbm=round(qbytes / us / 1e3 / PEAK_HBM_GBS, 4))
    del wb
    return out


def decode_leg(dev, rac):
    """The decode-shaped dense linear (16 x 4096 x 4096, bf16 input, NVFP4 + RAC
    of the input, pre-quantized weight): the GEMM's duration from a graph of
    back-to-back launches and with cold caches, against the bytes it must move
    and HBM peak; and two floors measured the same way on this machine: the
    duration of a one-element fill kernel (launch and completion alone) and
    of a 2 MiB device copy (one 16-byte load and store per lane over about as
    many lanes as the GEMM's grid)."""
    import torch

    from nvfp4_w4a4_moe_quant_amd import datagen as D
    from nvfp4_w4a4_moe_quant_amd import pipeline as P

    w = D.WORKLOADS[2]
    x = torch.from_numpy(D.bf16_bits(D.activations(w)).view(np.int16)).to(dev).view(
        torch.bfloat16)
    W = torch.from_numpy(D.bf16_bits(D.dense_weight(w)).view(np.int16)).to(dev).view(
        torch.bfloat16)
    wq = P.quantize_weights([(0, W)], 1, w.N, w.K, dev)
    offs = torch.tensor([0, w.rows], dtype=torch.int32, device=dev)
    nsx = w.n_select_x if rac else None
    x_in = P.quantize_input(x, nsx)
    torch.cuda.synchronize()
    nv = lambda r, k: r * k // 2 + r * k // 16
    g_bytes = nv(w.N, w.K) + (2 if rac else 1) * nv(w.rows, w.K) + 4 * w.rows * w.N
    t_b2b = dense_gemm_replay_ms(P, x_in, wq, offs, w.rows)
    t_cold = cold_ms(lambda: P.gemm(x_in, wq, offs, w.rows), dev)
    one = torch.zeros(1, dtype=torch.float32, device=dev)
    t_fill = replay_ms(lambda: one.fill_(1.0))
    src = torch.ones(2 << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t_copy = replay_ms(lambda: dst.copy_(src))
    gbs = lambda t: g_bytes / t / 1e6
    return dict(workload=w.name, bytes=g_bytes,
                back_to_back=dict(us=round(t_b2b * 1e3, 2), gbs=round(gbs(t_b2b), 1),
                                  frac_hbm=round(gbs(t_b2b) / PEAK_HBM_GBS, 4)),
                cold_cache=dict(us=round(t_cold * 1e3, 2), gbs=round(gbs(t_cold), 1),
                                frac_hbm=round(gbs(t_cold) / PEAK_HBM_GBS, 4)),
                hbm_time_us=round(g_bytes / PEAK_HBM_GBS / 1e3, 2),
                floor_fill_kernel_us=round(t_fill * 1e3, 2),
                floor_2mib_copy_us=round(t_copy * 1e3, 2))


def decode_moe_gemms(w, P, L, xd, lgd, args):
    """The two expert GEMMs of a decode step on their own (graph of back-to-
    back launches, HIP events), priced on the bytes they must move: the NVFP4
    weights (codes, block scales) of the experts the step routes to, the
    routed rows' main and residual codes and scales, and the output.  The
    touched weights (about 1.7 GB for gate/up on the large layer) exceed the
    256 MB Infinity Cache, so every launch streams them from HBM."""
    import torch
    d = P.moe_forward(xd, lgd, *args)
    rt = d["route"]
    rows = xd.shape[0] * w.topk
    offs = rt.expert_offsets.cpu().numpy().astype(np.int64)
    n_exp = int((np.diff(offs) > 0).sum())
    amax = torch.zeros(1, dtype=torch.float32, device=xd.device)
    res = dict(rows=rows, experts_touched=n_exp)
    for name, inp, wq, kw, out_b in (
            ("gate_up", d["x_in"], args[0],
             dict(gather=rt.gather_rows, epilogue=L.NVFP4_EPI_SILU_MUL_BF16, out_amax=amax),
             rows * (args[0].N // 2) * 2),
            ("down", d["h_in"], args[1], {}, rows * args[1].N * 4)):
        N, K = wq.N, wq.K
        passes = 2 if inp.rac is not None else 1
        byt = n_exp * (N * K // 2 + N * K // 16) + passes * rows * (K // 2 + K // 16) + out_b
        ms = replay_ms(lambda: P.gemm(inp, wq, rt.expert_offsets, rows, **kw))
        res[name] = dict(us=round(ms * 1e3, 1), bytes=int(byt),
                         gbs=round(byt / ms / 1e6, 1),
                         frac_hbm=round(byt / ms / 1e6 / PEAK_HBM_GBS, 4))
    return res


def replay_ms(fn, n=20, reps=10):
    """Mean duration of one fn() launch: n launches captured in one HIP graph,
    the replay timed with HIP events on the capture stream."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    b.synchronize()
    return a.elapsed_time(b) / (reps * n)


def dense_graph(w, dev, x, wq, nsx, flops):
    """The dense step (quantize + RAC + GEMM) eager against a HIP-graph
    replay of the same calls: at decode sizes the eager step is bound by host
    launch work, the replay by the kernels."""
    import torch

    from nvfp4_w4a4_moe_quant_amd import pipeline as P

    def per_call(fn, n=200):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n * 1e6
    eager = per_call(lambda: P.dense_forward(x, wq, nsx))
    g = P.GraphedDense(wq, nsx, w.rows, x.dtype, dev)
    graph = per_call(lambda: g(x))
    return dict(eager_us_per_step=round(eager, 2), graph_us_per_step=round(graph, 2),
                graph_tflops=round(flops / graph / 1e6, 3), speedup=round(eager / graph, 3))


def library_fp8_reference(w, dev):
    """hipBLASLt's FP8 GEMM (torch._scaled_mm with per-row and per-column
    scales, bf16 output) on the dense shape rows x N x K of each GEMM of the
    workload: no grouping, no gather, one weight matrix.  Beside it, this
    library's FP8 GEMM on the same operands with the same output type (one
    group, bf16 epilogue): the like-for-like kernel ratio."""
    import torch
    from nvfp4_w4a4_moe_quant_amd import _lib as L
    shapes = ([("gate_up", w.T * w.topk, 2 * w.I, w.H), ("down", w.T * w.topk, w.H, w.I)]
              if w.kind == "moe" else [("gemm", w.rows, w.N, w.K)])
    out = {}
    for name, M, N, K in shapes:
        a = (torch.randn(M, K, device=dev) * 0.5).to(torch.float8_e4m3fn)
        b = (torch.randn(N, K, device=dev) * 0.5).to(torch.float8_e4m3fn)
        sa = torch.ones((M, 1), device=dev)
        sb = torch.ones((1, N), device=dev)
        fn = lambda: torch._scaled_mm(a, b.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)
        try:
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
        except Exception as ex:  # the library may lack a kernel for the shape
            out[name] = dict(shape=[M, N, K], error=repr(ex)[:200])
            continue
        A = L.FP8(a.view(torch.uint8), sa.reshape(M))
        Wt = L.FP8(b.view(torch.uint8).reshape(1, N, K), sb.reshape(1, N))
        off = torch.tensor([0, M], dtype=torch.int32, device=dev)
        yb = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ours = lambda: L.fp8_grouped_gemm(A, Wt, off, N=N, K=K, total_rows=M,
                                          epilogue=L.NVFP4_EPI_BF16, out=yb)
        for _ in range(3):
            ours()
        torch.cuda.synchronize()
        # the two alternate in blocks of 10 calls, so that a drift of the
        # clock over the run falls on both; medians of the blocks
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        per = {"lib": [], "ours": []}
        for _ in range(4):
            for k, f in (("lib", fn), ("ours", ours)):
                e0.record()
                for _ in range(10):
                    f()
                e1.record()
                torch.cuda.synchronize()
                per[k].append(e0.elapsed_time(e1) / 10 * 1e3)
        us, ous = float(np.median(per["lib"])), float(np.median(per["ours"]))
        out[name] = dict(shape=[M, N, K], us=round(us, 1),
                         tflops=round(2.0 * M * N * K / us / 1e6, 1),
                         this_library_dense_bf16_us=round(ous, 1),
                         this_library_dense_over_library=round(ous / us, 3))
    return out


def dense_gemm_replay_ms(P, x_in, wq, offs, rows, n=20, reps=10):
    """Mean duration of one decode-shaped GEMM launch: n launches captured
    in one HIP graph (no host work between them), the replay timed with HIP
    events on the capture stream."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            P.gemm(x_in, wq, offs, rows)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = [P.gemm(x_in, wq, offs, rows) for _ in range(n)]
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    b.synchronize()
    del outs
    return a.elapsed_time(b) / (reps * n)


def cold_ms(fn, dev, n=20):
    """Mean duration of fn()'s GPU work with cold caches: a 512 MiB buffer
    is written before every call (more than the 256 MB Infinity Cache and
    the L2s), and only fn() is timed with HIP events (the fill keeps the
    queue ahead of the host)."""
    import torch
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for a, b in [(None, None)] * 2 + evs:
        scrub.fill_(1)
        if a is not None:
            a.record()
        fn()
        if b is not None:
            b.record()
    torch.cuda.synchronize()
    del scrub
    return float(np.mean([a.elapsed_time(b) for a, b in evs]))


def measured_traffic(summary_name):
    """HBM bytes per launch of the dominant GEMM from the committed counter
    summary profiles/<summary_name>_traffic.json (FETCH_SIZE + WRITE_SIZE,
    each scaled by a copy-kernel calibration), or None when there is none for
    this workload or the GEMM source has changed since the counters were
    taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{summary_name}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, rec["source"])
    if not os.path.exists(src) or \
            hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
        return None
    return int(round(rec["hbm_bytes"]))


def cpu_baseline(w, x_np, n_experts, rac):
    """The oracle, as it stands, on a bounded sample of the same workload:
    quantize + RAC of X, then the gate/up grouped GEMM (main + residual) over
    the routed rows of the first n_experts experts (0: as many experts as
    fit about 0.6 TFLOP of GEMM work, roughly 8 s for the oracle on 16
    threads)."""
    from nvfp4_w4a4_moe_quant_amd import datagen as D
    from oracle import oracle as O

    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t0 = time.perf_counter()
    if w.kind == "moe":
        d = O.quantize_rac(x_np, w.n_select_x)
        rt = O.route(D.router_logits(w), w.topk)
        if n_experts <= 0:
            per = 2.0 * (w.T * w.topk / w.E) * 2 * w.I * w.H * (2 if rac else 1)
            n_experts = max(1, int(0.6e12 // per))
        ex = sample_experts(rt["offsets"], min(n_experts, w.E), seed=1000 + w.seed)
        rows = np.concatenate([rt["gather"][rt["offsets"][e]:rt["offsets"][e + 1]] for e in ex])
        offs = np.concatenate([[0], np.cumsum([rt["offsets"][e + 1] - rt["offsets"][e] for e in ex])])
        wq = [O.quantize(m) for _, m in D.expert_weights(w, "gate_up", ex)]
        wst = (np.stack([q[0] for q in wq]), np.stack([q[1] for q in wq]),
               np.array([q[2] for q in wq], np.float32))
        t1 = time.perf_counter()
        O.grouped_gemm(2 * w.I, w.H, offs.astype(np.int32), rows.astype(np.int32),
                       (d["codes"], d["scales"], d["s_t"]),
                       (d["res_codes"], d["res_scales"], d["s_tr"]) if rac else None, wst)
        t2 = time.perf_counter()
        bx = int(d["active"].sum())
        flops = 2.0 * len(rows) * 2 * w.I * (w.H + (16 * bx if rac else 0))
        sample = (f"oracle quantize+RAC of X [{w.T}x{w.H}] and routing (not in the rate), then "
                  f"the gate/up grouped GEMM over the {len(rows)} routed rows of {len(ex)} of "
                  f"{w.E} experts (largest, median and smallest non-empty, then seeded random: "
                  f"{ex}; main + residual, exact int64 sums)")
    else:
        d = O.quantize_rac(x_np, w.n_select_x)
        c, s, t = O.quantize(D.dense_weight(w))
        t1 = time.perf_counter()
        O.grouped_gemm(w.N, w.K, np.array([0, w.rows], np.int32), None,
                       (d["codes"], d["scales"], d["s_t"]),
                       (d["res_codes"], d["res_scales"], d["s_tr"]) if rac else None,
                       (c[None], s[None], np.array([t], np.float32)))
        t2 = time.perf_counter()
        bx = int(d["active"].sum())
        flops = 2.0 * w.rows * w.N * (w.K + (16 * bx if rac else 0))
        sample = f"oracle quantize+RAC and the full dense GEMM {w.rows}x{w.K}x{w.N}"
    return {"value": round(flops / (t2 - t1) / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "sample": sample, "gemm_s": round(t2 - t1, 2),
            "total_s": round(t2 - t0, 2), "cpu_model": cpu_model(),
            "host_cpus": os.cpu_count()}


def sample_experts(offsets, n, seed):
    """n experts for the oracle's sample: the largest, median and smallest
    non-empty experts by routed rows, then seeded random non-empty ones."""
    cnt = np.diff(np.asarray(offsets))
    nz = np.flatnonzero(cnt)
    order = nz[np.argsort(cnt[nz], kind="stable")]
    pick = [int(order[-1]), int(order[len(order) // 2]), int(order[0])]
    rest = [int(e) for e in np.random.default_rng(seed).permutation(nz) if int(e) not in pick]
    out = []
    for e in pick + rest:
        if e not in out:
            out.append(e)
    return sorted(out[:max(1, n)])


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
