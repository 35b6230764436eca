"""Activation error of NVFP4 with and without RAC, per-tensor against
per-expert selection -- TEST INFRASTRUCTURE: a CPU analysis that calls only
the oracle, on the seeded inputs of a MoE workload.

    python -m oracle.rac_error [workload index]   (default 3)

For the gate/up input (the routed token rows, expert-major) and for the
down-projection input (the seeded stand-in for H, in the same grouped
order), it prints the relative Frobenius error ||X - X_hat|| / ||X|| of
  naive      X_hat = dequant(main codes)
  per-tensor X_hat = dequant(main) + dequant(residual), RAC over the whole
             GEMM-input tensor (one selection of n_select channels)
  per-expert the same with each expert's rows as their own tensor
(QUADS blog post, section "Two fixes, on two different sides": RAC corrects
the highest-error activation channels; the pages leave the granularity
open).
"""
import sys

import numpy as np

from nvfp4_w4a4_moe_quant_amd import datagen as D
from oracle import oracle as O


def _deq_grouped(d, off, key_c, key_s, key_t):
    out = np.zeros((int(off[-1]), d[key_c].shape[1] * 2), np.float32)
    for g in range(len(off) - 1):
        j0, j1 = off[g], off[g + 1]
        if j1 > j0:
            out[j0:j1] = O.dequantize(d[key_c][j0:j1], d[key_s][j0:j1], float(d[key_t][g]))
    return out


def errors(x_src, gather, off, n_sel):
    """Relative Frobenius errors over the grouped rows x_src[gather]."""
    xg = x_src[gather] if gather is not None else x_src
    nrm = np.linalg.norm(xg.astype(np.float64))
    rel = lambda xh: float(np.linalg.norm(xg.astype(np.float64) - xh) / nrm)
    # per-tensor: one tensor over the source rows, then gathered
    p = O.quantize_rac(x_src, n_sel)
    main = O.dequantize(p["codes"], p["scales"], p["s_t"]).astype(np.float64)
    res = O.dequantize(p["res_codes"], p["res_scales"], p["s_tr"]).astype(np.float64)
    if gather is not None:
        main, res = main[gather], res[gather]
    # per-expert: each group's gathered rows as their own tensor
    g = O.quantize_rac_grouped(x_src, off, gather, n_sel)
    gm = _deq_grouped(g, off, "codes", "scales", "s_t").astype(np.float64)
    gr = _deq_grouped(g, off, "res_codes", "res_scales", "s_tr").astype(np.float64)
    return dict(naive_per_tensor=rel(main), rac_per_tensor=rel(main + res),
                naive_per_expert=rel(gm), rac_per_expert=rel(gm + gr))


def main(wid=3):
    w = D.WORKLOADS[wid]
    rt = O.route(D.router_logits(w), w.topk)
    x = D.activations(w)
    print(f"workload {w.name}: gate/up input (X gathered, {w.T * w.topk}x{w.H}), "
          f"n_select {w.n_select_x}")
    for k, v in errors(x, rt["gather"], rt["offsets"], w.n_select_x).items():
        print(f"  {k:18s} {v:.5f}")
    h = D.hidden_like(w, w.T * w.topk)
    print(f"down input (seeded H stand-in, {w.T * w.topk}x{w.I}), n_select {w.n_select_h}")
    for k, v in errors(h, None, rt["offsets"], w.n_select_h).items():
        print(f"  {k:18s} {v:.5f}")


if __name__ == "__main__":
    main(int(sys.argv[1]) if len(sys.argv) > 1 else 3)
