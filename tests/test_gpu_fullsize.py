"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (same shapes, grids and call sequence).

Quantizer, RAC and routing are compared in full (bit-exact).  GEMM outputs are
compared on sampled (row, column) pairs that the oracle computes one by one:
the largest, median and smallest non-empty experts, each expert's first and
last rows (ragged tails), plus seeded random picks.  The down projection runs
on a seeded H-like input (the same bytes on both sides), never on the GPU's H.
For the 256-expert workload, only the sampled experts get their seeded
weights; the others reuse expert 0's quantized weights so that the launch is
the same without drawing 11G normals."""
import numpy as np
import pytest
import torch

from nvfp4_w4a4_moe_quant_amd import _lib as L
from nvfp4_w4a4_moe_quant_amd import datagen as D
from nvfp4_w4a4_moe_quant_amd import pipeline as P
from gpu_util import (DEV, REL_F, bf16_ulp_ok, check_quant_rac, eq, host, rel_frob, say,
                      to_dev)

pytestmark = pytest.mark.gpu


def test_full_decode_dense(orc):
    w = D.WORKLOADS[2]
    say(f"full {w.name}")
    x, W = D.activations(w), D.dense_weight(w)
    wq = P.quantize_weights([(0, to_dev(W, "bf16"))], 1, w.N, w.K, DEV)
    c, s, t = orc.quantize(W)
    eq(host(wq.w.codes[0]), c, "weight codes")
    eq(host(wq.w.scales[0]), s, "weight scales")
    _, _, d = check_quant_rac(orc, x, "bf16", w.n_select_x)
    out = P.dense_forward(to_dev(x, "bf16"), wq, w.n_select_x)
    y_ref = orc.grouped_gemm(w.N, w.K, np.array([0, w.rows], np.int32), None,
                             (d["codes"], d["scales"], d["s_t"]),
                             (d["res_codes"], d["res_scales"], d["s_tr"]),
                             (c[None], s[None], np.array([t], np.float32)))
    err = rel_frob(host(out["y"]), y_ref)
    say(f"  rel frob {err:.3e}")
    assert err <= REL_F


@pytest.mark.parametrize("wid", [3, 4, 5])
def test_full_quant_rac_x(orc, wid):
    w = D.WORKLOADS[wid]
    say(f"full X quant+rac {w.name}")
    check_quant_rac(orc, D.activations(w), "bf16", w.n_select_x)


@pytest.mark.parametrize("wid", [3, 4, 5])
def test_full_quant_rac_h(orc, wid):
    w = D.WORKLOADS[wid]
    rows = w.T * w.topk
    say(f"full H quant+rac {w.name} rows={rows}")
    h = D.hidden_like(w, rows)
    check_quant_rac(orc, h, "bf16", w.n_select_h, amax=float(np.abs(h).max()))


@pytest.mark.parametrize("wid", [3, 4, 5])
def test_full_route(orc, wid):
    w = D.WORKLOADS[wid]
    say(f"full route {w.name}")
    lg = D.router_logits(w)
    rt = L.moe_route(torch.from_numpy(lg).to(DEV), w.topk)
    d = orc.route(lg, w.topk)
    eq(host(rt.topk_ids), d["topk_ids"], "topk ids")
    eq(host(rt.expert_offsets), d["offsets"], "offsets")
    eq(host(rt.gather_rows), d["gather"], "gather")
    eq(host(rt.row_of), d["row_of"], "row_of")
    cnt = np.diff(d["offsets"])
    say(f"  rows per expert min {cnt.min()} median {np.median(cnt)} max {cnt.max()} "
        f"empty {(cnt == 0).sum()}")
    if w.routing == "zipf":
        assert (cnt == 0).sum() >= w.n_empty


def _sample_experts(offsets, seed, n_random=3):
    cnt = np.diff(offsets)
    nz = np.flatnonzero(cnt)
    order = nz[np.argsort(cnt[nz], kind="stable")]
    pick = {int(order[-1]), int(order[len(order) // 2]), int(order[0])}
    rng = np.random.default_rng(seed)
    pick |= set(int(e) for e in rng.choice(nz, size=min(n_random, len(nz)), replace=False))
    return sorted(pick)


def _sample_points(offsets, experts, ncols, seed, per_expert=40):
    rng = np.random.default_rng(seed)
    rows, cols = [], []
    for e in experts:
        b, t = int(offsets[e]), int(offsets[e + 1])
        rr = [b, t - 1] + list(rng.integers(b, t, per_expert - 2))
        rows += rr
        cols += list(rng.integers(0, ncols, len(rr)))
    return np.array(rows, np.int64), np.array(cols, np.int64)


def _expert_weights_subset(orc, w, which, experts):
    """Seeded weights for `experts` (checked bit-exact against the oracle),
    expert 0's quantized weights everywhere else (when w.E is large)."""
    N, K = (2 * w.I, w.H) if which == "gate_up" else (w.H, w.I)
    full = w.E <= 128
    src = None if full else sorted(set(experts) | {0})
    wq = P.quantize_weights(((e, to_dev(m, "bf16")) for e, m in D.expert_weights(w, which, src)),
                            w.E, N, K, DEV)
    if not full:
        rest = [e for e in range(w.E) if e not in set(src)]
        idx = torch.tensor(rest, device=DEV)
        wq.w.codes[idx] = wq.w.codes[0].clone()
        wq.w.scales[idx] = wq.w.scales[0].clone()
        wq.w.tscale[idx] = wq.w.tscale[0].clone()
    ref = {}
    for e, m in D.expert_weights(w, which, experts):
        c, s, t = orc.quantize(m)
        eq(host(wq.w.codes[e]), c, f"{which} weight codes e{e}")
        eq(host(wq.w.scales[e]), s, f"{which} weight scales e{e}")
        ref[e] = (c, s, t)
    return wq, ref


@pytest.mark.parametrize("wid", [3, 4, 5])
def test_full_moe_gemms_sampled(orc, wid):
    w = D.WORKLOADS[wid]
    rows_total = w.T * w.topk
    say(f"full moe gemms sampled {w.name}")
    x, lg = D.activations(w), D.router_logits(w)
    rt_ref = orc.route(lg, w.topk)
    offs = rt_ref["offsets"]
    experts = _sample_experts(offs, 100 + wid)
    say(f"  sampled experts {experts}")
    wgu, ref_gu = _expert_weights_subset(orc, w, "gate_up", experts)
    wd, ref_d = _expert_weights_subset(orc, w, "down", experts)

    # gate/up with SiLU*mul, exactly as in the benchmark's step
    rt = L.moe_route(torch.from_numpy(lg).to(DEV), w.topk)
    x_in = P.quantize_input(to_dev(x, "bf16"), w.n_select_x)
    amax_h = torch.zeros(1, dtype=torch.float32, device=DEV)
    h = P.gemm(x_in, wgu, rt.expert_offsets, rows_total, gather=rt.gather_rows,
               epilogue=L.NVFP4_EPI_SILU_MUL_BF16, out_amax=amax_h)
    d = orc.quantize_rac(x, w.n_select_x)
    eq(host(x_in.qo.q.codes), d["codes"], "X codes")
    eq(host(x_in.rac.r.codes), d["res_codes"], "X residual codes")
    h_gpu = host(h.view(torch.int16)).view(np.uint16)
    rows, cols = _sample_points(offs, experts, w.I, 200 + wid)
    ok_all = []
    for e in experts:
        sel = (rows >= offs[e]) & (rows < offs[e + 1])
        rr, cc = rows[sel], cols[sel]
        g_rows = rt_ref["gather"][offs[e]:offs[e + 1]].astype(np.int32)
        loc = rr - offs[e]
        a = (d["codes"], d["scales"], d["s_t"])
        r = (d["res_codes"], d["res_scales"], d["s_tr"])
        wst = tuple(np.asarray(v)[None] for v in ref_gu[e][:2]) + \
            (np.array([ref_gu[e][2]], np.float32),)
        off1 = np.array([0, len(g_rows)], np.int32)
        gate = orc.grouped_gemm_sample(2 * w.I, w.H, off1, g_rows, a, r, wst, loc, cc)
        up = orc.grouped_gemm_sample(2 * w.I, w.H, off1, g_rows, a, r, wst, loc, cc + w.I)
        h_ref, _ = orc.silu_mul(np.stack([gate, up], axis=1).astype(np.float32), 1)
        ok_all.append(bf16_ulp_ok(h_gpu[rr, cc], h_ref[:, 0]))
    ok = np.concatenate(ok_all)
    say(f"  H samples within 1 bf16 ulp: {ok.sum()}/{ok.size}")
    assert ok.all()

    # down projection on a seeded H-like input
    hl = D.hidden_like(w, rows_total)
    h_in = P.quantize_input(to_dev(hl, "bf16"), w.n_select_h, amax_in=torch.tensor(
        [float(np.abs(hl).max())], dtype=torch.float32, device=DEV))
    y = P.gemm(h_in, wd, rt.expert_offsets, rows_total)
    dh = orc.quantize_rac(hl, w.n_select_h, amax=float(np.abs(hl).max()))
    eq(host(h_in.qo.q.codes), dh["codes"], "H codes")
    eq(host(h_in.rac.r.codes), dh["res_codes"], "H residual codes")
    y_gpu = host(y)
    rows, cols = _sample_points(offs, experts, w.H, 300 + wid)
    got, want = [], []
    for e in experts:
        sel = (rows >= offs[e]) & (rows < offs[e + 1])
        rr, cc = rows[sel], cols[sel]
        wst = tuple(np.asarray(v)[None] for v in ref_d[e][:2]) + \
            (np.array([ref_d[e][2]], np.float32),)
        n_e = int(offs[e + 1] - offs[e])
        # rows of expert e are contiguous grouped rows: no gather, a one-group problem
        sub = (dh["codes"][offs[e]:offs[e + 1]], dh["scales"][offs[e]:offs[e + 1]], dh["s_t"])
        subr = (dh["res_codes"][offs[e]:offs[e + 1]], dh["res_scales"][offs[e]:offs[e + 1]],
                dh["s_tr"])
        want.append(orc.grouped_gemm_sample(w.H, w.I, np.array([0, n_e], np.int32), None, sub,
                                            subr, wst, rr - offs[e], cc))
        got.append(y_gpu[rr, cc])
    err = rel_frob(np.concatenate(got), np.concatenate(want))
    say(f"  down samples rel frob {err:.3e}")
    assert err <= REL_F
