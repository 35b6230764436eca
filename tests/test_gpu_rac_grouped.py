"""GPU parity of per-expert RAC (nvfp4_quantize_grouped,
rac_select_residual_grouped, and the grouped GEMM with per-group tensor
scales) through the C ABI against the CPU oracle.  Bars as for the
per-tensor path: every byte, scale, statistic and selection bit-exact; FP32
GEMM outputs within relative Frobenius 1e-5; SiLU*mul within one bf16 ulp.
GEMM inputs are the oracle's grouped operands."""
import numpy as np
import pytest
import torch

from nvfp4_w4a4_moe_quant_amd import _lib as L
from nvfp4_w4a4_moe_quant_amd import datagen as D
from nvfp4_w4a4_moe_quant_amd import pipeline as P

pytestmark = pytest.mark.gpu
from gpu_util import DEV, REL_F, bf16_ulp_ok, eq, host, rel_frob, say, to_dev


def _x(seed, rows, K, dtype):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, K)) * np.exp(rng.uniform(-1, 1, (rows, 1)))).astype(np.float32)
    x[:, rng.integers(0, K, 3)] *= 25.0
    if dtype == "bf16":
        x = D.bf16_to_f32(D.bf16_bits(x))
    return x


def _offsets(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


CASES = [  # (seed, group sizes, K, src rows or None (no gather), n_select, dtype)
    (0, [50, 0, 37, 64], 256, None, 128, "bf16"),
    (1, [20, 31, 1, 0, 44, 9, 17, 2], 512, 100, 256, "bf16"),
    (2, [77], 128, None, 64, "f32"),
    (3, [300, 12, 150, 1, 90, 0, 260, 40] * 2, 768, None, 384, "bf16"),
    (4, [5, 400, 3], 256, 64, 0, "f32"),
    (5, [33, 18], 256, None, 256, "bf16"),
]


@pytest.mark.parametrize("seed,sizes,K,src,n_sel,dtype", CASES)
def test_grouped_quant_rac_parity(orc, seed, sizes, K, src, n_sel, dtype):
    say(f"grouped quant+rac seed={seed} G={len(sizes)} K={K} gather={src is not None} n_sel={n_sel}")
    off = _offsets(sizes)
    total = int(off[-1])
    rng = np.random.default_rng(100 + seed)
    x = _x(seed, src if src is not None else total, K, dtype)
    gat = rng.integers(0, src, total).astype(np.int32) if src is not None else None
    d = orc.quantize_rac_grouped(x, off, gat, n_sel)
    xd, od = to_dev(x, dtype), _t(off)
    gd = None if gat is None else _t(gat)
    qo = L.nvfp4_quantize_grouped(xd, od, total, gather_rows=gd, stats=True)
    rac = L.rac_select_residual_grouped(xd, qo, od, total, n_sel, gather_rows=gd)
    eq(host(qo.q.tscale), d["s_t"], "tensor scales")
    eq(host(qo.q.scales), d["scales"], "block scales")
    eq(host(qo.q.codes), d["codes"], "codes")
    eq(host(qo.channel_score), d["score"], "channel scores")
    eq(host(qo.channel_max), d["chmax"], "channel max")
    eq(host(rac.selected), d["selected"], "selected")
    eq(host(rac.kblock_active), d["active"], "kblock_active")
    eq(host(rac.r.tscale), d["s_tr"], "residual tensor scales")
    eq(host(rac.r.scales), d["res_scales"], "residual scales")
    eq(host(rac.r.codes), d["res_codes"], "residual codes")
    qn = L.nvfp4_quantize_grouped(xd, od, total, gather_rows=gd, stats=True, channel_max=False)
    assert qn.channel_max is None
    rn = L.rac_select_residual_grouped(xd, qn, od, total, n_sel, gather_rows=gd)
    eq(host(qn.channel_score), d["score"], "channel scores (no channel max)")
    eq(host(qn.q.codes), d["codes"], "codes (no channel max)")
    eq(host(rn.selected), d["selected"], "selected (no channel max)")
    eq(host(rn.r.codes), d["res_codes"], "residual codes (no channel max)")


@pytest.mark.parametrize("silu,skip", [(False, False), (True, False), (False, True)])
def test_gemm_per_group_scales(orc, silu, skip):
    say(f"gemm per-group scales silu={silu} skip={skip}")
    sizes, K, N = [70, 0, 33, 130, 5], 256, 256
    off = _offsets(sizes)
    total, G = int(off[-1]), len(sizes)
    x = _x(7, 90, K, "bf16")
    gat = np.random.default_rng(8).integers(0, 90, total).astype(np.int32)
    n_sel = 32 if skip else 128
    d = orc.quantize_rac_grouped(x, off, gat, n_sel)
    rng = np.random.default_rng(9)
    ws = [orc.quantize((rng.standard_normal((N, K)) * 0.02).astype(np.float32)) for _ in range(G)]
    w = (np.stack([q[0] for q in ws]), np.stack([q[1] for q in ws]),
         np.array([q[2] for q in ws], np.float32))
    y = orc.grouped_gemm(N, K, off, None, (d["codes"], d["scales"], d["s_t"]),
                         (d["res_codes"], d["res_scales"], d["s_tr"]), w)
    a = L.NVFP4(_t(d["codes"]), _t(d["scales"]), _t(d["s_t"]))
    r = L.NVFP4(_t(d["res_codes"]), _t(d["res_scales"]), _t(d["s_tr"]))
    wq = L.NVFP4(_t(w[0]), _t(w[1]), _t(w[2]))
    out = L.w4a4_grouped_gemm_rac(a, wq, _t(off), N=N, K=K, total_rows=total, r=r,
                                  kblock_active=_t(d["active"]),
                                  epilogue=L.NVFP4_EPI_SILU_MUL_BF16 if silu else L.NVFP4_EPI_F32,
                                  skip_inactive=skip, per_group_scales=True)
    if silu:
        h_ref, _ = orc.silu_mul(y, N // 2)
        ok = bf16_ulp_ok(host(out.view(torch.int16)).view(np.uint16), h_ref)
        assert ok.all(), f"{(~ok).sum()} beyond one bf16 ulp"
    else:
        err = rel_frob(host(out), y)
        assert err <= REL_F, err


def test_per_expert_moe_gate_up(orc):
    """The per-expert MoE path's gate/up stage (routing, per-expert quantize +
    RAC of the gathered tokens, GEMM with SiLU*mul) against the oracle."""
    say("per-expert moe gate/up")
    T, E, k, H, I = 96, 8, 2, 256, 128
    rng = np.random.default_rng(11)
    x = _x(12, T, H, "bf16")
    logits = rng.standard_normal((T, E)).astype(np.float32)
    wgu_np = [(rng.standard_normal((2 * I, H)) * 0.02).astype(np.float32) for _ in range(E)]
    wd_np = [(rng.standard_normal((H, I)) * 0.02).astype(np.float32) for _ in range(E)]
    wgu = P.quantize_weights(((e, to_dev(m, "f32")) for e, m in enumerate(wgu_np)), E, 2 * I, H, DEV)
    wd = P.quantize_weights(((e, to_dev(m, "f32")) for e, m in enumerate(wd_np)), E, H, I, DEV)
    d = P.moe_forward(to_dev(x, "bf16"), _t(logits), wgu, wd, k, H // 2, I // 2, per_expert=True)
    rt = orc.route(logits, k)
    g = orc.quantize_rac_grouped(x, rt["offsets"], rt["gather"], H // 2)
    eq(host(d["x_in"].qo.q.codes), g["codes"], "gate/up input codes")
    eq(host(d["x_in"].rac.r.codes), g["res_codes"], "gate/up residual codes")
    wq = [orc.quantize(m) for m in wgu_np]
    w = (np.stack([q[0] for q in wq]), np.stack([q[1] for q in wq]),
         np.array([q[2] for q in wq], np.float32))
    y = orc.grouped_gemm(2 * I, H, rt["offsets"], None, (g["codes"], g["scales"], g["s_t"]),
                         (g["res_codes"], g["res_scales"], g["s_tr"]), w)
    h_ref, _ = orc.silu_mul(y, I)
    ok = bf16_ulp_ok(host(d["h"].view(torch.int16)).view(np.uint16), h_ref)
    assert ok.all(), f"{(~ok).sum()} beyond one bf16 ulp"


@pytest.mark.parametrize("K,n_sel", [(2048, 1024), (768, 384), (8192, 4096), (256, 1),
                                     (512, 511), (256, 256), (128, 0)])
def test_grouped_select_crafted_scores(orc, K, n_sel):
    """Per-group selection on hand-made int64 scores -- one group each of heavy
    ties, values near 2^63, all zeros, all equal, random -- against the
    oracle's per-group sort (score desc, index asc); the residual uses the
    real per-channel max |e|, so its scale and bytes are checked too."""
    say(f"grouped select crafted K={K} n_sel={n_sel}")
    rng = np.random.default_rng(K + 7 * n_sel)
    sizes = [3, 2, 4, 1, 3]
    off = _offsets(sizes)
    total, G = int(off[-1]), len(sizes)
    x = _x(K, total, K, "bf16")
    xd, od = to_dev(x, "bf16"), _t(off)
    qo = L.nvfp4_quantize_grouped(xd, od, total, stats=True)
    score = np.zeros((G, K), np.int64)
    score[0] = rng.integers(0, 5, K).astype(np.int64) << 40
    score[1] = (np.int64(2 ** 62) + rng.integers(0, 2 ** 61, K)).astype(np.int64)
    score[1, rng.integers(0, K, K // 8)] = np.iinfo(np.int64).max
    score[1, rng.integers(0, K, K // 8)] = 0
    score[2] = 0
    score[3] = 123456789
    score[4] = rng.integers(0, 2 ** 40, K)
    qo2 = L.QuantOut(qo.q, _t(score), qo.channel_max)
    rac = L.rac_select_residual_grouped(xd, qo2, od, total, n_sel)
    sel_g, act_g = host(rac.selected), host(rac.kblock_active)
    s_tr_g = host(rac.r.tscale)
    # the oracle's own per-group quantization and channel maxima
    q = orc.quantize_rac_grouped(x, off, None, None)
    codes, scales, s_t = q["codes"], q["scales"], q["s_t"]
    for g in range(G):
        j0, j1 = off[g], off[g + 1]
        _, chmax = orc.channel_stats(x[j0:j1], codes[j0:j1], scales[j0:j1], float(s_t[g]))
        sel, mask, active, _ = orc.rac_select(score[g], chmax, n_sel)
        eq(sel_g[g], sel, f"selected group {g}")
        eq(act_g[g], active, f"kblock_active group {g}")
        rc, rs, s_tr, _ = orc.rac_residual(x[j0:j1], codes[j0:j1], scales[j0:j1], float(s_t[g]),
                                           mask)
        eq(s_tr_g[g], np.float32(s_tr), f"residual tensor scale group {g}")
        eq(host(rac.r.codes)[j0:j1], rc, f"residual codes group {g}")
        eq(host(rac.r.scales)[j0:j1], rs, f"residual scales group {g}")
