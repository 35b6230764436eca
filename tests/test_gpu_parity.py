"""GPU parity of the HIP library against the CPU oracle, called through the
C ABI (via the ctypes binding).

Bars: bit-exact codes, scales, tensor scales, channel statistics, selected
channels, block activity, residual bytes and routing indices; FP32 GEMM
outputs within relative Frobenius error 1e-5 (only the FP32 accumulation
order differs from the oracle's exact sums); SiLU*mul output within one bf16
ulp (its exp() is not bit-defined across implementations).  The down
projection of the MoE chain is checked on an H that comes from the oracle (or
from the seeded generator), never from the GPU."""
import numpy as np
import pytest
import torch

from nvfp4_w4a4_moe_quant_amd import _lib as L
from nvfp4_w4a4_moe_quant_amd import datagen as D
from nvfp4_w4a4_moe_quant_amd import pipeline as P

pytestmark = pytest.mark.gpu
from gpu_util import (DEV, REL_F, bf16_ulp_ok, check_quant_rac, eq, host, rel_frob, say,
                      to_dev)


# ------------------------------------------------------------ quantizer
@pytest.mark.parametrize("wid", [1, 2])
def test_quant_rac_workloads_small(orc, wid):
    w = D.WORKLOADS[wid]
    say(f"quant+rac workload {wid} {w.name}")
    check_quant_rac(orc, D.activations(w), w.x_dtype, w.n_select_x)


@pytest.mark.parametrize("rows,K,dtype", [(1, 16, "bf16"), (3, 48, "f32"), (257, 272, "bf16"),
                                          (1000, 768, "bf16"), (33, 4112, "f32"),
                                          (5, 7168, "bf16"), (2, 16384, "bf16")])
def test_quant_rac_shapes(orc, rows, K, dtype):
    say(f"quant+rac shape {rows}x{K} {dtype}")
    rng = np.random.default_rng(rows * 7 + K)
    x = rng.standard_normal((rows, K)).astype(np.float32)
    x[:, rng.integers(0, K, 3)] *= 40.0
    if dtype == "bf16":
        x = D.bf16_to_f32(D.bf16_bits(x))
    check_quant_rac(orc, x, dtype, K // 2)


def test_quant_rac_edge_values(orc):
    say("quant+rac edge values")
    rng = np.random.default_rng(77)
    x = rng.standard_normal((40, 64)).astype(np.float32)
    x[0] = 0.0                                 # all-zero row
    x[1, :16] = 1e-30                          # tiny block -> subnormal/zero scale
    x[2, 16:32] = np.float32(3e-6)             # subnormal block scale
    x[3, 5] = 1e4                              # tensor amax dominated by one value
    x[4] = 2.5                                 # exact E2M1 ties after scaling
    check_quant_rac(orc, x, "f32", 32)
    check_quant_rac(orc, x, "f32", 0)
    check_quant_rac(orc, x, "f32", 64)


def test_quant_rac_ties_and_zero(orc):
    say("quant+rac all-zero and tied scores")
    check_quant_rac(orc, np.zeros((7, 128), np.float32), "f32", 64)
    x = np.tile(np.linspace(-3, 3, 32, dtype=np.float32), (9, 4))  # repeated channels
    check_quant_rac(orc, x, "f32", 50)


@pytest.mark.parametrize("K,n_sel,kind", [(2048, 1024, "ties"), (768, 384, "huge"),
                                           (16384, 8192, "ties"), (4112, 1, "huge"),
                                           (4096, 4095, "zeros"), (1024, 512, "equal")])
def test_select_crafted_scores(orc, K, n_sel, kind):
    """Selection on hand-made int64 scores (heavy ties, values near 2^63,
    all-zero, all-equal) against the oracle's sort; the residual uses the
    real per-channel max |e|, so its bytes are checked as well."""
    say(f"select crafted {kind} K={K} n_sel={n_sel}")
    rng = np.random.default_rng(K + n_sel)
    x = D.bf16_to_f32(D.bf16_bits(rng.standard_normal((3, K)).astype(np.float32)))
    xd = to_dev(x, "bf16")
    qo = L.nvfp4_quantize(xd, stats=True)
    if kind == "ties":
        score = rng.integers(0, 5, K).astype(np.int64) << 40
    elif kind == "huge":
        score = (np.int64(2 ** 62) + rng.integers(0, 2 ** 61, K)).astype(np.int64)
        score[rng.integers(0, K, K // 8)] = np.iinfo(np.int64).max
        score[rng.integers(0, K, K // 8)] = 0
    elif kind == "zeros":
        score = np.zeros(K, np.int64)
    else:
        score = np.full(K, 123456789, np.int64)
    qo2 = L.QuantOut(qo.q, torch.from_numpy(score).to(DEV), qo.channel_max)
    rac = L.rac_select_residual(xd, qo2, n_sel)
    # the oracle's own quantization and channel maxima, the crafted scores
    c, sc, t = orc.quantize(x)
    _, chmax = orc.channel_stats(x, c, sc, t)
    sel, mask, active, _ = orc.rac_select(score, chmax, n_sel)
    eq(host(rac.selected), sel, "selected")
    eq(host(rac.kblock_active), active, "kblock_active")
    rc, rs, s_tr, _ = orc.rac_residual(x, c, sc, t, mask)
    assert np.float32(s_tr) == np.float32(t)
    eq(host(rac.r.tscale)[0], np.float32(s_tr), "residual tensor scale")
    eq(host(rac.r.scales), rs, "residual scales")
    eq(host(rac.r.codes), rc, "residual codes")


def test_quant_amax_in_and_stride(orc):
    say("quant with amax_in and padded rows")
    rng = np.random.default_rng(78)
    x = D.bf16_to_f32(D.bf16_bits(rng.standard_normal((100, 256)).astype(np.float32)))
    check_quant_rac(orc, x, "bf16", 128, amax=float(np.abs(x).max()) * 1.5)
    check_quant_rac(orc, x, "bf16", 128, ldx_pad=32)


# Statistics buffers that start with garbage: with one row split (at most 128
# rows at this K) the workgroups store each channel's sums and nothing zeroes
# them first; with more rows k_amax, or k_zero_stats when amax_in is given,
# zeroes them before the atomic sums.  Called through the C ABI directly, so
# that the outputs can be pre-filled.
@pytest.mark.parametrize("rows,amax_in", [(16, False), (16, True), (128, True), (129, True),
                                          (1000, False), (1000, True)])
def test_quant_stats_overwrite_garbage(orc, rows, amax_in):
    say(f"quant stats over garbage rows={rows} amax_in={amax_in}")
    K = 2048
    rng = np.random.default_rng(800 + rows)
    x = D.bf16_to_f32(D.bf16_bits(rng.standard_normal((rows, K)).astype(np.float32)))
    amax = float(np.abs(x).max()) if amax_in else None
    d = orc.quantize_rac(x, K // 2, amax=amax)
    xd = to_dev(x, "bf16")
    am = None if amax is None else torch.tensor([amax], dtype=torch.float32, device=DEV)
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((rows, K // 16), dtype=torch.uint8, device=DEV)
    ts = torch.empty(1, dtype=torch.float32, device=DEV)
    score = torch.full((K,), 0x5A5A5A5A5A5A5A5A, dtype=torch.int64, device=DEV)
    chmax = torch.full((K,), 3.0e38, dtype=torch.float32, device=DEV)
    lib = L.lib()
    ws = torch.empty(max(int(lib.nvfp4_quantize_workspace_size(rows, K)), 256), dtype=torch.uint8,
                     device=DEV)
    for cm in (chmax, None):  # with the channel maximum, then without
        score.fill_(0x5A5A5A5A5A5A5A5A)
        st = lib.nvfp4_quantize(L._ptr(xd), L.NVFP4_IN_BF16, rows, K, xd.stride(0), L._ptr(am),
                                L._ptr(codes), L._ptr(scales), L._ptr(ts), L._ptr(score),
                                L._ptr(cm), L._ptr(ws), ws.numel(), L._stream(xd.device))
        assert st == 0, st
        eq(host(codes), d["codes"], "codes")
        eq(host(score), d["score"], "channel score")
        if cm is not None:
            eq(host(cm), d["chmax"], "channel max")


def test_quant_empty_rows(orc):
    say("quant rows=0")
    xd = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    qo = L.nvfp4_quantize(xd, stats=True)
    rac = L.rac_select_residual(xd, qo, 32)
    assert host(qo.q.tscale)[0] == 0.0
    assert not host(qo.channel_score).any()
    eq(host(rac.selected), np.arange(32), "selected of empty input")


# ------------------------------------------------------------- routing
# Up to 64 tokens one workgroup does all of the routing (the first five
# cases: a decode step, the largest E and k, every expert taken); 65 tokens is
# the first case of the three-launch path.  The last two cases are past the
# fused scan's bound (blocks^2 x E > 2^20): the separate one-workgroup scan of
# the expert counts runs there.
@pytest.mark.parametrize("T,E,k,routing", [(1, 4, 1, "normal"), (16, 256, 8, "normal"),
                                           (33, 100, 5, "zipf"), (64, 1024, 16, "normal"),
                                           (64, 16, 16, "normal"), (65, 512, 8, "zipf"),
                                           (300, 8, 2, "zipf"),
                                           (1000, 128, 8, "normal"), (777, 256, 8, "normal"),
                                           (513, 64, 6, "zipf"), (200, 384, 8, "normal"),
                                           (20000, 256, 8, "zipf"), (9000, 1024, 4, "normal")])
def test_route(orc, T, E, k, routing):
    say(f"route T={T} E={E} k={k} {routing}")
    w = D.small_moe(90 + T, T, E, k, 64, 32, routing=routing, n_empty=2 if routing == "zipf" else 0)
    lg = D.router_logits(w)
    rt = L.moe_route(torch.from_numpy(lg).to(DEV), k)
    d = orc.route(lg, k)
    eq(host(rt.topk_ids), d["topk_ids"], "topk ids")
    eq(host(rt.expert_offsets), d["offsets"], "offsets")
    eq(host(rt.gather_rows), d["gather"], "gather")
    eq(host(rt.row_of), d["row_of"], "row_of")
    np.testing.assert_allclose(host(rt.topk_weights), d["topk_weights"], rtol=2e-5, atol=1e-7)


def test_route_empty():
    say("route T=0")
    rt = L.moe_route(torch.zeros((0, 16), dtype=torch.float32, device=DEV), 4)
    eq(host(rt.expert_offsets), np.zeros(17, np.int32), "offsets of no tokens")
    assert rt.gather_rows.numel() == 0 and rt.row_of.numel() == 0


@pytest.mark.parametrize("T", [70, 40])  # three launches / one workgroup
def test_route_ties(orc, T):
    say(f"route with tied logits T={T}")
    lg = np.zeros((T, 16), np.float32)
    lg[::3, 5] = 1.0
    rt = L.moe_route(torch.from_numpy(lg).to(DEV), 4)
    d = orc.route(lg, 4)
    eq(host(rt.topk_ids), d["topk_ids"], "topk ids")
    eq(host(rt.expert_offsets), d["offsets"], "offsets")
    eq(host(rt.gather_rows), d["gather"], "gather")
    eq(host(rt.row_of), d["row_of"], "row_of")


# --------------------------------------------------------------- GEMM
def quant_weights_checked(orc, mats, G, N, K, dtype, check=None):
    """Quantize weights on the GPU; check the bytes of groups `check` against
    the oracle.  Returns (QuantWeights, {g: oracle (codes, scales, s_t)})."""
    mats = list(mats)
    wq = P.quantize_weights(((g, to_dev(m, dtype)) for g, m in mats), G, N, K, DEV)
    ref = {}
    for g, m in mats:
        if check is None or g in check:
            c, s, t = orc.quantize(m)
            ref[g] = (c, s, t)
            eq(host(wq.w.codes[g]), c, f"weight codes g{g}")
            eq(host(wq.w.scales[g]), s, f"weight scales g{g}")
            eq(host(wq.w.tscale[g:g + 1])[0], np.float32(t), f"weight tscale g{g}")
    return wq, ref


def w_stack(ref, G):
    return (np.stack([ref[g][0] for g in range(G)]), np.stack([ref[g][1] for g in range(G)]),
            np.array([ref[g][2] for g in range(G)], np.float32))


@pytest.mark.parametrize("wid,rac", [(1, True), (1, False)])
def test_dense_workload1(orc, wid, rac):
    w = D.WORKLOADS[wid]
    say(f"dense gemm workload {wid} rac={rac}")
    x, W = D.activations(w), D.dense_weight(w)
    wq, ref = quant_weights_checked(orc, [(0, W)], 1, w.N, w.K, w.x_dtype)
    out = P.dense_forward(to_dev(x, w.x_dtype), wq, w.n_select_x if rac else None)
    d = orc.quantize_rac(x, w.n_select_x)
    a = (d["codes"], d["scales"], d["s_t"])
    r = (d["res_codes"], d["res_scales"], d["s_tr"]) if rac else None
    y_ref = orc.grouped_gemm(w.N, w.K, np.array([0, w.rows], np.int32), None, a, r, w_stack(ref, 1))
    y = host(out["y"])
    err = rel_frob(y, y_ref)
    say(f"  rel frob {err:.3e}")
    assert err <= REL_F
    np.testing.assert_allclose(y, y_ref, rtol=1e-4, atol=1e-5 * np.abs(y_ref).max())


@pytest.mark.parametrize("rows,K,N", [(200, 384, 256), (1, 128, 128), (129, 256, 384)])
def test_dense_ragged(orc, rows, K, N):
    say(f"dense gemm ragged {rows}x{K}x{N}")
    w = D.small_dense(50 + rows, rows, K, N)
    x, W = D.activations(w), D.dense_weight(w)
    wq, ref = quant_weights_checked(orc, [(0, W)], 1, N, K, "bf16")
    out = P.dense_forward(to_dev(x, "bf16"), wq, K // 2)
    d = orc.quantize_rac(x, K // 2)
    y_ref = orc.grouped_gemm(N, K, np.array([0, rows], np.int32), None,
                             (d["codes"], d["scales"], d["s_t"]),
                             (d["res_codes"], d["res_scales"], d["s_tr"]), w_stack(ref, 1))
    err = rel_frob(host(out["y"]), y_ref)
    say(f"  rel frob {err:.3e}")
    assert err <= REL_F


def _nv(orc_triple):
    """Oracle NVFP4 (codes, scales, s_t) -> device NVFP4."""
    c, sc, t = orc_triple
    return L.NVFP4(torch.from_numpy(np.ascontiguousarray(c)).to(DEV),
                   torch.from_numpy(np.ascontiguousarray(sc)).to(DEV),
                   torch.tensor([t], dtype=torch.float32, device=DEV))


@pytest.mark.parametrize("rows,K,N,rac,gather", [
    (16, 4096, 256, True, False), (1, 512, 128, True, False), (5, 1536, 128, False, False),
    (33, 1024, 256, True, True), (64, 2048, 384, True, False), (17, 512, 128, False, True),
    (65, 512, 128, True, False), (16, 16384, 128, True, True), (3, 3072, 256, True, False),
    (64, 1024, 128, False, True), (9, 7168, 384, True, False), (16, 8192, 256, False, False)])
def test_decode_shaped_gemm(orc, rows, K, N, rac, gather):
    """One group with few rows (the decode kernel below 65 rows when K % 1024
    == 0 and K <= 16384: one to sixteen chunks of 1024 k, so the LDS chunk
    ring wraps up to four times, and scale rows of 4 to 64 pieces; other
    shapes take the prefill kernel), with and without RAC and a row gather,
    against the oracle GEMM on oracle-quantized operands."""
    say(f"decode gemm {rows}x{K}x{N} rac={rac} gather={gather}")
    rng = np.random.default_rng(rows * 31 + K + N)
    src = rows + 3 if gather else rows
    x = D.bf16_to_f32(D.bf16_bits(rng.standard_normal((src, K)).astype(np.float32)))
    x[:, rng.integers(0, K, 4)] *= 30.0
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    d = orc.quantize_rac(x, K // 2)
    a = (d["codes"], d["scales"], d["s_t"])
    r = (d["res_codes"], d["res_scales"], d["s_tr"]) if rac else None
    wc, ws, wt = orc.quantize(W)
    w = (wc[None], ws[None], np.array([wt], np.float32))
    g = rng.permutation(src)[:rows].astype(np.int32) if gather else None
    offsets = np.array([0, rows], np.int32)
    y_ref = orc.grouped_gemm(N, K, offsets, g, a, r, w)
    y = L.w4a4_grouped_gemm_rac(
        _nv(a), L.NVFP4(torch.from_numpy(w[0]).to(DEV), torch.from_numpy(w[1]).to(DEV),
                        torch.from_numpy(w[2]).to(DEV)),
        torch.from_numpy(offsets).to(DEV), N=N, K=K, total_rows=rows,
        gather_rows=None if g is None else torch.from_numpy(g).to(DEV),
        r=_nv(r) if rac else None)
    err = rel_frob(host(y), y_ref)
    say(f"  rel frob {err:.3e}")
    assert err <= REL_F


def test_gemm_onehot_reads_dequantized_weights(orc):
    """A = one-hot rows (value 1 at k = i): y[i, n] = s_ta * s_tw * W_deq[n, i]."""
    say("gemm one-hot")
    K, N = 128, 128
    x = np.zeros((K, K), np.float32)
    np.fill_diagonal(x, 2688.0)              # s_t = 1, s_b = 448, g = 6
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    wq, ref = quant_weights_checked(orc, [(0, W)], 1, N, K, "f32")
    out = P.dense_forward(to_dev(x, "f32"), wq, None)
    wdeq = orc.dequantize(ref[0][0], ref[0][1], ref[0][2])
    y = host(out["y"])
    np.testing.assert_allclose(y, 2688.0 * wdeq.T, rtol=1e-6)


def _moe_case(orc, w, check_experts=None):
    x, lg = D.activations(w), D.router_logits(w)
    wgu, ref_gu = quant_weights_checked(orc, D.expert_weights(w, "gate_up"), w.E, 2 * w.I, w.H,
                                        "bf16", check_experts)
    wd, ref_d = quant_weights_checked(orc, D.expert_weights(w, "down"), w.E, w.H, w.I, "bf16",
                                      check_experts)
    return x, lg, wgu, ref_gu, wd, ref_d


@pytest.mark.parametrize("T,E,k,H,I,routing", [(333, 6, 2, 256, 128, "zipf"),
                                               (200, 16, 4, 384, 256, "normal")])
def test_moe_chain_small(orc, T, E, k, H, I, routing):
    say(f"moe chain T={T} E={E} k={k} H={H} I={I} {routing}")
    w = D.small_moe(60 + T, T, E, k, H, I, routing=routing, n_empty=1 if routing == "zipf" else 0)
    x, lg, wgu, ref_gu, wd, ref_d = _moe_case(orc, w)
    out = P.moe_forward(to_dev(x, "bf16"), torch.from_numpy(lg).to(DEV), wgu, wd, k,
                        w.n_select_x, w.n_select_h)
    rt = orc.route(lg, k)
    eq(host(out["route"].gather_rows), rt["gather"], "gather")
    d = orc.quantize_rac(x, w.n_select_x)
    eq(host(out["x_in"].qo.q.codes), d["codes"], "X codes")
    eq(host(out["x_in"].rac.r.codes), d["res_codes"], "X residual codes")
    rows = T * k
    y_gu = orc.grouped_gemm(2 * I, H, rt["offsets"], rt["gather"],
                            (d["codes"], d["scales"], d["s_t"]),
                            (d["res_codes"], d["res_scales"], d["s_tr"]), w_stack(ref_gu, E))
    h_ref, amax_ref = orc.silu_mul(y_gu, I)
    h_gpu = host(out["h"].view(torch.int16)).view(np.uint16)
    ok = bf16_ulp_ok(h_gpu, h_ref)
    say(f"  H within 1 bf16 ulp: {ok.mean():.6f}, exact: {(h_gpu == h_ref).mean():.6f}")
    assert ok.all()
    amax_gpu = host(out["amax_h"])[0]
    assert abs(amax_gpu - amax_ref) <= amax_ref * 2.0 ** -7
    # down projection on the oracle's H (same bytes into both sides)
    h_ref_f = D.bf16_to_f32(h_ref)
    dh = orc.quantize_rac(h_ref_f, w.n_select_h)
    h_in = P.quantize_input(to_dev(h_ref_f, "bf16"), w.n_select_h)
    eq(host(h_in.qo.q.codes), dh["codes"], "H codes")
    eq(host(h_in.rac.selected), dh["selected"], "H selected")
    eq(host(h_in.rac.r.codes), dh["res_codes"], "H residual codes")
    y_gpu = P.gemm(h_in, wd, out["route"].expert_offsets, rows)
    y_ref = orc.grouped_gemm(H, I, rt["offsets"], None, (dh["codes"], dh["scales"], dh["s_t"]),
                             (dh["res_codes"], dh["res_scales"], dh["s_tr"]), w_stack(ref_d, E))
    err = rel_frob(host(y_gpu), y_ref)
    say(f"  down rel frob {err:.3e}")
    assert err <= REL_F
    # whole GPU chain against the oracle chain (loose: H differs by <= 1 ulp)
    err_chain = rel_frob(host(out["y"]), y_ref)
    say(f"  chained layer rel frob {err_chain:.3e}")
    assert err_chain <= 1e-2


def test_moe_naive_mode_matches_main_sum(orc):
    """RAC off on the GPU equals the oracle's naive W4A4 output (the main pass
    alone)."""
    say("moe naive mode")
    w = D.small_moe(71, 150, 5, 2, 256, 128)
    x, lg, wgu, ref_gu, wd, ref_d = _moe_case(orc, w)
    rt = L.moe_route(torch.from_numpy(lg).to(DEV), 2)
    x_in = P.quantize_input(to_dev(x, "bf16"), None)
    y = P.gemm(x_in, wgu, rt.expert_offsets, 300, gather=rt.gather_rows)
    r = orc.route(lg, 2)
    c, s, t = orc.quantize(x)
    y_ref = orc.grouped_gemm(256, 256, r["offsets"], r["gather"], (c, s, t), None,
                             w_stack(ref_gu, 5))
    assert rel_frob(host(y), y_ref) <= REL_F


@pytest.mark.parametrize("n_select", [16, 40])
def test_residual_skip_with_inactive_blocks(orc, n_select):
    """A sparse selection leaves most 16-blocks inactive: the step-skipping
    GEMM (NVFP4_GEMM_SKIP_INACTIVE_BLOCKS) and the branch-free residual pass
    both match the oracle, and each other."""
    say(f"residual skip, n_select={n_select}")
    rows, K, N = 150, 512, 256
    w = D.small_dense(81, rows, K, N, n_outliers=0)
    x = D.activations(w)
    x[:, 64:80] *= 30.0                      # errors concentrated in two blocks
    x[:, 200:216] *= 25.0
    x = D.bf16_to_f32(D.bf16_bits(x))
    W = D.dense_weight(w)
    wq, ref = quant_weights_checked(orc, [(0, W)], 1, N, K, "bf16")
    xd = to_dev(x, "bf16")
    inp = P.quantize_input(xd, n_select)
    kact = host(inp.rac.kblock_active)
    assert (kact == 0).sum() >= K // 16 - 4
    offs = torch.tensor([0, rows], dtype=torch.int32, device=DEV)
    y_skip = L.w4a4_grouped_gemm_rac(inp.qo.q, wq.w, offs, N=N, K=K, total_rows=rows,
                                     r=inp.rac.r, kblock_active=inp.rac.kblock_active,
                                     skip_inactive=True)
    y_full = L.w4a4_grouped_gemm_rac(inp.qo.q, wq.w, offs, N=N, K=K, total_rows=rows,
                                     r=inp.rac.r, kblock_active=inp.rac.kblock_active,
                                     skip_inactive=False)
    d = orc.quantize_rac(x, n_select)
    eq(kact, d["active"], "kblock_active")
    y_ref = orc.grouped_gemm(N, K, np.array([0, rows], np.int32), None,
                             (d["codes"], d["scales"], d["s_t"]),
                             (d["res_codes"], d["res_scales"], d["s_tr"]), w_stack(ref, 1))
    ys, yf = host(y_skip), host(y_full)
    assert rel_frob(ys, y_ref) <= REL_F and rel_frob(yf, y_ref) <= REL_F
    np.testing.assert_array_equal(ys, yf)
