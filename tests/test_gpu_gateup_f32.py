"""The gate/up GEMM with the SiLU*mul epilogue -- the largest kernel of the MoE
step -- checked at the FP32 tolerance.  The kernel's optional FP32 side
output (out_y) holds the gate/up values that enter the SiLU, from the same
instantiation, tiles and accumulation as the bf16 H it writes; they are
compared element by element with the oracle's exact GEMM (relative Frobenius
error <= 1e-5), and H with the oracle's SiLU*mul of the oracle's y (within one
bf16 ulp, with a floor on the fraction of bit-identical values).

Both sides read the same NVFP4 bytes: the oracle quantizes X and W, and those
bytes are uploaded for the GPU GEMM, so the comparison isolates the GEMM."""
import numpy as np
import pytest
import torch

from nvfp4_w4a4_moe_quant_amd import _lib as L
from nvfp4_w4a4_moe_quant_amd import datagen as D
from gpu_util import DEV, REL_F, bf16_ulp_ok, eq, host, rel_frob, say

pytestmark = pytest.mark.gpu

# Fraction of H values that must be bit-identical to the oracle's.  The GPU
# evaluates silu(g) * u in FP32 with the hardware exp and reciprocal, the
# oracle in double: only values within a few FP32 ulp of a bf16 rounding
# boundary may round the other way (about 2^-16 of them per FP32 ulp of
# difference), so a floor of 99% leaves a wide margin.
H_EXACT_FLOOR = 0.99


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t if dtype is None else t.view(dtype)


def _nv(c, s, t):
    return L.NVFP4(_dev(c), _dev(s), torch.tensor(np.atleast_1d(np.asarray(t, np.float32)),
                                                  device=DEV))


def _check_h(h_gpu, y_ref, y_gpu, I, what):
    """H against the oracle's SiLU*mul of the oracle's y.  Per element the bound
    is one bf16 ulp of the oracle's h plus the first-order change of
    silu(g) * u under the measured difference of the FP32 gate and up values
    (which is itself checked against the oracle in relative Frobenius norm):
    an output near zero by cancellation carries an FP32 accumulation error
    that is small against its row but not against itself."""
    h_ref, amax_ref = _silu(y_ref, I)
    a = D.bf16_to_f32(np.asarray(h_gpu, np.uint16)).astype(np.float64)
    b = D.bf16_to_f32(np.asarray(h_ref, np.uint16)).astype(np.float64)
    g, u = y_ref[:, :I].astype(np.float64), y_ref[:, I:].astype(np.float64)
    dg = np.abs(y_gpu[:, :I].astype(np.float64) - g)
    du = np.abs(y_gpu[:, I:].astype(np.float64) - u)
    sg = 0.5 * (1.0 + np.tanh(0.5 * g))                  # logistic sigmoid, no overflow
    dsilu = sg * (1.0 + g * (1.0 - sg))                  # d silu / d g
    prop = np.abs(dsilu * u) * dg + np.abs(g * sg) * du
    ulp = np.maximum(np.abs(b), 2.0 ** -126) * 2.0 ** -7
    bound = 1.0001 * ulp + 2.0 * prop
    ok = np.abs(a - b) <= bound
    ok1 = bf16_ulp_ok(h_gpu, h_ref)
    exact = float((h_gpu == h_ref).mean())
    say(f"  {what}: H within 1 bf16 ulp {ok1.mean():.7f}, within the propagated bound "
        f"{ok.mean():.7f}, bit-identical {exact:.7f}")
    assert ok.all()
    assert exact >= H_EXACT_FLOOR
    return amax_ref


_ORC = {}


def _silu(y, I):
    return _ORC["o"].silu_mul(np.ascontiguousarray(y, np.float32), I)


def _gateup_case(orc, T, E, k, H, I, *, rac=True, n_select=None, skip=False, seed=0):
    _ORC["o"] = orc
    rng = np.random.default_rng(seed)
    x = D.bf16_to_f32(D.bf16_bits(rng.standard_normal((T, H)).astype(np.float32)))
    x[:, rng.choice(H, max(1, H // 100), replace=False)] *= 20.0
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[:, E - 1] = -np.inf                       # one expert stays empty
    rt = orc.route(lg, k)
    rows = T * k
    ns = H // 2 if n_select is None else n_select
    d = orc.quantize_rac(x, ns)
    W = [(rng.standard_normal((2 * I, H)) * 0.02).astype(np.float32) for _ in range(E)]
    wq = [orc.quantize(m) for m in W]
    wst = (np.stack([q[0] for q in wq]), np.stack([q[1] for q in wq]),
           np.array([q[2] for q in wq], np.float32))
    a = (d["codes"], d["scales"], d["s_t"])
    r = (d["res_codes"], d["res_scales"], d["s_tr"]) if rac else None
    y_ref = orc.grouped_gemm(2 * I, H, rt["offsets"], rt["gather"], a, r, wst)

    out_y = torch.full((rows, 2 * I), float("nan"), dtype=torch.float32, device=DEV)
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    h = L.w4a4_grouped_gemm_rac(
        _nv(*a), _nv(*wst), _dev(rt["offsets"]), N=2 * I, K=H, total_rows=rows,
        gather_rows=_dev(rt["gather"]), r=_nv(*r) if rac else None,
        kblock_active=_dev(d["active"]) if rac else None,
        epilogue=L.NVFP4_EPI_SILU_MUL_BF16, out_amax=amax, skip_inactive=skip, out_y=out_y,
        validate=True)
    y = host(out_y)
    assert np.isfinite(y).all(), "every output row written"
    err = rel_frob(y, y_ref)
    say(f"  gate/up FP32 rel frob {err:.3e}")
    assert err <= REL_F
    h_gpu = host(h.view(torch.int16)).view(np.uint16)
    amax_ref = _check_h(h_gpu, y_ref, y, I, "gate/up")
    assert abs(host(amax)[0] - amax_ref) <= amax_ref * 2.0 ** -7
    return d


@pytest.mark.parametrize("T,E,k,H,I", [(300, 6, 2, 512, 256),    # 64 x 256 tiles
                                       (257, 5, 2, 384, 192),    # N % 256 != 0: 64 x 128
                                       (96, 3, 3, 1024, 128)])
def test_gate_up_f32(orc, T, E, k, H, I):
    say(f"gate/up SiLU FP32 side output T={T} E={E} k={k} H={H} I={I}")
    _gateup_case(orc, T, E, k, H, I, seed=T + E)


def test_gate_up_f32_rac_off(orc):
    say("gate/up SiLU FP32 side output, RAC off")
    _gateup_case(orc, 200, 4, 2, 512, 256, rac=False, seed=7)


@pytest.mark.parametrize("I", [256, 192])
def test_gate_up_f32_block_skipping(orc, I):
    """A sparse selection (most 16-blocks inactive) with the SiLU epilogue and
    NVFP4_GEMM_SKIP_INACTIVE_BLOCKS."""
    say(f"gate/up SiLU with block skipping I={I}")
    d = _gateup_case(orc, 180, 4, 2, 512, I, n_select=24, skip=True, seed=11)
    assert (d["active"] == 0).sum() >= 512 // 16 // 2


def test_full_moe_ffn_e128_gate_up_and_down(orc):
    """The MoE FFN workload (128 experts, top-8, 4096 tokens, H = 2048,
    I = 768) at full size: the whole gate/up FP32 output (32768 x 1536) and
    the whole down output (32768 x 2048, on the oracle's H) against the
    oracle's exact GEMMs; H in full within one bf16 ulp."""
    _ORC["o"] = orc
    w = D.WORKLOADS[3]
    rows = w.T * w.topk
    say(f"full gate/up + down FP32 {w.name}")
    x, lg = D.activations(w), D.router_logits(w)
    rt = orc.route(lg, w.topk)
    d = orc.quantize_rac(x, w.n_select_x)

    def bank(which, N, K):
        q = [orc.quantize(m) for _, m in D.expert_weights(w, which)]
        return (np.stack([t[0] for t in q]), np.stack([t[1] for t in q]),
                np.array([t[2] for t in q], np.float32))
    wgu = bank("gate_up", 2 * w.I, w.H)
    a = (d["codes"], d["scales"], d["s_t"])
    r = (d["res_codes"], d["res_scales"], d["s_tr"])
    y_ref = orc.grouped_gemm(2 * w.I, w.H, rt["offsets"], rt["gather"], a, r, wgu)
    offs, gat = _dev(rt["offsets"]), _dev(rt["gather"])
    out_y = torch.full((rows, 2 * w.I), float("nan"), dtype=torch.float32, device=DEV)
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    h = L.w4a4_grouped_gemm_rac(_nv(*a), _nv(*wgu), offs, N=2 * w.I, K=w.H, total_rows=rows,
                                gather_rows=gat, r=_nv(*r), kblock_active=_dev(d["active"]),
                                epilogue=L.NVFP4_EPI_SILU_MUL_BF16, out_amax=amax, out_y=out_y,
                                validate=True)
    y = host(out_y)
    err = rel_frob(y, y_ref)
    say(f"  gate/up FP32 rel frob {err:.3e} over {y.size} values")
    assert np.isfinite(y).all() and err <= REL_F
    h_gpu = host(h.view(torch.int16)).view(np.uint16)
    _check_h(h_gpu, y_ref, y, w.I, "gate/up")
    del y, out_y, wgu

    # down projection on the oracle's H, every output compared
    h_ref, amax_h = _silu(y_ref, w.I)
    hf = D.bf16_to_f32(h_ref)
    dh = orc.quantize_rac(hf, w.n_select_h, amax=float(amax_h))
    wd = bank("down", w.H, w.I)
    ad = (dh["codes"], dh["scales"], dh["s_t"])
    rd = (dh["res_codes"], dh["res_scales"], dh["s_tr"])
    yd_ref = orc.grouped_gemm(w.H, w.I, rt["offsets"], None, ad, rd, wd)
    yd = L.w4a4_grouped_gemm_rac(_nv(*ad), _nv(*wd), offs, N=w.H, K=w.I, total_rows=rows,
                                 r=_nv(*rd), kblock_active=_dev(dh["active"]))
    err = rel_frob(host(yd), yd_ref)
    say(f"  down FP32 rel frob {err:.3e} over {yd_ref.size} values")
    assert err <= REL_F


@pytest.mark.parametrize("silu", [True, False])
def test_tail_tiles_every_size(orc, silu):
    """Experts whose last 128-row m-tile holds 1, 31, 32, 33, 63, 64 or 65
    rows (and whole tiles) in the 128 x 512 configuration: tails of at most
    64 rows run with every wave on the same rows (narrow), longer ones with
    two wave rows.  FP32 outputs (or the FP32 side output of SiLU*mul) at
    1e-5, H against the oracle's SiLU*mul."""
    _ORC["o"] = orc
    sizes = [1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 160, 191, 192, 193, 256, 300, 0, 2]
    G, H, N = len(sizes), 512, 512
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    total = int(off[-1])
    say(f"tail tiles silu={silu} rows={total}")
    rng = np.random.default_rng(5 + silu)
    src = 150
    x = D.bf16_to_f32(D.bf16_bits(rng.standard_normal((src, H)).astype(np.float32)))
    x[:, rng.choice(H, 5, replace=False)] *= 20.0
    gat = rng.integers(0, src, total).astype(np.int32)
    d = orc.quantize_rac(x, H // 2)
    wq = [orc.quantize((rng.standard_normal((N, H)) * 0.02).astype(np.float32)) for _ in range(G)]
    w = (np.stack([q[0] for q in wq]), np.stack([q[1] for q in wq]),
         np.array([q[2] for q in wq], np.float32))
    a = (d["codes"], d["scales"], d["s_t"])
    r = (d["res_codes"], d["res_scales"], d["s_tr"])
    y_ref = orc.grouped_gemm(N, H, off, gat, a, r, w)
    kw = dict(N=N, K=H, total_rows=total, gather_rows=_dev(gat), r=_nv(*r),
              kblock_active=_dev(d["active"]), validate=True)
    if not silu:
        y = host(L.w4a4_grouped_gemm_rac(_nv(*a), _nv(*w), _dev(off), **kw))
        err = rel_frob(y, y_ref)
        say(f"  FP32 rel frob {err:.3e}")
        assert err <= REL_F
        return
    out_y = torch.full((total, N), float("nan"), dtype=torch.float32, device=DEV)
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    h = L.w4a4_grouped_gemm_rac(_nv(*a), _nv(*w), _dev(off), epilogue=L.NVFP4_EPI_SILU_MUL_BF16,
                                out_amax=amax, out_y=out_y, **kw)
    y = host(out_y)
    assert np.isfinite(y).all(), "every output row written"
    err = rel_frob(y, y_ref)
    say(f"  gate/up FP32 rel frob {err:.3e}")
    assert err <= REL_F
    amax_ref = _check_h(host(h.view(torch.int16)).view(np.uint16), y_ref, y, N // 2, "gate/up")
    assert abs(host(amax)[0] - amax_ref) <= amax_ref * 2.0 ** -7
