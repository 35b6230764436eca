"""GPU parity of the FP8 W8A8 comparator (fp8_quantize_rows and
fp8_grouped_gemm, through the C ABI) against the CPU oracle.

Bars: codes and row scales bit-exact.  GEMM outputs element by element
within a bound derived from the FP8 matrix instruction's arithmetic, measured
on MI355X with in-bounds single-instruction probes: v_mfma_scale_f32_32x32x64_
f8f6f4 forms exact products and adds them in groups of 8 consecutive k, each
group aligned to the exponent E of its largest product with the bits below
2^(E-13) truncated; groups and instructions are then added in FP32.  So per
output |y_gpu - y_exact| <= s_a s_w (sum over groups of 7 * 2^(E_g - 13)
+ (K/64 + 4) 2^-24 sum_k |a_k w_k|) + 2^-23 |y|.  (On rows without outliers
the truncation never triggers and the error is FP32 rounding alone; both are
reported.)  SiLU*mul within one bf16 ulp plus the propagated GEMM bound.
GEMM inputs are the oracle's own codes and scales, so the GEMM is checked
independently of the quantizer."""
import numpy as np
import pytest
import torch

from nvfp4_w4a4_moe_quant_amd import _lib as L
from nvfp4_w4a4_moe_quant_amd import datagen as D

pytestmark = pytest.mark.gpu
from gpu_util import DEV, REL_F, bf16_ulp_ok, eq, host, rel_frob, say, to_dev


def _edge_rows(rng, rows, K, dtype):
    x = (rng.standard_normal((rows, K)) * np.exp(rng.uniform(-3, 3, (rows, 1)))).astype(np.float32)
    x[:, rng.integers(0, K, 3)] *= 30.0
    if rows > 3:
        x[0] = 0.0                               # zero row: scale 0, zero codes
        x[1, :min(K, 16)] = -1e-30               # negatives that round to -0
        x[2, K // 2] = 1e5                       # one outlier, the rest tiny or subnormal
        x[3] = np.float32(448.0) * np.linspace(-1, 1, K, dtype=np.float32)  # scale 1
    if dtype == "bf16":
        x = D.bf16_to_f32(D.bf16_bits(x))
    return x


@pytest.mark.parametrize("rows,K,dtype", [(1, 16, "f32"), (7, 48, "bf16"), (1000, 768, "bf16"),
                                          (257, 2048, "bf16"), (33, 4112, "f32"),
                                          (5, 7168, "bf16"), (3, 16384, "bf16"),
                                          (6, 8208, "f32")])
def test_fp8_quantize_rows_parity(orc, rows, K, dtype):
    say(f"fp8 quantize rows {rows}x{K} {dtype}")
    rng = np.random.default_rng(rows * 11 + K)
    x = _edge_rows(rng, rows, K, dtype)
    q = L.fp8_quantize_rows(to_dev(x, dtype))
    codes, scales = orc.fp8_quantize_rows(x)
    eq(host(q.scales), scales, "row scales")
    eq(host(q.codes), codes, "codes")


def _weights(orc, rng, G, N, K):
    w = (rng.standard_normal((G, N, K)) * 0.03).astype(np.float32)
    w[:, :, rng.integers(0, K, 2)] *= 10.0
    parts = [orc.fp8_quantize_rows(w[g]) for g in range(G)]
    return np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts])


def _offsets(rng, G, mean):
    if mean < 0:                                 # exactly -mean rows per group
        return np.concatenate([[0], np.cumsum(np.full(G, -mean))]).astype(np.int32)
    sizes = rng.integers(0, 2 * mean + 1, G)
    if G > 2:
        sizes[1] = 0                             # an empty group
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


_E4M3 = None


def _decode(orc, codes):
    global _E4M3
    if _E4M3 is None:
        t = np.array([orc.e4m3_value(b & 0x7F) for b in range(256)], np.float64)
        t[[0x7F, 0xFF]] = 0.0                    # NaN bytes: never produced
        _E4M3 = np.where(np.arange(256) & 0x80, -t, t)
    return _E4M3[codes]


def _fp8_bound(orc, ac, as_, wc, wsc, off, gat):
    """Per-output error bound of the FP8 GEMM (module docstring)."""
    A = np.abs(_decode(orc, ac))
    W = np.abs(_decode(orc, wc))
    G, N, K = wc.shape
    total = int(off[-1])
    bound = np.zeros((total, N))
    for g in range(G):
        for j0 in range(int(off[g]), int(off[g + 1]), 16):
            j1 = min(j0 + 16, int(off[g + 1]))
            src = gat[j0:j1] if gat is not None else np.arange(j0, j1)
            P = A[src][:, None, :] * W[g][None, :, :]          # |a_k w_k|
            gm = P.reshape(len(src), N, K // 8, 8).max(-1)
            e = np.floor(np.log2(np.where(gm > 0, gm, 1.0)))
            trunc = np.where(gm > 0, 7.0 * np.exp2(e - 13), 0.0).sum(-1)
            fp32 = (K / 64 + 4) * 2.0 ** -24 * P.sum(-1)
            bound[j0:j1] = (as_[src].astype(np.float64)[:, None] *
                            wsc[g].astype(np.float64)[None, :] * (trunc + fp32))
    return bound


def _run(orc, seed, G, N, K, mean_rows, src_rows, gather, silu, bf16out=False):
    rng = np.random.default_rng(seed)
    x = D.bf16_to_f32(D.bf16_bits(_edge_rows(rng, src_rows, K, "f32")))
    ac, as_ = orc.fp8_quantize_rows(x)
    wc, wsc = _weights(orc, rng, G, N, K)
    off = _offsets(rng, G, mean_rows)
    total = int(off[-1])
    gat = rng.integers(0, src_rows, total).astype(np.int32) if gather else None
    y = orc.fp8_grouped_gemm(N, K, off, gat, (ac, as_), (wc, wsc))
    bound = _fp8_bound(orc, ac, as_, wc, wsc, off, gat) + 2.0 ** -23 * np.abs(y)
    a = L.FP8(torch.from_numpy(ac).to(DEV), torch.from_numpy(as_).to(DEV))
    w = L.FP8(torch.from_numpy(wc).to(DEV), torch.from_numpy(wsc).to(DEV))
    gd = None if gat is None else torch.from_numpy(gat).to(DEV)
    out = L.fp8_grouped_gemm(a, w, torch.from_numpy(off).to(DEV), N=N, K=K, total_rows=total,
                             gather_rows=gd,
                             epilogue=(L.NVFP4_EPI_SILU_MUL_BF16 if silu else
                                       L.NVFP4_EPI_BF16 if bf16out else L.NVFP4_EPI_F32))
    if silu:
        I = N // 2
        h_ref, _ = orc.silu_mul(y, I)
        h = D.bf16_to_f32(host(out.view(torch.int16)).view(np.uint16)).astype(np.float64)
        hr = D.bf16_to_f32(h_ref).astype(np.float64)
        g, u = y[:, :I].astype(np.float64), y[:, I:].astype(np.float64)
        silu_g = g * 0.5 * (1.0 + np.tanh(0.5 * g))     # g * sigmoid(g), no overflow
        # |d silu/dg| <= 1.1; one bf16 ulp for the final rounding
        tol = (np.maximum(np.abs(hr), 2.0 ** -126) * 2.0 ** -7 + 1.1 * np.abs(u) * bound[:, :I]
               + np.abs(silu_g) * bound[:, I:])
        bad = np.abs(h - hr) > tol * 1.0001
        assert not bad.any(), f"{bad.sum()} SiLU outputs beyond the bound"
    elif bf16out:
        # the FP32 value within the bound, then one rounding to bf16 (nearest
        # even, 7 fraction bits: at most half an ulp, 2^-8 of the value)
        yb = D.bf16_to_f32(host(out.view(torch.int16)).view(np.uint16)).astype(np.float64)
        tol = bound + 2.0 ** -8 * (np.abs(y) + bound) * 1.0001
        bad = np.abs(yb - y) > tol
        assert not bad.any(), f"{bad.sum()} bf16 outputs beyond the bound"
    else:
        yg = host(out).astype(np.float64)
        bad = np.abs(yg - y) > bound
        assert not bad.any(), f"{bad.sum()} outputs beyond the bound, first " \
                              f"{np.argwhere(bad)[:4].tolist()}"
        print(f"rel Frobenius error {rel_frob(yg, y):.3e}")


@pytest.mark.parametrize("seed,G,N,K,mean_rows,src_rows,gather,silu", [
    (0, 1, 256, 256, 100, 100, False, False),     # dense, 128 x 256 tiles, ragged tail
    (1, 5, 384, 384, 70, 90, True, False),        # N % 256 != 0: 128 x 128 tiles
    (2, 4, 512, 512, 150, 300, True, True),       # SiLU, gather
    (3, 3, 384, 128, 40, 64, True, True),         # SiLU on 128 x 128 tiles, one chunk
    (4, 6, 512, 1024, 100, 500, True, False),     # several chunks and m-tiles per group
    (5, 2, 256, 2048, 1, 4, False, False),        # one-row groups
    (6, 1, 512, 256, -2300, 2300, False, False),  # one long group: 9 m-tiles, bands of 8, tail
    (7, 1, 384, 128, -2500, 2600, True, False),   # 20 m-tiles of 128 rows: three bands
])
def test_fp8_gemm_parity(orc, seed, G, N, K, mean_rows, src_rows, gather, silu):
    say(f"fp8 gemm seed={seed} G={G} N={N} K={K} rows~{mean_rows} gather={gather} silu={silu}")
    _run(orc, seed, G, N, K, mean_rows, src_rows, gather, silu)


@pytest.mark.parametrize("seed,G,N,K,mean_rows,src_rows,gather", [
    (20, 1, 512, 256, -2300, 2300, False),      # dense, 256 x 256 tiles in bands, ragged tail
    (21, 5, 384, 384, 70, 90, True),            # grouped, gather, 128 x 128 tiles
    (22, 1, 256, 1024, -40, 40, False),         # one short group (not the decode kernel)
])
def test_fp8_gemm_bf16_out(orc, seed, G, N, K, mean_rows, src_rows, gather):
    say(f"fp8 gemm bf16 out seed={seed} G={G} N={N} K={K} rows~{mean_rows} gather={gather}")
    _run(orc, seed, G, N, K, mean_rows, src_rows, gather, False, bf16out=True)


@pytest.mark.parametrize("rows,N,K,gather", [(16, 4096, 4096, False), (1, 256, 512, False),
                                           (7, 384, 1024, True), (64, 128, 2048, False),
                                           (65, 256, 512, False)])
def test_fp8_gemm_decode_shape(orc, rows, N, K, gather):
    """One group and at most 64 rows run the decode kernel (65 rows: the
    prefill tiles), checked with the same bound."""
    say(f"fp8 decode-shaped gemm rows={rows} N={N} K={K} gather={gather}")
    rng = np.random.default_rng(rows * 3 + K)
    src_rows = rows + 5 if gather else rows
    x = D.bf16_to_f32(D.bf16_bits(_edge_rows(rng, src_rows, K, "f32")))
    ac, as_ = orc.fp8_quantize_rows(x)
    wc, wsc = _weights(orc, rng, 1, N, K)
    off = np.array([0, rows], np.int32)
    gat = rng.integers(0, src_rows, rows).astype(np.int32) if gather else None
    y = orc.fp8_grouped_gemm(N, K, off, gat, (ac, as_), (wc, wsc))
    bound = _fp8_bound(orc, ac, as_, wc, wsc, off, gat) + 2.0 ** -23 * np.abs(y)
    out = L.fp8_grouped_gemm(L.FP8(torch.from_numpy(ac).to(DEV), torch.from_numpy(as_).to(DEV)),
                             L.FP8(torch.from_numpy(wc).to(DEV), torch.from_numpy(wsc).to(DEV)),
                             torch.from_numpy(off).to(DEV), N=N, K=K, total_rows=rows,
                             gather_rows=None if gat is None else torch.from_numpy(gat).to(DEV))
    yg = host(out).astype(np.float64)
    bad = np.abs(yg - y) > bound
    assert not bad.any(), f"{bad.sum()} outputs beyond the bound"
    print(f"rel Frobenius error {rel_frob(yg, y):.3e}")


def test_fp8_gemm_empty(orc):
    say("fp8 gemm empty problem")
    a = L.FP8(torch.zeros((1, 128), dtype=torch.uint8, device=DEV),
              torch.zeros(1, dtype=torch.float32, device=DEV))
    w = L.FP8(torch.zeros((2, 128, 128), dtype=torch.uint8, device=DEV),
              torch.zeros((2, 128), dtype=torch.float32, device=DEV))
    off = torch.zeros(3, dtype=torch.int32, device=DEV)
    out = L.fp8_grouped_gemm(a, w, off, N=128, K=128, total_rows=0)
    assert out.shape == (0, 128)
