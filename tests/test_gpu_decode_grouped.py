"""The decode-shaped GEMM kernels on groups with few rows -- the experts of
a decode step, on average at most 32 rows per group, K % 512 == 0 (the wide
kernel: 128 columns per workgroup; 16-row tiles up to 16 rows per group on
average, 32-row tiles above, and above 8 and above 24 a second workgroup per
column block takes every other tile; a three-deep chunk ring for at most one
row per sixteen groups) -- and on one group with the
SiLU*mul epilogue (16-column slabs), against the oracle's exact grouped GEMM
on oracle-quantized operands.  FP32 outputs within relative Frobenius 1e-5;
with SiLU*mul, the FP32 gate/up side output within 1e-5, H within the
propagated one-ulp bound and max|H| within one bf16 ulp of the oracle's.
The cases cover empty groups, a group longer than one 16-row tile, a row
gather, RAC off, per-group tensor scales, K from 512 (two 256-k chunks) to
12288 with odd chunk counts, and grids of many groups with more workgroups
than the chip holds at once."""
import numpy as np
import pytest
import torch

import test_gpu_gateup_f32 as GU
from nvfp4_w4a4_moe_quant_amd import _lib as L
from nvfp4_w4a4_moe_quant_amd import datagen as D
from gpu_util import DEV, REL_F, host, rel_frob, say

pytestmark = pytest.mark.gpu


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _nv(c, s, t):
    return L.NVFP4(_t(c), _t(s), _t(np.atleast_1d(np.asarray(t, np.float32))))


def _x(rng, rows, K):
    x = (rng.standard_normal((rows, K)) * np.exp(rng.uniform(-1, 1, (rows, 1)))).astype(np.float32)
    x[:, rng.integers(0, K, 3)] *= 25.0
    return D.bf16_to_f32(D.bf16_bits(x))


CASES = [  # (seed, group sizes, K, N, rac, silu, gather source rows, per-group scales)
    (0, [1, 0, 2, 1, 0, 0, 3, 1, 0, 1, 2, 0] * 4, 1024, 256, True, True, 20, False),
    (1, [20, 1, 0, 2, 3, 0, 1, 5], 2048, 256, True, False, None, False),
    (2, [2, 1, 0, 0, 1, 3, 0, 1] * 2, 3072, 128, False, True, 9, False),
    (3, [1, 2, 0, 3, 1, 0, 4, 1, 0, 2, 1, 1], 1024, 384, True, False, 30, True),
    (4, [1, 2, 0, 1], 12288, 128, True, True, None, False),
    (5, [3, 0, 1, 17, 1, 2], 7168, 256, True, False, None, False),
    (6, [5], 2048, 256, True, True, None, False),
    (7, [9, 0, 1, 12, 0, 2, 2, 4], 4096, 512, True, True, 48, True),
    (8, [1, 0, 3, 2, 0, 1, 1, 0, 4, 1], 1536, 384, True, True, 12, False),
    (9, [2, 1, 0, 1], 512, 128, True, False, None, False),
    (10, [1, 1, 0, 2, 1, 0, 0, 3], 2560, 256, False, False, 7, True),
    # many groups, more workgroups than the chip holds at once (K = 512: two
    # chunks per workgroup)
    (11, [1, 2, 0, 3, 1, 2, 1, 1] * 12, 1024, 2048, True, True, 150, False),
    (12, [2, 1, 1, 3, 0, 1, 2, 1] * 16, 512, 2048, True, False, None, False),
    # 5-8 rows per group on average (one workgroup per column block walks a
    # 20-row group's two tiles), 9-16 (two workgroups take every other tile:
    # groups of 30 and 35 rows, three tiles), and 9-16 with every group
    # inside one tile (the second workgroups exit at once)
    (13, [9, 3, 0, 20, 6, 1, 8, 7] * 2, 2048, 256, True, True, 60, False),
    (14, [12, 30, 0, 9, 35, 3, 17, 20], 1024, 384, True, False, None, True),
    (15, [10, 11, 9, 12] * 8, 512, 2048, True, True, 200, False),
    # 32-row tiles: 17-24 rows per group on average (one workgroup per column
    # block; a 40-row group takes two tiles, a 1-row group one), and 25-32
    # (two workgroups take every other tile: a 70-row group, three tiles),
    # with the gather, RAC off, per-group scales and a padded last fragment
    (16, [20, 40, 1, 0, 17, 33, 24, 31], 2048, 256, True, True, 90, False),
    (17, [30, 70, 2, 0, 25, 40, 33, 31], 1024, 384, True, False, None, True),
    (18, [18, 23, 19, 21] * 4, 1536, 128, False, True, 40, False),
    (19, [29, 31, 27, 30, 26, 32, 28, 28] * 2, 512, 2048, True, False, None, False),
    # at most one row per sixteen groups (a one-token decode step): a
    # three-deep chunk ring
    (20, [0] * 60 + [1, 0, 2, 1], 1024, 256, True, True, 3, False),
    (21, [0, 1] + [0] * 30, 3072, 128, True, False, None, True),
]


@pytest.mark.parametrize("seed,sizes,K,N,rac,silu,src,per_group", CASES)
def test_decode_grouped_gemm(orc, seed, sizes, K, N, rac, silu, src, per_group):
    G = len(sizes)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    total = int(off[-1])
    assert total <= 32 * G or G == 1
    say(f"decode grouped gemm seed={seed} G={G} rows={total} K={K} N={N} rac={rac} "
        f"silu={silu} gather={src is not None} per_group={per_group}")
    rng = np.random.default_rng(1000 + seed)
    n_sel = K // 2
    x = _x(rng, src if src is not None else total, K)
    gat = rng.integers(0, src, total).astype(np.int32) if src is not None else None
    if per_group:
        d = orc.quantize_rac_grouped(x, off, gat, n_sel)
        gemm_gather = None                     # operands are already in grouped row order
    else:
        d = orc.quantize_rac(x, n_sel)
        gemm_gather = gat
    wq = [orc.quantize((rng.standard_normal((N, K)) * 0.02).astype(np.float32)) for _ in range(G)]
    w = (np.stack([q[0] for q in wq]), np.stack([q[1] for q in wq]),
         np.array([q[2] for q in wq], np.float32))
    a = (d["codes"], d["scales"], d["s_t"])
    r = (d["res_codes"], d["res_scales"], d["s_tr"]) if rac else None
    y_ref = orc.grouped_gemm(N, K, off, gemm_gather, a, r, w)
    kw = dict(N=N, K=K, total_rows=total, r=_nv(*r) if rac else None,
              kblock_active=_t(d["active"]) if rac else None,
              gather_rows=None if gemm_gather is None else _t(gemm_gather),
              per_group_scales=per_group, validate=True)
    if not silu:
        y = torch.full((total, N), float("nan"), dtype=torch.float32, device=DEV)
        L.w4a4_grouped_gemm_rac(_nv(*a), _nv(*w), _t(off), out=y, **kw)
        assert np.isfinite(host(y)).all(), "every output row written"
        err = rel_frob(host(y), y_ref)
        say(f"  FP32 rel frob {err:.3e}")
        assert err <= REL_F
        return
    out_y = torch.full((total, N), float("nan"), dtype=torch.float32, device=DEV)
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    h = L.w4a4_grouped_gemm_rac(_nv(*a), _nv(*w), _t(off), epilogue=L.NVFP4_EPI_SILU_MUL_BF16,
                                out_amax=amax, out_y=out_y, **kw)
    yg = host(out_y)
    assert np.isfinite(yg).all(), "every output row written"
    err = rel_frob(yg, y_ref)
    say(f"  gate/up FP32 rel frob {err:.3e}")
    assert err <= REL_F
    GU._ORC["o"] = orc
    amax_ref = GU._check_h(host(h.view(torch.int16)).view(np.uint16), y_ref, yg, N // 2, "gate/up")
    assert abs(host(amax)[0] - amax_ref) <= amax_ref * 2.0 ** -7
