"""Seeded synthetic inputs for the NVFP4 W4A4 + RAC hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, so both the GPU path and the CPU oracle take their inputs
from here.  Every stream is ``numpy.random.default_rng([workload, stream,
expert])`` (PCG64 seeded through SeedSequence); floats are drawn in FP32 and
cast to bf16 with round-to-nearest-even where a workload says bf16.

The workloads stand in for the MoE rollout GEMMs of the QUADS pages (the
pages evaluate on public benchmarks with a trained model; none of that is
reproduced).  Shapes and value distributions:

  1 dense      X fp32 [64, 256] ~ N(0,1), 4 channels x20; W fp32 [256, 256]
               ~ N(0, 0.02^2); select 128.
  2 decode     X bf16 [16, 4096] ~ N(0,1), 41 channels (1%) x30; W bf16
               [4096, 4096] ~ N(0, 0.02^2); select 2048.
  3 moe        T=4096, E=128, top-8, H=2048, I=768; X bf16 ~ N(0,1), 20
               channels (1%) x20; logits ~ N(0,1); per expert W_gu [1536, 2048]
               and W_d [2048, 768] ~ N(0, 0.02^2) bf16.
  4 moe-skew   as 3 with T=16384, 10 channels (0.5%) x50; expert popularity
               p_e ~ rank^-1.2 (Zipf) over 120 experts with 8 experts never
               chosen; logits = ln p_e + Gumbel(0,1) (-inf when p_e = 0), so
               top-8 is popularity-proportional sampling without replacement.
  5 moe-large  T=8192, E=256, top-8, H=7168, I=2048; X bf16 ~ Student-t(3);
               logits ~ N(0,1).

Streams: 1 = X, 2 = outlier channels, 3 = W (dense or gate/up), 4 = W_down,
5 = routing, 6 = expert popularity permutation.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

S_X, S_OUTLIER, S_W, S_WDOWN, S_ROUTE, S_PERM = 1, 2, 3, 4, 5, 6


@dataclasses.dataclass(frozen=True)
class Workload:
    seed: int            # first SeedSequence word
    name: str
    kind: str            # "dense" | "moe"
    x_dtype: str         # "f32" | "bf16"
    x_dist: str = "normal"          # "normal" | "student_t3"
    n_outliers: int = 0
    outlier_scale: float = 1.0
    w_std: float = 0.02
    # dense
    rows: int = 0
    K: int = 0
    N: int = 0
    # moe
    T: int = 0
    E: int = 0
    topk: int = 0
    H: int = 0
    I: int = 0
    routing: str = "normal"         # "normal" | "zipf"
    zipf_s: float = 1.2
    n_empty: int = 0

    @property
    def n_select_x(self) -> int:
        return (self.K if self.kind == "dense" else self.H) // 2

    @property
    def n_select_h(self) -> int:
        return self.I // 2


WORKLOADS = {
    1: Workload(1, "dense_linear_64x256x256_f32", "dense", "f32", n_outliers=4,
                outlier_scale=20.0, rows=64, K=256, N=256),
    2: Workload(2, "decode_linear_16x4096x4096_bf16", "dense", "bf16",
                n_outliers=41, outlier_scale=30.0, rows=16, K=4096, N=4096),
    3: Workload(3, "moe_ffn_e128_top8_t4096_h2048_i768", "moe", "bf16",
                n_outliers=20, outlier_scale=20.0, T=4096, E=128, topk=8,
                H=2048, I=768),
    4: Workload(4, "moe_ffn_skew_zipf1.2_e128_top8_t16384_h2048_i768", "moe",
                "bf16", n_outliers=10, outlier_scale=50.0, T=16384, E=128,
                topk=8, H=2048, I=768, routing="zipf", n_empty=8),
    5: Workload(5, "moe_ffn_e256_top8_t8192_h7168_i2048", "moe", "bf16",
                x_dist="student_t3", T=8192, E=256, topk=8, H=7168, I=2048),
}


def small_moe(seed: int, T: int, E: int, topk: int, H: int, I: int, *,
              n_outliers: int = 2, outlier_scale: float = 20.0,
              routing: str = "normal", n_empty: int = 0,
              x_dist: str = "normal") -> Workload:
    """A reduced MoE workload with the same recipe (for parity tests)."""
    return Workload(seed, f"moe_small_s{seed}_t{T}_e{E}_h{H}_i{I}", "moe",
                    "bf16", x_dist=x_dist, n_outliers=n_outliers,
                    outlier_scale=outlier_scale, T=T, E=E, topk=topk, H=H, I=I,
                    routing=routing, n_empty=n_empty)


def small_dense(seed: int, rows: int, K: int, N: int, *, x_dtype="bf16",
                n_outliers: int = 2, outlier_scale: float = 20.0) -> Workload:
    return Workload(seed, f"dense_small_s{seed}_{rows}x{K}x{N}", "dense",
                    x_dtype, n_outliers=n_outliers, outlier_scale=outlier_scale,
                    rows=rows, K=K, N=N)


def rng(w: Workload, stream: int, expert: int = 0) -> np.random.Generator:
    return np.random.default_rng([w.seed, stream, expert])


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """FP32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _round_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_to_f32(bf16_bits(a)) if dtype == "bf16" else a.astype(np.float32)


def activations(w: Workload) -> np.ndarray:
    """X as FP32 values (exactly bf16-representable when x_dtype is bf16)."""
    rows, K = (w.rows, w.K) if w.kind == "dense" else (w.T, w.H)
    g = rng(w, S_X)
    if w.x_dist == "student_t3":
        x = g.standard_t(3, size=(rows, K)).astype(np.float32)
    else:
        x = g.standard_normal((rows, K), dtype=np.float32)
    if w.n_outliers:
        ch = rng(w, S_OUTLIER).choice(K, size=w.n_outliers, replace=False)
        x[:, ch] *= np.float32(w.outlier_scale)
    return _round_dtype(x, w.x_dtype)


def outlier_channels(w: Workload) -> np.ndarray:
    K = w.K if w.kind == "dense" else w.H
    if not w.n_outliers:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rng(w, S_OUTLIER).choice(K, size=w.n_outliers, replace=False))


def _normal_w(w: Workload, stream: int, expert: int, shape) -> np.ndarray:
    a = rng(w, stream, expert).standard_normal(shape, dtype=np.float32)
    a *= np.float32(w.w_std)
    return _round_dtype(a, "f32" if w.x_dtype == "f32" else "bf16")


def dense_weight(w: Workload) -> np.ndarray:
    """W [N, K] (out x in), y = x W^T."""
    return _normal_w(w, S_W, 0, (w.N, w.K))


def expert_gate_up(w: Workload, e: int) -> np.ndarray:
    """Fused gate/up weight of expert e: [2I, H], gate rows first."""
    return _normal_w(w, S_W, e, (2 * w.I, w.H))


def expert_down(w: Workload, e: int) -> np.ndarray:
    """Down weight of expert e: [H, I]."""
    return _normal_w(w, S_WDOWN, e, (w.H, w.I))


def expert_weights(w: Workload, which: str, experts=None, threads: int = 8):
    """Yield (e, W_e) over experts, drawn on a thread pool (NumPy releases
    the GIL while filling)."""
    fn = expert_gate_up if which == "gate_up" else expert_down
    experts = list(range(w.E)) if experts is None else list(experts)
    with ThreadPoolExecutor(max(1, threads)) as ex:
        chunk = max(1, threads * 2)
        for i in range(0, len(experts), chunk):
            part = experts[i:i + chunk]
            for e, a in zip(part, ex.map(lambda e: fn(w, e), part)):
                yield e, a


def router_logits(w: Workload) -> np.ndarray:
    """FP32 router logits [T, E]."""
    if w.routing == "zipf":
        perm = rng(w, S_PERM).permutation(w.E)      # expert -> popularity slot
        empty = perm[w.E - w.n_empty:]               # the n_empty least popular
        ranks = np.empty(w.E, dtype=np.float64)
        ranks[perm] = np.arange(1, w.E + 1, dtype=np.float64)
        logp = -w.zipf_s * np.log(ranks)
        logp[empty] = -np.inf
        gum = rng(w, S_ROUTE).gumbel(size=(w.T, w.E))
        return (logp[None, :] + gum).astype(np.float32)
    return rng(w, S_ROUTE).standard_normal((w.T, w.E), dtype=np.float32)


S_HIDDEN = 7


def hidden_like(w: Workload, rows: int) -> np.ndarray:
    """A seeded stand-in for the expert intermediate H [rows, I] (bf16 values):
    the product of two N(0, 0.05^2) draws through silu, i.e. the distribution
    silu(g) * u of a gate/up output, for testing the H-side quantizer and the
    down projection on their own."""
    g = rng(w, S_HIDDEN)
    a = g.standard_normal((rows, w.I), dtype=np.float32) * np.float32(0.05)
    b = g.standard_normal((rows, w.I), dtype=np.float32) * np.float32(0.05)
    h = a / (np.float32(1.0) + np.exp(-a)) * b
    return _round_dtype(h.astype(np.float32), "bf16")
