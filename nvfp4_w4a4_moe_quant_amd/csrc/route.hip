// MoE top-k routing and the gather map of the grouped GEMM.
//
// The QUADS pages run an MoE LLM in rollout (arXiv abstract, mlsanity page
// "Abstract (arXiv)") but describe no router; this is the plain reading:
// per token the k largest logits (ties toward the lower expert index), groups
// ordered by expert with tokens ascending inside each group.  Everything is
// integer work after the logit comparisons, so the indices are bit-exact.
//
//   k_topk     one wave per token: k rounds of a wave arg-max (logits held in
//              registers, E/64 per lane rounded up to a power of two)
//   k_counts   per 256-token block, per-expert counts (LDS histogram)
//   k_scan     one workgroup: per-expert running sums over blocks, then an
//              exclusive scan of the expert totals for the offsets
//   k_scatter  per 256-token block: rank of each token inside its expert via
//              LDS bit masks, then gather_rows / row_of
#include "common.h"

namespace {

constexpr int kTok = 256;
constexpr int kMaxE = 1024;
constexpr int kMaxK = 16;

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// PER logits per lane (E <= 64 * PER), so the per-lane scan is unrolled to
// exactly the lanes' share and has no branches.
template <int PER>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int64_t T, int E,
                                              int k, int32_t* __restrict__ ids,
                                              float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float l[PER];
  bool live[PER];  // a real logit not taken yet
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = lane + 64 * j;
    live[j] = e < E;
    l[j] = live[j] ? logits[t * E + e] : -__builtin_inff();
  }
  float chosen[kMaxK];
  for (int s = 0; s < k; ++s) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = lane + 64 * j;
      const bool take = live[j] && better(l[j], e, bv, bi);
      bv = take ? l[j] : bv;
      bi = take ? e : bi;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      const bool take = better(ov, oi, bv, bi);
      bv = take ? ov : bv;
      bi = take ? oi : bi;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (bi == lane + 64 * j) live[j] = false;
    chosen[s] = bv;  // wave-uniform after the reduction
    if (lane == 0) ids[t * k + s] = bi;
  }
  if (wts) {
    const float mx = chosen[0];
    float den = 0.0f;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = lane + 64 * j;
      if (e < E) den += __expf(l[j] - mx);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o, 64);
    for (int s = 0; s < k; ++s)
      if (lane == s) wts[t * k + s] = __expf(chosen[s] - mx) / den;
  }
}

__global__ __launch_bounds__(kTok) void k_counts(const int32_t* __restrict__ ids, int64_t T, int E,
                                                 int k, int32_t* __restrict__ cnt) {
  __shared__ uint32_t hist[kMaxE];
  for (int e = threadIdx.x; e < E; e += kTok) hist[e] = 0u;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kTok + threadIdx.x;
  if (t < T)
    for (int s = 0; s < k; ++s) atomicAdd(&hist[ids[t * k + s]], 1u);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kTok) cnt[(int64_t)blockIdx.x * E + e] = (int32_t)hist[e];
}

// One workgroup, thread e = expert: running sums over the blocks (the loads of
// 8 blocks are issued before their stores), then an exclusive scan of the
// per-expert totals across the workgroup for the offsets.
__global__ __launch_bounds__(kMaxE) void k_scan(int32_t* __restrict__ cnt, int nblk, int E,
                                                int32_t* __restrict__ offsets) {
  __shared__ int32_t wtot[kMaxE / 64];
  const int e = threadIdx.x, lane = e & 63, w = e >> 6;
  int32_t run = 0;
  if (e < E) {
    for (int b0 = 0; b0 < nblk; b0 += 8) {
      int32_t c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = b0 + u < nblk ? cnt[(int64_t)(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (b0 + u < nblk) {
          cnt[(int64_t)(b0 + u) * E + e] = run;  // rows of expert e before block b0 + u
          run += c[u];
        }
    }
  }
  // exclusive scan of run over e
  int32_t inc = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t n = __shfl_up(inc, o, 64);
    if (lane >= o) inc += n;
  }
  if (lane == 63) wtot[w] = inc;
  __syncthreads();
  int32_t before = 0;
  for (int i = 0; i < w; ++i) before += wtot[i];
  if (e < E) offsets[e] = before + inc - run;
  if (e == E - 1) offsets[E] = before + inc;
}

__global__ __launch_bounds__(kTok) void k_scatter(const int32_t* __restrict__ ids, int64_t T,
                                                  int E, int k, const int32_t* __restrict__ base,
                                                  const int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ gather,
                                                  int32_t* __restrict__ row_of) {
  __shared__ uint32_t bits[kMaxE * (kTok / 32)];
  for (int i = threadIdx.x; i < E * (kTok / 32); i += kTok) bits[i] = 0u;
  __syncthreads();
  const int tl = threadIdx.x;
  const int64_t t = (int64_t)blockIdx.x * kTok + tl;
  int32_t my[kMaxK];
  if (t < T) {
    for (int s = 0; s < k; ++s) {
      my[s] = ids[t * k + s];
      atomicOr(&bits[my[s] * (kTok / 32) + (tl >> 5)], 1u << (tl & 31));
    }
  }
  __syncthreads();
  if (t < T) {
    for (int s = 0; s < k; ++s) {
      const int e = my[s];
      const uint32_t* m = bits + e * (kTok / 32);
      int rank = __builtin_popcount(m[tl >> 5] & ((1u << (tl & 31)) - 1u));
      for (int w = 0; w < (tl >> 5); ++w) rank += __builtin_popcount(m[w]);
      const int32_t pos = offsets[e] + base[(int64_t)blockIdx.x * E + e] + rank;
      gather[pos] = (int32_t)t;
      row_of[t * k + s] = pos;
    }
  }
}

}  // namespace

extern "C" {

size_t moe_route_workspace_size(int64_t T, int64_t E, int64_t) {
  const int64_t nblk = (T + kTok - 1) / kTok;
  return nv_round256(sizeof(int32_t) * (size_t)((nblk > 0 ? nblk : 1) * (E > 0 ? E : 1)));
}

int moe_route(const float* logits, int64_t T, int64_t E, int64_t k, int32_t* topk_ids,
              float* topk_weights, int32_t* expert_offsets, int32_t* gather_rows,
              int32_t* row_of, void* ws, size_t ws_bytes, void* stream) {
  NV_RETURN_IF(!logits || !topk_ids || !expert_offsets || !gather_rows || !row_of,
               NVFP4_ERR_NULL);
  NV_RETURN_IF(T < 0 || E < 1 || E > kMaxE || k < 1 || k > E || k > kMaxK ||
                   T * k > INT32_MAX,
               NVFP4_ERR_SHAPE);
  NV_RETURN_IF(!ws || ws_bytes < moe_route_workspace_size(T, E, k) ||
                   (reinterpret_cast<uintptr_t>(ws) & 3),
               NVFP4_ERR_WORKSPACE);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws);
  const int64_t nblk = (T + kTok - 1) / kTok;
  if (T > 0) {
    const dim3 grid((unsigned)((T + 3) / 4));
#define NV_TOPK(PER)                                                                        \
  hipLaunchKernelGGL(k_topk<PER>, grid, dim3(256), 0, s, logits, T, (int)E, (int)k, topk_ids, \
                     topk_weights)
    if (E <= 64) NV_TOPK(1);
    else if (E <= 128) NV_TOPK(2);
    else if (E <= 256) NV_TOPK(4);
    else if (E <= 512) NV_TOPK(8);
    else NV_TOPK(16);
#undef NV_TOPK
    hipLaunchKernelGGL(k_counts, dim3((unsigned)nblk), dim3(kTok), 0, s, topk_ids, T, (int)E,
                       (int)k, cnt);
  }
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(kMaxE), 0, s, cnt, (int)nblk, (int)E, expert_offsets);
  if (T > 0)
    hipLaunchKernelGGL(k_scatter, dim3((unsigned)nblk), dim3(kTok), 0, s, topk_ids, T, (int)E,
                       (int)k, cnt, expert_offsets, gather_rows, row_of);
  return nv_launch_status();
}

}  // extern "C"
