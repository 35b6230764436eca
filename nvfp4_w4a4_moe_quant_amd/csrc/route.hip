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
//              LDS bit masks, then gather_rows / row_of.  When blocks^2 x E
//              is small, each block sums the counts itself (the earlier
//              blocks' for its base, all blocks' for the offsets) and k_scan
//              is not launched.
//   k_route1   at most 64 tokens (a decode step): all of the above in one
//              workgroup, the ids, counts and ranks kept in LDS -- one launch
//              instead of three.
#include "common.h"

namespace {

constexpr int kTok = 256;
constexpr int kMaxE = 1024;
constexpr int kMaxK = 16;
constexpr int64_t kSelfScanLoads = 1 << 20;  // nblk^2 x E bound of the fused scan

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Top-k of token t by one wave: k rounds of a wave arg-max.  PER logits per
// lane (E <= 64 * PER), so the per-lane scan is unrolled to exactly the
// lanes' share and has no branches.  Lane 0 writes the ids (and, with sid, a
// copy to LDS); wts, when given, gets the softmax weights of the k chosen.
template <int PER>
__device__ __forceinline__ void topk_token(const float* __restrict__ logits, int64_t t, int E,
                                           int k, int32_t* __restrict__ ids,
                                           float* __restrict__ wts, int32_t* sid) {
  const int lane = threadIdx.x & 63;
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
    if (lane == 0) {
      ids[t * k + s] = bi;
      if (sid) sid[t * k + s] = bi;
    }
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

// One wave per token.
template <int PER>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int64_t T, int E,
                                              int k, int32_t* __restrict__ ids,
                                              float* __restrict__ wts) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_token<PER>(logits, t, E, k, ids, wts, nullptr);
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

// kSelf: the block computes its own base and the expert offsets from the
// per-block counts cnt[nblk][E] (block 0 writes offsets); otherwise base and
// offsets come from k_scan.
template <bool kSelf>
__global__ __launch_bounds__(kTok) void k_scatter(const int32_t* __restrict__ ids, int64_t T,
                                                  int E, int k, const int32_t* __restrict__ base,
                                                  int nblk, int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ gather,
                                                  int32_t* __restrict__ row_of) {
  __shared__ uint32_t bits[kMaxE * (kTok / 32)];
  __shared__ int32_t sbase[kSelf ? kMaxE : 1];  // first row of expert e in this block
  for (int i = threadIdx.x; i < E * (kTok / 32); i += kTok) bits[i] = 0u;
  const int tl = threadIdx.x;
  // the token's experts are loaded first, so that their latency overlaps the
  // count sums below
  const int64_t t = (int64_t)blockIdx.x * kTok + tl;
  int32_t my[kMaxK];
  if (t < T)
    for (int s = 0; s < k; ++s) my[s] = ids[t * k + s];
  if constexpr (kSelf) {
    // thread tl owns experts [per tl, per tl + per): rows in earlier blocks
    // (run) and in all blocks (tot), then a scan of the totals.  The counts
    // of 16 blocks are loaded before any is added.
    constexpr int kPer = kMaxE / kTok, kB = 16;
    __shared__ int32_t wtot[kTok / 64];
    const int per = (E + kTok - 1) / kTok;
    int32_t run[kPer], tot[kPer], mine = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) run[j] = tot[j] = 0;
    for (int b0 = 0; b0 < nblk; b0 += kB) {
      int32_t c[kB][kPer];
#pragma unroll
      for (int u = 0; u < kB; ++u)
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int e = tl * per + j;
          c[u][j] = (j < per && e < E && b0 + u < nblk) ? base[(int64_t)(b0 + u) * E + e] : 0;
        }
#pragma unroll
      for (int u = 0; u < kB; ++u)
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          tot[j] += c[u][j];
          run[j] += b0 + u < (int)blockIdx.x ? c[u][j] : 0;
        }
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) mine += tot[j];
    const int lane = tl & 63, w = tl >> 6;
    int32_t inc = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t n = __shfl_up(inc, o, 64);
      if (lane >= o) inc += n;
    }
    if (lane == 63) wtot[w] = inc;
    __syncthreads();
    int32_t off = inc - mine;
    for (int i = 0; i < w; ++i) off += wtot[i];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = tl * per + j;
      if (j < per && e < E) {
        sbase[e] = off + run[j];
        if (blockIdx.x == 0) offsets[e] = off;
      }
      off += tot[j];
    }
    if (blockIdx.x == 0 && tl == kTok - 1) offsets[E] = off;  // the total
  }
  __syncthreads();
  if (t < T)
    for (int s = 0; s < k; ++s) atomicOr(&bits[my[s] * (kTok / 32) + (tl >> 5)], 1u << (tl & 31));
  __syncthreads();
  if (t < T) {
    for (int s = 0; s < k; ++s) {
      const int e = my[s];
      const uint32_t* m = bits + e * (kTok / 32);
      int rank = __builtin_popcount(m[tl >> 5] & ((1u << (tl & 31)) - 1u));
      for (int w = 0; w < (tl >> 5); ++w) rank += __builtin_popcount(m[w]);
      const int32_t pos =
          (kSelf ? sbase[e] : offsets[e] + base[(int64_t)blockIdx.x * E + e]) + rank;
      gather[pos] = (int32_t)t;
      row_of[t * k + s] = pos;
    }
  }
}

// ------------------------------------------------- one-workgroup routing
// T <= kR1MaxT: wave w takes tokens w, w + 16, ... (at most four: beyond
// that the separate top-k launch, a wave per token over many CUs, is
// faster); then, from LDS, the expert counts, their exclusive scan (the
// offsets; thread e holds expert e) and the rank of each token inside its
// expert by bit masks, as k_counts, k_scan and k_scatter do for one block.
constexpr int kR1Threads = 1024;
constexpr int kR1MaxT = 4 * (kR1Threads / 64);
constexpr int kR1Words = kR1MaxT / 32;  // token bit-mask words per expert

template <int PER>
__global__ __launch_bounds__(kR1Threads) void k_route1(const float* __restrict__ logits, int T,
                                                       int E, int k, int32_t* __restrict__ ids,
                                                       float* __restrict__ wts,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ gather,
                                                       int32_t* __restrict__ row_of) {
  __shared__ int32_t sid[kR1MaxT * kMaxK];
  __shared__ int32_t sbase[kMaxE];  // counts, then each expert's first row
  __shared__ uint32_t bits[kMaxE * kR1Words];
  __shared__ int32_t wtot[kR1Threads / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < E; i += kR1Threads) sbase[i] = 0;
  for (int i = tid; i < E * kR1Words; i += kR1Threads) bits[i] = 0u;
  for (int t = w; t < T; t += kR1Threads / 64) topk_token<PER>(logits, t, E, k, ids, wts, sid);
  __syncthreads();
  if (tid < T)
    for (int s = 0; s < k; ++s) {
      const int e = sid[tid * k + s];
      atomicAdd(&sbase[e], 1);
      atomicOr(&bits[e * kR1Words + (tid >> 5)], 1u << (tid & 31));
    }
  __syncthreads();
  // exclusive scan of the counts over the experts
  const int32_t c = tid < E ? sbase[tid] : 0;
  int32_t inc = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t n = __shfl_up(inc, o, 64);
    if (lane >= o) inc += n;
  }
  if (lane == 63) wtot[w] = inc;
  __syncthreads();
  int32_t before = 0, total = 0;
  for (int i = 0; i < kR1Threads / 64; ++i) {
    before += i < w ? wtot[i] : 0;
    total += wtot[i];
  }
  const int32_t off = before + inc - c;
  if (tid < E) {
    offsets[tid] = off;
    sbase[tid] = off;
  }
  if (tid == 0) offsets[E] = total;
  __syncthreads();
  if (tid < T) {
    for (int s = 0; s < k; ++s) {
      const int e = sid[tid * k + s];
      const uint32_t* m = bits + e * kR1Words;
      int rank = __builtin_popcount(m[tid >> 5] & ((1u << (tid & 31)) - 1u));
      for (int i = 0; i < (tid >> 5); ++i) rank += __builtin_popcount(m[i]);
      const int32_t pos = sbase[e] + rank;
      gather[pos] = tid;
      row_of[tid * k + s] = pos;
    }
  }
}

// ---------------------------------------------------------------- combine
// out[t, :] = sum over the token's k slots, in slot order, of
// w[t, s] * y[row_of[t, s], :]: one FP32 product and one FP32 addition per
// slot (unfused, the same order for every element), then FP32 or bf16.  A
// thread owns 8 consecutive columns of one token and loads all k rows before
// the first addition; consecutive threads read consecutive 32-byte pieces.
template <int KMAX, bool kBf16Out>
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y,
                                                 const int32_t* __restrict__ row_of,
                                                 const float* __restrict__ w, int64_t T, int k,
                                                 int64_t H, void* __restrict__ out) {
  const int64_t nv = H >> 3;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * nv) return;
  const int64_t t = i / nv, hv = i - t * nv;
  float4 a[KMAX], b[KMAX];
  float ws[KMAX];
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    if (s < k) {
      const int64_t r = row_of[t * k + s];
      ws[s] = w[t * k + s];
      const float4* p = reinterpret_cast<const float4*>(y + r * H + hv * 8);
      a[s] = p[0];
      b[s] = p[1];
    }
  }
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    if (s < k) {
      const float v[8] = {a[s].x, a[s].y, a[s].z, a[s].w, b[s].x, b[s].y, b[s].z, b[s].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] + ws[s] * v[e];
    }
  }
  if constexpr (kBf16Out) {
    uint4 o;
    o.x = nv_f32_to_bf16(acc[0]) | (nv_f32_to_bf16(acc[1]) << 16);
    o.y = nv_f32_to_bf16(acc[2]) | (nv_f32_to_bf16(acc[3]) << 16);
    o.z = nv_f32_to_bf16(acc[4]) | (nv_f32_to_bf16(acc[5]) << 16);
    o.w = nv_f32_to_bf16(acc[6]) | (nv_f32_to_bf16(acc[7]) << 16);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + t * H + hv * 8) = o;
  } else {
    float4* d = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + t * H + hv * 8);
    d[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    d[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

template <int KMAX>
int launch_combine(const float* y, const int32_t* row_of, const float* w, int64_t T, int k,
                   int64_t H, bool bf16, void* out, hipStream_t s) {
  const unsigned grid = (unsigned)((T * (H >> 3) + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL((k_combine<KMAX, true>), dim3(grid), dim3(256), 0, s, y, row_of, w, T, k,
                       H, out);
  else
    hipLaunchKernelGGL((k_combine<KMAX, false>), dim3(grid), dim3(256), 0, s, y, row_of, w, T, k,
                       H, out);
  return nv_launch_status();
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
  // per-token buffers may be NULL when T == 0 (empty tensors have no storage)
  NV_RETURN_IF(!expert_offsets || (T > 0 && (!logits || !topk_ids || !gather_rows || !row_of)),
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
  if (T > 0 && T <= kR1MaxT) {
#define NV_ROUTE1(PER)                                                                       \
  hipLaunchKernelGGL(k_route1<PER>, dim3(1), dim3(kR1Threads), 0, s, logits, (int)T, (int)E, \
                     (int)k, topk_ids, topk_weights, expert_offsets, gather_rows, row_of)
    if (E <= 64) NV_ROUTE1(1);
    else if (E <= 128) NV_ROUTE1(2);
    else if (E <= 256) NV_ROUTE1(4);
    else if (E <= 512) NV_ROUTE1(8);
    else NV_ROUTE1(16);
#undef NV_ROUTE1
    return nv_launch_status();
  }
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
  // Every scatter block reads all nblk x E counts when it sums them itself;
  // beyond kSelfScanLoads in total the one-workgroup scan is cheaper.
  if (nblk * nblk * E <= kSelfScanLoads) {
    // at least one block: block 0 writes the offsets (all zero when T == 0)
    hipLaunchKernelGGL(k_scatter<true>, dim3((unsigned)(nblk > 0 ? nblk : 1)), dim3(kTok), 0, s,
                       topk_ids, T, (int)E, (int)k, cnt, (int)nblk, expert_offsets, gather_rows,
                       row_of);
    return nv_launch_status();
  }
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(kMaxE), 0, s, cnt, (int)nblk, (int)E, expert_offsets);
  hipLaunchKernelGGL(k_scatter<false>, dim3((unsigned)nblk), dim3(kTok), 0, s, topk_ids, T,
                     (int)E, (int)k, cnt, (int)nblk, expert_offsets, gather_rows, row_of);
  return nv_launch_status();
}

int moe_combine(const float* y, const int32_t* row_of, const float* topk_weights, int64_t T,
                int64_t k, int64_t H, int out_dtype, void* out, void* stream) {
  NV_RETURN_IF(out_dtype != NVFP4_IN_F32 && out_dtype != NVFP4_IN_BF16, NVFP4_ERR_DTYPE);
  NV_RETURN_IF(T < 0 || k < 1 || k > kMaxK || H <= 0 || H % 8 || T * (H >> 3) > (1LL << 38),
               NVFP4_ERR_SHAPE);
  if (T == 0) return NVFP4_OK;
  NV_RETURN_IF(!y || !row_of || !topk_weights || !out, NVFP4_ERR_NULL);
  NV_RETURN_IF(!nv_aligned16(y) || !nv_aligned16(out), NVFP4_ERR_ALIGN);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool bf = out_dtype == NVFP4_IN_BF16;
  if (k <= 1) return launch_combine<1>(y, row_of, topk_weights, T, (int)k, H, bf, out, s);
  if (k <= 2) return launch_combine<2>(y, row_of, topk_weights, T, (int)k, H, bf, out, s);
  if (k <= 4) return launch_combine<4>(y, row_of, topk_weights, T, (int)k, H, bf, out, s);
  if (k <= 8) return launch_combine<8>(y, row_of, topk_weights, T, (int)k, H, bf, out, s);
  return launch_combine<16>(y, row_of, topk_weights, T, (int)k, H, bf, out, s);
}

}  // extern "C"
