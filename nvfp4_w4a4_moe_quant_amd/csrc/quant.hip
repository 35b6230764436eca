// Online NVFP4 quantizer and Residual Activation Compensation (RAC) kernels.
//
// QUADS arXiv abstract (mlsanity page, "Abstract (arXiv)"): rollout
// activations are new at every step, so they are quantized to E2M1 with
// per-block scales at run time.  QUADS blog post ("Why 4-bit RL rollout collapses"), section "Two
// fixes, on two different sides": RAC ranks activation channels by
// quantization error, keeps about the worse half, and re-quantizes their
// residual for a second FP4 pass.
//
// Passes over x (row-major [rows, K], 16-element blocks along K):
//   k_amax      partial max|x| per workgroup (tensor amax); zeroes the RAC
//               statistics when k_quant adds them atomically
//   k_quant     tensor scale, block scales, E2M1 codes; optionally the exact
//               per-channel error statistics (score = sum q^2, max |e|)
//   k_rank      rank of every channel by (score desc, index asc); the
//               first n are selected; block masks and activity flags
//   k_residual  r = mask * e re-quantized in the same blocks with the
//               activation's tensor scale; the ascending selected indices
// All reductions are max or integer sums, so results are order-independent.

#include <mutex>

#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxParts = 1024;

// ------------------------------------------------------------------ amax
__global__ __launch_bounds__(kThreads) void k_amax(const void* __restrict__ x, int bf16,
                                                   int64_t rows, int64_t K, int64_t ldx,
                                                   float* __restrict__ partials,
                                                   int64_t* __restrict__ score,
                                                   uint32_t* __restrict__ chmax) {
  const int64_t cb_per_row = K >> 4;
  const int64_t nblk = rows * cb_per_row;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  // (row, block) advance incrementally: one 64-bit division per thread
  const int64_t srow = stride / cb_per_row, scb = stride - srow * cb_per_row;
  int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  int64_t r = b / cb_per_row, cb = b - r * cb_per_row;
  float m = 0.0f;
  for (; b < nblk; b += stride) {
    float v[16];
    nv_load16(x, bf16, r * ldx + cb * 16, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
    r += srow;
    cb += scb;
    if (cb >= cb_per_row) {
      cb -= cb_per_row;
      ++r;
    }
  }
  if (score) {
    for (int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x; k < K; k += stride) {
      score[k] = 0;
      if (chmax) chmax[k] = 0u;
    }
  }
  __shared__ float red[kThreads / 64];
  m = nv_wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = red[0];
    for (int w = 1; w < kThreads / 64; ++w) t = __builtin_fmaxf(t, red[w]);
    partials[blockIdx.x] = t;
  }
}

// Per-group tensor amax (per-expert RAC): workgroup (p, g) takes part p of
// the 16-element blocks of group g's rows, read through the gather when one
// is given, and writes partials[g * gridDim.x + p].  The grid also zeroes the
// per-group statistics [G, K].
__global__ __launch_bounds__(kThreads) void k_amax_grouped(
    const void* __restrict__ x, int bf16, int64_t K, int64_t ldx,
    const int32_t* __restrict__ goff, const int32_t* __restrict__ gather, int G,
    float* __restrict__ partials, int64_t* __restrict__ score, uint32_t* __restrict__ chmax) {
  const int g = blockIdx.y;
  const int CB = (int)(K >> 4);
  const int row0 = goff[g];
  const int nblk = (goff[g + 1] - row0) * CB;
  float m = 0.0f;
  for (int b = blockIdx.x * kThreads + threadIdx.x; b < nblk; b += gridDim.x * kThreads) {
    const int j = row0 + b / CB, cb = b - (b / CB) * CB;
    const int64_t src = gather ? (int64_t)gather[j] : (int64_t)j;
    float v[16];
    nv_load16(x, bf16, src * ldx + (int64_t)cb * 16, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
  }
  if (score) {
    const int64_t nwg = (int64_t)gridDim.x * gridDim.y;
    const int64_t wg = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    for (int64_t k = wg * kThreads + threadIdx.x; k < (int64_t)G * K; k += nwg * kThreads) {
      score[k] = 0;
      if (chmax) chmax[k] = 0u;
    }
  }
  __shared__ float red[kThreads / 64];
  m = nv_wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = red[0];
    for (int w = 1; w < kThreads / 64; ++w) t = __builtin_fmaxf(t, red[w]);
    partials[g * gridDim.x + blockIdx.x] = t;
  }
}

__global__ void k_zero_stats(int64_t K, int64_t* __restrict__ score, uint32_t* __restrict__ chmax) {
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < K;
       k += (int64_t)gridDim.x * blockDim.x) {
    score[k] = 0;
    if (chmax) chmax[k] = 0u;
  }
}

// Reduce the amax partials (or take amax_in) inside every workgroup.
__device__ float workgroup_amax(const float* __restrict__ partials, int nparts,
                                const float* __restrict__ amax_in, float* red) {
  if (amax_in) return *amax_in;
  float m = 0.0f;
  for (int i = threadIdx.x; i < nparts; i += blockDim.x) m = __builtin_fmaxf(m, partials[i]);
  m = nv_wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float t = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) t = __builtin_fmaxf(t, red[w]);
  return t;
}

// ------------------------------------------------------------- quantize
// grid.x: column tiles of `tpr` column blocks; grid.y: row splits.  Thread t
// handles column block (blockIdx.x * tpr + t % tpr) for rows
// start + t / tpr, start + t / tpr + rpi, ...  With statistics, per-channel
// partial sums of q^2 (q < 2^17) are accumulated in 64-bit integer registers
// (one v_mad_u64_u32 per element), combined in LDS, then added to the global
// int64 sums.  That costs one
// global atomic pair per channel and workgroup, and atomics on one address
// are serialized, so the host keeps the row splits few (about two
// workgroups per CU).  Workgroups of 8 waves, two per CU, run out of step,
// so one's loads overlap the other's arithmetic better than one 16-wave
// workgroup per CU.
constexpr int kQThreads = 512;

// Raw 16-element block as loaded (bf16: 8 dwords, fp32: 16 dwords); it is
// widened to FP32 only when used, which keeps several rows in flight within
// the 128 registers that four waves per SIMD leave.
template <bool kBf16>
struct RawBlock {
  uint32_t w[kBf16 ? 8 : 16];
  __device__ __forceinline__ void load(const void* x, int64_t off) {
    if constexpr (kBf16) {
      const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + off);
      const uint4 a = p[0], b = p[1];
      w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
      w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(x) + off);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 q = p[i];
        w[4 * i] = q.x; w[4 * i + 1] = q.y; w[4 * i + 2] = q.z; w[4 * i + 3] = q.w;
      }
    }
  }
  __device__ __forceinline__ void widen(float* v) const {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (kBf16)
        v[i] = __uint_as_float((i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16));
      else
        v[i] = __uint_as_float(w[i]);
    }
  }
};

// 16 dequantized values RN32(RN32(g s_b) s_t) of one block -> FP32 (kDq 1) or
// bf16 nearest even (kDq 2) at element offset o of out (row stride K).
template <int kDq>
__device__ __forceinline__ void dq_store16(void* out, int64_t o, uint32_t lo, uint32_t hi, float sb,
                                           float s_t) {
  float g[16];
  nv_decode8(lo, g);
  nv_decode8(hi, g + 8);
#pragma unroll
  for (int i = 0; i < 16; ++i) g[i] = (g[i] * sb) * s_t;
  if constexpr (kDq == 1) {
    float4* d = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + o);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = make_float4(g[4 * i], g[4 * i + 1], g[4 * i + 2], g[4 * i + 3]);
  } else {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = nv_f32_to_bf16(g[2 * i]) | (nv_f32_to_bf16(g[2 * i + 1]) << 16);
    uint4* d = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + o);
    d[0] = make_uint4(w[0], w[1], w[2], w[3]);
    d[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// kDq 0: codes and block scales.  kDq 1 / 2: the dequantized values instead
// (FP32 / bf16, row stride K) -- the trainer's weight fake-quantization runs
// the same quantizer and stores what the rollout's dequantization would give.
// kMax: with the statistics, also the per-channel max|e| (the selection does
// not read it; without it the kernel saves its arithmetic and atomics).
template <bool kStats, bool kBf16, int kDq = 0, bool kMax = true>
__global__ __launch_bounds__(kQThreads) void k_quant(
    const void* __restrict__ x, int64_t rows, int64_t K, int64_t ldx,
    const float* __restrict__ partials, int nparts, const float* __restrict__ amax_in,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ tscale_out,
    int64_t* __restrict__ score, uint32_t* __restrict__ chmax, int tpr, int rpi,
    int64_t rows_per_split, void* __restrict__ dq_out, const int32_t* __restrict__ goff,
    const int32_t* __restrict__ gather, int store_sums) {
  extern __shared__ unsigned char dyn_lds[];
  __shared__ float red[kQThreads / 64];
  // With goff (per-expert RAC) workgroup z quantizes group z's rows, grouped
  // rows [goff[z], goff[z+1]) read through the gather, as their own tensor:
  // its partial maxima, tensor scale and statistics are the group's.
  int64_t row0 = 0;
  if (goff) {
    const int g = blockIdx.z;
    row0 = goff[g];
    rows = goff[g + 1] - row0;
    partials += (int64_t)g * nparts;
    tscale_out += g;
    if (kStats) {
      score += (int64_t)g * K;
      if (kMax) chmax += (int64_t)g * K;
    }
    rows_per_split = (rows + gridDim.y - 1) / gridDim.y;
  }
  const float amax = workgroup_amax(partials, nparts, goff ? nullptr : amax_in, red);
  const float s_t = nv_tensor_scale(amax);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *tscale_out = s_t;
  // per-tensor constants of the block scales: c6 for the FP32 fast path of
  // the scale code, and rb of every code (one double division each, here)
  __shared__ float rb_lut[128];
  nv_fill_recip_lut(rb_lut, s_t);
  const float c6 = (float)(1.0 / (6.0 * (double)s_t));
  __syncthreads();

  const int64_t CB = K >> 4;
  const int sub = threadIdx.x / tpr;
  const int cbl = threadIdx.x - sub * tpr;
  const int64_t cb = (int64_t)blockIdx.x * tpr + cbl;
  const bool active = sub < rpi && cb < CB;
  const int64_t r0 = row0 + (int64_t)blockIdx.y * rows_per_split;
  const int64_t r1 = r0 + rows_per_split < row0 + rows ? r0 + rows_per_split : row0 + rows;
  const int shift = nv_score_shift(s_t);

  uint64_t acc[16];
  float emax[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    acc[i] = 0u;
    emax[i] = 0.0f;
  }

  auto block = [&](const RawBlock<kBf16>& raw, int64_t r) {
    float v[16];
    raw.widen(v);
    float amax_b = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax_b = __builtin_fmaxf(amax_b, __builtin_fabsf(v[i]));
    const uint32_t sc = nv_block_scale_c6(amax_b, s_t, c6);
    const float sb = nv_e4m3_to_f32(sc);
    const float rb = rb_lut[sc];
    const uint32_t lo = nv_encode8(v, rb), hi = nv_encode8(v + 8, rb);
    if constexpr (kStats) {
      float g[16];
      nv_decode8(lo, g);
      nv_decode8(hi, g + 8);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = v[i] - (g[i] * sb) * s_t;
        const uint32_t q = nv_score_qi(e, shift);
        acc[i] += (uint64_t)q * q;
        if constexpr (kMax) emax[i] = __builtin_fmaxf(emax[i], __builtin_fabsf(e));
      }
    }
    if constexpr (kDq == 0) {
      *reinterpret_cast<uint2*>(codes + r * (K >> 1) + cb * 8) = make_uint2(lo, hi);
      scales[r * CB + cb] = (uint8_t)sc;
    } else {
      dq_store16<kDq>(dq_out, r * K + cb * 16, lo, hi, sb, s_t);
    }
  };

  // kIn rows per iteration, all their loads issued before any is used.  The
  // statistics pass takes four bf16 rows (128 bytes a lane); two otherwise:
  // fp32 blocks are twice as large, the per-channel maxima leave no registers
  // for more, and without statistics a thread has only two rows (the row
  // splits are many).  The loads are unconditional -- a row past the end
  // reads row r again, a cache hit -- so the compiler can wait for each row's
  // own load only.
  constexpr int kIn = kBf16 && kStats && !kMax ? 4 : 2;
  if (active) {
    for (int64_t r = r0 + sub; r < r1; r += kIn * (int64_t)rpi) {
      int64_t src[kIn];
#pragma unroll
      for (int u = 0; u < kIn; ++u) src[u] = r + u * rpi < r1 ? r + u * rpi : r;
      if (gather) {
#pragma unroll
        for (int u = 0; u < kIn; ++u) src[u] = gather[src[u]];
      }
      RawBlock<kBf16> b[kIn];
#pragma unroll
      for (int u = 0; u < kIn; ++u) b[u].load(x, src[u] * ldx + cb * 16);
#pragma unroll
      for (int u = 0; u < kIn; ++u)
        if (r + u * rpi < r1) block(b[u], r + u * rpi);
    }
  }

  if constexpr (kStats) {
    // LDS: int64 sums then uint32 maxima, both [16][tpr] (element-in-block
    // major), so the lanes of a wave, which hold consecutive column blocks,
    // hit consecutive words and the atomics are free of bank conflicts.
    unsigned long long* lsum = reinterpret_cast<unsigned long long*>(dyn_lds);
    uint32_t* lmax = reinterpret_cast<uint32_t*>(lsum + tpr * 16);  // kMax only
    for (int i = threadIdx.x; i < tpr * 16; i += kQThreads) {
      lsum[i] = 0ull;
      if constexpr (kMax) lmax[i] = 0u;
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (acc[i] != 0u) atomicAdd(&lsum[i * tpr + cbl], (unsigned long long)acc[i]);
        if constexpr (kMax) {
          if (emax[i] != 0.0f) atomicMax(&lmax[i * tpr + cbl], __float_as_uint(emax[i]));
        }
      }
    }
    __syncthreads();
    // slot j holds channel (tile start) + 16 * (j % tpr) + j / tpr.  With
    // one row split (store_sums) this workgroup holds the channels' whole
    // sums and stores them; otherwise it adds them to the zeroed totals.
    for (int j = threadIdx.x; j < tpr * 16; j += kQThreads) {
      const int64_t k = ((int64_t)blockIdx.x * tpr + j % tpr) * 16 + j / tpr;
      if (k < K) {
        if (store_sums) {
          score[k] = (int64_t)lsum[j];
          if constexpr (kMax) chmax[k] = lmax[j];
        } else {
          if (lsum[j]) atomicAdd(reinterpret_cast<unsigned long long*>(score) + k, lsum[j]);
          if constexpr (kMax) {
            if (lmax[j]) atomicMax(chmax + k, lmax[j]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- select
// Channel k is selected iff its rank in the order (score desc, index asc),
//   rank_k = #{j : s_j > s_k} + #{j < k : s_j == s_k},
// is below n_sel: exactly the first n_sel channels of that order.  The ranks
// are counted directly, which needs no sort and no serial passes.
// k_rank: workgroup b ranks the 16 channels of block b.  Lane l of wave w
// holds channel 16b + l % 16 and counts over part 4w + l / 16 of the 64
// parts of the j range, reading the scores from LDS tiles; the 64 partial
// counts of a channel are summed in LDS.  The workgroup also writes the
// block's mask and its activity flag.
constexpr int kRankWaves = 16;
constexpr int kRankParts = 4 * kRankWaves;  // j parts per channel
constexpr int kRankTile = 4096;             // scores staged in LDS per pass (32 KiB)
constexpr int kSelThreads = 1024;
constexpr int kMaxSelectK = 16384;

__global__ __launch_bounds__(64 * kRankWaves) void k_rank(
    const int64_t* __restrict__ score_in, int K, int n_sel, uint16_t* __restrict__ mask16,
    uint8_t* __restrict__ kact) {
  __shared__ uint64_t tile[kRankTile];
  __shared__ uint32_t cnt[kRankParts][16];
  {  // group blockIdx.y (per-expert RAC): its statistics and outputs
    const int64_t g = blockIdx.y;
    score_in += g * K;
    mask16 += g * (K >> 4);
    kact += g * (K >> 4);
  }
  const uint64_t* score = reinterpret_cast<const uint64_t*>(score_in);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int part = 4 * w + (lane >> 4);
  const int k0 = blockIdx.x * 16;
  const int k = k0 + (lane & 15);  // K % 16 == 0: always a valid channel
  const uint64_t sk = score[k];
  const int d0 = k0, d1 = k0 + 16;  // this workgroup's own channels

  uint32_t c = 0;
  for (int t0 = 0; t0 < K; t0 += kRankTile) {
    const int n = K - t0 < kRankTile ? K - t0 : kRankTile;
    __syncthreads();  // the previous tile is consumed
#pragma unroll 4
    for (int i = threadIdx.x; i < n; i += 64 * kRankWaves) tile[i] = score[t0 + i];
    __syncthreads();
    // this lane's part of the tile, split where the tie rule changes
    const int per = (n + kRankParts - 1) / kRankParts;
    const int j0 = t0 + part * per < t0 + n ? t0 + part * per : t0 + n;
    const int j1 = j0 + per < t0 + n ? j0 + per : t0 + n;
    {  // j below every channel of this workgroup: a tie ranks j first
      const int e = j1 < d0 ? j1 : d0;
#pragma unroll 8
      for (int j = j0; j < e; ++j) c += tile[j - t0] >= sk ? 1u : 0u;
    }
    {
      const int bj = j0 > d0 ? j0 : d0, e = j1 < d1 ? j1 : d1;
      for (int j = bj; j < e; ++j) {
        const uint64_t sj = tile[j - t0];
        c += (sj > sk || (sj == sk && j < k)) ? 1u : 0u;
      }
    }
    {  // j above every channel of this workgroup: a tie ranks j after
      const int bj = j0 > d1 ? j0 : d1;
#pragma unroll 8
      for (int j = bj; j < j1; ++j) c += tile[j - t0] > sk ? 1u : 0u;
    }
  }
  cnt[part][lane & 15] = c;
  __syncthreads();
  if (w == 0) {
    uint32_t rank = 0;
    if (lane < 16)
      for (int i = 0; i < kRankParts; ++i) rank += cnt[i][lane];
    const bool sel = lane < 16 && rank < (uint32_t)n_sel;
    const uint32_t bits = (uint32_t)__ballot(sel) & 0xFFFFu;
    if (lane == 0) {
      mask16[blockIdx.x] = (uint16_t)bits;
      kact[blockIdx.x] = bits ? 1 : 0;
    }
  }
}

// Exclusive prefix sum over a workgroup of kNT threads; returns the total
// in *total.  wsum holds kNT / 64 entries.
template <int kNT>
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t n = __shfl_up(inc, o, 64);
    if (lane >= o) inc += n;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kNT / 64; ++i) {
    const uint32_t s = wsum[i];
    if (i < w) before += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// ------------------------------------------------ per-group selection
// Per-expert RAC selects within each of many groups, where the all-pairs rank
// count (K^2 compares per group) is too costly.  k_select_group takes one
// group per workgroup with its scores staged in LDS and finds the n-th
// largest score by an MSB-first radix select (8 passes of 8 bits: histogram
// of the candidates' digit, then the digit where the count from the top
// reaches n).  Scores above that threshold are selected; of the scores equal
// to it, the lowest-index ones fill the remaining places (a prefix count in
// index order) -- the same set as the first n of (score desc, index asc).
constexpr int kGroupSelectMaxK = 8192;  // scores staged in LDS (64 KiB)

__global__ __launch_bounds__(kSelThreads) void k_select_group(
    const int64_t* __restrict__ score_in, int K, int n_sel, uint16_t* __restrict__ mask16,
    uint8_t* __restrict__ kact) {
  __shared__ uint64_t sc[kGroupSelectMaxK];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[kSelThreads / 64];
  __shared__ uint32_t res_digit, res_above;
  const int64_t g = blockIdx.x;
  const uint64_t* score = reinterpret_cast<const uint64_t*>(score_in + g * K);
  mask16 += g * (K >> 4);
  kact += g * (K >> 4);
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < K; i += kSelThreads) sc[i] = score[i];

  uint64_t prefix = 0, pmask = 0;
  uint32_t remaining = (uint32_t)n_sel;  // places left among the candidates
  if (n_sel > 0) {
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
      __syncthreads();  // also publishes sc on the first pass
      for (int i = tid; i < K; i += kSelThreads) {
        const uint64_t v = sc[i];
        if ((v & pmask) == prefix) atomicAdd(&hist[(uint32_t)(v >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l holds digits 4l .. 4l+3; counts from the top (digit 255 down)
        uint32_t h[4], sfx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = hist[4 * lane + i];
        sfx[3] = h[3];
        sfx[2] = sfx[3] + h[2];
        sfx[1] = sfx[2] + h[1];
        sfx[0] = sfx[1] + h[0];
        // sum over the lanes above this one (higher digits)
        uint32_t above = 0, inc = sfx[0];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t n = __shfl_down(inc, o, 64);
          if (lane + o < 64) inc += n;
        }
        above = inc - sfx[0];
        // the digit d with count(>= d) >= remaining > count(> d) is unique
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t ge = above + sfx[i], gt = ge - h[i];
          if (ge >= remaining && gt < remaining) {
            res_digit = (uint32_t)(4 * lane + i);
            res_above = gt;
          }
        }
      }
      __syncthreads();
      prefix |= (uint64_t)res_digit << shift;
      pmask |= (uint64_t)255u << shift;
      remaining -= res_above;
    }
  } else {
    __syncthreads();
  }
  // threshold T = prefix; `remaining` of the scores equal to T are taken,
  // lowest index first.  Thread t owns block t (channels 16t .. 16t+15).
  const int nb = K >> 4;
  uint32_t eqbits = 0, gtbits = 0;
  if (tid < nb && n_sel > 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint64_t v = sc[tid * 16 + i];
      if (v > prefix) gtbits |= 1u << i;
      if (v == prefix) eqbits |= 1u << i;
    }
  }
  uint32_t total;
  const uint32_t before = block_exclusive_scan<kSelThreads>((uint32_t)__builtin_popcount(eqbits), wsum, &total);
  if (tid < nb) {
    uint32_t bits = gtbits, rank = before;
    for (uint32_t m = eqbits; m; m &= m - 1) {
      if (rank < remaining) bits |= m & (~m + 1u);
      ++rank;
    }
    mask16[tid] = (uint16_t)bits;
    kact[tid] = bits ? 1 : 0;
  }
}

// -------------------------------------------------------------- residual
// r = mask * e in every block with a selected channel, e = x - deq(q(x)).
// The main codes are recomputed from x, the block scale and the tensor scale
// (the same operations as k_quant, so the same codes) rather than read back:
// that saves a quarter of this pass's reads.  The residual is quantized with
// the activation's tensor scale s_t (the residual pass of the GEMM shares
// it), so its block scales are E4M3(max|r_b| / (6 s_t)); |r| <= max|x| keeps
// them within E4M3's range.  Workgroup 0 writes the residual tensor scale
// (= s_t) and lists the selected channels in ascending order (a prefix sum of
// the block masks' popcounts).
// A thread takes kResU blocks per iteration and issues all their x and block
// scale loads before it computes any of them, so each wave keeps kResU
// blocks' loads in flight instead of waiting out one load round trip per
// block (bf16: 4 blocks, 128 bytes a lane; FP32 blocks are twice as large).
// The loads are unconditional -- a block without selected channels, or past
// the end, reads the tensors' first element instead, one cache line for the
// whole wave -- so the compiler can wait for each block's own loads only.
template <bool kBf16, bool kGather>
__global__ __launch_bounds__(kThreads) void k_residual(
    const void* __restrict__ x, int64_t rows, int64_t K, int64_t ldx,
    const uint8_t* __restrict__ scales, const float* __restrict__ tscale,
    const uint16_t* __restrict__ mask16, int nparts,
    int32_t* __restrict__ selected,
    float* __restrict__ res_ts, uint8_t* __restrict__ res_codes,
    uint8_t* __restrict__ res_scales, const int32_t* __restrict__ goff,
    const int32_t* __restrict__ gather, int n_sel) {
  __shared__ uint32_t wred[kThreads / 64];
  // With goff (per-expert RAC) workgroups y handle group y: grouped rows
  // [goff[y], goff[y+1]) read through the gather, the group's masks, tensor
  // scales and selected list.
  int64_t row0 = 0;
  if (goff) {
    const int g = blockIdx.y;
    row0 = goff[g];
    rows = goff[g + 1] - row0;
    mask16 += (int64_t)g * nparts;
    tscale += g;
    res_ts += g;
    if (selected) selected += (int64_t)g * n_sel;
  }
  __shared__ uint16_t lmask[kMaxSelectK / 16];  // block masks, so x loads wait on nothing
  for (int i = threadIdx.x; i < nparts; i += kThreads) lmask[i] = mask16[i];  // K / 16 blocks
  __syncthreads();
  const float s_tr = *tscale;  // the residual pass shares the activation's tensor scale
  if (blockIdx.x == 0) {
    if (threadIdx.x == 0) *res_ts = s_tr;
    // thread t lists the selected channels of blocks [t*pb, t*pb + pb)
    constexpr int kPb = (kMaxSelectK / 16 + kThreads - 1) / kThreads;
    const int nb = (int)(K >> 4);
    const int pb = (nb + kThreads - 1) / kThreads;
    const int b0 = threadIdx.x * pb;
    uint32_t bits[kPb];
    uint32_t n = 0;
#pragma unroll
    for (int i = 0; i < kPb; ++i) {
      bits[i] = (i < pb && b0 + i < nb) ? (uint32_t)mask16[b0 + i] : 0u;
      n += __builtin_popcount(bits[i]);
    }
    uint32_t tot;
    uint32_t pos = block_exclusive_scan<kThreads>(n, wred, &tot);
#pragma unroll
    for (int i = 0; i < kPb; ++i)
      for (uint32_t m = bits[i]; m; m &= m - 1) selected[pos++] = (b0 + i) * 16 + __builtin_ctz(m);
  }

  const int64_t CB = K >> 4;
  const int64_t nblk = rows * CB;
  const float s_t = *tscale;
  // rb of every E4M3 code and c6 for the FP32 fast path of the residual's
  // scale codes (main and residual share the tensor scale)
  __shared__ float rb_lut[128];
  nv_fill_recip_lut(rb_lut, s_t);
  const float c6 = (float)(1.0 / (6.0 * (double)s_t));
  __syncthreads();
  // Blocks b = row * CB + cb, grid-stride; (row, cb) advance incrementally
  // (one 64-bit division per thread).
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int64_t srow = stride / CB, scb = stride - srow * CB;
  int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  int64_t r = b / CB, cb = b - r * CB;
  auto advance = [&](int64_t& rr, int64_t& cc) {
    rr += srow;
    cc += scb;
    if (cc >= CB) {
      cc -= CB;
      ++rr;
    }
  };
  // block (grouped row rr, column block cc) with mask m, its x and its main
  // scale code sm
  auto one = [&](int64_t rr, int64_t cc, uint32_t m, const RawBlock<kBf16>& raw, uint32_t sm) {
    uint32_t packed[2] = {0u, 0u};
    uint32_t sc = 0u;
    if (m) {
      float v[16];
      raw.widen(v);
      const float sb = nv_e4m3_to_f32(sm);
      const float rm = rb_lut[sm];
      float g[16], e[16];
      nv_decode8(nv_encode8(v, rm), g);
      nv_decode8(nv_encode8(v + 8, rm), g + 8);
      float amax_b = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float d = (g[i] * sb) * s_t;
        e[i] = ((m >> i) & 1u) ? v[i] - d : 0.0f;
        amax_b = __builtin_fmaxf(amax_b, __builtin_fabsf(e[i]));
      }
      sc = nv_block_scale_c6(amax_b, s_tr, c6);
      const float rb = rb_lut[sc];  // nv_block_recip(RN32(E4M3(sc) s_t))
      packed[0] = nv_encode8(e, rb);
      packed[1] = nv_encode8(e + 8, rb);
    }
    *reinterpret_cast<uint2*>(res_codes + rr * (K >> 1) + cc * 8) = make_uint2(packed[0], packed[1]);
    res_scales[rr * CB + cc] = (uint8_t)sc;
  };
  constexpr int kResU = kBf16 ? 4 : 2;
  for (; b < nblk; b += kResU * stride) {
    RawBlock<kBf16> raw[kResU];
    uint32_t m[kResU], sm[kResU];
    int64_t jj[kResU], cc[kResU], src[kResU];
#pragma unroll
    for (int u = 0; u < kResU; ++u) {
      jj[u] = row0 + r;  // grouped row
      cc[u] = cb;
      m[u] = b + u * stride < nblk ? lmask[cb] : 0u;
      advance(r, cb);
    }
#pragma unroll
    for (int u = 0; u < kResU; ++u) {
      if constexpr (kGather)
        src[u] = gather[m[u] ? jj[u] : 0];
      else
        src[u] = jj[u];
    }
#pragma unroll
    for (int u = 0; u < kResU; ++u) {
      raw[u].load(x, m[u] ? src[u] * ldx + cc[u] * 16 : 0);
      sm[u] = scales[m[u] ? jj[u] * CB + cc[u] : 0];
    }
#pragma unroll
    for (int u = 0; u < kResU; ++u)
      if (b + u * stride < nblk) one(jj[u], cc[u], m[u], raw[u], sm[u]);
  }
}

// k_residual for the input type and for a gather or none.
void residual_launch(dim3 grid, hipStream_t s, const void* x, int dtype, int64_t rows, int64_t K,
                     int64_t ldx, const uint8_t* scales, const float* tscale,
                     const uint16_t* mask16, int nparts, int32_t* selected, float* res_ts,
                     uint8_t* res_codes, uint8_t* res_scales, const int32_t* goff,
                     const int32_t* gather, int n_sel) {
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s, x, rows, K, ldx, scales, tscale, mask16,
                       nparts, selected, res_ts, res_codes, res_scales, goff, gather, n_sel);
  };
  const bool bf = dtype == NVFP4_IN_BF16;
  if (gather)
    bf ? go(k_residual<true, true>) : go(k_residual<false, true>);
  else
    bf ? go(k_residual<true, false>) : go(k_residual<false, false>);
}

int64_t blocks_for(int64_t work, int64_t per_block, int64_t cap) {
  int64_t b = (work + per_block - 1) / per_block;
  if (b < 1) b = 1;
  return b < cap ? b : cap;
}

// Per-row buffers may be NULL when rows == 0 (empty tensors have no storage).
int check_x(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx) {
  NV_RETURN_IF(!x && rows > 0, NVFP4_ERR_NULL);
  NV_RETURN_IF(dtype != NVFP4_IN_F32 && dtype != NVFP4_IN_BF16, NVFP4_ERR_DTYPE);
  NV_RETURN_IF(rows < 0 || K <= 0 || (K & 15) || ldx < K, NVFP4_ERR_SHAPE);
  NV_RETURN_IF((ldx & 15) || !nv_aligned16(x), NVFP4_ERR_ALIGN);
  return NVFP4_OK;
}

}  // namespace

extern "C" {

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "invalid size or divisibility";
    case NVFP4_ERR_DTYPE: return "unknown dtype or epilogue";
    case NVFP4_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t nvfp4_quantize_workspace_size(int64_t, int64_t) {
  return nv_round256(sizeof(float) * kMaxParts);
}

}  // extern "C"

// The quantizer's launches (after validation): tensor amax, then k_quant with
// output mode dq (0: codes/scales, 1: FP32 dequantized, 2: bf16 dequantized).
static int quantize_launch(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx,
                           const float* amax_in, uint8_t* codes, uint8_t* scales,
                           float* tensor_scale, int64_t* channel_score, float* channel_max,
                           void* ws, int dq, void* dq_out, hipStream_t s) {
  const bool stats = channel_score != nullptr;
  uint32_t* chm = reinterpret_cast<uint32_t*>(channel_max);  // nullable with stats
  const bool cmax = stats && chm != nullptr;
  float* partials = reinterpret_cast<float*>(ws);
  const int bf16 = dtype == NVFP4_IN_BF16;
  const int64_t CB = K / 16;
  // Column tiles of at most tile_max column blocks (16: 256 channels, 512 B
  // of bf16 per row), rpi rows in flight per pass.  Narrow tiles keep the
  // global atomics per workgroup few.
  constexpr int tile_max = 16;
  const int64_t ntile = (CB + tile_max - 1) / tile_max;
  const int tpr = (int)((CB + ntile - 1) / ntile);
  const int rpi = kQThreads / tpr;
  // Row splits: with statistics every workgroup adds one atomic per channel
  // to the global sums, so the splits stay few (about two workgroups per CU
  // over all column tiles) and each thread takes at least two rows.  With a
  // single split (few rows) the workgroups store the sums instead, and
  // nothing needs zeroing first.
  constexpr int wg_target = 512, min_rows = 2;
  int64_t splits = blocks_for(rows, (int64_t)rpi * min_rows, 65535);
  const int64_t max_splits = stats ? (wg_target / ntile > 0 ? wg_target / ntile : 1) : 65535;
  if (splits > max_splits) splits = max_splits;
  // with amax_in, one split also saves the launch that zeroes the sums: worth
  // it while a thread has at most eight rows
  if (amax_in && stats && rows <= (int64_t)rpi * 8) splits = 1;
  const int64_t rows_per_split = rows > 0 ? (rows + splits - 1) / splits : 1;
  const int store = stats && splits == 1 ? 1 : 0;
  int nparts = 0;
  if (!amax_in) {
    nparts = (int)blocks_for(rows * CB, kThreads * 4, kMaxParts);
    hipLaunchKernelGGL(k_amax, dim3(nparts), dim3(kThreads), 0, s, x, bf16, rows, K, ldx,
                       partials, stats && !store ? channel_score : nullptr,
                       store ? nullptr : chm);
  } else if (stats && !store) {
    hipLaunchKernelGGL(k_zero_stats, dim3((unsigned)blocks_for(K, 256, 1024)), dim3(256), 0, s,
                       K, channel_score, chm);
  }
  const size_t lds =
      stats ? (size_t)tpr * 16 * (sizeof(uint64_t) + (cmax ? sizeof(uint32_t) : 0)) : 0;
  const dim3 grid((unsigned)ntile, (unsigned)splits);
  int64_t* sc = stats ? channel_score : nullptr;
  uint32_t* cm = cmax ? chm : nullptr;
#define NV_QUANT_LAUNCH(ST, BF, MX)                                                              \
  hipLaunchKernelGGL((k_quant<ST, BF, 0, MX>), grid, dim3(kQThreads), ST ? lds : 0, s, x, rows, K, \
                     ldx, partials, nparts, amax_in, codes, scales, tensor_scale, sc, cm, tpr,    \
                     rpi, rows_per_split, nullptr, nullptr, nullptr, store)
#define NV_QUANT_LAUNCH_DQ(DQ, BF)                                                              \
  hipLaunchKernelGGL((k_quant<false, BF, DQ>), grid, dim3(kQThreads), 0, s, x, rows, K, ldx,    \
                     partials, nparts, amax_in, nullptr, nullptr, tensor_scale, nullptr, nullptr, \
                     tpr, rpi, rows_per_split, dq_out, nullptr, nullptr, 0)
  if (dq == 1 && bf16) NV_QUANT_LAUNCH_DQ(1, true);
  else if (dq == 1) NV_QUANT_LAUNCH_DQ(1, false);
  else if (dq == 2 && bf16) NV_QUANT_LAUNCH_DQ(2, true);
  else if (dq == 2) NV_QUANT_LAUNCH_DQ(2, false);
  else if (cmax && bf16) NV_QUANT_LAUNCH(true, true, true);
  else if (cmax) NV_QUANT_LAUNCH(true, false, true);
  else if (stats && bf16) NV_QUANT_LAUNCH(true, true, false);
  else if (stats) NV_QUANT_LAUNCH(true, false, false);
  else if (bf16) NV_QUANT_LAUNCH(false, true, false);
  else NV_QUANT_LAUNCH(false, false, false);
#undef NV_QUANT_LAUNCH
#undef NV_QUANT_LAUNCH_DQ
  return nv_launch_status();
}

// k_dequant: one thread per 16-element block (grid-stride).
template <int kDq>
__global__ __launch_bounds__(kThreads) void k_dequant(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ tscale,
                                                      int64_t rows, int64_t K, void* __restrict__ out) {
  const float s_t = *tscale;
  const int64_t CB = K >> 4, nblk = rows * CB;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * kThreads) {
    const int64_t r = b / CB, cb = b - r * CB;
    const uint2 c = *reinterpret_cast<const uint2*>(codes + r * (K >> 1) + cb * 8);
    dq_store16<kDq>(out, r * K + cb * 16, c.x, c.y, nv_e4m3_to_f32(scales[b]), s_t);
  }
}

extern "C" {

int nvfp4_quantize(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx,
                   const float* amax_in, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                   int64_t* channel_score, float* channel_max, void* ws, size_t ws_bytes,
                   void* stream) {
  int st = check_x(x, dtype, rows, K, ldx);
  if (st) return st;
  NV_RETURN_IF(!tensor_scale || (rows > 0 && (!codes || !scales)), NVFP4_ERR_NULL);
  NV_RETURN_IF(channel_max && !channel_score, NVFP4_ERR_NULL);
  NV_RETURN_IF(!nv_aligned16(codes), NVFP4_ERR_ALIGN);
  NV_RETURN_IF((reinterpret_cast<uintptr_t>(channel_score) & 7) ||
                   (reinterpret_cast<uintptr_t>(channel_max) & 3),
               NVFP4_ERR_ALIGN);
  NV_RETURN_IF(!amax_in && (!ws || ws_bytes < nvfp4_quantize_workspace_size(rows, K)),
               NVFP4_ERR_WORKSPACE);
  return quantize_launch(x, dtype, rows, K, ldx, amax_in, codes, scales, tensor_scale,
                         channel_score, channel_max, ws, 0, nullptr,
                         reinterpret_cast<hipStream_t>(stream));
}

size_t nvfp4_qdq_workspace_size(int64_t rows, int64_t K) {
  return nvfp4_quantize_workspace_size(rows, K);
}

int nvfp4_qdq(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx,
              const float* amax_in, int out_dtype, void* out, float* tensor_scale, void* ws,
              size_t ws_bytes, void* stream) {
  int st = check_x(x, dtype, rows, K, ldx);
  if (st) return st;
  NV_RETURN_IF(out_dtype != NVFP4_IN_F32 && out_dtype != NVFP4_IN_BF16, NVFP4_ERR_DTYPE);
  NV_RETURN_IF(!tensor_scale || (rows > 0 && !out), NVFP4_ERR_NULL);
  NV_RETURN_IF(!nv_aligned16(out), NVFP4_ERR_ALIGN);
  NV_RETURN_IF(!amax_in && (!ws || ws_bytes < nvfp4_qdq_workspace_size(rows, K)),
               NVFP4_ERR_WORKSPACE);
  return quantize_launch(x, dtype, rows, K, ldx, amax_in, nullptr, nullptr, tensor_scale,
                         nullptr, nullptr, ws, out_dtype == NVFP4_IN_F32 ? 1 : 2, out,
                         reinterpret_cast<hipStream_t>(stream));
}

int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                     int64_t rows, int64_t K, int out_dtype, void* out, void* stream) {
  NV_RETURN_IF(out_dtype != NVFP4_IN_F32 && out_dtype != NVFP4_IN_BF16, NVFP4_ERR_DTYPE);
  NV_RETURN_IF(rows < 0 || K <= 0 || K % 16 || K > (1LL << 40) / (rows > 0 ? rows : 1),
               NVFP4_ERR_SHAPE);
  if (rows == 0) return NVFP4_OK;
  NV_RETURN_IF(!codes || !scales || !tensor_scale || !out, NVFP4_ERR_NULL);
  NV_RETURN_IF((reinterpret_cast<uintptr_t>(codes) & 7) || !nv_aligned16(out), NVFP4_ERR_ALIGN);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const unsigned grid = (unsigned)blocks_for(rows * (K >> 4), kThreads, 8192);
  if (out_dtype == NVFP4_IN_F32)
    hipLaunchKernelGGL(k_dequant<1>, dim3(grid), dim3(kThreads), 0, s, codes, scales,
                       tensor_scale, rows, K, out);
  else
    hipLaunchKernelGGL(k_dequant<2>, dim3(grid), dim3(kThreads), 0, s, codes, scales,
                       tensor_scale, rows, K, out);
  return nv_launch_status();
}

// The RAC launches of one tensor (after validation): the rank count writes the
// block masks into mask16 [K/16] and kblock_active; the residual pass writes
// the residual, its tensor scale and the selected list.
static int rac_launch(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx,
                      const uint8_t* scales, const float* tensor_scale,
                      const int64_t* channel_score, int64_t n_select, int32_t* selected,
                      uint8_t* kblock_active, uint8_t* res_codes, uint8_t* res_scales,
                      float* res_tensor_scale, uint16_t* mask16, hipStream_t s) {
  const int nrank = (int)(K / 16);
  hipLaunchKernelGGL(k_rank, dim3(nrank), dim3(64 * kRankWaves), 0, s, channel_score, (int)K,
                     (int)n_select, mask16, kblock_active);
  int st = nv_launch_status();
  if (st) return st;
  // at least one workgroup: it also writes selected[] and the tensor scale
  const int64_t nblk = rows * (K / 16);
  residual_launch(dim3((unsigned)blocks_for(nblk, 2 * kThreads, 2048)), s, x, dtype, rows, K, ldx,
                  scales, tensor_scale, mask16, nrank, selected, res_tensor_scale, res_codes,
                  res_scales, nullptr, nullptr, 0);
  return nv_launch_status();
}

// Workspace of rac_select_residual: the selection's block masks [K/16] u16.
static size_t rac_ws_bytes(int64_t K) {
  return nv_round256(sizeof(uint16_t) * (size_t)(K > 0 ? K / 16 : 0));
}

size_t rac_select_residual_workspace_size(int64_t, int64_t K) { return rac_ws_bytes(K); }

int rac_select_residual(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx,
                        const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                        const int64_t* channel_score, const float* channel_max, int64_t n_select,
                        int32_t* selected, uint8_t* kblock_active, uint8_t* res_codes,
                        uint8_t* res_scales, float* res_tensor_scale, void* ws, size_t ws_bytes,
                        void* stream) {
  int st = check_x(x, dtype, rows, K, ldx);
  if (st) return st;
  (void)codes;  // recomputed from x, scales and tensor_scale
  (void)channel_max;  // the selection needs the scores only
  NV_RETURN_IF(!tensor_scale || !channel_score || !kblock_active || !res_tensor_scale,
               NVFP4_ERR_NULL);
  NV_RETURN_IF(rows > 0 && (!scales || !res_codes || !res_scales), NVFP4_ERR_NULL);
  NV_RETURN_IF(n_select < 0 || n_select > K || K > kMaxSelectK, NVFP4_ERR_SHAPE);
  NV_RETURN_IF(n_select > 0 && !selected, NVFP4_ERR_NULL);
  NV_RETURN_IF(!nv_aligned16(res_codes) || (reinterpret_cast<uintptr_t>(channel_score) & 7),
               NVFP4_ERR_ALIGN);
  NV_RETURN_IF(!ws || ws_bytes < rac_select_residual_workspace_size(rows, K) ||
                   (reinterpret_cast<uintptr_t>(ws) & 3),
               NVFP4_ERR_WORKSPACE);
  return rac_launch(x, dtype, rows, K, ldx, scales, tensor_scale, channel_score, n_select,
                    selected, kblock_active, res_codes, res_scales, res_tensor_scale,
                    reinterpret_cast<uint16_t*>(ws), reinterpret_cast<hipStream_t>(stream));
}

// --------------------------------------------- allocation-free quantize + RAC
// Scratch of nvfp4_quantize_rac_static on each device: the tensor-amax
// partials (kMaxParts floats) at offset 0, then the selection's block masks
// (kMaxSelectK / 16 u16).  Every byte is written by a kernel of the call before
// any kernel of the call reads it, so nothing needs clearing between calls.
constexpr size_t kStaticMaskOff = sizeof(float) * kMaxParts;             // 4096, 256-aligned
constexpr size_t kScratchBytes = kStaticMaskOff + sizeof(uint16_t) * (kMaxSelectK / 16);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static void* g_scratch[kMaxDevices];
static std::once_flag g_scratch_once[kMaxDevices];

// The device address of `scratch` on the current device, looked up once per
// device with that device current (the array's name is a host-side handle,
// not a device address).
static int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_HIP;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch[dev] = ptr;
  });
  if (!g_scratch[dev]) return NVFP4_ERR_HIP;
  *out = g_scratch[dev];
  return NVFP4_OK;
}

extern "C" int nvfp4_quantize_rac_static(
    const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx, const float* amax_in,
    uint8_t* codes, uint8_t* scales, float* tensor_scale, int64_t* channel_score,
    float* channel_max, int64_t n_select, int32_t* selected, uint8_t* kblock_active,
    uint8_t* res_codes, uint8_t* res_scales, float* res_tensor_scale, void* stream) {
  int st = check_x(x, dtype, rows, K, ldx);
  if (st) return st;
  NV_RETURN_IF(K > kMaxSelectK || n_select < 0 || n_select > K, NVFP4_ERR_SHAPE);
  NV_RETURN_IF(!tensor_scale || !channel_score || !kblock_active || !res_tensor_scale ||
                   (n_select > 0 && !selected),
               NVFP4_ERR_NULL);
  NV_RETURN_IF(rows > 0 && (!codes || !scales || !res_codes || !res_scales), NVFP4_ERR_NULL);
  NV_RETURN_IF(!nv_aligned16(codes) || !nv_aligned16(res_codes) ||
                   (reinterpret_cast<uintptr_t>(channel_score) & 7) ||
                   (reinterpret_cast<uintptr_t>(channel_max) & 3),
               NVFP4_ERR_ALIGN);
  void* base = nullptr;
  st = scratch_on_current_device(&base);
  if (st) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  st = quantize_launch(x, dtype, rows, K, ldx, amax_in, codes, scales, tensor_scale,
                       channel_score, channel_max, base, 0, nullptr, s);
  if (st) return st;
  return rac_launch(x, dtype, rows, K, ldx, scales, tensor_scale, channel_score, n_select,
                    selected, kblock_active, res_codes, res_scales, res_tensor_scale,
                    reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(base) + kStaticMaskOff), s);
}

// ------------------------------------------------------- per-expert RAC
constexpr int kGroupParts = 8;  // amax partials per group

static int check_grouped(const void* x, int dtype, int64_t K, int64_t ldx, const int32_t* goff,
                         int64_t G, int64_t total_rows) {
  NV_RETURN_IF(!goff || (!x && total_rows > 0), NVFP4_ERR_NULL);
  NV_RETURN_IF(dtype != NVFP4_IN_F32 && dtype != NVFP4_IN_BF16, NVFP4_ERR_DTYPE);
  NV_RETURN_IF(G < 1 || G > 65535 || total_rows < 0 || K <= 0 || (K & 15) || ldx < K ||
                   total_rows * (K >> 4) > 0x7fffffffLL,
               NVFP4_ERR_SHAPE);
  NV_RETURN_IF((ldx & 15) || !nv_aligned16(x), NVFP4_ERR_ALIGN);
  return NVFP4_OK;
}

size_t nvfp4_quantize_grouped_workspace_size(int64_t G, int64_t) {
  return nv_round256(sizeof(float) * (size_t)(G > 0 ? G : 0) * kGroupParts);
}

int nvfp4_quantize_grouped(const void* x, int dtype, int64_t K, int64_t ldx,
                           const int32_t* group_offsets, int64_t G, int64_t total_rows,
                           const int32_t* gather_rows, uint8_t* codes, uint8_t* scales,
                           float* tensor_scales, int64_t* channel_score, float* channel_max,
                           void* ws, size_t ws_bytes, void* stream) {
  int st = check_grouped(x, dtype, K, ldx, group_offsets, G, total_rows);
  if (st) return st;
  NV_RETURN_IF(!tensor_scales || (total_rows > 0 && (!codes || !scales)), NVFP4_ERR_NULL);
  NV_RETURN_IF(channel_max && !channel_score, NVFP4_ERR_NULL);
  NV_RETURN_IF(!nv_aligned16(codes) || (reinterpret_cast<uintptr_t>(channel_score) & 7) ||
                   (reinterpret_cast<uintptr_t>(channel_max) & 3),
               NVFP4_ERR_ALIGN);
  NV_RETURN_IF(!ws || ws_bytes < nvfp4_quantize_grouped_workspace_size(G, K),
               NVFP4_ERR_WORKSPACE);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool stats = channel_score != nullptr;
  uint32_t* chm = reinterpret_cast<uint32_t*>(channel_max);  // nullable with stats
  const bool cmax = stats && chm != nullptr;
  float* partials = reinterpret_cast<float*>(ws);
  const int bf16 = dtype == NVFP4_IN_BF16;
  hipLaunchKernelGGL(k_amax_grouped, dim3(kGroupParts, (unsigned)G), dim3(kThreads), 0, s, x,
                     bf16, K, ldx, group_offsets, gather_rows, (int)G, partials,
                     stats ? channel_score : nullptr, chm);
  // the column tiles of k_quant; row splits per group from the mean group size
  const int64_t CB = K / 16;
  const int tile_max = 16;
  const int64_t ntile = (CB + tile_max - 1) / tile_max;
  const int tpr = (int)((CB + ntile - 1) / ntile);
  const int rpi = kQThreads / tpr;
  int64_t splits = blocks_for((total_rows + G - 1) / G, (int64_t)rpi * 2, 64);
  const size_t lds =
      stats ? (size_t)tpr * 16 * (sizeof(uint64_t) + (cmax ? sizeof(uint32_t) : 0)) : 0;
  const dim3 grid((unsigned)ntile, (unsigned)splits, (unsigned)G);
  int64_t* sc = stats ? channel_score : nullptr;
  uint32_t* cm = cmax ? chm : nullptr;
#define NV_QUANT_LAUNCH_G(ST, BF, MX)                                                            \
  hipLaunchKernelGGL((k_quant<ST, BF, 0, MX>), grid, dim3(kQThreads), ST ? lds : 0, s, x,        \
                     total_rows, K, ldx, partials, kGroupParts, nullptr, codes, scales,          \
                     tensor_scales, sc, cm, tpr, rpi, (int64_t)0, nullptr, group_offsets,        \
                     gather_rows, 0)
  if (cmax && bf16) NV_QUANT_LAUNCH_G(true, true, true);
  else if (cmax) NV_QUANT_LAUNCH_G(true, false, true);
  else if (stats && bf16) NV_QUANT_LAUNCH_G(true, true, false);
  else if (stats) NV_QUANT_LAUNCH_G(true, false, false);
  else if (bf16) NV_QUANT_LAUNCH_G(false, true, false);
  else NV_QUANT_LAUNCH_G(false, false, false);
#undef NV_QUANT_LAUNCH_G
  return nv_launch_status();
}

size_t rac_select_residual_grouped_workspace_size(int64_t G, int64_t K) {
  return rac_ws_bytes((G > 0 ? G : 0) * K);
}

int rac_select_residual_grouped(const void* x, int dtype, int64_t K, int64_t ldx,
                                const int32_t* group_offsets, int64_t G, int64_t total_rows,
                                const int32_t* gather_rows, const uint8_t* scales,
                                const float* tensor_scales, const int64_t* channel_score,
                                const float* channel_max, int64_t n_select, int32_t* selected,
                                uint8_t* kblock_active, uint8_t* res_codes, uint8_t* res_scales,
                                float* res_tensor_scales, void* ws, size_t ws_bytes,
                                void* stream) {
  int st = check_grouped(x, dtype, K, ldx, group_offsets, G, total_rows);
  if (st) return st;
  (void)channel_max;  // the selection needs the scores only
  NV_RETURN_IF(!tensor_scales || !channel_score || !kblock_active || !res_tensor_scales,
               NVFP4_ERR_NULL);
  NV_RETURN_IF(total_rows > 0 && (!scales || !res_codes || !res_scales), NVFP4_ERR_NULL);
  NV_RETURN_IF(n_select < 0 || n_select > K || K > kMaxSelectK, NVFP4_ERR_SHAPE);
  NV_RETURN_IF(n_select > 0 && !selected, NVFP4_ERR_NULL);
  NV_RETURN_IF(!nv_aligned16(res_codes) || (reinterpret_cast<uintptr_t>(channel_score) & 7),
               NVFP4_ERR_ALIGN);
  NV_RETURN_IF(!ws || ws_bytes < rac_select_residual_grouped_workspace_size(G, K) ||
                   (reinterpret_cast<uintptr_t>(ws) & 3),
               NVFP4_ERR_WORKSPACE);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint16_t* mask16 = reinterpret_cast<uint16_t*>(ws);
  const int nrank = (int)(K / 16);
  // many groups: a radix select per group; very long rows: the rank count
  if (K <= kGroupSelectMaxK)
    hipLaunchKernelGGL(k_select_group, dim3((unsigned)G), dim3(kSelThreads), 0, s, channel_score,
                       (int)K, (int)n_select, mask16, kblock_active);
  else
    hipLaunchKernelGGL(k_rank, dim3(nrank, (unsigned)G), dim3(64 * kRankWaves), 0, s,
                       channel_score, (int)K, (int)n_select, mask16, kblock_active);
  st = nv_launch_status();
  if (st) return st;
  // at least one workgroup per group: it writes the group's selected[] and
  // residual tensor scale
  const int64_t per_group = ((total_rows + G - 1) / G) * (K / 16);
  residual_launch(dim3((unsigned)blocks_for(per_group, 2 * kThreads, 256), (unsigned)G), s, x,
                  dtype, total_rows, K, ldx, scales, tensor_scales, mask16, nrank, selected,
                  res_tensor_scales, res_codes, res_scales, group_offsets, gather_rows,
                  (int)n_select);
  return nv_launch_status();
}

}  // extern "C"
