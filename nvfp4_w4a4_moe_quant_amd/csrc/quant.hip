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
//   k_amax      partial max|x| per workgroup (tensor amax), zeroes RAC stats
//   k_quant     tensor scale, block scales, E2M1 codes; optionally the exact
//               per-channel error statistics (score = sum q^2, max |e|)
//   k_select    one workgroup: top-n channels by (score desc, index asc)
//               via radix select, block-activity flags, residual tensor scale
//   k_residual  r = mask * e re-quantized in the same blocks
// All reductions are max or integer sums, so results are order-independent.
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
  float m = 0.0f;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblk; b += stride) {
    const int64_t r = b / cb_per_row, cb = b - r * cb_per_row;
    float v[16];
    nv_load16(x, bf16, r * ldx + cb * 16, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
  }
  if (score) {
    for (int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x; k < K; k += stride) {
      score[k] = 0;
      chmax[k] = 0u;
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

__global__ void k_zero_stats(int64_t K, int64_t* __restrict__ score, uint32_t* __restrict__ chmax) {
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < K;
       k += (int64_t)gridDim.x * blockDim.x) {
    score[k] = 0;
    chmax[k] = 0u;
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
// partial sums are accumulated in registers (FP64, exact integers below 2^53),
// combined in LDS, then added to the global int64 sums.
template <bool kStats>
__global__ __launch_bounds__(kThreads) void k_quant(
    const void* __restrict__ x, int bf16, int64_t rows, int64_t K, int64_t ldx,
    const float* __restrict__ partials, int nparts, const float* __restrict__ amax_in,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ tscale_out,
    int64_t* __restrict__ score, uint32_t* __restrict__ chmax, int tpr, int rpi,
    int64_t rows_per_split) {
  extern __shared__ unsigned char dyn_lds[];
  __shared__ float red[kThreads / 64];
  const float amax = workgroup_amax(partials, nparts, amax_in, red);
  const float s_t = nv_tensor_scale(amax);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *tscale_out = s_t;

  const int64_t CB = K >> 4;
  const int sub = threadIdx.x / tpr;
  const int cbl = threadIdx.x - sub * tpr;
  const int64_t cb = (int64_t)blockIdx.x * tpr + cbl;
  const bool active = sub < rpi && cb < CB;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_split;
  const int64_t r1 = r0 + rows_per_split < rows ? r0 + rows_per_split : rows;
  const int shift = nv_score_shift(s_t);

  double acc[16];
  float emax[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    acc[i] = 0.0;
    emax[i] = 0.0f;
  }

  if (active) {
    for (int64_t r = r0 + sub; r < r1; r += rpi) {
      float v[16];
      nv_load16(x, bf16, r * ldx + cb * 16, v);
      float amax_b = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax_b = __builtin_fmaxf(amax_b, __builtin_fabsf(v[i]));
      const uint32_t sc = nv_block_scale(amax_b, s_t);
      const float sb = nv_e4m3_to_f32(sc);
      const float Sb = sb * s_t;
      const float rb = nv_block_recip(Sb);
      uint32_t packed[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t c = nv_e2m1_encode(v[i] * rb);
        packed[i >> 3] |= c << ((i & 7) * 4);
        if constexpr (kStats) {
          const float d = (nv_e2m1_to_f32(c) * sb) * s_t;
          const float e = v[i] - d;
          const float q = nv_score_q(e, shift);
          acc[i] = __builtin_fma((double)q, (double)q, acc[i]);
          emax[i] = __builtin_fmaxf(emax[i], __builtin_fabsf(e));
        }
      }
      *reinterpret_cast<uint2*>(codes + r * (K >> 1) + cb * 8) = make_uint2(packed[0], packed[1]);
      scales[r * CB + cb] = (uint8_t)sc;
    }
  }

  if constexpr (kStats) {
    // LDS: tpr*16 int64 sums, then tpr*16 uint32 maxima.
    unsigned long long* lsum = reinterpret_cast<unsigned long long*>(dyn_lds);
    uint32_t* lmax = reinterpret_cast<uint32_t*>(lsum + tpr * 16);
    for (int i = threadIdx.x; i < tpr * 16; i += kThreads) {
      lsum[i] = 0ull;
      lmax[i] = 0u;
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (acc[i] != 0.0) atomicAdd(&lsum[cbl * 16 + i], (unsigned long long)acc[i]);
        if (emax[i] != 0.0f) atomicMax(&lmax[cbl * 16 + i], __float_as_uint(emax[i]));
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < tpr * 16; i += kThreads) {
      const int64_t k = (int64_t)blockIdx.x * tpr * 16 + i;
      if (k < K) {
        if (lsum[i]) atomicAdd(reinterpret_cast<unsigned long long*>(score) + k, lsum[i]);
        if (lmax[i]) atomicMax(chmax + k, lmax[i]);
      }
    }
  }
}

// ---------------------------------------------------------------- select
constexpr int kSelThreads = 1024;
constexpr int kSelPer = 16;  // K <= 16384

// Exclusive prefix sum over the workgroup; returns the total in *total.
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
  for (int i = 0; i < kSelThreads / 64; ++i) {
    const uint32_t s = wsum[i];
    if (i < w) before += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

__global__ __launch_bounds__(kSelThreads) void k_select(
    const int64_t* __restrict__ score_in, const uint32_t* __restrict__ chmax, int K, int n_sel,
    int32_t* __restrict__ selected, uint8_t* __restrict__ kact, uint16_t* __restrict__ mask16,
    float* __restrict__ res_ts) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t found[2];
  __shared__ uint32_t wsum[kSelThreads / 64];
  __shared__ uint32_t wmax[kSelThreads / 64];
  __shared__ uint8_t lmask[kSelPer * kSelThreads];
  const int t = threadIdx.x;
  const int per = (K + kSelThreads - 1) / kSelThreads;
  const int base = t * per;

  uint64_t v[kSelPer];
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int k = base + i;
    v[i] = (i < per && k < K) ? (uint64_t)score_in[k] : 0ull;
  }
  auto valid = [&](int i) { return i < per && base + i < K; };

  // Radix select (8-bit digits, most significant first) of the n_sel-th
  // largest score T; `remaining` ends as the number of channels equal to T
  // that are taken (the lowest-index ones).
  uint64_t prefix = 0, pmask = 0;
  uint32_t remaining = (uint32_t)n_sel;
  if (n_sel > 0) {
    for (int shift = 56; shift >= 0; shift -= 8) {
      if (t < 256) hist[t] = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kSelPer; ++i)
        if (valid(i) && (v[i] & pmask) == prefix) atomicAdd(&hist[(v[i] >> shift) & 255u], 1u);
      __syncthreads();
      if (t < 64) {
        // lane t owns digits 255-4t .. 252-4t (descending order)
        uint32_t c[4], s = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[j] = hist[255 - (4 * t + j)];
          s += c[j];
        }
        uint32_t inc = s;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t n = __shfl_up(inc, o, 64);
          if (t >= o) inc += n;
        }
        uint32_t run = inc - s;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (run < remaining && remaining <= run + c[j]) {
            found[0] = 255u - (uint32_t)(4 * t + j);
            found[1] = run;
          }
          run += c[j];
        }
      }
      __syncthreads();
      prefix |= (uint64_t)found[0] << shift;
      pmask |= (uint64_t)0xFF << shift;
      remaining -= found[1];
      __syncthreads();
    }
  }
  const uint64_t T = prefix;

  // rank among channels equal to T (ascending index)
  uint32_t eq = 0;
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) eq += (n_sel > 0 && valid(i) && v[i] == T) ? 1u : 0u;
  uint32_t tot;
  uint32_t eq_before = block_exclusive_scan(eq, wsum, &tot);

  uint32_t nsel_local = 0;
  float amax_r = 0.0f;
  uint8_t m[kSelPer];
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    bool s = false;
    if (n_sel > 0 && valid(i)) {
      if (v[i] > T) s = true;
      else if (v[i] == T) { s = eq_before < remaining; ++eq_before; }
    }
    m[i] = s ? 1 : 0;
    if (s) {
      ++nsel_local;
      amax_r = __builtin_fmaxf(amax_r, __uint_as_float(chmax[base + i]));
    }
    if (valid(i)) lmask[base + i] = m[i];
  }
  uint32_t pos = block_exclusive_scan(nsel_local, wsum, &tot);
#pragma unroll
  for (int i = 0; i < kSelPer; ++i)
    if (m[i]) selected[pos++] = base + i;

  amax_r = nv_wave_max(amax_r);
  if ((t & 63) == 0) wmax[t >> 6] = __float_as_uint(amax_r);
  __syncthreads();  // also publishes lmask
  if (t == 0) {
    float a = 0.0f;
    for (int w = 0; w < kSelThreads / 64; ++w) a = __builtin_fmaxf(a, __uint_as_float(wmax[w]));
    *res_ts = nv_tensor_scale(a);
  }
  for (int b = t; b < (K >> 4); b += kSelThreads) {
    uint32_t bits = 0;
    for (int j = 0; j < 16; ++j) bits |= (uint32_t)lmask[b * 16 + j] << j;
    mask16[b] = (uint16_t)bits;
    kact[b] = bits ? 1 : 0;
  }
}

// -------------------------------------------------------------- residual
__global__ __launch_bounds__(kThreads) void k_residual(
    const void* __restrict__ x, int bf16, int64_t rows, int64_t K, int64_t ldx,
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ tscale, const uint16_t* __restrict__ mask16,
    const float* __restrict__ res_ts, uint8_t* __restrict__ res_codes,
    uint8_t* __restrict__ res_scales) {
  const int64_t CB = K >> 4;
  const int64_t nblk = rows * CB;
  const float s_t = *tscale;
  const float s_tr = *res_ts;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblk;
       b += (int64_t)gridDim.x * kThreads) {
    const int64_t r = b / CB, cb = b - r * CB;
    const uint32_t m = mask16[cb];
    uint32_t packed[2] = {0u, 0u};
    uint32_t sc = 0u;
    if (m) {
      float v[16];
      nv_load16(x, bf16, r * ldx + cb * 16, v);
      const uint2 cw = *reinterpret_cast<const uint2*>(codes + r * (K >> 1) + cb * 8);
      const float sb = nv_e4m3_to_f32(scales[r * CB + cb]);
      float e[16];
      float amax_b = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t c = ((i < 8 ? cw.x : cw.y) >> ((i & 7) * 4)) & 15u;
        const float d = (nv_e2m1_to_f32(c) * sb) * s_t;
        e[i] = ((m >> i) & 1u) ? v[i] - d : 0.0f;
        amax_b = __builtin_fmaxf(amax_b, __builtin_fabsf(e[i]));
      }
      sc = nv_block_scale(amax_b, s_tr);
      const float Sb = nv_e4m3_to_f32(sc) * s_tr;
      const float rb = nv_block_recip(Sb);
#pragma unroll
      for (int i = 0; i < 16; ++i) packed[i >> 3] |= nv_e2m1_encode(e[i] * rb) << ((i & 7) * 4);
    }
    *reinterpret_cast<uint2*>(res_codes + r * (K >> 1) + cb * 8) = make_uint2(packed[0], packed[1]);
    res_scales[r * CB + cb] = (uint8_t)sc;
  }
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

int nvfp4_quantize(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx,
                   const float* amax_in, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                   int64_t* channel_score, float* channel_max, void* ws, size_t ws_bytes,
                   void* stream) {
  int st = check_x(x, dtype, rows, K, ldx);
  if (st) return st;
  NV_RETURN_IF(!tensor_scale || (rows > 0 && (!codes || !scales)), NVFP4_ERR_NULL);
  NV_RETURN_IF((channel_score == nullptr) != (channel_max == nullptr), NVFP4_ERR_NULL);
  NV_RETURN_IF(!nv_aligned16(codes), NVFP4_ERR_ALIGN);
  NV_RETURN_IF(channel_score && ((reinterpret_cast<uintptr_t>(channel_score) & 7) ||
                                 (reinterpret_cast<uintptr_t>(channel_max) & 3)),
               NVFP4_ERR_ALIGN);
  NV_RETURN_IF(!amax_in && (!ws || ws_bytes < nvfp4_quantize_workspace_size(rows, K)),
               NVFP4_ERR_WORKSPACE);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool stats = channel_score != nullptr;
  uint32_t* chm = reinterpret_cast<uint32_t*>(channel_max);
  float* partials = reinterpret_cast<float*>(ws);
  const int bf16 = dtype == NVFP4_IN_BF16;
  const int64_t CB = K / 16;
  int nparts = 0;
  if (!amax_in) {
    nparts = (int)blocks_for(rows * CB, kThreads * 4, kMaxParts);
    hipLaunchKernelGGL(k_amax, dim3(nparts), dim3(kThreads), 0, s, x, bf16, rows, K, ldx,
                       partials, stats ? channel_score : nullptr, chm);
  } else if (stats) {
    hipLaunchKernelGGL(k_zero_stats, dim3((unsigned)blocks_for(K, 256, 1024)), dim3(256), 0, s,
                       K, channel_score, chm);
  }
  // column tiles of at most 256 column blocks, rows_per_iter sub-rows
  const int64_t ntile = (CB + kThreads - 1) / kThreads;
  const int tpr = (int)((CB + ntile - 1) / ntile);
  const int rpi = kThreads / tpr;
  int64_t splits = blocks_for(rows, (int64_t)rpi * 16, 65535);
  const int64_t max_splits = 512 / ntile > 0 ? 512 / ntile : 1;
  if (splits > max_splits) splits = max_splits;
  const int64_t rows_per_split = rows > 0 ? (rows + splits - 1) / splits : 1;
  const size_t lds = stats ? (size_t)tpr * 16 * (sizeof(uint64_t) + sizeof(uint32_t)) : 0;
  if (stats)
    hipLaunchKernelGGL(k_quant<true>, dim3((unsigned)ntile, (unsigned)splits), dim3(kThreads), lds,
                       s, x, bf16, rows, K, ldx, partials, nparts, amax_in, codes, scales,
                       tensor_scale, channel_score, chm, tpr, rpi, rows_per_split);
  else
    hipLaunchKernelGGL(k_quant<false>, dim3((unsigned)ntile, (unsigned)splits), dim3(kThreads), 0,
                       s, x, bf16, rows, K, ldx, partials, nparts, amax_in, codes, scales,
                       tensor_scale, nullptr, nullptr, tpr, rpi, rows_per_split);
  return nv_launch_status();
}

size_t rac_select_residual_workspace_size(int64_t, int64_t K) {
  return nv_round256(sizeof(uint16_t) * (size_t)(K > 0 ? K / 16 : 0));
}

int rac_select_residual(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx,
                        const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                        const int64_t* channel_score, const float* channel_max, int64_t n_select,
                        int32_t* selected, uint8_t* kblock_active, uint8_t* res_codes,
                        uint8_t* res_scales, float* res_tensor_scale, void* ws, size_t ws_bytes,
                        void* stream) {
  int st = check_x(x, dtype, rows, K, ldx);
  if (st) return st;
  NV_RETURN_IF(!tensor_scale || !channel_score || !channel_max || !kblock_active ||
                   !res_tensor_scale,
               NVFP4_ERR_NULL);
  NV_RETURN_IF(rows > 0 && (!codes || !scales || !res_codes || !res_scales), NVFP4_ERR_NULL);
  NV_RETURN_IF(n_select < 0 || n_select > K || K > kSelPer * kSelThreads, NVFP4_ERR_SHAPE);
  NV_RETURN_IF(n_select > 0 && !selected, NVFP4_ERR_NULL);
  NV_RETURN_IF(!nv_aligned16(codes) || !nv_aligned16(res_codes) ||
                   (reinterpret_cast<uintptr_t>(channel_score) & 7),
               NVFP4_ERR_ALIGN);
  NV_RETURN_IF(!ws || ws_bytes < rac_select_residual_workspace_size(rows, K) ||
                   (reinterpret_cast<uintptr_t>(ws) & 1),
               NVFP4_ERR_WORKSPACE);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint16_t* mask16 = reinterpret_cast<uint16_t*>(ws);
  hipLaunchKernelGGL(k_select, dim3(1), dim3(kSelThreads), 0, s, channel_score,
                     reinterpret_cast<const uint32_t*>(channel_max), (int)K, (int)n_select,
                     selected, kblock_active, mask16, res_tensor_scale);
  st = nv_launch_status();
  if (st) return st;
  const int64_t nblk = rows * (K / 16);
  hipLaunchKernelGGL(k_residual, dim3((unsigned)blocks_for(nblk, kThreads, 8192)), dim3(kThreads),
                     0, s, x, dtype == NVFP4_IN_BF16, rows, K, ldx, codes, scales, tensor_scale,
                     mask16, res_tensor_scale, res_codes, res_scales);
  return nv_launch_status();
}

}  // extern "C"
