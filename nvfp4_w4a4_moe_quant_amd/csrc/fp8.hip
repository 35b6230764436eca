// FP8 (E4M3) W8A8 comparator: per-row quantizer and grouped GEMM.
//
// The QUADS pages measure their rollout throughput against FP8 rollout (arXiv
// abstract on the mlsanity page; blog post "Why 4-bit RL rollout collapses",
// section "What it buys") without saying how the FP8 engine scales its
// tensors.  This file implements the usual dynamic per-token / static
// per-channel form: one FP32 scale per activation row and per weight output
// channel, s = RN32(amax / 448), r = RN32(1 / s), element = E4M3(RN32(x r))
// rounded to nearest even with saturation, the sign kept.
//
// MI355X design:
//  * Quantizer: one wave per row; rows up to 8192 elements stay in registers
//    between the max and the encode, longer rows are read twice (the second
//    read hits the caches).  The hardware FP8 conversion rounds to nearest
//    even; a clamp to +-448 before it gives the saturation.
//  * GEMM: v_mfma_scale_f32_32x32x64_f8f6f4 with FP8 operands and unit block
//    scales (E8M0 127).  The operands go from LDS to the matrix cores as they
//    are; the row and channel scales factor out of the K sum and are applied
//    in the epilogue.
//  * Decode shape (one group, <= 64 rows): k_fp8_gemv16, the FP8 counterpart
//    of the NVFP4 decode kernel (16 columns per workgroup, waves split K).
//  * Grouping, gather, XCD-aware tile order and the SiLU gate/up pairing are
//    those of the NVFP4 kernel.  K is consumed in chunks of 128 bytes per row
//    (two MFMA steps of 64); the global->LDS DMA runs NSTAGE - 1 chunks ahead.
//    16-byte pieces are XOR-swizzled per row so that fragment reads hit
//    distinct banks.
//  * Measured on MI355X (MoE gate/up shape, 32768 x 1536 x 2048 grouped over
//    128 experts): with 128 x 128 tiles the kernel was bound by its
//    global->LDS copies (about 1.8 GB per call), not by the matrix cores;
//    256 x 256 tiles of eight waves halve the copies per MFMA.

#include <type_traits>

#include "common.h"

namespace {

typedef int int8v __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// ------------------------------------------------------------------ quantizer

__device__ __forceinline__ float f8_clamp(float v) {
  return __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f);
}

// 8 values times r -> 8 E4M3 bytes, value i in byte i (little-endian order).
__device__ __forceinline__ uint2 f8_encode8(const float* x, float r) {
  uint32_t w[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int acc = 0;
    acc = __builtin_amdgcn_cvt_pk_fp8_f32(f8_clamp(x[4 * j] * r), f8_clamp(x[4 * j + 1] * r),
                                          acc, false);
    acc = __builtin_amdgcn_cvt_pk_fp8_f32(f8_clamp(x[4 * j + 2] * r),
                                          f8_clamp(x[4 * j + 3] * r), acc, true);
    w[j] = (uint32_t)acc;
  }
  return make_uint2(w[0], w[1]);
}

// 8 consecutive inputs at element offset `off` (16-byte aligned for bf16,
// 32-byte aligned for FP32).
template <bool BF16>
__device__ __forceinline__ void f8_load8(const void* x, int64_t off, float* v) {
  if constexpr (BF16) {
    const uint4 a = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + off);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* q = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
    const float4 a = q[0], b = q[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Row scale and reciprocal: s = RN32(amax / 448) (double quotient, rounded
// once), r = RN32(1 / s), both 0 for an all-zero row.
__device__ __forceinline__ void f8_row_scale(float amax, float& s, float& r) {
  s = (float)((double)amax / 448.0);
  r = s > 0.0f ? (float)(1.0 / (double)s) : 0.0f;
}

// One wave per row, four rows per workgroup.  VPL > 0: each lane holds VPL
// vectors of 8 elements (K <= 512 VPL); VPL == 0: two passes over the row.
template <bool BF16, int VPL>
__global__ __launch_bounds__(256) void k_fp8_rows(const void* x, int64_t rows, int K,
                                                  uint8_t* codes, float* scales) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  const int nv = K >> 3;
  const int64_t base = row * (int64_t)K;
  float amax = 0.0f, s, r;
  if constexpr (VPL > 0) {
    float v[VPL][8];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int c = lane + 64 * i;
      if (c < nv) {
        f8_load8<BF16>(x, base + 8 * c, v[i]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i][e]));
    }
    f8_row_scale(nv_wave_max(amax), s, r);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int c = lane + 64 * i;
      if (c < nv) *reinterpret_cast<uint2*>(codes + base + 8 * c) = f8_encode8(v[i], r);
    }
  } else {
    for (int c = lane; c < nv; c += 64) {
      float v[8];
      f8_load8<BF16>(x, base + 8 * c, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[e]));
    }
    f8_row_scale(nv_wave_max(amax), s, r);
    for (int c = lane; c < nv; c += 64) {
      float v[8];
      f8_load8<BF16>(x, base + 8 * c, v);
      *reinterpret_cast<uint2*>(codes + base + 8 * c) = f8_encode8(v, r);
    }
  }
  if (lane == 0) scales[row] = s;
}

template <bool BF16>
int launch_rows(const void* x, int64_t rows, int K, uint8_t* codes, float* scales,
                hipStream_t st) {
  const int per_lane = (K / 8 + 63) / 64;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (per_lane <= 1)
    hipLaunchKernelGGL((k_fp8_rows<BF16, 1>), grid, block, 0, st, x, rows, K, codes, scales);
  else if (per_lane <= 2)
    hipLaunchKernelGGL((k_fp8_rows<BF16, 2>), grid, block, 0, st, x, rows, K, codes, scales);
  else if (per_lane <= 4)
    hipLaunchKernelGGL((k_fp8_rows<BF16, 4>), grid, block, 0, st, x, rows, K, codes, scales);
  else if (per_lane <= 8)
    hipLaunchKernelGGL((k_fp8_rows<BF16, 8>), grid, block, 0, st, x, rows, K, codes, scales);
  else if (per_lane <= 16)
    hipLaunchKernelGGL((k_fp8_rows<BF16, 16>), grid, block, 0, st, x, rows, K, codes, scales);
  else
    hipLaunchKernelGGL((k_fp8_rows<BF16, 0>), grid, block, 0, st, x, rows, K, codes, scales);
  return nv_launch_status();
}

// ----------------------------------------------------------------------- GEMM

struct F8Params {
  int G, N, K, total_rows;
  const int32_t* offsets;
  const int32_t* gather;
  const uint8_t* a_codes;
  const float* a_scales;
  const uint8_t* w_codes;
  const float* w_scales;
  void* out;
  int m_slots, n_tiles;
};

constexpr int KB = 128;  // largest k (= bytes) per row per chunk; K % KB == 0

// Position of logical 16-byte piece lp of a row of PPR pieces is
// lp ^ f8_swz<PPR>(row): the rows one ds_read_b128 phase touches land on
// distinct banks.  128-byte rows (8 pieces): 8 rows of a 32-bank or 16 of a
// 64-bank LDS phase; 64-byte rows (4 pieces): 16 rows of a 64-bank phase
// (row % 4 picks the bank quarter, the swizzle spreads row / 4 over it).
template <int PPR>
__device__ __forceinline__ uint32_t f8_swz(uint32_t row) {
  return PPR == 8 ? ((row ^ (row >> 3)) & 7u) : ((row >> 2) & 3u);
}

// silu(g) * u in FP32 with the hardware exp and reciprocal.
__device__ __forceinline__ float f8_silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int NSTAGE, int MINW, bool SILU, bool GATHER,
          int KC = KB, bool OUT_BF16 = false>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, MINW) void k_fp8_gemm(F8Params p) {
  static_assert(KC == 64 || KC == 128, "64- or 128-byte chunks");
  constexpr int PPR = KC / 16;  // 16-byte pieces per row per chunk
  constexpr int NW = WAVES_M * WAVES_N;  // waves per workgroup
  constexpr int NT = 64 * NW;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "tile");
  static_assert(!SILU || FN % 2 == 0, "SiLU pairs gate/up fragments");
  constexpr int ROWS = BM + BN;  // A rows, then W rows
  constexpr int PIECES = ROWS * PPR;
  static_assert(PIECES % NT == 0, "whole wave-loads");
  constexpr int NPI = PIECES / NT;  // 16-byte pieces per thread per chunk
  constexpr int STAGE = ROWS * KC;
  static_assert(NSTAGE >= 2 && (NSTAGE - 2) * NPI <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NSTAGE * STAGE];
  __shared__ float sc_lds[ROWS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lr = lane & 31, lh = lane >> 5;

  // long groups in bands of 8 m-tiles (a dense GEMM shares A and W in L2)
  const NvTile tile = nv_find_tile<8>(p.offsets, p.G, BM, p.m_slots, p.n_tiles);
  if (tile.grp < 0) return;  // wave-uniform and identical in every wave
  const int grp = tile.grp, nt = tile.nt;
  const int row_beg = p.offsets[grp] + tile.local * BM;
  const int row_end = p.offsets[grp + 1];
  const int K = p.K, I = p.N >> 1;

  auto src_row = [&](int i) -> int64_t {  // i in [0, BM); padding rows repeat the last
    int m = row_beg + i;
    if (m >= row_end) m = row_end - 1;
    return GATHER ? (int64_t)p.gather[m] : (int64_t)m;
  };
  auto w_row = [&](int i) -> int64_t {  // i in [0, BN)
    int n;
    if constexpr (SILU) {
      const int wv = i / WTN, f = (i % WTN) / 32, rr = i % 32;
      n = ((f & 1) ? I : 0) + nt * (BN / 2) + wv * (WTN / 2) + (f >> 1) * 32 + rr;
    } else {
      n = nt * BN + i;
    }
    return (int64_t)grp * p.N + n;
  };

  for (int i = tid; i < ROWS; i += NT)
    sc_lds[i] = i < BM ? p.a_scales[src_row(i)] : p.w_scales[w_row(i - BM)];

  // wave-instruction j of a chunk writes 1 KiB (8 rows x 128 B) contiguously;
  // lane l fetches the piece that the swizzle places in its slot
  const uint8_t* gsrc[NPI];
#pragma unroll
  for (int j = 0; j < NPI; ++j) {
    const int slot = (j * NW + wave) * 64 + lane;
    const int row = slot / PPR;
    const uint32_t piece = (uint32_t)(slot % PPR) ^ f8_swz<PPR>((uint32_t)row);
    const uint8_t* base = row < BM ? p.a_codes + src_row(row) * K : p.w_codes + w_row(row - BM) * K;
    gsrc[j] = base + piece * 16;
  }
  auto issue = [&](int chunk, int buf) {
    const uint32_t st = (uint32_t)(uintptr_t)(lds_ptr_t)(lds + buf * STAGE);
#pragma unroll
    for (int j = 0; j < NPI; ++j) {
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(st + (j * NW + wave) * 1024);
      const uint8_t* g = gsrc[j] + (int64_t)chunk * KC;
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                   :: "s"(m0), "v"(g) : "memory", "m0");
    }
  };

  float16v acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  const bool wave_live = row_beg + wm * WTM < row_end;  // wave-uniform
  // 32 contiguous k of row i starting at logical piece lp (two pieces)
  auto frag = [&](const uint8_t* base, uint32_t i, uint32_t lp) -> int8v {
    const uint8_t* rp = base + i * KC;
    const uint4 x = *reinterpret_cast<const uint4*>(rp + ((lp ^ f8_swz<PPR>(i)) << 4));
    const uint4 y = *reinterpret_cast<const uint4*>(rp + (((lp + 1) ^ f8_swz<PPR>(i)) << 4));
    int8v v;
    v[0] = (int)x.x; v[1] = (int)x.y; v[2] = (int)x.z; v[3] = (int)x.w;
    v[4] = (int)y.x; v[5] = (int)y.y; v[6] = (int)y.z; v[7] = (int)y.w;
    return v;
  };
  constexpr int STEPS = KC / 64;
  // operands of one 64-k step; lanes 32-63 take the upper 32 k of the step
  auto load_step = [&](const uint8_t* base, int s, int8v* av, int8v* wv) {
    const uint32_t lp = 4 * s + 2 * lh;
#pragma unroll
    for (int a = 0; a < FM; ++a) av[a] = frag(base, wm * WTM + a * 32 + lr, lp);
#pragma unroll
    for (int b = 0; b < FN; ++b) wv[b] = frag(base, BM + wn * WTN + b * 32 + lr, lp);
  };
  auto mfma_step = [&](const int8v* av, const int8v* wv) {
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av[a], wv[b], acc[a][b],
                                                                    0, 0, 0, 127, 0, 127);
  };

  const int nchunks = K / KC;
#pragma unroll
  for (int c = 0; c < NSTAGE - 1; ++c)
    if (c < nchunks) issue(c, c);
  if (nchunks > 1 && NSTAGE > 2)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NSTAGE - 2) * NPI) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int buf = 0;
  for (int ch = 0; ch < nchunks; ++ch) {
    const int nxt = ch + NSTAGE - 1;
    if (nxt < nchunks) issue(nxt, nxt % NSTAGE);
    if (wave_live) {
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        int8v av[FM], wv[FN];
        load_step(lds + buf * STAGE, s, av, wv);
        mfma_step(av, wv);
      }
    }
    if (nxt < nchunks && NSTAGE > 2)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NSTAGE - 2) * NPI) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    buf = buf + 1 == NSTAGE ? 0 : buf + 1;
  }
  if (!wave_live) return;

  // ---- epilogue: element e of fragment (a, b) sits at tile row
  // wm*WTM + a*32 + (e>>2)*8 + lh*4 + (e&3) and tile column wn*WTN + b*32 + lr
  const int m0 = row_beg + wm * WTM + lh * 4;
  const bool full = row_beg + (wm + 1) * WTM <= row_end;  // wave-uniform
  const float* sa = sc_lds + wm * WTM + lh * 4;
  const float* sw = sc_lds + BM + wn * WTN + lr;
  if constexpr (!SILU) {
    using OutT = std::conditional_t<OUT_BF16, uint16_t, float>;
    OutT* ob = reinterpret_cast<OutT*>(p.out) + (int64_t)m0 * p.N + nt * BN + wn * WTN + lr;
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b) {
        const float swb = sw[b * 32];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int dm = a * 32 + (e >> 2) * 8 + (e & 3);
          if (full || m0 + dm < row_end) {
            const float y = (sa[dm] * swb) * acc[a][b][e];
            if constexpr (OUT_BF16)
              ob[(int64_t)dm * p.N + b * 32] = (uint16_t)nv_f32_to_bf16(y);
            else
              ob[(int64_t)dm * p.N + b * 32] = y;
          }
        }
      }
  } else {
    uint16_t* ob = reinterpret_cast<uint16_t*>(p.out) + (int64_t)m0 * I + nt * (BN / 2) +
                   wn * (WTN / 2) + lr;
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; b += 2) {
        const float swg = sw[b * 32], swu = sw[(b + 1) * 32];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int dm = a * 32 + (e >> 2) * 8 + (e & 3);
          if (full || m0 + dm < row_end) {
            const float g = (sa[dm] * swg) * acc[a][b][e];
            const float u = (sa[dm] * swu) * acc[a][b + 1][e];
            ob[(int64_t)dm * I + (b >> 1) * 32] = (uint16_t)nv_f32_to_bf16(f8_silu_mul(g, u));
          }
        }
      }
  }
}

template <int BM, int BN, int WM, int WN, int NS, int MINW, bool SILU, bool GATHER, int KC = KB,
          bool OUT_BF16 = false>
int launch_f8(F8Params& p, hipStream_t s) {
  if (p.N % BN) return NVFP4_ERR_SHAPE;
  p.m_slots = (p.total_rows + BM - 1) / BM + p.G;
  p.n_tiles = p.N / BN;
  const int64_t nb = (int64_t)p.m_slots * p.n_tiles;
  if (nb > 0x7fffffff) return NVFP4_ERR_SHAPE;
  hipLaunchKernelGGL((k_fp8_gemm<BM, BN, WM, WN, NS, MINW, SILU, GATHER, KC, OUT_BF16>), dim3((unsigned)nb),
                     dim3(64 * WM * WN), 0, s, p);
  return nv_launch_status();
}

// N % 256 == 0: 256 x 256 tiles of eight 64 x 128 waves, two stages, one
// workgroup per CU (twice the MFMAs per staged byte and per LDS fragment read
// of 128 x 128 tiles with 64 x 64 waves, which were bound by the copies into
// LDS).  Other N: 128 x 128 tiles (waves of 64 x 64), two workgroups per CU.
template <bool SILU, bool GATHER, bool OUT_BF16 = false>
int launch_f8_cfg(F8Params& p, hipStream_t s) {
  if (p.N % 256 == 0) return launch_f8<256, 256, 4, 2, 2, 1, SILU, GATHER, KB, OUT_BF16>(p, s);
  return launch_f8<128, 128, 2, 2, 2, 2, SILU, GATHER, KB, OUT_BF16>(p, s);
}

// ---------------------------------------------------------------------------
// Decode shape (one group, at most 64 rows, K % 512 == 0, F32 epilogue): a
// workgroup owns 16 output columns and one 16-row tile over the whole of K,
// so N/16 workgroups stream W once; its waves split K.  Each 128-k group is
// one v_mfma_scale_f32_16x16x128_f8f6f4: lane l feeds row (or column) l % 16
// with the 32 contiguous bytes k = 32 (l / 16) + 0..31 of the group, the same
// layout for both operands.  Every lane issues all its loads of a pass before
// the first use; the waves add their accumulators through LDS in a fixed
// order.
typedef float float4v __attribute__((ext_vector_type(4)));
constexpr int kF8GvGroups = 4;   // 128-k groups per wave per load pass
constexpr int kF8GvMaxRows = 64;

template <int WAVES, bool GATHER>
__global__ __launch_bounds__(64 * WAVES) void k_fp8_gemv16(F8Params p) {
  __shared__ float4v red[WAVES][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int w = (wave + (int)blockIdx.x) % WAVES;  // spread the A reads over lines
  const int c = lane & 15, q = lane >> 4;
  const int K = p.K, kw = K / WAVES;
  const int m = (int)blockIdx.y * 16 + c;  // A row fed by this lane
  const bool mv = m < p.total_rows;
  const int64_t n = (int64_t)blockIdx.x * 16 + c;  // W row fed by this lane
  const uint8_t* wr = p.w_codes + n * K;
  const int64_t src = mv ? (GATHER ? (int64_t)p.gather[m] : (int64_t)m) : 0;
  const uint8_t* ar = p.a_codes + src * K;
  float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int g0 = 0; g0 < kw; g0 += 128 * kF8GvGroups) {
    const int ng = (kw - g0) / 128 < kF8GvGroups ? (kw - g0) / 128 : kF8GvGroups;
    uint4 wv[kF8GvGroups][2], av[kF8GvGroups][2];
#pragma unroll
    for (int g = 0; g < kF8GvGroups; ++g) {
      const int kb = w * kw + g0 + g * 128 + q * 32;
      wv[g][0] = wv[g][1] = av[g][0] = av[g][1] = make_uint4(0u, 0u, 0u, 0u);
      if (g < ng) {
        wv[g][0] = *reinterpret_cast<const uint4*>(wr + kb);
        wv[g][1] = *reinterpret_cast<const uint4*>(wr + kb + 16);
        if (mv) {
          av[g][0] = *reinterpret_cast<const uint4*>(ar + kb);
          av[g][1] = *reinterpret_cast<const uint4*>(ar + kb + 16);
        }
      }
    }
#pragma unroll
    for (int g = 0; g < kF8GvGroups; ++g) {
      if (g >= ng) break;
      int8v a, b;
      a[0] = (int)av[g][0].x; a[1] = (int)av[g][0].y; a[2] = (int)av[g][0].z; a[3] = (int)av[g][0].w;
      a[4] = (int)av[g][1].x; a[5] = (int)av[g][1].y; a[6] = (int)av[g][1].z; a[7] = (int)av[g][1].w;
      b[0] = (int)wv[g][0].x; b[1] = (int)wv[g][0].y; b[2] = (int)wv[g][0].z; b[3] = (int)wv[g][0].w;
      b[4] = (int)wv[g][1].x; b[5] = (int)wv[g][1].y; b[6] = (int)wv[g][1].z; b[7] = (int)wv[g][1].w;
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
    }
  }
  red[w][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  float4v sum = red[0][lane];
#pragma unroll
  for (int i = 1; i < WAVES; ++i) sum += red[i][lane];
  const float sw = p.w_scales[n];
  float* out = reinterpret_cast<float*>(p.out);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (int)blockIdx.y * 16 + 4 * q + i;  // D row of element i
    if (row < p.total_rows) {
      const int64_t sr = GATHER ? (int64_t)p.gather[row] : (int64_t)row;
      out[(int64_t)row * p.N + n] = (p.a_scales[sr] * sw) * sum[i];
    }
  }
}

template <bool GATHER>
int launch_f8_gemv(F8Params& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.N / 16), (unsigned)((p.total_rows + 15) / 16));
  if (p.K % 1024 == 0)
    hipLaunchKernelGGL((k_fp8_gemv16<8, GATHER>), grid, dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL((k_fp8_gemv16<4, GATHER>), grid, dim3(256), 0, s, p);
  return nv_launch_status();
}

}  // namespace

extern "C" {

int fp8_quantize_rows(const void* x, int in_dtype, int64_t rows, int64_t K, uint8_t* codes,
                      float* row_scales, void* stream) {
  NV_RETURN_IF(in_dtype != NVFP4_IN_F32 && in_dtype != NVFP4_IN_BF16, NVFP4_ERR_DTYPE);
  NV_RETURN_IF(rows < 0 || K <= 0 || K % 16 || K > (1 << 24) || rows > 0x7fffffffLL * 4,
               NVFP4_ERR_SHAPE);
  if (rows == 0) return NVFP4_OK;
  NV_RETURN_IF(!x || !codes || !row_scales, NVFP4_ERR_NULL);
  NV_RETURN_IF(!nv_aligned16(x) || (reinterpret_cast<uintptr_t>(codes) & 7) ||
                   (reinterpret_cast<uintptr_t>(row_scales) & 3),
               NVFP4_ERR_ALIGN);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return in_dtype == NVFP4_IN_BF16 ? launch_rows<true>(x, rows, (int)K, codes, row_scales, s)
                                   : launch_rows<false>(x, rows, (int)K, codes, row_scales, s);
}

int fp8_grouped_gemm(const fp8_gemm_args_t* a, void* stream) {
  NV_RETURN_IF(!a, NVFP4_ERR_NULL);
  NV_RETURN_IF(a->epilogue != NVFP4_EPI_F32 && a->epilogue != NVFP4_EPI_SILU_MUL_BF16 &&
                   a->epilogue != NVFP4_EPI_BF16,
               NVFP4_ERR_DTYPE);
  NV_RETURN_IF(a->num_groups < 1 || a->total_rows < 0 || a->N <= 0 || a->K <= 0 ||
                   a->K % KB || a->N % 128 || a->N > (1 << 24) || a->K > (1 << 24) ||
                   a->total_rows > 0x7fffffff || a->num_groups > (1 << 20),
               NVFP4_ERR_SHAPE);
  NV_RETURN_IF(!a->group_offsets || !a->w_codes || !a->w_scales, NVFP4_ERR_NULL);
  if (a->total_rows == 0) return NVFP4_OK;
  NV_RETURN_IF(!a->a_codes || !a->a_scales || !a->out, NVFP4_ERR_NULL);
  NV_RETURN_IF(!nv_aligned16(a->a_codes) || !nv_aligned16(a->w_codes) ||
                   (reinterpret_cast<uintptr_t>(a->a_scales) & 3) ||
                   (reinterpret_cast<uintptr_t>(a->w_scales) & 3),
               NVFP4_ERR_ALIGN);
  F8Params p{};
  p.G = (int)a->num_groups;
  p.N = (int)a->N;
  p.K = (int)a->K;
  p.total_rows = (int)a->total_rows;
  p.offsets = a->group_offsets;
  p.gather = a->gather_rows;
  p.a_codes = a->a_codes;
  p.a_scales = a->a_scales;
  p.w_codes = a->w_codes;
  p.w_scales = a->w_scales;
  p.out = a->out;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool silu = a->epilogue == NVFP4_EPI_SILU_MUL_BF16, gather = a->gather_rows != nullptr;
  const bool bf16 = a->epilogue == NVFP4_EPI_BF16;
  if (p.G == 1 && p.total_rows <= kF8GvMaxRows && p.K % 512 == 0 && !silu && !bf16)
    return gather ? launch_f8_gemv<true>(p, s) : launch_f8_gemv<false>(p, s);
  if (silu) return gather ? launch_f8_cfg<true, true>(p, s) : launch_f8_cfg<true, false>(p, s);
  if (bf16)
    return gather ? launch_f8_cfg<false, true, true>(p, s) : launch_f8_cfg<false, false, true>(p, s);
  return gather ? launch_f8_cfg<false, true>(p, s) : launch_f8_cfg<false, false>(p, s);
}

}  // extern "C"
