// Grouped W4A4 GEMM over experts with the RAC residual pass fused in.
//
// QUADS arXiv abstract (mlsanity page, "Abstract (arXiv)"): native W4A4 FP4
// GEMMs on NVFP4 operands.  QUADS blog post, section "Two fixes, on two
// different sides": a second, residual FP4 pass over the selected channels is
// fused into the existing kernel and layered on top of the intact main pass.
//
// MI355X design:
//  * Operands stay NVFP4 in HBM and LDS (4 bits per element plus one E4M3
//    byte per 16).  Each wave dequantizes the fragments it feeds to the matrix
//    cores: an E2M1 value times an E4M3 scale has at most 6 significant bits
//    and lies in [2^-10, 2688], so g * s_b is exact in fp16; the FP4->fp16
//    conversion and the scale multiply are packed VALU ops.
//  * v_mfma_f32_32x32x16_f16 (gfx950) accumulates exact fp16 products in FP32.
//    K = 16 per instruction is exactly one NVFP4 block.
//  * Main and residual rows share every W fragment; they keep separate FP32
//    accumulators because their tensor scales differ:
//        y = s_tw * (s_ta * acc_main + s_tr * acc_res).
//  * K is consumed in chunks of 128 (8 MFMA steps).  Inside a chunk, lanes
//    32-63 take the upper 64 k of the chunk instead of the next 8 (a fixed
//    permutation of k applied identically to A, R and W, so the contraction is
//    unchanged); each lane then reads 32 contiguous code bytes per row.
//  * Tiles: (group, m-tile, n-tile) from the device-side group offsets; every
//    workgroup finds its tile with a wave scan, tiles past the real count exit.
//    Workgroup ids are remapped so that consecutive tiles (same expert, same
//    rows) run on the same XCD and share its L2.
//  * Double-buffered LDS; 16-byte code pieces are XOR-swizzled per row so that
//    the fragment reads of 8 (or 16) consecutive rows hit distinct banks.
#include "common.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int KC = 128;            // k per chunk
constexpr int CODE_ROW = KC / 2;   // 64 code bytes per row per chunk
constexpr int SCALE_ROW = KC / 16; // 8 scale bytes per row per chunk

__device__ __forceinline__ uint32_t swz(uint32_t i) { return ((i >> 1) ^ (i >> 3)) & 3u; }

// 8 E2M1 codes (one dword) times one E4M3 scale -> 8 exact fp16 values.
__device__ __forceinline__ half8 dequant8(uint32_t codes, _Float16 sb) {
  const half2v s2 = {sb, sb};
  half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0);
  half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1);
  half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2);
  half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3);
  p0 *= s2;
  p1 *= s2;
  p2 *= s2;
  p3 *= s2;
  half8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ _Float16 scale_f16(uint32_t byte) {
  return (_Float16)nv_e4m3_to_f32(byte);  // exact: E4M3 values are fp16 values
}

struct GemmParams {
  int G, N, K, total_rows;
  const int32_t* offsets;
  const int32_t* gather;
  const uint8_t *a_codes, *a_scales;
  const float* a_ts;
  const uint8_t *r_codes, *r_scales;
  const float* r_ts;
  const uint8_t* kact;
  const uint8_t *w_codes, *w_scales;
  const float* w_ts;
  void* out;
  float* out_amax;
  int silu;
  int m_slots;  // m-tile slots in the grid
  int n_tiles;
};

template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(kThreads) void k_gemm(GemmParams p) {
  static_assert(WAVES_M * WAVES_N == 4, "4 waves");
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "tile");
  constexpr int ROWS = 2 * BM + BN;  // A rows, R rows, W rows
  constexpr int NP = (ROWS * 4 + kThreads - 1) / kThreads;  // 16B code pieces per thread
  constexpr int NS = (ROWS * 2 + kThreads - 1) / kThreads;  // scale dwords per thread
  constexpr int STAGE_CODES = ROWS * CODE_ROW;
  constexpr int STAGE = STAGE_CODES + ROWS * SCALE_ROW;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lr = lane & 31, lh = lane >> 5;

  // ---- tile: XCD-aware remap of the workgroup id, then (m slot, n tile)
  const int nblocks = p.m_slots * p.n_tiles;
  const int bid = blockIdx.x;
  const int per = nblocks / 8, rem = nblocks % 8, xcd = bid % 8;
  const int L = xcd * per + (xcd < rem ? xcd : rem) + bid / 8;
  const int mt = L / p.n_tiles, nt = L % p.n_tiles;

  // ---- find the group that owns m-tile `mt`
  int grp = -1, local = 0;
  {
    int run = 0;
    for (int c = 0; c < p.G; c += 64) {
      const int g = c + lane;
      int tiles = 0;
      if (g < p.G) tiles = (p.offsets[g + 1] - p.offsets[g] + BM - 1) / BM;
      int inc = tiles;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int n = __shfl_up(inc, o, 64);
        if (lane >= o) inc += n;
      }
      const int excl = inc - tiles;
      const bool hit = g < p.G && mt >= run + excl && mt < run + inc;
      const unsigned long long bal = __ballot(hit);
      if (bal) {
        const int hl = __ffsll((long long)bal) - 1;
        grp = c + hl;
        local = mt - run - __shfl(excl, hl, 64);
        break;
      }
      run += __shfl(inc, 63, 64);
    }
  }
  if (grp < 0) return;  // wave-uniform and identical in every wave
  const int row_beg = p.offsets[grp] + local * BM;
  const int row_end = p.offsets[grp + 1];
  const bool rac = p.r_codes != nullptr;
  const int K2 = p.K >> 1, K16 = p.K >> 4;
  const int I = p.N >> 1;

  // ---- per-thread load assignments (pointers advance by one chunk per step)
  auto src_row = [&](int i) -> int64_t {
    int m = row_beg + i;
    if (m >= row_end) m = row_end - 1;
    return p.gather ? (int64_t)p.gather[m] : (int64_t)m;
  };
  auto w_row = [&](int i) -> int64_t {
    int n;
    if (p.silu) {
      const int wv = i / WTN, f = (i % WTN) / 32, rr = i % 32;
      n = ((f & 1) ? I : 0) + nt * (BN / 2) + wv * (WTN / 2) + (f >> 1) * 32 + rr;
    } else {
      n = nt * BN + i;
    }
    return (int64_t)grp * p.N + n;
  };
  const uint8_t* cptr[NP];
  uint32_t cdst[NP];
  const uint8_t* sptr[NS];
  uint32_t sdst[NS];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int q = tid + kThreads * j;
    const int i = q >> 2, pc = q & 3;
    cptr[j] = nullptr;
    cdst[j] = 0;
    if (i < ROWS) {
      if (i < BM) cptr[j] = p.a_codes + src_row(i) * K2 + pc * 16;
      else if (i < 2 * BM) cptr[j] = rac ? p.r_codes + src_row(i - BM) * K2 + pc * 16 : nullptr;
      else cptr[j] = p.w_codes + w_row(i - 2 * BM) * K2 + pc * 16;
      cdst[j] = i * CODE_ROW + ((pc ^ swz(i)) << 4);
    }
  }
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int q = tid + kThreads * j;
    const int i = q >> 1, d = q & 1;
    sptr[j] = nullptr;
    sdst[j] = 0;
    if (i < ROWS) {
      if (i < BM) sptr[j] = p.a_scales + src_row(i) * K16 + d * 4;
      else if (i < 2 * BM) sptr[j] = rac ? p.r_scales + src_row(i - BM) * K16 + d * 4 : nullptr;
      else sptr[j] = p.w_scales + w_row(i - 2 * BM) * K16 + d * 4;
      sdst[j] = STAGE_CODES + i * SCALE_ROW + d * 4;
    }
  }

  uint4 creg[NP];
  uint32_t sreg[NS];
  auto gload = [&](int chunk) {
#pragma unroll
    for (int j = 0; j < NP; ++j)
      if (cptr[j]) creg[j] = *reinterpret_cast<const uint4*>(cptr[j] + (int64_t)chunk * CODE_ROW);
#pragma unroll
    for (int j = 0; j < NS; ++j)
      if (sptr[j]) sreg[j] = *reinterpret_cast<const uint32_t*>(sptr[j] + (int64_t)chunk * SCALE_ROW);
  };
  auto lstore = [&](int buf) {
    uint8_t* base = lds + buf * STAGE;
#pragma unroll
    for (int j = 0; j < NP; ++j)
      if (cptr[j]) *reinterpret_cast<uint4*>(base + cdst[j]) = creg[j];
#pragma unroll
    for (int j = 0; j < NS; ++j)
      if (sptr[j]) *reinterpret_cast<uint32_t*>(base + sdst[j]) = sreg[j];
  };

  float16v accm[FM][FN], accr[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        accm[a][b][e] = 0.0f;
        accr[a][b][e] = 0.0f;
      }
    }

  // fragment rows in the LDS tile
  const int arow0 = wm * WTM + lr;            // + fm*32
  const int wrow0 = 2 * BM + wn * WTN + lr;   // + fn*32

  const int nchunks = p.K / KC;
  gload(0);
  lstore(0);
  __syncthreads();

  for (int ch = 0; ch < nchunks; ++ch) {
    const int buf = ch & 1;
    if (ch + 1 < nchunks) gload(ch + 1);
    const uint8_t* base = lds + buf * STAGE;

    // residual activity of the 8 blocks of this chunk
    uint64_t act = ~0ull;
    if (rac && p.kact) act = *reinterpret_cast<const uint64_t*>(p.kact + (int64_t)ch * 8);

    uint32_t sa[FM], sr[FM], sw[FN];
#pragma unroll
    for (int a = 0; a < FM; ++a) {
      const int i = arow0 + a * 32;
      sa[a] = *reinterpret_cast<const uint32_t*>(base + STAGE_CODES + i * SCALE_ROW + lh * 4);
      if (rac) sr[a] = *reinterpret_cast<const uint32_t*>(base + STAGE_CODES + (i + BM) * SCALE_ROW + lh * 4);
    }
#pragma unroll
    for (int b = 0; b < FN; ++b) {
      const int i = wrow0 + b * 32;
      sw[b] = *reinterpret_cast<const uint32_t*>(base + STAGE_CODES + i * SCALE_ROW + lh * 4);
    }

#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      const uint32_t pc = 2 * lh + hp;
      uint4 ca[FM], cr[FM], cw[FN];
#pragma unroll
      for (int a = 0; a < FM; ++a) {
        const uint32_t i = arow0 + a * 32;
        ca[a] = *reinterpret_cast<const uint4*>(base + i * CODE_ROW + ((pc ^ swz(i)) << 4));
        if (rac) {
          const uint32_t ir = i + BM;
          cr[a] = *reinterpret_cast<const uint4*>(base + ir * CODE_ROW + ((pc ^ swz(ir)) << 4));
        }
      }
#pragma unroll
      for (int b = 0; b < FN; ++b) {
        const uint32_t i = wrow0 + b * 32;
        cw[b] = *reinterpret_cast<const uint4*>(base + i * CODE_ROW + ((pc ^ swz(i)) << 4));
      }
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int s = hp * 4 + s4;        // MFMA step in the chunk
        const int sbyte = s >> 1;         // scale byte within the lane's dword
        half8 av[FM], wv[FN];
#pragma unroll
        for (int b = 0; b < FN; ++b) {
          const uint32_t c = s4 == 0 ? cw[b].x : s4 == 1 ? cw[b].y : s4 == 2 ? cw[b].z : cw[b].w;
          wv[b] = dequant8(c, scale_f16((sw[b] >> (8 * sbyte)) & 0xFFu));
        }
#pragma unroll
        for (int a = 0; a < FM; ++a) {
          const uint32_t c = s4 == 0 ? ca[a].x : s4 == 1 ? ca[a].y : s4 == 2 ? ca[a].z : ca[a].w;
          av[a] = dequant8(c, scale_f16((sa[a] >> (8 * sbyte)) & 0xFFu));
        }
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
          for (int b = 0; b < FN; ++b)
            accm[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[a], wv[b], accm[a][b], 0, 0, 0);
        // blocks s/2 (lanes 0-31) and 4 + s/2 (lanes 32-63) of the chunk
        const bool ract = rac && (((act >> (8 * sbyte)) & 0xFFull) | ((act >> (8 * (4 + sbyte))) & 0xFFull));
        if (ract) {
          half8 rv[FM];
#pragma unroll
          for (int a = 0; a < FM; ++a) {
            const uint32_t c = s4 == 0 ? cr[a].x : s4 == 1 ? cr[a].y : s4 == 2 ? cr[a].z : cr[a].w;
            rv[a] = dequant8(c, scale_f16((sr[a] >> (8 * sbyte)) & 0xFFu));
          }
#pragma unroll
          for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
              accr[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(rv[a], wv[b], accr[a][b], 0, 0, 0);
        }
      }
    }
    if (ch + 1 < nchunks) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  const float s_ta = *p.a_ts;
  const float s_tr = rac ? *p.r_ts : 0.0f;
  const float s_tw = p.w_ts[grp];
  if (!p.silu) {
    float* out = reinterpret_cast<float*>(p.out);
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = row_beg + wm * WTM + a * 32 + (e >> 2) * 8 + lh * 4 + (e & 3);
          const int n = nt * BN + wn * WTN + b * 32 + lr;
          if (m < row_end) {
            float y = s_ta * accm[a][b][e];
            if (rac) y = y + s_tr * accr[a][b][e];
            out[(int64_t)m * p.N + n] = s_tw * y;
          }
        }
  } else {
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
    float hmax = 0.0f;
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; b += 2)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = row_beg + wm * WTM + a * 32 + (e >> 2) * 8 + lh * 4 + (e & 3);
          const int hc = nt * (BN / 2) + wn * (WTN / 2) + (b >> 1) * 32 + lr;
          if (m < row_end) {
            float g = s_ta * accm[a][b][e], u = s_ta * accm[a][b + 1][e];
            if (rac) {
              g = g + s_tr * accr[a][b][e];
              u = u + s_tr * accr[a][b + 1][e];
            }
            g *= s_tw;
            u *= s_tw;
            const float hv = g / (1.0f + expf(-g)) * u;
            const uint32_t hb = nv_f32_to_bf16(hv);
            out[(int64_t)m * I + hc] = (uint16_t)hb;
            hmax = __builtin_fmaxf(hmax, __builtin_fabsf(nv_bf16_to_f32(hb)));
          }
        }
    if (p.out_amax) {
      hmax = nv_wave_max(hmax);
      if (lane == 0 && hmax > 0.0f)
        atomicMax(reinterpret_cast<uint32_t*>(p.out_amax), __float_as_uint(hmax));
    }
  }
}

template <int BM, int BN, int WM, int WN>
int launch(GemmParams& p, hipStream_t s) {
  p.m_slots = (p.total_rows + BM - 1) / BM + p.G;
  p.n_tiles = p.N / BN;
  const int64_t nb = (int64_t)p.m_slots * p.n_tiles;
  if (nb > 0x7fffffff) return NVFP4_ERR_SHAPE;
  hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN>), dim3((unsigned)nb), dim3(kThreads), 0, s, p);
  return nv_launch_status();
}

}  // namespace

extern "C" {

size_t w4a4_grouped_gemm_rac_workspace_size(const w4a4_gemm_args_t*) { return 0; }

int w4a4_grouped_gemm_rac(const w4a4_gemm_args_t* a, void*, size_t, void* stream) {
  NV_RETURN_IF(!a, NVFP4_ERR_NULL);
  NV_RETURN_IF(a->epilogue != NVFP4_EPI_F32 && a->epilogue != NVFP4_EPI_SILU_MUL_BF16,
               NVFP4_ERR_DTYPE);
  NV_RETURN_IF(a->num_groups < 1 || a->total_rows < 0 || a->N <= 0 || a->K <= 0 ||
                   a->K % KC || a->N % 128 || a->N > (1 << 24) || a->K > (1 << 24) ||
                   a->total_rows > 0x7fffffff || a->num_groups > (1 << 20),
               NVFP4_ERR_SHAPE);
  NV_RETURN_IF(!a->group_offsets || !a->w_codes || !a->w_scales || !a->w_tscale ||
                   !a->a_tscale,
               NVFP4_ERR_NULL);
  if (a->total_rows == 0) return NVFP4_OK;  // nothing to compute; row buffers may be empty
  NV_RETURN_IF(!a->a_codes || !a->a_scales || !a->out, NVFP4_ERR_NULL);
  NV_RETURN_IF(a->r_codes && (!a->r_scales || !a->r_tscale), NVFP4_ERR_NULL);
  NV_RETURN_IF(!nv_aligned16(a->a_codes) || !nv_aligned16(a->w_codes) ||
                   (a->r_codes && !nv_aligned16(a->r_codes)) ||
                   (reinterpret_cast<uintptr_t>(a->a_scales) & 3) ||
                   (reinterpret_cast<uintptr_t>(a->w_scales) & 3) ||
                   (a->r_scales && (reinterpret_cast<uintptr_t>(a->r_scales) & 3)) ||
                   (a->kblock_active && (reinterpret_cast<uintptr_t>(a->kblock_active) & 7)),
               NVFP4_ERR_ALIGN);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  GemmParams p{};
  p.G = (int)a->num_groups;
  p.N = (int)a->N;
  p.K = (int)a->K;
  p.total_rows = (int)a->total_rows;
  p.offsets = a->group_offsets;
  p.gather = a->gather_rows;
  p.a_codes = a->a_codes;
  p.a_scales = a->a_scales;
  p.a_ts = a->a_tscale;
  p.r_codes = a->r_codes;
  p.r_scales = a->r_codes ? a->r_scales : nullptr;
  p.r_ts = a->r_codes ? a->r_tscale : nullptr;
  p.kact = a->kblock_active;
  p.w_codes = a->w_codes;
  p.w_scales = a->w_scales;
  p.w_ts = a->w_tscale;
  p.out = a->out;
  p.out_amax = a->epilogue == NVFP4_EPI_SILU_MUL_BF16 ? a->out_amax : nullptr;
  p.silu = a->epilogue == NVFP4_EPI_SILU_MUL_BF16;
  return launch<128, 128, 2, 2>(p, s);
}

}  // extern "C"
