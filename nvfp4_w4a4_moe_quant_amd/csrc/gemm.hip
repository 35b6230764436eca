// Grouped W4A4 GEMM over experts with the RAC residual pass fused in.
//
// QUADS arXiv abstract (mlsanity page, "Abstract (arXiv)"): 4-bit weights
// times 4-bit activations on NVFP4 operands.  QUADS blog post, section "Two
// fixes, on two different sides": the selected channels' residual gets its
// own 4-bit pass inside the same kernel, added to the unchanged main pass.
//
// MI355X design:
//  * Operands stay NVFP4 in HBM and LDS (4 bits per element plus one E4M3
//    byte per 16).  Each wave dequantizes the fragments it feeds to the matrix
//    cores: an E2M1 value times an E4M3 scale has at most 6 significant bits
//    and lies in [2^-10, 2688], so g * s_b is exact in fp16; the FP4->fp16
//    conversion and the scale multiply are packed VALU ops.
//  * v_mfma_f32_32x32x16_f16 (gfx950) accumulates exact fp16 products in FP32.
//    K = 16 per instruction is exactly one NVFP4 block.
//  * Main and residual rows share every W fragment and, since the residual is
//    quantized with the activation's own tensor scale, one FP32 accumulator:
//        y = s_tw * s_ta * (sum A W + sum R W).
//    One accumulator set per fragment leaves the registers for 64 x 128 wave
//    tiles, which dequantize half an operand fragment per MFMA.
//  * K is consumed in chunks of 128 (8 MFMA steps).  Inside a chunk, lanes
//    32-63 take the upper 64 k of the chunk instead of the next 8 (a fixed
//    permutation of k applied identically to A, R and W, so the contraction is
//    unchanged); each lane then reads 32 contiguous code bytes per row.
//  * Tiles: (group, m-tile, n-tile) from the device-side group offsets; every
//    workgroup finds its tile with a wave scan, tiles past the real count exit.
//    Workgroup ids are remapped so that consecutive tiles run on the same XCD
//    and share its L2; within an expert the m-tiles vary fastest, so the
//    workgroups reading one W tile are adjacent.
//  * Double-buffered LDS; 16-byte code pieces are XOR-swizzled per row so that
//    the fragment reads of 8 (or 16) consecutive rows hit distinct banks.
#include <type_traits>

#include "common.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int KC = 128;            // k per chunk
constexpr int CODE_ROW = KC / 2;   // 64 code bytes per row per chunk
constexpr int SCALE_ROW = KC / 16; // 8 scale bytes per row per chunk
constexpr int kMaxKChunks = 256;   // K <= 32768

__device__ __forceinline__ uint32_t swz(uint32_t i) { return ((i >> 1) ^ (i >> 3)) & 3u; }

// 8 E2M1 codes (one dword) times one E4M3 scale (as an fp16 pair) -> 8 exact
// fp16 values.  The hardware FP4 conversion only applies the exponent of its
// scale operand, so it runs with scale 1 and the packed multiply applies s_b.
__device__ __forceinline__ half8 dequant8(uint32_t codes, half2v s2) {
  half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0);
  half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1);
  half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2);
  half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3);
  p0 *= s2;
  p1 *= s2;
  p2 *= s2;
  p3 *= s2;
  return __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                 __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4,
                                 5, 6, 7);
}

// Four E4M3 scale bytes -> four exact fp16 values (OCP E4M3 conversion, scale 1).
__device__ __forceinline__ void scales4(uint32_t w, half2v& s01, half2v& s23) {
  s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
}

__device__ __forceinline__ half2v pick_scale(half2v s01, half2v s23, int blk) {
  return blk == 0 ? __builtin_shufflevector(s01, s01, 0, 0)
       : blk == 1 ? __builtin_shufflevector(s01, s01, 1, 1)
       : blk == 2 ? __builtin_shufflevector(s23, s23, 0, 0)
                  : __builtin_shufflevector(s23, s23, 1, 1);
}

// silu(g) * u in FP32 with the hardware exp and reciprocal (each within a few
// FP32 ulp; the result is rounded to bf16, whose ulp is 2^16 times larger).
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

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
  int m_slots;  // m-tile slots in the grid
  int n_tiles;
  int skip;     // NVFP4_GEMM_SKIP_INACTIVE_BLOCKS
  int per_group;  // NVFP4_GEMM_PER_GROUP_SCALES: a_ts, r_ts [G], kact [G, K/16]
  float* out_y;   // SiLU*mul epilogue only, nullable: FP32 gate/up outputs [rows, N]
};

// Rows of A and R past an expert's last row (the padding of its last m-tile)
// are read from this zero row: zero codes and zero block scales dequantize to
// 0, so the matrix cores spend little power on them.  K <= 32768.
__device__ uint8_t nv_zero_row[kMaxKChunks * CODE_ROW];

// The grouped GEMM.  BM x BN output tile per workgroup, WAVES_M x WAVES_N
// waves of (BM / WAVES_M) x (BN / WAVES_N), NSTAGE LDS stages of KC k.
template <int BM, int BN, int WAVES_M, int WAVES_N, int NSTAGE, int MINW, bool RAC, bool SILU,
          bool GATHER, bool RSKIP>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, MINW) void k_gemm(GemmParams p) {
  constexpr int NW = WAVES_M * WAVES_N, NT = 64 * NW;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM >= 1 && FM <= 2 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "tile");
  static_assert(!SILU || FN % 2 == 0, "SiLU pairs gate/up fragments");
  constexpr int AR = RAC ? 2 * BM : BM;  // A rows then R rows
  constexpr int ROWS = AR + BN;          // then W rows
  static_assert((ROWS * 2) % NT == 0, "whole wave-loads of codes and scales");
  constexpr int NPI = ROWS * 4 / NT;  // 16-byte code pieces per thread per chunk
  constexpr int NSI = ROWS * 2 / NT;  // 4-byte scale words per thread per chunk
  constexpr int STAGE_CODES = ROWS * CODE_ROW;
  constexpr int STAGE = STAGE_CODES + ROWS * SCALE_ROW;
  static_assert(NSTAGE >= 2 && (NSTAGE - 2) * (NPI + NSI) <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NSTAGE * STAGE];
  __shared__ uint64_t kact_lds[kMaxKChunks];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lr = lane & 31, lh = lane >> 5;

  // ---- tile (group, m-tile, n-tile), XCD-aware, m-tiles fastest in a group
  const NvTile tile = nv_find_tile(p.offsets, p.G, BM, p.m_slots, p.n_tiles);
  const int grp = tile.grp, local = tile.local, nt = tile.nt;
  if (grp < 0) return;  // wave-uniform and identical in every wave
  const int row_beg = p.offsets[grp] + local * BM;
  const int row_end = p.offsets[grp + 1];
  const int K2 = p.K >> 1, K16 = p.K >> 4;
  const int I = p.N >> 1;

  // ---- source rows of the LDS tile rows; rows past the group's end read zeros
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
  auto act_row = [&](const uint8_t* base, int i, int per_row) -> const uint8_t* {
    const int m = row_beg + i;
    if (m >= row_end) return nv_zero_row;
    return base + (GATHER ? (int64_t)p.gather[m] : (int64_t)m) * per_row;
  };
  auto code_row_ptr = [&](int i) -> const uint8_t* {
    if (i < BM) return act_row(p.a_codes, i, K2);
    if (RAC && i < AR) return act_row(p.r_codes, i - BM, K2);
    return p.w_codes + w_row(i - AR) * K2;
  };
  auto scale_row_ptr = [&](int i) -> const uint8_t* {
    if (i < BM) return act_row(p.a_scales, i, K16);
    if (RAC && i < AR) return act_row(p.r_scales, i - BM, K16);
    return p.w_scales + w_row(i - AR) * K16;
  };

  // Direct global->LDS loads: wave-instruction j writes 1 KiB of codes
  // (16 rows x 64 B) or 256 B of scales (32 rows x 8 B) contiguously; lane l
  // fetches the 16-byte piece that the swizzle places in its slot.
  const uint8_t* gcode[NPI];
  const uint8_t* gscale[NSI];
#pragma unroll
  for (int j = 0; j < NPI; ++j) {
    const int slot = (j * NW + wave) * 64 + lane;
    const int row = slot >> 2;
    const uint32_t piece = (uint32_t)(slot & 3) ^ swz((uint32_t)row);
    gcode[j] = code_row_ptr(row) + piece * 16;
  }
#pragma unroll
  for (int j = 0; j < NSI; ++j) {
    const int slot = (j * NW + wave) * 64 + lane;
    gscale[j] = scale_row_ptr(slot >> 1) + (slot & 1) * 4;
  }
  // The DMA is issued through inline asm: the compiler cannot tell that the
  // next stage never aliases the stage being read and would otherwise wait for
  // the DMA before every LDS read.  Completion is awaited explicitly (vmcnt)
  // before the barrier that publishes a stage.
  auto issue = [&](int chunk, int buf) {
    const uint32_t st = (uint32_t)(uintptr_t)(lds_ptr_t)(lds + buf * STAGE);
#pragma unroll
    for (int j = 0; j < NPI; ++j) {
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(st + (j * NW + wave) * 1024);
      const uint8_t* g = gcode[j] + (int64_t)chunk * CODE_ROW;
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                   :: "s"(m0), "v"(g) : "memory", "m0");
    }
#pragma unroll
    for (int j = 0; j < NSI; ++j) {
      const uint32_t m0 =
          __builtin_amdgcn_readfirstlane(st + STAGE_CODES + (j * NW + wave) * 256);
      const uint8_t* g = gscale[j] + (int64_t)chunk * SCALE_ROW;
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                   :: "s"(m0), "v"(g) : "memory", "m0");
    }
  };

  // One FP32 accumulator per fragment: the residual shares the activation's
  // tensor scale, so both passes add into it.
  float16v acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  const int arow0 = wm * WTM + lr;       // + a*32 (A), + BM (R)
  const int wrow0 = AR + wn * WTN + lr;  // + b*32
  // live 32-row fragments of this wave: rows past the group's end are padding
  const int wave_rows = row_end - (row_beg + wm * WTM);  // wave-uniform
  const int fm_live = wave_rows <= 0 ? 0 : (wave_rows <= 32 ? 1 : FM);

  const int nchunks = p.K / KC;
  // residual block activity, 8 blocks (one chunk) per 64-bit word
  if constexpr (RAC && RSKIP) {
    for (int c = tid; c < nchunks; c += NT)
      kact_lds[c] = p.kact ? *reinterpret_cast<const uint64_t*>(
                                 p.kact + (p.per_group ? (int64_t)grp * (p.K >> 4) : 0) +
                                 (int64_t)c * 8)
                           : ~0ull;
  }

  // One chunk (8 MFMA steps) over the first FMX fragments of the wave.  With
  // RSKIP, the residual MFMAs of a step run only when one of its two blocks
  // holds a selected channel; inactive blocks carry all-zero residual codes,
  // so running them is exact as well.
  auto compute = [&](auto fmx_c, int ch, const uint8_t* base) {
    constexpr int FMX = decltype(fmx_c)::value;
    uint32_t act = 0xFFu;  // activity of the chunk's 8 blocks (SGPR)
    if constexpr (RAC && RSKIP) {
      const uint64_t w = kact_lds[ch];
      uint32_t m = 0;
#pragma unroll
      for (int b = 0; b < 8; ++b) m |= ((w >> (8 * b)) & 0xFFull) ? (1u << b) : 0u;
      act = __builtin_amdgcn_readfirstlane(m);
    }
    // scales of the lane's 4 blocks for every fragment row
    half2v sa01[FMX], sa23[FMX], sr01[RAC ? FMX : 1], sr23[RAC ? FMX : 1], sw01[FN], sw23[FN];
#pragma unroll
    for (int a = 0; a < FMX; ++a) {
      const int i = arow0 + a * 32;
      scales4(*reinterpret_cast<const uint32_t*>(base + STAGE_CODES + i * SCALE_ROW + lh * 4),
              sa01[a], sa23[a]);
      if constexpr (RAC)
        scales4(*reinterpret_cast<const uint32_t*>(base + STAGE_CODES + (i + BM) * SCALE_ROW +
                                                   lh * 4),
                sr01[a], sr23[a]);
    }
#pragma unroll
    for (int b = 0; b < FN; ++b) {
      const int i = wrow0 + b * 32;
      scales4(*reinterpret_cast<const uint32_t*>(base + STAGE_CODES + i * SCALE_ROW + lh * 4),
              sw01[b], sw23[b]);
    }
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      const uint32_t pc = 2 * lh + hp;
      uint4 ca[FMX], cr[RAC ? FMX : 1], cw[FN];
#pragma unroll
      for (int a = 0; a < FMX; ++a) {
        const uint32_t i = arow0 + a * 32;
        ca[a] = *reinterpret_cast<const uint4*>(base + i * CODE_ROW + ((pc ^ swz(i)) << 4));
        if constexpr (RAC) {
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
        const int blk = (hp * 4 + s4) >> 1;  // block among the lane's four
        half8 av[FMX], wv[FN];
#pragma unroll
        for (int b = 0; b < FN; ++b) {
          const uint32_t c = s4 == 0 ? cw[b].x : s4 == 1 ? cw[b].y : s4 == 2 ? cw[b].z : cw[b].w;
          wv[b] = dequant8(c, pick_scale(sw01[b], sw23[b], blk));
        }
#pragma unroll
        for (int a = 0; a < FMX; ++a) {
          const uint32_t c = s4 == 0 ? ca[a].x : s4 == 1 ? ca[a].y : s4 == 2 ? ca[a].z : ca[a].w;
          av[a] = dequant8(c, pick_scale(sa01[a], sa23[a], blk));
        }
#pragma unroll
        for (int a = 0; a < FMX; ++a)
#pragma unroll
          for (int b = 0; b < FN; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[a], wv[b], acc[a][b], 0, 0, 0);
        if (RAC && (!RSKIP || (act & ((1u << blk) | (1u << (4 + blk)))))) {
          half8 rv[RAC ? FMX : 1];
#pragma unroll
          for (int a = 0; a < FMX; ++a) {
            const uint32_t c = s4 == 0 ? cr[a].x : s4 == 1 ? cr[a].y : s4 == 2 ? cr[a].z : cr[a].w;
            rv[a] = dequant8(c, pick_scale(sr01[a], sr23[a], blk));
          }
#pragma unroll
          for (int a = 0; a < FMX; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
              acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(rv[a], wv[b], acc[a][b], 0, 0, 0);
        }
      }
    }
  };

  // Two-deep pipeline: chunk ch is computed while chunk ch + NSTAGE - 1 is in
  // flight; before the barrier that ends the iteration, chunk ch + 1 must have
  // landed.  Waves without live rows (the padded part of an expert's last
  // tile) still load and synchronize.
  constexpr int PER_CHUNK = NPI + NSI;
  constexpr int AHEAD = NSTAGE - 1;
  auto run = [&](auto fmx_c) {
#pragma unroll
    for (int c = 0; c < AHEAD; ++c)
      if (c < nchunks) issue(c, c);
    if (nchunks > 1 && NSTAGE > 2)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NSTAGE - 2) * PER_CHUNK) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int ch = 0; ch < nchunks; ++ch) {
      const int nxt = ch + AHEAD;
      if (nxt < nchunks) issue(nxt, nxt % NSTAGE);
      if constexpr (decltype(fmx_c)::value > 0) compute(fmx_c, ch, lds + (ch % NSTAGE) * STAGE);
      if (ch + AHEAD < nchunks && NSTAGE > 2)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NSTAGE - 2) * PER_CHUNK) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
  };
  if (fm_live == FM) run(std::integral_constant<int, FM>{});
  else if (fm_live == 1) run(std::integral_constant<int, 1>{});
  else run(std::integral_constant<int, 0>{});

  // ---- epilogue: y = s_tw * s_ta * acc.  The residual pass assumed the
  // activation's tensor scale; a residual tensor scale that differs makes the
  // group's outputs NaN rather than silently wrong.
  const float s_ta = p.a_ts[p.per_group ? grp : 0];
  float scale = p.w_ts[grp] * s_ta;
  if constexpr (RAC) {
    if (p.r_ts[p.per_group ? grp : 0] != s_ta) scale = __builtin_nanf("");
  }
  auto yval = [&](int a, int b, int e) -> float { return scale * acc[a][b][e]; };
  // Element e of fragment (a, b) sits at row m0 + a*32 + (e>>2)*8 + (e&3) of
  // the lane's column; the base pointer is formed once, and a wave whose 32
  // x FM rows all lie inside the group stores without per-element checks.
  const int m0 = row_beg + wm * WTM + lh * 4;
  const bool full = row_beg + (wm + 1) * WTM <= row_end;  // wave-uniform
  if constexpr (!SILU) {
    float* ob = reinterpret_cast<float*>(p.out) + (int64_t)m0 * p.N + nt * BN + wn * WTN + lr;
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int dm = a * 32 + (e >> 2) * 8 + (e & 3);
          if (full || m0 + dm < row_end) ob[(int64_t)dm * p.N + b * 32] = yval(a, b, e);
        }
  } else {
    // Elements e and e + 1 (e even) of a lane are rows dm and dm + 1 of its
    // column.  Lanes l and l ^ 1 hold neighbouring columns, so one swap gives
    // the even lane both columns of row dm and the odd lane both of row
    // dm + 1, and each stores them as one 32-bit word.  Every lane computes
    // its values (padded rows carry finite accumulators) so the swap is
    // uniform; only rows inside the group are stored or enter the max.
    if (p.out_y) {  // the FP32 gate/up values before the SiLU (verification)
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) {
          const int64_t n = ((b & 1) ? I : 0) + nt * (BN / 2) + wn * (WTN / 2) + (b >> 1) * 32 + lr;
          float* yb = p.out_y + (int64_t)m0 * p.N + n;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int dm = a * 32 + (e >> 2) * 8 + (e & 3);
            if (full || m0 + dm < row_end) yb[(int64_t)dm * p.N] = yval(a, b, e);
          }
        }
    }
    const bool odd = (lr & 1) != 0;
    uint32_t* ob = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(p.out) +
                                               (int64_t)m0 * I + nt * (BN / 2) +
                                               wn * (WTN / 2) + (lr & ~1));
    float hmax = 0.0f;
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; b += 2)
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const int dm = a * 32 + (e >> 2) * 8 + (e & 3);
          const uint32_t h0 = nv_f32_to_bf16(silu_mul(yval(a, b, e), yval(a, b + 1, e)));
          const uint32_t h1 = nv_f32_to_bf16(silu_mul(yval(a, b, e + 1), yval(a, b + 1, e + 1)));
          const bool v0 = full || m0 + dm < row_end, v1 = full || m0 + dm + 1 < row_end;
          if (v0) hmax = __builtin_fmaxf(hmax, __builtin_fabsf(nv_bf16_to_f32(h0)));
          if (v1) hmax = __builtin_fmaxf(hmax, __builtin_fabsf(nv_bf16_to_f32(h1)));
          // DPP quad_perm [1, 0, 3, 2]: lane l reads lane l ^ 1
          const uint32_t got =
              (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? h0 : h1), 0xB1, 0xF, 0xF, false);
          const int64_t col = (b >> 1) * 32;  // in bf16 elements, even
          if (!odd) {
            if (v0) ob[((int64_t)dm * I + col) >> 1] = h0 | (got << 16);
          } else {
            if (v1) ob[((int64_t)(dm + 1) * I + col) >> 1] = got | (h1 << 16);
          }
        }
    if (p.out_amax) {
      hmax = nv_wave_max(hmax);
      if (lane == 0 && hmax > 0.0f)
        atomicMax(reinterpret_cast<uint32_t*>(p.out_amax), __float_as_uint(hmax));
    }
  }
}

template <int BM, int BN, int WM, int WN, int NS, int MINW, bool RAC, bool SILU, bool GATHER,
          bool RSKIP>
int launch_t(GemmParams& p, hipStream_t s) {
  constexpr int rows = (RAC ? 2 * BM : BM) + BN;
  static_assert((rows * 2) % (64 * WM * WN) == 0, "whole wave-loads of codes and scales");
  {
    if (p.N % BN) return NVFP4_ERR_SHAPE;
    p.m_slots = (p.total_rows + BM - 1) / BM + p.G;
    p.n_tiles = p.N / BN;
    const int64_t nb = (int64_t)p.m_slots * p.n_tiles;
    if (nb > 0x7fffffff) return NVFP4_ERR_SHAPE;
    hipLaunchKernelGGL((k_gemm<BM, BN, WM, WN, NS, MINW, RAC, SILU, GATHER, RSKIP>), dim3((unsigned)nb),
                       dim3(64 * WM * WN), 0, s, p);
    return nv_launch_status();
  }
}

// ---------------------------------------------------------------------------
// Decode-shaped GEMM for one group with at most 64 rows (a 16 x 4096 x 4096
// linear layer is the model case), K % 1024 == 0, K <= 16384 (12288 with
// SiLU*mul).  A workgroup owns one 16-column slab of W (with the SiLU*mul
// epilogue two: gate columns j .. j+15 and the up columns I + j ..) over the
// whole of K, and one 16-row tile (grid y; the kernel is written for any
// group count, grid z, but many small groups take k_gemv_wide below): N/16
// workgroups stream W once.
//  * Every operand goes through LDS by coalesced DMA: each wave-instruction
//    fetches 1 KiB of whole 128-byte lines (two rows' 512-byte pieces of a
//    chunk).  Fetching MFMA fragments straight from global memory would make
//    every load instruction touch 16 rows, and the A and R rows that every
//    workgroup re-reads from L2 then cost more than streaming W.
//  * K is consumed in chunks of 1024 k (128 per wave) through a ring of LDS
//    chunk buffers; the block scales of the whole K land first.  Chunk c is
//    computed as soon as its DMA has landed while later chunks are in flight.
//  * v_mfma_f32_16x16x32_f16 matches the 16-row tile.  Inside a 128-k group,
//    lane quarter q takes k = 32q .. 32q + 31 (16 contiguous code bytes) for
//    four MFMA steps of 8 k: a fixed permutation of k applied to A, R and W
//    alike, so the contraction is unchanged.  The eight waves split each
//    chunk and add their accumulators through LDS in wave order.
//  * Code pieces (16 bytes) are XOR-swizzled by row within 16-piece groups,
//    scale pieces likewise, so the fragment reads of 16 rows hit distinct
//    banks.
// Rows of a tile past the group's end read the zero row.  The kernel is
// bound by dequantization VALU (A, R and W each once per element; every
// workgroup dequantizes its A and R rows again) and DMA latency, not MFMA.
typedef float float4v __attribute__((ext_vector_type(4)));
constexpr int kGvMaxRows = 64;      // one group: rows up to which this kernel is used
constexpr int kGvAvgRows = 32;      // many groups: average rows per group
constexpr int kGvWaves = 8;
constexpr int kGvKC = 128 * kGvWaves;  // k per chunk
constexpr int kGvCRow = kGvKC / 2;     // code bytes per row per chunk
constexpr int kGvMaxK = 16384;      // 12288 with the SiLU*mul epilogue (two W slabs)

template <bool RAC, bool SILU, bool GATHER>
__global__ __launch_bounds__(64 * kGvWaves) void k_gemv(GemmParams p) {
  constexpr int NS = SILU ? 2 : 1;           // 16-column W slabs per workgroup
  constexpr int AROWS = RAC ? 32 : 16;       // A 16 | R 16
  constexpr int ROWS = AROWS + 16 * NS;      // then the W slabs
  constexpr int CHUNK = ROWS * kGvCRow;
  constexpr int NBUF = ROWS <= 48 ? 4 : 3;   // chunk buffers
  constexpr int NCI = CHUNK / 1024 / kGvWaves;  // code DMA instructions per wave per chunk
  static_assert(CHUNK % (1024 * kGvWaves) == 0 && (NBUF - 1) * NCI <= 63, "DMA, vmcnt");
  constexpr int SCODES = NBUF * CHUNK;
  constexpr int MAXK = SILU ? 12288 : kGvMaxK;
  static_assert(kGvWaves * NS * 64 * 16 <= CHUNK, "reduction fits in a chunk buffer");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[SCODES + ROWS * (MAXK / 16)];
  float4v* red = reinterpret_cast<float4v*>(lds);  // [wave][slab][lane], after the last chunk

  const int grp = blockIdx.z;
  const int row_beg = p.offsets[grp], row_end = p.offsets[grp + 1];
  const int nrows = row_end - row_beg;
  if ((int)blockIdx.y * 16 >= nrows) return;  // workgroup-uniform

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = p.K, K2 = K >> 1, K16 = K >> 4;
  const int nch = K / kGvKC;
  const int I = p.N >> 1;
  const int j0 = (int)blockIdx.x * 16;  // first column of slab 0
  auto w_row = [&](int i) -> int64_t {  // W row of LDS W row i (0 .. 16 NS - 1)
    const int n = SILU ? ((i >> 4) ? I : 0) + j0 + (i & 15) : j0 + i;
    return (int64_t)grp * p.N + n;
  };
  const float s_ta = p.a_ts[p.per_group ? grp : 0];
  float scale = p.w_ts[grp] * s_ta;
  if constexpr (RAC) {
    if (p.r_ts[p.per_group ? grp : 0] != s_ta) scale = __builtin_nanf("");  // shares s_ta
  }
  const uint32_t lbase = (uint32_t)(uintptr_t)(lds_ptr_t)lds;
  const int spr = K16 >> 4;  // 16-byte pieces per scale row (a multiple of 4)
  const int smask = (spr & 15) == 0 ? 15 : (spr & 7) == 0 ? 7 : 3;
  const int nsi = ROWS * spr / 64;  // scale DMA instructions (whole K)
  const int c = lane & 15, q = lane >> 4;
  float hmax = 0.0f;

  for (int tile = blockIdx.y; tile * 16 < nrows; tile += gridDim.y) {
    const int m0 = row_beg + tile * 16;
    auto act = [&](const uint8_t* base, int i, int per_row) -> const uint8_t* {
      const int m = m0 + i;
      if (m >= row_end) return nv_zero_row;
      return base + (GATHER ? (int64_t)p.gather[m] : (int64_t)m) * per_row;
    };
    auto code_row = [&](int r) -> const uint8_t* {
      if (r < 16) return act(p.a_codes, r, K2);
      if (RAC && r < 32) return act(p.r_codes, r - 16, K2);
      return p.w_codes + w_row(r - AROWS) * K2;
    };
    auto scale_row = [&](int r) -> const uint8_t* {
      if (r < 16) return act(p.a_scales, r, K16);
      if (RAC && r < 32) return act(p.r_scales, r - 16, K16);
      return p.w_scales + w_row(r - AROWS) * K16;
    };
    __syncthreads();  // the previous tile's reduction has been read
    // block scales of the whole K: ROWS rows of K/16 bytes in 16-byte pieces,
    // swizzled within groups of smask + 1 pieces
    for (int j = wave; j < nsi; j += kGvWaves) {
      const int slot = j * 64 + lane, r = slot / spr, pc = (slot % spr) ^ (r & smask);
      const uint8_t* g = scale_row(r) + pc * 16;
      const uint32_t m0r = __builtin_amdgcn_readfirstlane(lbase + SCODES + j * 1024);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                   :: "s"(m0r), "v"(g) : "memory", "m0");
    }
    // code pieces: slot -> (row, piece), 32 pieces per row per chunk
    const uint8_t* gcode[NCI];
#pragma unroll
    for (int j = 0; j < NCI; ++j) {
      const int slot = (j * kGvWaves + wave) * 64 + lane, r = slot >> 5;
      gcode[j] = code_row(r) + (((slot & 31) ^ (r & 15)) << 4);
    }
    auto issue = [&](int ch) {
      const uint32_t st = lbase + (ch % NBUF) * CHUNK;
#pragma unroll
      for (int j = 0; j < NCI; ++j) {
        const uint32_t m0r = __builtin_amdgcn_readfirstlane(st + (j * kGvWaves + wave) * 1024);
        const uint8_t* g = gcode[j] + (int64_t)ch * kGvCRow;
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                     :: "s"(m0r), "v"(g) : "memory", "m0");
      }
    };
    for (int ch = 0; ch < NBUF && ch < nch; ++ch) issue(ch);

    auto code16 = [&](const uint8_t* buf, int r, int kl) -> uint4 {
      return *reinterpret_cast<const uint4*>(buf + r * kGvCRow + (((kl >> 5) ^ (r & 15)) << 4));
    };
    auto scale2 = [&](int r, int k) -> half2v {  // the two block scales of k .. k + 31
      const int b = k >> 4, pc = (b >> 4) ^ (r & smask);
      const uint32_t v =
          *reinterpret_cast<const uint16_t*>(lds + SCODES + r * K16 + pc * 16 + (b & 15));
      return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, false);
    };
    float4v acc[NS];  // main and residual passes (one tensor scale)
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) acc[sl] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    for (int ch = 0; ch < nch; ++ch) {
      // chunks issued after ch whose DMA may still be in flight
      const int pend = nch - 1 - ch < NBUF - 1 ? nch - 1 - ch : NBUF - 1;
      if (pend >= 3)
        asm volatile("s_waitcnt vmcnt(%0)" :: "n"(3 * NCI) : "memory");
      else if (pend == 2)
        asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * NCI) : "memory");
      else if (pend == 1)
        asm volatile("s_waitcnt vmcnt(%0)" :: "n"(NCI) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const uint8_t* buf = lds + (ch % NBUF) * CHUNK;
      const int kl = wave * 128 + q * 32;  // this lane's 32 k within the chunk
      const int k = ch * kGvKC + kl;
      const uint4 av = code16(buf, c, kl);
      const half2v sa = scale2(c, k);
      uint4 rv = av;
      half2v sr = sa;
      if constexpr (RAC) {
        rv = code16(buf, 16 + c, kl);
        sr = scale2(16 + c, k);
      }
      uint4 wv[NS];
      half2v sw[NS];
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) {
        wv[sl] = code16(buf, AROWS + 16 * sl + c, kl);
        sw[sl] = scale2(AROWS + 16 * sl + c, k);
      }
      const uint32_t aw[4] = {av.x, av.y, av.z, av.w}, rw[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int hi = st >> 1;  // steps 0-1: first block of the 32 k, 2-3: second
        const half2v s_a = hi ? __builtin_shufflevector(sa, sa, 1, 1)
                              : __builtin_shufflevector(sa, sa, 0, 0);
        const half8 ba = dequant8(aw[st], s_a);
        half8 br;
        if constexpr (RAC) {
          const half2v s_r = hi ? __builtin_shufflevector(sr, sr, 1, 1)
                                : __builtin_shufflevector(sr, sr, 0, 0);
          br = dequant8(rw[st], s_r);
        }
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
          const uint32_t ww = st == 0 ? wv[sl].x : st == 1 ? wv[sl].y : st == 2 ? wv[sl].z
                                                                              : wv[sl].w;
          const half2v s_w = hi ? __builtin_shufflevector(sw[sl], sw[sl], 1, 1)
                                : __builtin_shufflevector(sw[sl], sw[sl], 0, 0);
          const half8 bw = dequant8(ww, s_w);
          acc[sl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ba, bw, acc[sl], 0, 0, 0);
          if constexpr (RAC)
            acc[sl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(br, bw, acc[sl], 0, 0, 0);
        }
      }
      if (ch + NBUF < nch) {
        __syncthreads();  // every wave is done with this buffer
        issue(ch + NBUF);
      }
    }

    __syncthreads();  // every wave is done with the last chunk: its buffer holds the sums
#pragma unroll
    for (int sl = 0; sl < NS; ++sl) red[(wave * NS + sl) * 64 + lane] = acc[sl];
    __syncthreads();
    if (wave == 0) {
      float4v sm[NS];
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) {
        sm[sl] = red[sl * 64 + lane];
#pragma unroll
        for (int i = 1; i < kGvWaves; ++i) sm[sl] += red[(i * NS + sl) * 64 + lane];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + 4 * q + i;  // D row of element i
        if (row >= row_end) continue;
        if constexpr (!SILU) {
          float* out = reinterpret_cast<float*>(p.out);
          out[(int64_t)row * p.N + j0 + c] = scale * sm[0][i];
        } else {
          const float g = scale * sm[0][i], u = scale * sm[1][i];
          if (p.out_y) {
            p.out_y[(int64_t)row * p.N + j0 + c] = g;
            p.out_y[(int64_t)row * p.N + I + j0 + c] = u;
          }
          const uint32_t h = nv_f32_to_bf16(silu_mul(g, u));
          reinterpret_cast<uint16_t*>(p.out)[(int64_t)row * I + j0 + c] = (uint16_t)h;
          hmax = __builtin_fmaxf(hmax, __builtin_fabsf(nv_bf16_to_f32(h)));
        }
      }
    }
  }
  if constexpr (SILU) {
    if (wave == 0 && p.out_amax) {
      hmax = nv_wave_max(hmax);
      if (lane == 0 && hmax > 0.0f)
        atomicMax(reinterpret_cast<uint32_t*>(p.out_amax), __float_as_uint(hmax));
    }
  }
}

// Many groups with few rows each (the experts of a decode step): there is
// parallelism to spare across groups, so a workgroup owns 128 columns (eight
// 16-column slabs; with SiLU*mul four gate and the four matching up slabs)
// and one group, and takes MT 16-row fragments of the group per pass over W
// (MT = 1 or 2).  A wave dequantizes its A and R fragments once for four
// slabs, which keeps the VALU work per streamed W byte low.  K goes in
// 256-k chunks (codes, then the chunk's block scales, of 128 + 32 MT LDS
// rows) through NB buffers (23 KiB with MT = 1, 27 KiB with MT = 2): with
// two, one chunk is in flight while the other is computed, and three
// workgroups (MT = 1) or two (MT = 2, registers) fit on a CU; a handful of
// rows over many groups takes three.  (A three-deep ring with two workgroups
// per CU keeps more bytes in flight but streams 3-10% slower: more
// independent workgroups hide each one's start and finish better.)  Wave w
// takes k-slice w % 2 (128 k) of every chunk for slabs 4 (w / 2) .. 4 (w / 2)
// + 3; the two slices of a slab are added in slice order.
constexpr int kGwWaves = 4;
constexpr int kGwSlices = 2;               // 128-k slices per chunk
constexpr int kGwKC = 128 * kGwSlices;     // k per chunk
constexpr int kGwSlabs = 8;                // 16-column W slabs per workgroup
constexpr int kGwWaveSlabs = kGwSlabs * kGwSlices / kGwWaves;  // slabs per wave
constexpr int kGwBufs = 2;

template <bool RAC, bool SILU, bool GATHER, int MT, int NB = kGwBufs>
__global__ __launch_bounds__(64 * kGwWaves) void k_gemv_wide(GemmParams p) {
  constexpr int TR = 16 * MT;                 // rows of a group per pass over W
  constexpr int ROWS = 2 * TR + 16 * kGwSlabs;  // A TR | R TR (zero rows without RAC) | W
  constexpr int CROW = kGwKC / 2;            // code bytes per row per chunk (8 pieces)
  constexpr int SROW = kGwKC / 16;           // scale bytes per row per chunk
  constexpr int CODES = ROWS * CROW;
  constexpr int NCI = CODES / 1024 / kGwWaves;  // code DMA (16 B per lane) per wave
  // scale DMA (4 B per lane), rounded up to whole instructions per wave: the
  // extra lanes fetch zero-row words into padding past the scales
  constexpr int NSI = (ROWS * SROW + 256 * kGwWaves - 1) / (256 * kGwWaves);
  constexpr int SCALE_WORDS = ROWS * SROW / 4;
  constexpr int CHUNK = CODES + NSI * kGwWaves * 256;
  constexpr int PER = NCI + NSI;             // DMA instructions per wave per chunk
  static_assert(CODES % (1024 * kGwWaves) == 0 && (NB - 1) * PER <= 63, "DMA, vmcnt");
  static_assert(kGwWaves * kGwWaveSlabs * MT * 64 * 16 <= NB * CHUNK, "reduction fits");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NB * CHUNK];
  float4v* red = reinterpret_cast<float4v*>(lds);  // [wave][wave slab][lane], after the last chunk

  const int grp = blockIdx.z;
  const int row_beg = p.offsets[grp], row_end = p.offsets[grp + 1];
  const int nrows = row_end - row_beg;
  if ((int)blockIdx.y * TR >= nrows) return;  // workgroup-uniform

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ks = wave % kGwSlices, sh = wave / kGwSlices;  // k-slice, slab group
  const int K = p.K, K2 = K >> 1, K16 = K >> 4;
  const int nch = K / kGwKC;
  const int I = p.N >> 1;
  constexpr int HS = SILU ? kGwSlabs / 2 : kGwSlabs;  // slabs per half (gate, up)
  const int j0 = (int)blockIdx.x * 16 * HS;           // first column of slab 0
  auto w_row = [&](int i) -> int64_t {  // W row of LDS W row i
    const int sl = i >> 4;
    const int n = SILU ? (sl >= HS ? I : 0) + j0 + (sl % HS) * 16 + (i & 15) : j0 + i;
    return (int64_t)grp * p.N + n;
  };
  const float s_ta = p.a_ts[p.per_group ? grp : 0];
  float scale = p.w_ts[grp] * s_ta;
  if constexpr (RAC) {
    if (p.r_ts[p.per_group ? grp : 0] != s_ta) scale = __builtin_nanf("");  // shares s_ta
  }
  const uint32_t lbase = (uint32_t)(uintptr_t)(lds_ptr_t)lds;
  const int c = lane & 15, q = lane >> 4;
  float hmax = 0.0f;

  for (int tile = blockIdx.y; tile * TR < nrows; tile += gridDim.y) {
    const int m0 = row_beg + tile * TR;
    auto act = [&](const uint8_t* base, int i, int per_row) -> const uint8_t* {
      const int m = m0 + i;
      if (m >= row_end) return nv_zero_row;
      return base + (GATHER ? (int64_t)p.gather[m] : (int64_t)m) * per_row;
    };
    auto code_row = [&](int r) -> const uint8_t* {
      if (r < TR) return act(p.a_codes, r, K2);
      if (r < 2 * TR) return RAC ? act(p.r_codes, r - TR, K2) : nv_zero_row;
      return p.w_codes + w_row(r - 2 * TR) * K2;
    };
    auto scale_row = [&](int r) -> const uint8_t* {
      if (r < TR) return act(p.a_scales, r, K16);
      if (r < 2 * TR) return RAC ? act(p.r_scales, r - TR, K16) : nv_zero_row;
      return p.w_scales + w_row(r - 2 * TR) * K16;
    };
    // per-lane sources: code pieces (8 per row per chunk, XOR-swizzled by
    // row) and scale words (4 per row per chunk); chunk ch adds ch * CROW
    // or ch * SROW (the zero row is long enough for every chunk)
    const uint8_t* gcode[NCI];
    const uint8_t* gscale[NSI];
#pragma unroll
    for (int j = 0; j < NCI; ++j) {
      const int slot = (j * kGwWaves + wave) * 64 + lane, r = slot >> 3;
      gcode[j] = code_row(r) + (((slot & 7) ^ (r & 7)) << 4);
    }
#pragma unroll
    for (int j = 0; j < NSI; ++j) {
      const int slot = (j * kGwWaves + wave) * 64 + lane;
      gscale[j] = slot < SCALE_WORDS ? scale_row(slot >> 2) + (slot & 3) * 4 : nv_zero_row;
    }
    auto issue = [&](int ch) {
      const uint32_t st = lbase + (ch % NB) * CHUNK;
#pragma unroll
      for (int j = 0; j < NCI; ++j) {
        const uint32_t m0r = __builtin_amdgcn_readfirstlane(st + (j * kGwWaves + wave) * 1024);
        const uint8_t* g = gcode[j] + (int64_t)ch * CROW;
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                     :: "s"(m0r), "v"(g) : "memory", "m0");
      }
#pragma unroll
      for (int j = 0; j < NSI; ++j) {
        const uint32_t m0r =
            __builtin_amdgcn_readfirstlane(st + CODES + (j * kGwWaves + wave) * 256);
        const uint8_t* g = gscale[j] + (int64_t)ch * SROW;
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                     :: "s"(m0r), "v"(g) : "memory", "m0");
      }
    };
    __syncthreads();  // the previous tile's reduction has been read
    for (int ch = 0; ch < NB - 1 && ch < nch; ++ch) issue(ch);

    auto code16 = [&](const uint8_t* buf, int r, int kl) -> uint4 {
      return *reinterpret_cast<const uint4*>(buf + r * CROW + (((kl >> 5) ^ (r & 7)) << 4));
    };
    auto scale2 = [&](const uint8_t* buf, int r, int kl) -> half2v {  // blocks of kl .. kl+31
      const uint32_t v = *reinterpret_cast<const uint16_t*>(buf + CODES + r * SROW + (kl >> 4));
      return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, false);
    };
    float4v acc[MT][kGwWaveSlabs];  // main and residual passes (one tensor scale)
#pragma unroll
    for (int f = 0; f < MT; ++f)
#pragma unroll
      for (int t = 0; t < kGwWaveSlabs; ++t) acc[f][t] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
    for (int ch = 0; ch < nch; ++ch) {
      // issue chunk ch + 1 into the buffer computed in the previous iteration
      // (the barrier at its end ended its reads), then wait for chunk ch:
      // the chunk issued after it may stay in flight
      if (ch + NB - 1 < nch) issue(ch + NB - 1);
      const int pend = nch - 1 - ch < NB - 1 ? nch - 1 - ch : NB - 1;
      if (pend >= 2)
        asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * PER) : "memory");
      else if (pend == 1)
        asm volatile("s_waitcnt vmcnt(%0)" :: "n"(PER) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const uint8_t* buf = lds + (ch % NB) * CHUNK;
      const int kl = ks * 128 + q * 32;  // this lane's 32 k within the chunk
      uint32_t aw[MT][4], rw[MT][4];
      half2v sa[MT], sr[MT];
#pragma unroll
      for (int f = 0; f < MT; ++f) {
        const uint4 av = code16(buf, 16 * f + c, kl);
        sa[f] = scale2(buf, 16 * f + c, kl);
        uint4 rv = av;
        sr[f] = sa[f];
        if constexpr (RAC) {
          rv = code16(buf, TR + 16 * f + c, kl);
          sr[f] = scale2(buf, TR + 16 * f + c, kl);
        }
        aw[f][0] = av.x; aw[f][1] = av.y; aw[f][2] = av.z; aw[f][3] = av.w;
        rw[f][0] = rv.x; rw[f][1] = rv.y; rw[f][2] = rv.z; rw[f][3] = rv.w;
      }
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {  // the two 16-k blocks of the lane's 32 k
        half8 ba0[MT], ba1[MT], br0[MT], br1[MT];
#pragma unroll
        for (int f = 0; f < MT; ++f) {
          const half2v s_a = hi ? __builtin_shufflevector(sa[f], sa[f], 1, 1)
                                : __builtin_shufflevector(sa[f], sa[f], 0, 0);
          ba0[f] = dequant8(aw[f][2 * hi], s_a);
          ba1[f] = dequant8(aw[f][2 * hi + 1], s_a);
          if constexpr (RAC) {
            const half2v s_r = hi ? __builtin_shufflevector(sr[f], sr[f], 1, 1)
                                  : __builtin_shufflevector(sr[f], sr[f], 0, 0);
            br0[f] = dequant8(rw[f][2 * hi], s_r);
            br1[f] = dequant8(rw[f][2 * hi + 1], s_r);
          }
        }
#pragma unroll
        for (int t = 0; t < kGwWaveSlabs; ++t) {
          const int r = 2 * TR + 16 * (sh * kGwWaveSlabs + t) + c;
          const uint4 wv = code16(buf, r, kl);
          const half2v sw = scale2(buf, r, kl);
          const half2v s_w = hi ? __builtin_shufflevector(sw, sw, 1, 1)
                                : __builtin_shufflevector(sw, sw, 0, 0);
          const half8 bw0 = dequant8(hi ? wv.z : wv.x, s_w), bw1 = dequant8(hi ? wv.w : wv.y, s_w);
#pragma unroll
          for (int f = 0; f < MT; ++f) {
            acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ba0[f], bw0, acc[f][t], 0, 0, 0);
            acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ba1[f], bw1, acc[f][t], 0, 0, 0);
            if constexpr (RAC) {
              acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(br0[f], bw0, acc[f][t], 0, 0, 0);
              acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(br1[f], bw1, acc[f][t], 0, 0, 0);
            }
          }
        }
      }
      __syncthreads();  // every wave is done with this buffer
    }

#pragma unroll
    for (int f = 0; f < MT; ++f)
#pragma unroll
      for (int t = 0; t < kGwWaveSlabs; ++t)
        red[((f * kGwWaves + wave) * kGwWaveSlabs + t) * 64 + lane] = acc[f][t];
    __syncthreads();
    // wave w finishes slabs w and w + 4 (with SiLU: gate slab w, up slab w + 4)
    // of every 16-row fragment; slab sl's two k-slices sit with the waves of
    // slab group sl / 4
    constexpr int PERW = kGwSlabs / kGwWaves;
#pragma unroll
    for (int f = 0; f < MT; ++f) {
      const float4v* rf = red + f * kGwWaves * kGwWaveSlabs * 64;
      float4v sm[PERW];
#pragma unroll
      for (int t = 0; t < PERW; ++t) {
        const int sl = wave + t * kGwWaves;
        const int g = sl / kGwWaveSlabs, u = sl % kGwWaveSlabs;
        sm[t] = rf[((g * kGwSlices + 0) * kGwWaveSlabs + u) * 64 + lane];
#pragma unroll
        for (int i = 1; i < kGwSlices; ++i)
          sm[t] += rf[((g * kGwSlices + i) * kGwWaveSlabs + u) * 64 + lane];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + 16 * f + 4 * q + i;  // D row of element i
        if (row >= row_end) continue;
        if constexpr (!SILU) {
          float* out = reinterpret_cast<float*>(p.out);
#pragma unroll
          for (int t = 0; t < PERW; ++t)
            out[(int64_t)row * p.N + j0 + (wave + t * kGwWaves) * 16 + c] = scale * sm[t][i];
        } else {
          static_assert(!SILU || (PERW == 2 && HS == kGwWaves), "gate slab w, up slab w + HS");
          const int j = j0 + wave * 16 + c;
          const float g = scale * sm[0][i], u = scale * sm[1][i];
          if (p.out_y) {
            p.out_y[(int64_t)row * p.N + j] = g;
            p.out_y[(int64_t)row * p.N + I + j] = u;
          }
          const uint32_t h = nv_f32_to_bf16(silu_mul(g, u));
          reinterpret_cast<uint16_t*>(p.out)[(int64_t)row * I + j] = (uint16_t)h;
          hmax = __builtin_fmaxf(hmax, __builtin_fabsf(nv_bf16_to_f32(h)));
        }
      }
    }
  }
  if constexpr (SILU) {
    if (p.out_amax) {
      hmax = nv_wave_max(hmax);
      if (lane == 0 && hmax > 0.0f)
        atomicMax(reinterpret_cast<uint32_t*>(p.out_amax), __float_as_uint(hmax));
    }
  }
}

// Up to 16 rows per group on average a group's 16-row tiles are few, and one
// workgroup per column block walks them.  Above 8, a second workgroup per
// column block takes every other tile, so that groups of more than 16 rows
// do not stream their weights twice in a row; it exits at once where a
// group has one tile.  From 16 to 32 rows per group the workgroups take
// 32-row tiles (two 16-row fragments per pass over W; two workgroups per CU
// instead of three), and above 24 a second workgroup per column block again
// takes every other tile.
template <bool RAC, bool SILU, bool GATHER>
int launch_gemv_wide(GemmParams& p, hipStream_t s) {
  const int cols = 16 * kGwSlabs;  // output columns (SiLU: gate + up columns) per workgroup
  if (p.total_rows > 16 * (int64_t)p.G) {
    const unsigned yt = p.total_rows > 24 * (int64_t)p.G ? 2u : 1u;
    const dim3 grid((unsigned)(p.N / cols), yt, (unsigned)p.G);
    hipLaunchKernelGGL((k_gemv_wide<RAC, SILU, GATHER, 2>), grid, dim3(64 * kGwWaves), 0, s, p);
    return nv_launch_status();
  }
  const unsigned ytiles = p.total_rows > 8 * (int64_t)p.G ? 2u : 1u;
  const dim3 grid((unsigned)(p.N / cols), ytiles, (unsigned)p.G);
  // a handful of rows over many groups (one or two tokens through a large
  // MoE layer): few workgroups have work, one per CU, so each keeps two
  // chunks in flight through a three-deep ring
  if (p.total_rows * 16 <= (int64_t)p.G) {
    hipLaunchKernelGGL((k_gemv_wide<RAC, SILU, GATHER, 1, 3>), grid, dim3(64 * kGwWaves), 0, s, p);
    return nv_launch_status();
  }
  hipLaunchKernelGGL((k_gemv_wide<RAC, SILU, GATHER, 1>), grid, dim3(64 * kGwWaves), 0, s, p);
  return nv_launch_status();
}

template <bool RAC, bool SILU, bool GATHER>
int launch_gemv(GemmParams& p, hipStream_t s) {
  const int slabs = SILU ? p.N / 32 : p.N / 16;
  const int ytiles = p.G == 1 ? (p.total_rows + 15) / 16 : 1;
  const dim3 grid((unsigned)slabs, (unsigned)ytiles, (unsigned)p.G);
  hipLaunchKernelGGL((k_gemv<RAC, SILU, GATHER>), grid, dim3(64 * kGvWaves), 0, s, p);
  return nv_launch_status();
}

// 0: tile kernel; 1: decode kernel (one group); 2: wide decode kernel (groups)
int gemv_kind(const GemmParams& p, bool silu) {
  if (p.G == 1)
    return p.total_rows <= kGvMaxRows && p.K % kGvKC == 0 &&
                   p.K <= (silu ? 12288 : kGvMaxK) && p.N / 16 <= 65535
               ? 1 : 0;
  return p.total_rows <= (int64_t)kGvAvgRows * p.G && p.K % kGwKC == 0 && p.G <= 65535 ? 2 : 0;
}

int launch_gemv_wide_any(GemmParams& p, bool rac, bool silu, bool gather, hipStream_t s) {
  if (rac) {
    if (silu) return gather ? launch_gemv_wide<true, true, true>(p, s) : launch_gemv_wide<true, true, false>(p, s);
    return gather ? launch_gemv_wide<true, false, true>(p, s) : launch_gemv_wide<true, false, false>(p, s);
  }
  if (silu) return gather ? launch_gemv_wide<false, true, true>(p, s) : launch_gemv_wide<false, true, false>(p, s);
  return gather ? launch_gemv_wide<false, false, true>(p, s) : launch_gemv_wide<false, false, false>(p, s);
}

int launch_gemv_any(GemmParams& p, bool rac, bool silu, bool gather, hipStream_t s) {
  if (rac) {
    if (silu) return gather ? launch_gemv<true, true, true>(p, s) : launch_gemv<true, true, false>(p, s);
    return gather ? launch_gemv<true, false, true>(p, s) : launch_gemv<true, false, false>(p, s);
  }
  if (silu) return gather ? launch_gemv<false, true, true>(p, s) : launch_gemv<false, true, false>(p, s);
  return gather ? launch_gemv<false, false, true>(p, s) : launch_gemv<false, false, false>(p, s);
}

// Tile configurations (rows x cols per workgroup, waves, LDS stages, min waves
// per SIMD, residual step skipping).  Waves compute 64 x 128 (two 32-row
// fragments; a wave whose second fragment is all padding skips it).  With
// RAC and N % 512 == 0: 128 x 512 tiles of 2 x 4 waves, one workgroup (two
// waves per SIMD) per CU -- each staged byte feeds a third more MFMAs than
// in a 128 x 256 tile, which the copy into LDS dominates.  N % 256 == 0:
// 128 x 256 tiles of 2 x 2 waves, two workgroups per CU.  Other N, and
// residual block skipping: with RAC, 64 x 128 tiles (waves of 32 x 64); RAC
// off, 128 x 128 (waves of 64 x 64), so that the staged rows fill whole
// wave-loads.
template <bool RAC, bool SILU, bool GATHER>
int launch_cfg(GemmParams& p, hipStream_t s) {
  // block skipping needs registers for its activity mask: 64 x 128 tiles
  if constexpr (RAC) {
    if (p.skip) return launch_t<64, 128, 2, 2, 2, 2, RAC, SILU, GATHER, true>(p, s);
  }
  if constexpr (RAC) {
    if (p.N % 512 == 0) return launch_t<128, 512, 2, 4, 2, 1, RAC, SILU, GATHER, false>(p, s);
  }
  if (p.N % 256 == 0) return launch_t<128, 256, 2, 2, 2, 2, RAC, SILU, GATHER, false>(p, s);
  if constexpr (RAC) {
    return launch_t<64, 128, 2, 2, 2, 2, RAC, SILU, GATHER, false>(p, s);
  } else {
    return launch_t<128, 128, 2, 2, 2, 2, RAC, SILU, GATHER, false>(p, s);
  }
}

int launch(GemmParams& p, bool rac, bool silu, bool gather, hipStream_t s) {
  if (rac) {
    if (silu) return gather ? launch_cfg<true, true, true>(p, s) : launch_cfg<true, true, false>(p, s);
    return gather ? launch_cfg<true, false, true>(p, s) : launch_cfg<true, false, false>(p, s);
  }
  if (silu) return gather ? launch_cfg<false, true, true>(p, s) : launch_cfg<false, true, false>(p, s);
  return gather ? launch_cfg<false, false, true>(p, s) : launch_cfg<false, false, false>(p, s);
}

}  // namespace

extern "C" {

int nvfp4_check_groups(const int32_t* offsets, int64_t G, int64_t total_rows,
                       const int32_t* gather, int64_t src_rows) {
  NV_RETURN_IF(!offsets, NVFP4_ERR_NULL);
  NV_RETURN_IF(G < 1 || total_rows < 0 || offsets[0] != 0 || offsets[G] != total_rows,
               NVFP4_ERR_SHAPE);
  for (int64_t g = 0; g < G; ++g) NV_RETURN_IF(offsets[g + 1] < offsets[g], NVFP4_ERR_SHAPE);
  if (gather) {
    for (int64_t j = 0; j < total_rows; ++j)
      NV_RETURN_IF(gather[j] < 0 || gather[j] >= src_rows, NVFP4_ERR_SHAPE);
  }
  return NVFP4_OK;
}

size_t w4a4_grouped_gemm_rac_workspace_size(const w4a4_gemm_args_t*) { return 0; }

int w4a4_grouped_gemm_rac(const w4a4_gemm_args_t* a, void*, size_t, void* stream) {
  NV_RETURN_IF(!a, NVFP4_ERR_NULL);
  NV_RETURN_IF(a->epilogue != NVFP4_EPI_F32 && a->epilogue != NVFP4_EPI_SILU_MUL_BF16,
               NVFP4_ERR_DTYPE);
  NV_RETURN_IF(a->num_groups < 1 || a->total_rows < 0 || a->N <= 0 || a->K <= 0 ||
                   a->K % KC || a->N % 128 || a->N > (1 << 24) || a->K > (1 << 24) ||
                   a->total_rows > 0x7fffffff || a->num_groups > (1 << 20) ||
                   a->K > KC * kMaxKChunks,
               NVFP4_ERR_SHAPE);
  NV_RETURN_IF(!a->group_offsets || !a->w_codes || !a->w_scales || !a->w_tscale ||
                   !a->a_tscale,
               NVFP4_ERR_NULL);
  if (a->total_rows == 0) return NVFP4_OK;  // nothing to compute; row buffers may be empty
  NV_RETURN_IF(!a->a_codes || !a->a_scales || !a->out, NVFP4_ERR_NULL);
  NV_RETURN_IF(a->r_codes && (!a->r_scales || !a->r_tscale), NVFP4_ERR_NULL);
  NV_RETURN_IF(!nv_aligned16(a->a_codes) || !nv_aligned16(a->w_codes) ||
                   !nv_aligned16(a->out) || (a->r_codes && !nv_aligned16(a->r_codes)) ||
                   (a->epilogue == NVFP4_EPI_SILU_MUL_BF16 && a->out_y &&
                    (reinterpret_cast<uintptr_t>(a->out_y) & 3)) ||
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
  p.out_y = a->epilogue == NVFP4_EPI_SILU_MUL_BF16 ? a->out_y : nullptr;
  p.skip = (a->flags & NVFP4_GEMM_SKIP_INACTIVE_BLOCKS) && a->kblock_active ? 1 : 0;
  p.per_group = (a->flags & NVFP4_GEMM_PER_GROUP_SCALES) ? 1 : 0;
  const bool rac = a->r_codes != nullptr, gather = a->gather_rows != nullptr;
  const bool silu = a->epilogue == NVFP4_EPI_SILU_MUL_BF16;
  const int kind = gemv_kind(p, silu);
  if (kind == 1) return launch_gemv_any(p, rac, silu, gather, s);
  if (kind == 2) return launch_gemv_wide_any(p, rac, silu, gather, s);
  return launch(p, rac, silu, gather, s);
}

}  // extern "C"
