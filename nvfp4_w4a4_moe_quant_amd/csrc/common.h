// Internal helpers shared by the HIP translation units of libnvfp4rac.
// gfx950 only; compiled with -ffp-contract=off so that the quantizer's FP32
// steps stay the single IEEE operations the format definition names.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4rac.h"

#define NV_RETURN_IF(cond, code) \
  do {                           \
    if (cond) return (code);     \
  } while (0)

static inline int nv_launch_status() {
  return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

static inline bool nv_aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

static inline size_t nv_round256(size_t n) { return (n + 255) & ~size_t(255); }

// ---------------------------------------------------------------- formats

// E4M3 byte (0..0x7E) -> float value.  Exponent field 0 is subnormal b*2^-9.
__device__ __forceinline__ float nv_e4m3_to_f32(uint32_t b) {
  return (b < 8u) ? (float)b * 0.001953125f
                  : __uint_as_float((((b >> 3) + 120u) << 23) | ((b & 7u) << 20));
}

// Nearest E4M3 to rho >= 0 (finite), ties to even, saturating at 448.
// Normal range: round the FP32 mantissa to 3 bits with the carry running into
// the exponent; below 2^-6 the grid is uniform with step 2^-9.
__device__ __forceinline__ uint32_t nv_e4m3_encode(float rho) {
  if (!(rho > 0.0f)) return 0u;
  if (rho >= 448.0f) return 0x7Eu;
  if (rho < 0.015625f) return (uint32_t)__builtin_rintf(rho * 512.0f);
  const uint32_t u = __float_as_uint(rho);
  const uint32_t c = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - (120u << 3);
  return c > 0x7Eu ? 0x7Eu : c;
}

// Nearest E2M1 code to v, ties to the even magnitude index, saturating at 6;
// the thresholds are the midpoints of {0, .5, 1, 1.5, 2, 3, 4, 6}, strict where
// the lower neighbour has the even index.
__device__ __forceinline__ uint32_t nv_e2m1_encode(float v) {
  const float a = __builtin_fabsf(v);
  const uint32_t idx = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) +
                       (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
                       (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                       (uint32_t)(a > 5.0f);
  return (v < 0.0f && idx != 0u) ? (idx | 8u) : idx;
}

// E2M1 code -> signed float value.
__device__ __forceinline__ float nv_e2m1_to_f32(uint32_t c) {
  const uint32_t idx = c & 7u;
  const float g = (idx < 2u) ? (float)idx * 0.5f
                             : __uint_as_float((((idx >> 1) + 126u) << 23) | ((idx & 1u) << 22));
  return (c & 8u) ? -g : g;
}

// Tensor scale s_t = RN32(amax / 2688) (double quotient rounded once).
__device__ __forceinline__ float nv_tensor_scale(float amax) {
  return (float)((double)amax / 2688.0);
}

// Block scale code from the block amax: rho = RN32(amax_b / (6 s_t)).
__device__ __forceinline__ uint32_t nv_block_scale(float amax_b, float s_t) {
  if (s_t == 0.0f) return 0u;
  const float rho = (float)((double)amax_b / (6.0 * (double)s_t));
  return nv_e4m3_encode(rho);
}

// Reciprocal of the effective block scale, correctly rounded (0 for S_b = 0).
__device__ __forceinline__ float nv_block_recip(float Sb) {
  return (Sb > 0.0f) ? (float)(1.0 / (double)Sb) : 0.0f;
}

// nv_block_scale from an FP32 product instead of the double-precision
// quotient.  c6 = RN32(1 / (6 s_t)) (per tensor) makes r = RN32(amax_b c6)
// agree with y = amax_b / (6 s_t) to within 1.5 * 2^-23 relative (two FP32
// roundings), and the quotient rounded to FP32 agrees with y to 2^-24: the two
// lie less than three FP32 ulp apart.  In E4M3's normal range the code only
// changes at the midpoints between grid values, which sit at 0x80000 in the
// low 20 mantissa bits of each binade (powers of two are grid values, not
// boundaries); so when r is at least 16 ulp from a midpoint, r and the
// quotient round to the same code.  Near a midpoint, below the normal range
// (2^-6, with a margin) and for zero or non-finite products the exact path
// decides.
__device__ __forceinline__ uint32_t nv_block_scale_c6(float amax_b, float s_t, float c6) {
  if (amax_b == 0.0f) return 0u;
  const float r = amax_b * c6;
  const uint32_t u = __float_as_uint(r);
  const bool near_mid = ((u & 0xFFFFFu) - 0x7FFF0u) < 0x20u;
  if (r >= 0.0157f && r < 448.0f && !near_mid) {
    const uint32_t c = ((u + 0x80000u) >> 20) - (120u << 3);  // round half up: no ties here
    return c > 0x7Eu ? 0x7Eu : c;
  }
  if (r >= 448.0f && r <= 3.4e38f) return 0x7Eu;  // the quotient is at least 447.99: saturates
  return nv_block_scale(amax_b, s_t);
}

// rb of every E4M3 code for one tensor scale: lut[c] = nv_block_recip(
// RN32(E4M3(c) s_t)), filled by the first 128 threads (the caller
// synchronizes before reading it).
__device__ __forceinline__ void nv_fill_recip_lut(float* lut, float s_t) {
  if (threadIdx.x < 128) lut[threadIdx.x] = nv_block_recip(nv_e4m3_to_f32(threadIdx.x) * s_t);
}

// Score shift 8 - Es where s_t = f * 2^Es, f in [0.5, 1).
__device__ __forceinline__ int nv_score_shift(float s_t) {
  return (s_t == 0.0f) ? 8 : 8 - __builtin_amdgcn_frexp_expf(s_t);
}

// Fixed-point magnitude q = min(floor(|e| 2^shift), 2^17 - 1).  The clamp
// comes first and the conversion truncates, which is the floor of a
// non-negative value (2^17 - 1 is an integer, so clamping and flooring
// commute).
__device__ __forceinline__ uint32_t nv_score_qi(float e, int shift) {
  const float t = __builtin_fminf(__builtin_ldexpf(__builtin_fabsf(e), shift), 131071.0f);
  return (uint32_t)t;
}

// bf16 bits -> float.
__device__ __forceinline__ float nv_bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t nv_f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Load 16 consecutive inputs starting at element offset `off` (16-byte aligned).
__device__ __forceinline__ void nv_load16(const void* x, int bf16, int64_t off, float* v) {
  if (bf16) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + off);
    const uint4 a = p[0], b = p[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 q = p[i];
      v[4 * i] = q.x;
      v[4 * i + 1] = q.y;
      v[4 * i + 2] = q.z;
      v[4 * i + 3] = q.w;
    }
  }
}

// Wave-wide max of a non-negative float (64 lanes).
__device__ __forceinline__ float nv_wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Clear the sign of E2M1 codes whose magnitude index is 0 (no -0), for the 8
// codes of a word: bit 3 of a nibble survives only if its low 3 bits are not 0.
__device__ __forceinline__ uint32_t nv_clear_neg_zero(uint32_t w) {
  const uint32_t nz = ((w & 0x77777777u) + 0x77777777u) & 0x88888888u;
  return w & (nz | 0x77777777u);
}

// 8 values times r -> 8 E2M1 codes (element 2j in the low nibble of byte j).
// The gfx950 packed FP4 conversion rounds to nearest even and saturates at 6;
// each product x*r is one FP32 multiply before it.
__device__ __forceinline__ uint32_t nv_encode8(const float* v, float r) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0] * r, v[1] * r, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2] * r, v[3] * r, 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4] * r, v[5] * r, 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6] * r, v[7] * r, 1.0f, 3);
  return nv_clear_neg_zero(w);
}

typedef float nv_float2 __attribute__((ext_vector_type(2)));

// 8 E2M1 codes -> 8 signed grid values (FP32, exact).
__device__ __forceinline__ void nv_decode8(uint32_t w, float* g) {
  const nv_float2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const nv_float2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const nv_float2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const nv_float2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  g[0] = a.x; g[1] = a.y; g[2] = b.x; g[3] = b.y;
  g[4] = c.x; g[5] = c.y; g[6] = d.x; g[7] = d.y;
}

// ---------------------------------------------------------- grouped tiles

// Tile of a grouped-GEMM workgroup: group `grp` (-1 for a surplus
// workgroup), m-tile `local` inside the group, n-tile `nt`.  The grid holds
// m_slots x n_tiles workgroups, m_slots an upper bound on the groups'
// m-tiles; the real count is only known on the device.
//  * A first wave-wide pass sums the groups' m-tiles, so the real tiles --
//    not the grid's upper bound -- are split evenly over the eight XCDs (the
//    hardware deals workgroups round-robin over them).  Each XCD gets one
//    contiguous range of tile indices, so consecutive tiles run on one XCD
//    and share its L2; workgroups past their XCD's share exit.
//  * Inside a group the m-tiles vary fastest: the workgroups that read one W
//    tile (one n-tile of one group) are adjacent.  With BAND_M > 0 they vary
//    fastest in bands of at most BAND_M m-tiles, each band running through
//    every n-tile before the next starts.  A group of at most BAND_M m-tiles
//    keeps the plain order; in a long group (a dense GEMM) the tiles an XCD
//    runs at once then cover a few m-tiles by a few n-tiles and share both
//    their A and their W tiles in its L2, where the plain order has them all
//    read one W tile and each its own A tile, streaming A from HBM once per
//    n-tile.
//  * A second wave scan finds the group of the tile; every wave of the
//    workgroup computes the same result.
struct NvTile {
  int grp, local, nt;
};

__device__ __forceinline__ int nv_group_tiles(const int32_t* offsets, int G, int g, int bm) {
  return g < G ? (offsets[g + 1] - offsets[g] + bm - 1) / bm : 0;
}

template <int BAND_M = 0>
__device__ __forceinline__ NvTile nv_find_tile(const int32_t* offsets, int G, int bm,
                                               int m_slots, int n_tiles) {
  (void)m_slots;
  const int lane = threadIdx.x & 63;
  NvTile t{-1, 0, 0};
  int total = 0;
  for (int c = 0; c < G; c += 64) {
    int v = nv_group_tiles(offsets, G, c + lane, bm);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    total += v;
  }
  const int nblocks = total * n_tiles;  // real tiles
  const int bid = blockIdx.x;
  const int per = nblocks / 8, rem = nblocks % 8, xcd = bid % 8, li = bid / 8;
  if (li >= per + (xcd < rem ? 1 : 0)) return t;
  const int L = xcd * per + (xcd < rem ? xcd : rem) + li;
  const int mt = L / n_tiles;
  int run = 0;
  for (int c = 0; c < G; c += 64) {
    const int g = c + lane;
    const int tiles = nv_group_tiles(offsets, G, g, bm);
    int inc = tiles;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int n = __shfl_up(inc, o, 64);
      if (lane >= o) inc += n;
    }
    const int excl = inc - tiles;
    const bool hit = g < G && mt >= run + excl && mt < run + inc;
    const unsigned long long bal = __ballot(hit);
    if (bal) {
      const int hl = __ffsll((long long)bal) - 1;
      const int first = run + __shfl(excl, hl, 64);
      const int gt = __shfl(tiles, hl, 64);
      const int i = L - first * n_tiles;  // tile inside the group
      t.grp = c + hl;
      if constexpr (BAND_M > 0) {
        const int band = i / (BAND_M * n_tiles);
        const int gm = min(BAND_M, gt - band * BAND_M);  // m-tiles of the band
        const int j = i - band * BAND_M * n_tiles;
        t.local = band * BAND_M + j % gm;
        t.nt = j / gm;
      } else {
        t.local = i % gt;
        t.nt = i / gt;
      }
      return t;
    }
    run += __shfl(inc, 63, 64);
  }
  return t;
}
