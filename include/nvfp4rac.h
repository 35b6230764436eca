/*
 * nvfp4rac -- NVFP4 W4A4 MoE GEMMs with Residual Activation Compensation,
 * native on AMD Instinct MI355X (gfx950).  C ABI.
 *
 * What the calls compute (cited by page title and section):
 *  - QUADS arXiv abstract (mlsanity paper page, "Abstract (arXiv)"): NVFP4
 *    pairs per-block scale factors with 4-bit E2M1 values and multiplies
 *    4-bit weights by 4-bit activations; rollout activations are new at
 *    every step and are quantized at run time; Residual Activation
 *    Compensation (RAC) repairs the activation channels with the worst
 *    quantization error and keeps the 4-bit GEMMs.
 *  - Blog post "Why 4-bit RL rollout collapses - and it isn't the weights",
 *    section "The failure mode": E2M1 can represent eight magnitudes for
 *    each sign; every engine quantizes the synchronized weights the same way.
 *  - Same post, section "Two fixes, on two different sides": about half of
 *    the activation channels, those with the largest error, also go through
 *    a second 4-bit GEMM on their quantized residual, in the same kernels;
 *    the ordinary 4-bit pass is unchanged.
 *
 * Number formats (the pages name no block size or scale encoding; this library
 * implements the standard NVFP4 layout):
 *  - element: E2M1 code, 4 bits, sign in bit 3, magnitude index in bits 0-2
 *    over {0, 0.5, 1, 1.5, 2, 3, 4, 6}; -0 is never produced.
 *  - block scale: one OCP E4M3 byte (bias 7, max 448, never NaN, sign 0) per
 *    16 consecutive elements along K, blocks starting at k = 0.
 *  - tensor scale: FP32 s_t = RN32(amax / 2688), 2688 = 6 * 448.
 *  - layout: codes[rows, K/2] bytes, element 2j in the low nibble of byte j;
 *    scales[rows, K/16] bytes.  Weights are [N, K] (out x in), y = x W^T.
 *  - rounding: round-to-nearest-even with saturation for both encodings.
 *    rho_b = RN32(amax_b / (6 s_t)), s_b = E4M3(rho_b), S_b = RN32(s_b s_t),
 *    r_b = RN32(1 / S_b), code = E2M1(RN32(x r_b)).
 *
 * Conventions for every call:
 *  - Pointers are device pointers unless stated; the caller owns all memory.
 *    Calls allocate nothing; scratch comes from the caller's workspace `ws`
 *    of at least the size the matching *_workspace_size call returns.
 *  - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL is
 *    the default stream).  Arguments are validated on the host before
 *    anything is enqueued; a failed check returns its status and enqueues no
 *    work.  Launch failures return NVFP4_ERR_HIP.  Device faults surface at
 *    the caller's next synchronization.
 *  - Not checked on the device (preconditions): finite inputs; group offsets
 *    non-decreasing with the last equal to total_rows; gather indices in
 *    range; an `amax_in` not smaller than the true max|x|.  The group and
 *    gather rules can be checked on host copies with nvfp4_check_groups.
 *  - Re-entrant on distinct buffers; results are bit-reproducible (integer
 *    and max reductions only; no floating-point atomics).
 */
#ifndef NVFP4RAC_H
#define NVFP4RAC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = 1,      /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = 2,     /* a size is negative or violates a divisibility rule */
  NVFP4_ERR_DTYPE = 3,     /* unknown dtype or epilogue enum */
  NVFP4_ERR_ALIGN = 4,     /* a pointer or leading dimension is misaligned */
  NVFP4_ERR_WORKSPACE = 5, /* workspace missing or too small */
  NVFP4_ERR_HIP = 6        /* a kernel launch failed */
} nvfp4_status_t;

typedef enum { NVFP4_IN_F32 = 0, NVFP4_IN_BF16 = 1 } nvfp4_in_dtype_t;

typedef enum {
  NVFP4_EPI_F32 = 0,           /* out: float [total_rows, N] */
  NVFP4_EPI_SILU_MUL_BF16 = 1, /* out: bf16 [total_rows, N/2], h = silu(gate) * up */
  NVFP4_EPI_BF16 = 2           /* out: bf16 [total_rows, N], y rounded to nearest even
                                  (fp8_grouped_gemm only) */
} nvfp4_epilogue_t;

/* Text for a status code (static storage). */
const char* nvfp4_status_string(int status);

/* ------------------------------------------------------------------------
 * nvfp4_quantize -- run-time NVFP4 quantization of one tensor (abstract:
 * activations are quantized at every step; blog, "The failure mode": the
 * weights go through the same quantizer once per synchronization).
 *
 * x        [rows, K] row-major, row stride ldx elements, dtype F32 or BF16.
 *          Requires K % 16 == 0, ldx % 16 == 0, ldx >= K, x 16-byte aligned.
 * amax_in  nullable device float: the tensor amax to use instead of max|x|
 *          (a producer that already knows it, e.g. the SiLU*mul epilogue).
 * codes    out [rows, K/2];  scales out [rows, K/16];  tensor_scale out [1].
 * channel_score  nullable.  When given, the RAC per-channel error statistics
 *          are computed in the same pass over x:  e = x - deq(q(x)) in FP32;
 *          with Es the exponent of s_t (s_t = f 2^Es, f in [0.5, 1)) and
 *          q = min(floor(|e| 2^(8-Es)), 2^17 - 1):  channel_score[k] = sum
 *          over rows of q^2 (int64, exact).  It feeds rac_select_residual.
 *          (Blog, "Two fixes": channels ranked by quantization error; the
 *          metric is this library's reading: the sum of squared errors, in
 *          fixed point so that it is exact.)
 * channel_max  nullable; requires channel_score.  When given, also
 *          channel_max[k] = max over rows of |e| (float), a diagnostic the
 *          selection does not read; leaving it NULL saves its arithmetic and
 *          atomics (about a tenth of the call).
 * rows == 0 is allowed (writes s_t = RN32(amax_in/2688) or 0, and zero stats).
 * ------------------------------------------------------------------------ */
size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t K);
int nvfp4_quantize(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx,
                   const float* amax_in, uint8_t* codes, uint8_t* scales,
                   float* tensor_scale, int64_t* channel_score, float* channel_max,
                   void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * rac_select_residual -- RAC channel selection and residual re-quantization
 * (blog, "Two fixes, on two different sides": the activation channels with
 * the largest errors, about half of them, get a second 4-bit GEMM pass on
 * their quantized residual).
 *
 * Inputs: the same x, scales, tensor_scale that nvfp4_quantize used and
 * wrote, and its channel_score.  codes is not read and may be NULL: the main
 * codes are a function of x, scales and tensor_scale, and the residual pass
 * recomputes them, which costs less than reading them back.  channel_max is
 * not read either (the selection ranks the scores) and may be NULL.
 * n_select (0 <= n_select <= K; K/2 in the workloads): the channels with the
 *          largest channel_score are selected, ties toward the lower channel
 *          index.
 * selected out [n_select] int32, ascending channel indices.
 * kblock_active out [K/16]: 1 where the 16-block holds a selected channel.
 * res_codes/res_scales out, same layout as codes/scales; res_tensor_scale out:
 *          r = e on selected channels and 0 elsewhere, quantized to NVFP4 in
 *          the same 16-element blocks with the activation's own tensor scale
 *          s_t (the residual pass shares the main pass's tensor scale, so the
 *          GEMM adds both passes in one accumulator): block scale
 *          E4M3(RN32(max|r_b| / (6 s_t))), codes as nvfp4_quantize.
 *          *res_tensor_scale receives s_t.
 * Requires K <= 16384 and the layout rules of nvfp4_quantize; ws 4-byte
 * aligned.  The result is deterministic (integer ranks, max reductions).
 * ------------------------------------------------------------------------ */
size_t rac_select_residual_workspace_size(int64_t rows, int64_t K);
int rac_select_residual(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx,
                        const uint8_t* codes, const uint8_t* scales,
                        const float* tensor_scale, const int64_t* channel_score,
                        const float* channel_max, int64_t n_select,
                        int32_t* selected, uint8_t* kblock_active,
                        uint8_t* res_codes, uint8_t* res_scales,
                        float* res_tensor_scale, void* ws, size_t ws_bytes,
                        void* stream);

/* ------------------------------------------------------------------------
 * nvfp4_quantize_rac_static -- nvfp4_quantize (with statistics) followed by
 * rac_select_residual, in one call that allocates nothing and takes no
 * workspace: for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Arguments and
 * results are those of the two calls (channel_score is required,
 * channel_max may be NULL).  Scratch (6 KiB: amax partials and block masks) lives in a
 * device array of the library, one per GPU, held until the process ends; its
 * address is looked up on the first call on each device (which must be the
 * current device, the stream's device).  Every call on a GPU shares that
 * GPU's array: calls that overlap on one GPU race (serialize them on one
 * stream).  Nothing in it needs to start at zero.  Limit: K <= 16384
 * (NVFP4_ERR_SHAPE beyond); otherwise the rules of nvfp4_quantize and
 * rac_select_residual.  NVFP4_ERR_HIP if the array's address cannot be found.
 * ------------------------------------------------------------------------ */
int nvfp4_quantize_rac_static(const void* x, int dtype, int64_t rows, int64_t K, int64_t ldx,
                              const float* amax_in, uint8_t* codes, uint8_t* scales,
                              float* tensor_scale, int64_t* channel_score, float* channel_max,
                              int64_t n_select, int32_t* selected, uint8_t* kblock_active,
                              uint8_t* res_codes, uint8_t* res_scales, float* res_tensor_scale,
                              void* stream);

/* ------------------------------------------------------------------------
 * moe_route -- top-k routing of T tokens over E experts and the gather map
 * for the grouped GEMM (the MoE layer of the rollout model; the pages give no
 * routing details, so this is the plain reading).
 *
 * logits   [T, E] float.  Per token, the k experts with the largest logit,
 *          ties toward the lower expert index, in (logit desc, index asc)
 *          order -> topk_ids [T, k].
 * topk_weights nullable [T, k]: softmax(logits) of the chosen experts (not
 *          renormalized; FP32, not bit-defined).
 * expert_offsets [E+1]: exclusive prefix sum of per-expert counts.
 * gather_rows [T*k]: source token of each grouped row, expert-major, tokens
 *          ascending within an expert.  row_of [T, k]: grouped row of
 *          (token, slot).
 * Requires 1 <= k <= min(E, 16), E <= 1024.  With T == 0 the per-token
 * pointers may be NULL and expert_offsets is all zero.
 * ------------------------------------------------------------------------ */
size_t moe_route_workspace_size(int64_t T, int64_t E, int64_t k);
int moe_route(const float* logits, int64_t T, int64_t E, int64_t k,
              int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
              int32_t* gather_rows, int32_t* row_of, void* ws, size_t ws_bytes,
              void* stream);

/* ------------------------------------------------------------------------
 * Per-expert RAC.  The pages leave open over which rows RAC's tensor scale and
 * channel selection are taken (blog post, section "Two fixes, on two
 * different sides").  The calls above take one GEMM-input tensor; these take
 * each expert group on its own: the grouped rows j of group g,
 * group_offsets[g] <= j < group_offsets[g+1], read from x row gather_rows[j]
 * (or row j when gather_rows is NULL), form a tensor with its own amax and
 * tensor scale, channel statistics, selection of n_select channels and
 * residual tensor scale.  Every step is the per-tensor definition applied to
 * that tensor.  Outputs are in grouped row order: codes / res_codes
 * [total_rows, K/2], scales / res_scales [total_rows, K/16]; per group:
 * tensor_scales / res_tensor_scales [G], channel_score [G, K] (int64),
 * channel_max [G, K] (nullable, requires channel_score), selected
 * [G, n_select] (ascending per group), kblock_active [G, K/16].  The GEMM then runs without a gather, with
 * NVFP4_GEMM_PER_GROUP_SCALES.  Requires 1 <= G <= 65535, K % 16 == 0,
 * total_rows * K / 16 < 2^31, x 16-byte aligned, ldx % 16 == 0; the
 * selection needs K <= 16384.  Empty groups get zero tensor scales and the
 * n_select lowest channels.
 * ------------------------------------------------------------------------ */
size_t nvfp4_quantize_grouped_workspace_size(int64_t G, int64_t K);
int nvfp4_quantize_grouped(const void* x, int in_dtype, int64_t K, int64_t ldx,
                           const int32_t* group_offsets, int64_t G, int64_t total_rows,
                           const int32_t* gather_rows, uint8_t* codes, uint8_t* scales,
                           float* tensor_scales, int64_t* channel_score, float* channel_max,
                           void* ws, size_t ws_bytes, void* stream);
size_t rac_select_residual_grouped_workspace_size(int64_t G, int64_t K);
int rac_select_residual_grouped(const void* x, int in_dtype, int64_t K, int64_t ldx,
                                const int32_t* group_offsets, int64_t G, int64_t total_rows,
                                const int32_t* gather_rows, const uint8_t* scales,
                                const float* tensor_scales, const int64_t* channel_score,
                                const float* channel_max, int64_t n_select, int32_t* selected,
                                uint8_t* kblock_active, uint8_t* res_codes, uint8_t* res_scales,
                                float* res_tensor_scales, void* ws, size_t ws_bytes,
                                void* stream);

/* ------------------------------------------------------------------------
 * moe_combine -- weighted combine of the expert outputs back to token order
 * (the end of the MoE layer whose expert GEMMs the pages quantize).  For each
 * token t, in slot order s = 0 .. k-1 (the order moe_route writes):
 *   acc = RN32(acc + RN32(topk_weights[t, s] * y[row_of[t, s], :])), acc from 0
 * then out[t, :] = acc (FP32, out_dtype NVFP4_IN_F32) or bf16(acc) (nearest
 * even, NVFP4_IN_BF16).  A gather, not an atomic scatter-add, so the result
 * is deterministic.  y is float [rows, H] in grouped order; row_of and
 * topk_weights are [T, k] from moe_route; out is [T, H].  Requires 1 <= k <=
 * 16, H % 8 == 0, y and out 16-byte aligned.  No workspace.
 * ------------------------------------------------------------------------ */
int moe_combine(const float* y, const int32_t* row_of, const float* topk_weights, int64_t T,
                int64_t k, int64_t H, int out_dtype, void* out, void* stream);

/* ------------------------------------------------------------------------
 * w4a4_grouped_gemm_rac -- grouped (per-expert) W4A4 GEMM with the RAC
 * residual pass fused into the same kernel (abstract: 4-bit by 4-bit GEMMs;
 * blog, "Two fixes": the selected channels' residual pass adds to the
 * unchanged main pass).
 *
 * For grouped row j of group g (offsets[g] <= j < offsets[g+1]) and src =
 * gather_rows[j] (or j when gather_rows is NULL):
 *   y[j, n] = s_tw[g] * s_ta * ( sum_k A[src,k] W_g[n,k]
 *                              + sum_{k in active blocks} R[src,k] W_g[n,k] )
 * with A, R, W the exact dequantized values g * s_b, both passes accumulated
 * in one FP32 accumulator.  The residual shares the activation's tensor
 * scale (rac_select_residual writes *r_tscale = s_ta): the call requires
 * *r_tscale == *a_tscale (per group with NVFP4_GEMM_PER_GROUP_SCALES) and
 * writes NaN outputs for a group where they differ.
 * r_codes == NULL turns RAC off (naive W4A4).  kblock_active == NULL means
 * every block is active.  With NVFP4_GEMM_SKIP_INACTIVE_BLOCKS in `flags`, the
 * residual MFMAs of each 32-k step run only if one of its two 16-blocks is
 * active; without it the residual pass runs over every block.  Both are exact
 * (an inactive block's residual codes are zero); the flag pays off when the
 * selection leaves many blocks inactive, and costs a few percent otherwise.
 * Epilogue F32 writes y.  Epilogue SILU_MUL_BF16 treats W as the fused
 * gate/up weight [N = 2I, K] with the gate in rows [0, I) and writes
 * h[j, i] = bf16(silu(y[j, i]) * y[j, I + i]) to out [total_rows, I] and, if
 * out_amax is given, max-combines max|h| into *out_amax (an atomic max on the
 * float bits; the caller initializes *out_amax, normally to 0, so that the
 * call launches the GEMM kernel alone).  With SILU_MUL, a non-NULL out_y
 * (float [total_rows, N], 4-byte aligned) also receives the FP32 values y
 * that enter the SiLU*mul, gate columns then up columns as in W: the same
 * kernel and accumulation, plus these stores (for verification).
 * Requires K % 128 == 0, N % 128 == 0, all tensors 16-byte aligned.
 * ------------------------------------------------------------------------ */
typedef struct {
  int64_t num_groups;           /* G >= 1 */
  int64_t N;                    /* output columns (2I for SILU_MUL) */
  int64_t K;                    /* contraction length */
  int64_t total_rows;           /* rows of the grouped output */
  const int32_t* group_offsets; /* [G+1], ascending, [0] = 0, [G] = total_rows */
  const int32_t* gather_rows;   /* [total_rows] or NULL (identity) */
  const uint8_t* a_codes;       /* [src_rows, K/2] */
  const uint8_t* a_scales;      /* [src_rows, K/16] */
  const float* a_tscale;        /* [1] */
  const uint8_t* r_codes;       /* residual, or NULL for RAC off */
  const uint8_t* r_scales;
  const float* r_tscale;
  const uint8_t* kblock_active; /* [K/16] or NULL */
  const uint8_t* w_codes;       /* [G, N, K/2] */
  const uint8_t* w_scales;      /* [G, N, K/16] */
  const float* w_tscale;        /* [G] */
  int64_t epilogue;             /* nvfp4_epilogue_t */
  void* out;                    /* float [total_rows, N] or bf16 [total_rows, N/2] */
  float* out_amax;              /* SILU_MUL only, nullable, caller-initialized */
  int64_t flags;                /* NVFP4_GEMM_* bits */
  float* out_y;                 /* SILU_MUL only, nullable: FP32 y [total_rows, N] */
} w4a4_gemm_args_t;

/* nvfp4_check_groups -- host-side check of the grouped GEMM's preconditions
 * that the device does not check (a violation would read out of bounds).
 * All pointers are HOST pointers (copies of the device arrays).
 * offsets [G+1]: offsets[0] == 0, non-decreasing, offsets[G] == total_rows.
 * gather [total_rows] (nullable): every index in [0, src_rows).
 * Returns NVFP4_OK, NVFP4_ERR_NULL (offsets NULL) or NVFP4_ERR_SHAPE (the
 * first violated rule).  Reads only; no device work. */
int nvfp4_check_groups(const int32_t* offsets, int64_t G, int64_t total_rows,
                       const int32_t* gather, int64_t src_rows);

#define NVFP4_GEMM_SKIP_INACTIVE_BLOCKS 1
/* Per-expert RAC: a_tscale and r_tscale are [G] (group g's tensor scales) and
 * kblock_active is [G, K/16], as nvfp4_quantize_grouped and
 * rac_select_residual_grouped write them. */
#define NVFP4_GEMM_PER_GROUP_SCALES 2

size_t w4a4_grouped_gemm_rac_workspace_size(const w4a4_gemm_args_t* args);
int w4a4_grouped_gemm_rac(const w4a4_gemm_args_t* args, void* ws, size_t ws_bytes,
                          void* stream);

/* ------------------------------------------------------------------------
 * Trainer-side weight fake-quantization (Asymmetric QAT).  The trainer
 * fake-quantizes its weights, and only its weights, with the rollout's own
 * NVFP4 quantize-dequantize path, so the two sides see the same weight error
 * (blog post, section "Two fixes, on two different sides"; arXiv abstract:
 * weights align through a shared quantization-dequantization path).
 *
 * nvfp4_qdq: runs the quantizer of nvfp4_quantize (same kernel, same
 * arithmetic, tensor scale from max|x| or from amax_in) and stores, instead of
 * codes and scales, the dequantized values v = RN32(RN32(g s_b) s_t) -- the
 * exact product g s_b s_t rounded once -- to out [rows, K] (row stride K):
 * FP32 for out_dtype NVFP4_IN_F32, bf16 (nearest even of v) for
 * NVFP4_IN_BF16.  *tensor_scale receives s_t.  Workspace as
 * nvfp4_quantize (none with amax_in).  Requires K % 16 == 0, x and out
 * 16-byte aligned, ldx % 16 == 0 (elements), as nvfp4_quantize.
 *
 * nvfp4_dequantize: the same values from stored codes [rows, K/2], scales
 * [rows, K/16] and tensor scale; nvfp4_qdq(x) equals
 * nvfp4_dequantize(nvfp4_quantize(x)) bit for bit.  Requires K % 16 == 0,
 * codes 8-byte aligned, out 16-byte aligned.  No workspace.
 * ------------------------------------------------------------------------ */
size_t nvfp4_qdq_workspace_size(int64_t rows, int64_t K);
int nvfp4_qdq(const void* x, int in_dtype, int64_t rows, int64_t K, int64_t ldx,
              const float* amax_in, int out_dtype, void* out, float* tensor_scale, void* ws,
              size_t ws_bytes, void* stream);
int nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                     int64_t rows, int64_t K, int out_dtype, void* out, void* stream);

/* ------------------------------------------------------------------------
 * FP8 (E4M3) W8A8 comparator.  The pages measure QUADS against FP8 rollout
 * (arXiv abstract on the mlsanity page; blog post, section "What it buys")
 * without saying how the FP8 engine scales its tensors; these calls
 * implement one FP32 scale per activation row (token) and per weight output
 * channel, so that a QUADS step can be timed beside an FP8 step on the same
 * workload.
 *
 * fp8_quantize_rows: for each row of x [rows, K] (FP32 or bf16, row-major):
 *   s = RN32(amax_row / 448)   (double quotient rounded once; 0 for a zero row)
 *   r = RN32(1 / s)            (0 when s == 0)
 *   codes[row, k] = E4M3(RN32(x r)): OCP E4M3 (bias 7, max 448), nearest
 *   even, saturating at +-448, sign bit from the product (so -0 may occur).
 * codes is uint8 [rows, K]; row_scales is float [rows].  Requires K % 16 == 0,
 * x 16-byte aligned, codes 8-byte aligned.
 * ------------------------------------------------------------------------ */
int fp8_quantize_rows(const void* x, int in_dtype, int64_t rows, int64_t K, uint8_t* codes,
                      float* row_scales, void* stream);

/* fp8_grouped_gemm: grouped (per-expert) FP8 GEMM with the grouping, gather
 * and epilogues of w4a4_grouped_gemm_rac:
 *   y[j, n] = a_scales[src] * w_scales[g*N + n] * sum_k A[src,k] W_g[n,k]
 * with A, W the E4M3 values (products exact, FP32 accumulation).  Epilogue
 * SILU_MUL_BF16 writes h[j, i] = bf16(silu(y[j, i]) * y[j, I + i]) to out
 * [total_rows, I] (no amax: the FP8 quantizer scales per row); epilogue
 * BF16 writes bf16(y) to out [total_rows, N] (the output type of the vendor
 * FP8 GEMM it is compared with).  Requires
 * K % 128 == 0, N % 128 == 0, codes 16-byte aligned, scales 4-byte aligned.
 * No workspace. */
typedef struct {
  int64_t num_groups;           /* G >= 1 */
  int64_t N;                    /* output columns (2I for SILU_MUL) */
  int64_t K;                    /* contraction length */
  int64_t total_rows;           /* rows of the grouped output */
  const int32_t* group_offsets; /* [G+1], ascending, [0] = 0, [G] = total_rows */
  const int32_t* gather_rows;   /* [total_rows] or NULL (identity) */
  const uint8_t* a_codes;       /* [src_rows, K] E4M3 */
  const float* a_scales;        /* [src_rows] */
  const uint8_t* w_codes;       /* [G, N, K] E4M3 */
  const float* w_scales;        /* [G, N] */
  int64_t epilogue;             /* nvfp4_epilogue_t */
  void* out;                    /* float or bf16 [total_rows, N], or bf16 [total_rows, N/2] */
} fp8_gemm_args_t;

int fp8_grouped_gemm(const fp8_gemm_args_t* args, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4RAC_H */
