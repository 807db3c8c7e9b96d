/*
 * sbl.h -- C ABI of the Sparse-BitLinear library for AMD MI355X (gfx950).
 *
 * Sparse-BitLinear is the layer of Sparse-BitNet that replaces every linear
 * layer: a BF16 master weight W [d_out, d_in] is quantized to ternary codes
 * {-1, 0, +1} with the absmean scale gamma, masked to N kept slots in every
 * group of 8 consecutive d_in positions (top-N by |W| of the master weight),
 * and multiplied with per-token absmax int8 activations.  The backward pass is
 * the Dual straight-through estimator: dW flows densely to every master
 * weight, masked ones included, and dX goes through the effective weight.
 *
 * Sources, cited by page and section:
 *   [SUM]  "Sparse-BitNet: 1.58-bit LLMs are Naturally Friendly to
 *          Semi-Structured Sparsity" -- structured summary of arXiv
 *          2603.05168 (paper.rainbus.top).  Sections: 前置知识 (prerequisites)
 *          > "1.58-bit BitNet 量化", "半结构化 N:M 稀疏",
 *          "Straight-Through Estimator (STE)"; 核心方法 (core method);
 *          方法步骤详情 (method steps).
 *   [GIST] gist.science summary of arXiv 2603.05168, section
 *          "2.2 Sparse-BitNet 框架".
 *   [EXPL] "什麼是 Sparse-BitNet？核心概念一次搞懂" (openclaw-pages), section
 *          "1.58 位元量化的技術原理" (ternary threshold form).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (memory on the current HIP
 *     device) unless stated otherwise; all tensors are dense row-major.
 *     bfloat16 values are passed as their uint16 bit patterns.
 *   - The caller owns every buffer.  The library never allocates or frees
 *     device memory; scratch space is a caller-provided workspace.
 *   - `hip_stream` is a hipStream_t passed as void*; NULL means the default
 *     stream.  Every call only enqueues work on that stream and returns
 *     without synchronizing.  gamma and absmax stay in device memory and are
 *     read by later calls in stream order.
 *   - Every function returns an sbl_status.  Arguments are validated on the
 *     host before anything is enqueued, so an error return means no work was
 *     enqueued.  A HIP launch failure returns SBL_ERR_HIP with detail text in
 *     sbl_last_error().  Faults inside kernels surface at the caller's next
 *     synchronization, as with any HIP work.
 *   - Inputs must be finite; non-finite inputs give unspecified results.
 *   - All outputs are bitwise deterministic: no floating-point atomics, and
 *     every reduction runs in a fixed order.
 *   - Device pointers must be 16-byte aligned, except absmax/gamma (4-byte).
 *   - Calls on different streams that write the same buffers race; ordering
 *     across streams is the caller's job.
 */
#ifndef SBL_H_
#define SBL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define SBL_API __attribute__((visibility("default")))
#else
#define SBL_API
#endif

typedef enum {
  SBL_OK = 0,
  SBL_ERR_INVALID_ARG = -1, /* NULL or misaligned pointer, unknown dtype/flag */
  SBL_ERR_SHAPE = -2,       /* a size outside the supported range           */
  SBL_ERR_UNSUPPORTED = -3, /* a valid but unimplemented option (e.g. n_keep) */
  SBL_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than required      */
  SBL_ERR_HIP = -5          /* a HIP runtime call failed                    */
} sbl_status;

typedef enum {
  SBL_F32 = 0,  /* float32                                    */
  SBL_BF16 = 1, /* bfloat16 (round to nearest even)           */
  SBL_I32 = 2   /* raw int32 accumulators (sbl_forward only)  */
} sbl_dtype;

/* sbl_backward flags: which gradients to compute. */
enum { SBL_BWD_DX = 1, SBL_BWD_DW = 2 };

/* Weight planes the decode-size forward reads (sbl_forward_plane_multi). */
enum { SBL_PLANE_CODES = 0, SBL_PLANE_PAIRS = 1 };

/* Size limits checked by every entry point. */
#define SBL_MAX_DIM ((int64_t)1 << 21)      /* d_in, d_out, T each <= 2,097,152 */
#define SBL_MAX_WEIGHTS ((int64_t)1 << 36)  /* d_out * d_in                       */

/* ------------------------------------------------------------------------ */
/* Weight side: gamma, N:8 mask, ternary codes                               */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace sbl_quant_mask_pack needs for a [d_out, d_in] weight.
 * Returns 0 for shapes sbl_quant_mask_pack would reject. */
SBL_API size_t sbl_quant_mask_pack_workspace_size(int64_t d_out, int64_t d_in);

/* Quant-then-mask of a BF16 master weight ([SUM] 核心方法 (i)-(iii);
 * 方法步骤详情 steps (2), (4), (5); [GIST] 2.2):
 *
 *   gamma  = mean |W| over the full, unmasked matrix ([SUM] 前置知识 >
 *            1.58-bit BitNet 量化), as the correctly rounded (nearest-even)
 *            float32 of the exact mean, so it is independent of summation
 *            order;
 *   mask   = in every group of 8 consecutive d_in positions, keep the n_keep
 *            slots of largest |W| (bf16 magnitude; ties to the lower index)
 *            ([SUM] 前置知识 > 半结构化 N:M 稀疏; 核心方法 (i));
 *   W_q    = RoundClip(W/gamma, -1, 1) = sign(W) if |W| > gamma/2 else 0
 *            (tie goes to 0; [EXPL] threshold form);
 *   W_eff  = W_q * mask.
 *
 * W_bf16 : [d_out, d_in] bf16 bits.           d_in % 8 == 0, d_in >= 8.
 * n_keep : N of N:8, 1 <= N <= 8.             d_out >= 1.
 * codes  : [d_out, d_in/8] uint16 code plane.  Slot j (d_in position 8g+j)
 *          of group g sits at bits 2j..2j+1: 00 = 0, 01 = +1, 11 = -1 (10 is
 *          never written).  Masked slots hold 00.
 * mask   : [d_out, d_in/8] uint8 mask plane, bit j = slot j kept.  May be
 *          NULL when the caller does not need it.
 * gamma  : one float32 in device memory.
 * workspace: at least sbl_quant_mask_pack_workspace_size(d_out, d_in) bytes,
 *          device memory; contents need no initialization and are clobbered.
 */
SBL_API int sbl_quant_mask_pack(const uint16_t* W_bf16, int64_t d_out, int64_t d_in, int n_keep,
                                uint16_t* codes, uint8_t* mask, float* gamma, void* workspace,
                                size_t workspace_bytes, void* hip_stream);

/* sbl_quant_mask_pack without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * sbl_quant_mask_pack with n_keep 1..8 (N:8); it calls no allocator.
 *
 * Its scratch (the partial sums of the gamma reduction) is a static device
 * array of sbl_quant_mask_pack_noalloc_scratch_bytes() bytes (2,129,920: the
 * reduction never launches more than 1024 blocks, so every shape accepted by
 * sbl_quant_mask_pack fits; a larger need returns SBL_ERR_WORKSPACE).  Each
 * GPU holds one copy until the process ends, located on that GPU's first
 * call.  All calls on one GPU share it and it keeps the last call's contents
 * (no clearing is needed: each call writes what it reads), so calls that
 * overlap on one GPU (concurrent streams or host threads) race: serialize
 * them.
 */
SBL_API int sbl_quant_mask_pack_noalloc(const uint16_t* W_bf16, int64_t d_out, int64_t d_in, int n_keep,
                                        uint16_t* codes, uint8_t* mask, float* gamma, void* hip_stream);
SBL_API size_t sbl_quant_mask_pack_noalloc_scratch_bytes(void);

/* sbl_quant_mask_pack_nm flags. */
enum { SBL_MASK_FROM_QUANTIZED = 1 };

/* sbl_quant_mask_pack with the mask pattern and the mask source chosen:
 *
 *   m_group : M of N:M, 8 or 4 ([SUM] 前置知识 > 半结构化 N:M 稀疏 names 2:4 as
 *             the hardware pattern and 6:8 as the one studied; 方法步骤详情
 *             compares the two).  M = 4 keeps n_keep of every 4 consecutive
 *             d_in positions; the planes keep their 8-slot words (two mask
 *             groups per word), so every other entry point takes them as is.
 *   n_keep  : 1 <= n_keep <= m_group (the N:8 sweep of [GIST] 4.1 runs 8:8 to 2:8).
 *   flags   : 0, or SBL_MASK_FROM_QUANTIZED for the ablation of [GIST] 4.3 消融实验
 *             ("mask from quantized weight", which the pages report as
 *             unstable): the mask ranks |W_q| in {0, 1} instead of |W|, ties
 *             to the lower index as in the main rule, so a group keeps its
 *             non-zero ternary slots in index order, then zero slots.
 *
 * Everything else (gamma, codes, planes, workspace, errors) as for
 * sbl_quant_mask_pack, which is this call with m_group = 8 and flags = 0.
 * Unsupported (n_keep, m_group) return SBL_ERR_UNSUPPORTED; unknown flag bits
 * SBL_ERR_INVALID_ARG.
 */
SBL_API int sbl_quant_mask_pack_nm(const uint16_t* W_bf16, int64_t d_out, int64_t d_in, int n_keep, int m_group,
                                   int flags, uint16_t* codes, uint8_t* mask, float* gamma, void* workspace,
                                   size_t workspace_bytes, void* hip_stream);

/* sbl_quant_mask_pack_nm for several matrices at once (a layer's linears):
 * the same results, bit for bit, as one call per matrix, in three launches in
 * all instead of three per matrix.
 *
 * items : HOST array of `count` descriptors, 1 <= count <= SBL_PACK_BATCH_MAX;
 *         each as the arguments of the single call (W, d_out, d_in, codes,
 *         mask or NULL, gamma).  Matrices must not overlap.
 * n_keep, m_group, flags : as sbl_quant_mask_pack_nm, for every matrix.
 * workspace : sbl_quant_mask_pack_batch_workspace_size(count, items) bytes.
 */
#define SBL_PACK_BATCH_MAX 16
typedef struct {
  const uint16_t* W_bf16;
  int64_t d_out, d_in;
  uint16_t* codes;
  uint8_t* mask;
  float* gamma;
} sbl_pack_item;

SBL_API size_t sbl_quant_mask_pack_batch_workspace_size(int count, const sbl_pack_item* items);
SBL_API int sbl_quant_mask_pack_batch(int count, const sbl_pack_item* items, int n_keep, int m_group, int flags,
                                      void* workspace, size_t workspace_bytes, void* hip_stream);

/* "Mask without grad" ablation ([SUM] 核心方法, second design point; 4.3
 * 消融实验 of [GIST]): the gradient of masked master weights is dropped, i.e. applied
 * after sbl_backward, dW[o, i] = +0 wherever bit (i % 8) of mask[o, i / 8] is
 * clear; kept entries are unchanged.  In place.
 *
 * dW   : [d_out, d_in] float32, 16-byte aligned.  d_in % 8 == 0.
 * mask : [d_out, d_in/8] mask plane from sbl_quant_mask_pack(_nm).
 */
SBL_API int sbl_mask_grad(float* dW, const uint8_t* mask, int64_t d_out, int64_t d_in, void* hip_stream);

/* Optimizer step followed by the next step's packing ([SUM] 方法步骤详情 step
 * (8): AdamW updates the master weight, with beta = (0.9, 0.95), eps = 1e-5,
 * weight decay 0.1 and gradient clipping at 1.0; step (2) of the next step
 * recomputes the mask from the new W; the mask flip count is the training
 * diagnostic behind the masks-recomputed-every-step design of 核心方法).
 *
 * In place on W, m, v, one read of each:
 *   g      = dW * grad_scale        (grad_scale: the caller's global-norm clip
 *                                    factor, min(1, clip / ||g||) over every
 *                                    parameter, which no single layer sees)
 *   m'     = beta1 m + (1 - beta1) g,   v' = beta2 v + (1 - beta2) g^2
 *   W'     = W (1 - lr wd) - (lr / (1 - beta1^t)) m' / (sqrt(v') / sqrt(1 - beta2^t) + eps)
 *            in float32 (the form of torch.optim.AdamW), rounded once to bf16;
 * then, from W', what sbl_quant_mask_pack_nm(W', n_keep, m_group, 0) returns
 * (gamma, codes, mask plane; bit-identical to calling it on W'), and the
 * number of slots whose mask bit differs from mask_prev.
 *
 * W_bf16      : [d_out, d_in] bf16, updated.        d_in % 8 == 0.
 * dW          : [d_out, d_in] float32 gradient (sbl_backward's dW).
 * m, v        : [d_out, d_in] float32 AdamW moments, updated (zeros at t = 1).
 * hp          : HOST pointer; step t >= 1, 0 <= beta < 1, eps > 0, lr >= 0,
 *               weight_decay >= 0, grad_scale >= 0, all finite.
 * mask_prev   : the previous mask plane, or NULL (then no flip count).  May
 *               equal mask (each byte is read before it is overwritten).
 * mask        : [d_out, d_in/8] new mask plane (required).
 * codes, gamma: as sbl_quant_mask_pack.
 * flips       : one uint64 in device memory, written when mask_prev is given;
 *               may be NULL.
 * workspace   : sbl_adamw_repack_workspace_size(d_out, d_in) bytes.
 * All 16-byte aligned except gamma, flips (4 / 8) and the mask planes.
 */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay, grad_scale;
  int64_t step;
} sbl_adamw_params;

SBL_API size_t sbl_adamw_repack_workspace_size(int64_t d_out, int64_t d_in);
SBL_API int sbl_adamw_repack(uint16_t* W_bf16, const float* dW, float* m, float* v, int64_t d_out, int64_t d_in,
                             const sbl_adamw_params* hp, int n_keep, int m_group, const uint8_t* mask_prev,
                             uint8_t* mask, uint16_t* codes, float* gamma, uint64_t* flips, void* workspace,
                             size_t workspace_bytes, void* hip_stream);

/* ------------------------------------------------------------------------ */
/* Activation side                                                            */
/* ------------------------------------------------------------------------ */

/* Per-token absmax 8-bit quantization ([SUM] 前置知识 > 1.58-bit BitNet 量化,
 * last sentence; 方法步骤详情 step (3)):
 *
 *   absmax[t] = max_i |x[t, i]|;
 *   x_q[t, i] = round-half-even(127 * x[t, i] / absmax[t])  (|x_q| <= 127),
 *   a zero row gives x_q = 0 and absmax = 0.
 *
 * x_bf16 : [T, d_in] bf16 bits.  T >= 0 (T = 0 is a no-op), d_in % 8 == 0.
 * x_q    : [T, d_in] int8.
 * absmax : [T] float32 (the exact bf16 value of the row maximum).
 */
SBL_API int sbl_act_quant(const uint16_t* x_bf16, int64_t T, int64_t d_in, int8_t* x_q, float* absmax,
                          void* hip_stream);

/* Q_a(Norm(x)) in one pass ([SUM] 方法步骤详情 step (3)): RMSNorm of each row,
 * rounded to bf16, then the activation quantization of sbl_act_quant on it.
 *
 *   ms     = RN32(sum_i x[t, i]^2 / d_in)      (the exact mean, rounded once)
 *   r      = RN32(1 / sqrt(RN32(ms + eps)))   (correctly rounded)
 *   y      = bf16(RN32(RN32(x * r) * g))
 *   absmax, x_q as sbl_act_quant(y).
 *
 * The pages name Norm(x) without its kind; RMSNorm with a bf16 weight g is
 * the reading.  Each step is one correctly rounded binary32 operation on an
 * exact value (RN32: nearest, ties to even), so the result does not depend on
 * any summation order and x_q is reproducible bit for bit.  A row whose mean
 * square overflows binary32 gives r = 0 and y = 0.
 *
 * x_bf16 : [T, d_in] bf16 bits.   d_in % 8 == 0, d_in <= 16384 (else
 *          SBL_ERR_UNSUPPORTED).
 * g_bf16 : [d_in] bf16 weight, or NULL for ones.
 * eps    : > 0, finite (else SBL_ERR_INVALID_ARG).
 * x_q, absmax : as sbl_act_quant.
 * rstd   : [T] float32, r of each row (what the norm's backward needs), or
 *          NULL.
 * T = 0 is a no-op.  Outputs are defined while y stays finite.
 */
SBL_API int sbl_rmsnorm_act_quant(const uint16_t* x_bf16, const uint16_t* g_bf16, float eps, int64_t T, int64_t d_in,
                                  int8_t* x_q, float* absmax, float* rstd, void* hip_stream);

/* ------------------------------------------------------------------------ */
/* Forward                                                                    */
/* ------------------------------------------------------------------------ */

/* Forward product ([SUM] 前置知识 > 半结构化 N:M 稀疏: y = (W (.) M) x;
 * 方法步骤详情 step (6): y ~= s * W_eff x~, s absorbing the scales):
 *
 *   acc[t, o] = sum_i x_q[t, i] * W_eff[o, i]        (exact int32)
 *   y[t, o]   = acc[t, o] * gamma * absmax[t] / 127
 *
 * codes, gamma : from sbl_quant_mask_pack for W [d_out, d_in].
 * x_q, absmax  : from sbl_act_quant, [T, d_in] and [T].
 * y            : [T, d_out] of y_dtype: SBL_F32, SBL_BF16, or SBL_I32 (acc).
 * T = 0 is a no-op.  Decode-sized T (T <= 64, d_in % 64 == 0) uses a kernel
 * that streams the code plane once with a split K range per block; larger T
 * uses tiled int8 matrix-core kernels.  All paths compute the same exact
 * int32 sums, so the results are identical.
 */
SBL_API int sbl_forward(const uint16_t* codes, const float* gamma, const int8_t* x_q, const float* absmax,
                        int64_t T, int64_t d_in, int64_t d_out, void* y, int y_dtype, void* hip_stream);

/* Decode step: sbl_act_quant followed by sbl_forward in one launch, for
 * decode-sized token counts ([SUM] Table 3, decode rows: the activation
 * quantization and the product of one generated token batch).
 *
 *   absmax[t] = max_i |x[t, i]|,  x_q = round-half-even(127 x / absmax[t]),
 *   y[t, o]   = (sum_i x_q[t, i] W_eff[o, i]) * gamma * absmax[t] / 127,
 *
 * with x_q, absmax and the int32 sums bit-identical to the two-call path
 * (the quantization runs the same arithmetic), so y is too.  x_q and absmax
 * are not written.
 *
 * codes, gamma : from sbl_quant_mask_pack for W [d_out, d_in].
 * x_bf16       : [T, d_in] bf16 bits.
 * y            : [T, d_out] of y_dtype: SBL_F32, SBL_BF16 or SBL_I32.
 * Supported (sbl_decode_supported): 1 <= T <= 16, d_in % 64 == 0,
 * T * d_in <= 65536 and T * (d_in + 16) <= 56832 (the int8 tile each block
 * keeps in LDS); other shapes return SBL_ERR_UNSUPPORTED and enqueue nothing
 * (use sbl_act_quant + sbl_forward).  T = 0 is a no-op.
 * Cost: each resident block quantizes the T rows once for all the output
 * rows it walks, a few blocks per compute unit, which is cheaper than the
 * launch and the memory round trip of a separate quantization.
 */
SBL_API int sbl_decode(const uint16_t* codes, const float* gamma, const uint16_t* x_bf16, int64_t T, int64_t d_in,
                       int64_t d_out, void* y, int y_dtype, void* hip_stream);

/* 1 if sbl_decode takes this (T, d_in), else 0. */
SBL_API int sbl_decode_supported(int64_t T, int64_t d_in);

/* Decode of several matrices that read the same activations, in one launch:
 * a layer's q, k and v projections (one normed hidden state), or gate and up
 * ([SUM] Table 3, decode rows: every linear of the decoder layer runs per
 * generated token batch).  Each item is one matrix of the same d_in:
 *
 *   y_i[t, o] = (sum_k x_q[t, k] W_eff,i[o, k]) * gamma_i * absmax[t] / 127
 *
 * bit-identical to one sbl_decode (sbl_decode_multi, x as bf16, the
 * activation quantization fused in; sbl_decode_supported(T, d_in) must hold)
 * or one sbl_forward (sbl_forward_decode_multi, x_q and absmax from
 * sbl_act_quant; 0 <= T <= 64 and d_in % 64 == 0) per item.  Blocks of 16
 * output rows of every item share the launch, so the fixed cost of a launch
 * (several us at these sizes) is paid once per group instead of per matrix.
 *
 * items : HOST array of `count` descriptors, 1 <= count <= SBL_DECODE_MULTI_MAX;
 *         codes and gamma as from sbl_quant_mask_pack for W_i [d_out, d_in];
 *         y [T, d_out] of y_dtype (SBL_F32, SBL_BF16 or SBL_I32); codes and y
 *         16-byte aligned, gamma 4-byte aligned.
 * Errors: SBL_ERR_INVALID_ARG (count, NULL or misaligned pointers, y_dtype),
 * SBL_ERR_SHAPE, SBL_ERR_UNSUPPORTED (T or d_in outside the range above);
 * nothing is enqueued then.  T = 0 is a no-op.
 */
#define SBL_DECODE_MULTI_MAX 4
typedef struct sbl_decode_item {
  const uint16_t* codes;
  const float* gamma;
  int64_t d_out;
  void* y;
} sbl_decode_item;

SBL_API int sbl_decode_multi(int count, const sbl_decode_item* items, const uint16_t* x_bf16, int64_t T,
                             int64_t d_in, int y_dtype, void* hip_stream);
SBL_API int sbl_forward_decode_multi(int count, const sbl_decode_item* items, const int8_t* x_q, const float* absmax,
                                     int64_t T, int64_t d_in, int y_dtype, void* hip_stream);

/* Pair plane of a weight whose mask keeps at most 2 of every 8 (2:8, 1:8):
 * one byte per group of 8 instead of two, for decoding, which streams the
 * weights once per generated token batch ([SUM] Table 3 decode rows; the
 * packed format is precomputed once for inference).  Group g of row o gets
 *
 *   plane[o, g] = 9 * rank(p0, p1) + 3 * digit(v0) + digit(v1)   (< 252)
 *
 * where p0 < p1 are the positions (0..7) of its stored slots, rank their
 * index among the 28 pairs in lexicographic order, v0, v1 the ternary values
 * there and digit(0, +1, -1) = 0, 1, 2.  The stored slots are the group's
 * non-zeros, padded with zeros at the lowest free positions (one non-zero at
 * a: (0, a), or (0, 1) when a = 0; none: (0, 1)), so every group has one byte.
 *
 * codes : [d_out, d_in/8] code plane (sbl_quant_mask_pack with N <= 2).
 * plane : [d_out, d_in/8] uint8.
 * bad   : one uint64 in device memory or NULL; the number of groups with more
 *         than 2 non-zeros (their byte is written as 0 and the plane is then
 *         not valid) is ADDED to it, so the caller zeroes it first.
 * Pointers 16-byte aligned (bad: 8).  d_in % 8 == 0.
 */
SBL_API int sbl_pack_pairs(const uint16_t* codes, int64_t d_out, int64_t d_in, uint8_t* plane, uint64_t* bad,
                           void* hip_stream);

/* sbl_forward_decode_multi (x_q and absmax given) and sbl_decode_multi (x as
 * bf16, the activation quantization fused in: x_q = NULL, x_bf16 given,
 * absmax = NULL) on either weight plane: format SBL_PLANE_CODES (items[i].codes
 * is the code plane) or SBL_PLANE_PAIRS (items[i].codes points at the pair
 * plane of sbl_pack_pairs, uint8 [d_out, d_in/8]).  The int32 sums, hence y,
 * are identical for the two planes of one weight.
 * T <= 64 and d_in % 64 == 0 (codes) or % 128 == 0 (pairs); the fused form
 * takes what sbl_decode_supported accepts (pairs: d_in % 128 == 0 and
 * T * (d_in + 16) <= 54784; sbl_decode_plane_supported).  Otherwise
 * SBL_ERR_UNSUPPORTED.
 */
SBL_API int sbl_decode_plane_supported(int format, int64_t T, int64_t d_in); /* the fused form: 1 or 0 */
SBL_API int sbl_forward_plane_multi(int format, int count, const sbl_decode_item* items, const int8_t* x_q,
                                    const float* absmax, const uint16_t* x_bf16, int64_t T, int64_t d_in,
                                    int y_dtype, void* hip_stream);

/* Kept-only 2:4 operand plane for 2:8 and 2:4 masks, and the forward on it,
 * which runs on gfx950's sparse int8 matrix instruction (2 stored values of
 * every 4 k): half the matrix work of sbl_forward for the same result ([SUM]
 * 前置知识 > 半结构化 N:M 稀疏 names 2:4 the hardware pattern; [SUM] Table 3,
 * the sparse kernels' speed-ups).
 *
 * sbl_pack_sparse24: codes [d_out, d_in/8] (from sbl_quant_mask_pack(_nm) with
 * a 2:8, 2:4 or 1:4 pattern) -> plane uint8 [d_out, d_in/64, 16], the same size.
 * Per row and 64-wide step, for each half h (32 positions, 8 groups of 4): a
 * 32-bit word of 16 two-bit codes (slot 2 g + i = the i-th stored value of
 * group g) at bytes 4 h, and a 32-bit word of their positions (bits 4 g ..
 * 4 g + 3: first | second << 2, first < second) at bytes 8 + 4 h.  A group's
 * non-zeros are stored in position order, padded with zeros at the next free
 * positions.  Groups with more than 2 non-zeros (other patterns) cannot be
 * represented: their count is added to *bad (device uint64, may be NULL; the
 * caller zeroes it) and the plane is then not valid for sbl_forward_sparse24.
 * d_in % 64 == 0.
 *
 * sbl_forward_sparse24: as sbl_forward with the plane in place of the codes
 * (the same int32 sums, so the same y bit for bit).  d_in % 128 == 0.
 */
SBL_API int sbl_pack_sparse24(const uint16_t* codes, int64_t d_out, int64_t d_in, uint8_t* plane, uint64_t* bad,
                              void* hip_stream);
SBL_API int sbl_forward_sparse24(const uint8_t* plane, const float* gamma, const int8_t* x_q, const float* absmax,
                                 int64_t T, int64_t d_in, int64_t d_out, void* y, int y_dtype, void* hip_stream);

/* ------------------------------------------------------------------------ */
/* Backward (Dual STE)                                                        */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace sbl_backward needs for these flags.  It holds the
 * per-call operands of the matrix-core path, in private layouts: the code
 * plane transposed for the dX product (2 bits per weight, d_in rows of d_out
 * rounded up to 64); dY^T in bf16, run-major ([T8 / 8][d_out][8] with T8 = T
 * rounded up to 8), for the dW product: scaled to bf16(dY[t, o] absmax[t] /
 * 127) when that product reads x_q as it is (d_in % 16 == 0), else unscaled
 * next to x~ = bf16(x_q absmax / 127) in the same run-major form; and split-K
 * partial sums of dW (float32, one [d_out, d_in] slice per split).  With
 * SBL_BWD_DX | SBL_BWD_DW on shapes that take the matrix-core path for both,
 * the dX product writes dY^T while it runs and the dW product reads it;
 * otherwise dW makes it itself.  Shapes off the matrix-core path need at most
 * the split-K partials.  0 when nothing is needed (e.g. T = 0). */
SBL_API size_t sbl_backward_workspace_size(int64_t T, int64_t d_in, int64_t d_out, int flags);

/* Dual-STE backward ([SUM] 前置知识 > Straight-Through Estimator (STE);
 * 核心方法 (dense gradient flow); 方法步骤详情 step (7); [GIST] 2.2).  The
 * straight-through estimator replaces the ternary quantizer, the N:M
 * selector and the activation quantizer by the identity, so for the forward
 * y = x~ (gamma W_eff)^T with x~ = x_q * absmax / 127:
 *
 *   dX[t, i] = gamma * sum_o dY[t, o] * W_eff[o, i]      (flags & SBL_BWD_DX)
 *   dW[o, i] = sum_t dY[t, o] * x~[t, i]                 (flags & SBL_BWD_DW)
 *
 * dW is dense: every (o, i), masked positions included, gets its gradient.
 * Both products run on bf16 matrix cores with float32 accumulation (x~ is
 * rounded to bf16 once, W_eff in {-1,0,1} is exact in bf16).
 *
 * dY_bf16 : [T, d_out] bf16 bits.
 * dX      : [T, d_in] of dx_dtype (SBL_BF16 or SBL_F32); may be NULL without
 *           SBL_BWD_DX.
 * dW      : [d_out, d_in] float32; may be NULL without SBL_BWD_DW.  With
 *           T = 0, dW is set to zero.
 * workspace: at least sbl_backward_workspace_size(...) bytes for the same
 *           flags (may be NULL when that size is 0).  Asking for both
 *           gradients in one call costs less than two calls: dY is
 *           transposed once, by the dX product, for both.
 */
SBL_API int sbl_backward(const uint16_t* codes, const float* gamma, const int8_t* x_q, const float* absmax,
                         const uint16_t* dY_bf16, int64_t T, int64_t d_in, int64_t d_out, void* dX,
                         int dx_dtype, float* dW, int flags, void* workspace, size_t workspace_bytes,
                         void* hip_stream);

/* ------------------------------------------------------------------------ */
/* Status and test hooks                                                      */
/* ------------------------------------------------------------------------ */

/* Static English text for a status code. */
SBL_API const char* sbl_status_string(int status);

/* Detail of the last error on the calling thread (thread-local, static
 * storage valid until the next failing call on that thread). */
SBL_API const char* sbl_last_error(void);

/* Library version string. */
SBL_API const char* sbl_version(void);

/* HOST-side test hook for the exact gamma rounding that the device code uses
 * (the same function, compiled for the host).  S is an unsigned integer of
 * n_words little-endian 32-bit words holding sum|W| in units of 2^-133;
 * count = d_out * d_in.  Writes RN_float32(S * 2^-133 / count) to *out (host
 * pointer).  n_words <= 10. */
SBL_API int sbl_test_round_mean(const uint32_t* S_words, int n_words, int64_t count, float* out);

/* ------------------------------------------------------------------------ */
/* Measurement helpers (not part of the operator)                            */
/* ------------------------------------------------------------------------ */

/* The matrix instruction the operator uses, on register operands only, so
 * that its rate can be read against a measured ceiling beside the datasheet
 * one: kind 0 = int8 32x32x32 (forward), 1 = bf16 32x32x16 (backward).
 * blocks x 4 waves each issue 4 independent chains of iters instructions:
 * blocks * 4 * 4 * iters instructions of 65,536 (int8) or 32,768 (bf16)
 * operations.  sink: [blocks] float32, device memory, never read back.
 */
SBL_API int sbl_peak_mfma(int kind, int64_t iters, int blocks, float* sink, void* hip_stream);

/* A streaming read of `bytes` bytes at `src` (device, 16-byte aligned, a
 * multiple of 16), four 16-byte loads in flight per lane; sink: one uint32.
 */
SBL_API int sbl_peak_read(const void* src, int64_t bytes, uint32_t* sink, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SBL_H_ */
