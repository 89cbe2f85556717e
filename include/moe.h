/*
 * moe.h — C ABI of the single-GPU Mixture-of-Experts layer for MI355X (gfx950).
 *
 * The layer, as the Tutel and DeepSpeed-MoE pages describe it:
 *   1. gate: per token, softmax over E gate logits and the k largest experts
 *      (Tutel catalogue page, "key configuration": gate_type
 *      {'type': 'top', 'k': ..., 'capacity_factor': ...});
 *   2. capacity-bounded slots: each route's location is the count of earlier
 *      routes to the same expert; capacity C follows capacity_factor (catalogue
 *      page FAQ: positive = fixed factor X, 0 = max needed volume, negative =
 *      min(-X, max needed); MoE training blog, part 3 section 3.5, "dynamic
 *      capacity factor"); routes at or beyond C are dropped;
 *   3. fast encode: tokens are copied into a flat [E*C, M] expert buffer by
 *      index (blog part 3 section 3.5 "fast encode/decode"; DeepSpeed PR #8195
 *      sections 2 and 3);
 *   4. expert FFN: fc1 + bias, activation, fc2 + bias per expert (catalogue
 *      page: experts {'type': 'ffn', hidden size per expert, has_fc1_bias,
 *      has_fc2_bias}, biases default on);
 *   5. fast decode: out[s] = sum of gate * expert output over the token's kept
 *      routes, accumulated in fp32 (DeepSpeed PR #8195 section 3).
 * The backward covers decode (gate-weighted scatter of dout and the gate
 * gradient, kernels K1/K2 of blog part 3 section 3.5), the expert FFN (data
 * and fp32 weight/bias gradients), encode (gather-sum, kernel K0) and the
 * gate itself: the softmax's gradient, the auxiliary load-balance loss (blog
 * part 2 section 2.1) and the gate projection's weight and input gradients.
 *
 * Conventions shared by every call:
 *  - Pointers named *_host are host memory; every other pointer is device
 *    memory allocated and owned by the caller. The library allocates nothing
 *    and keeps no state between calls; calls on different streams may overlap.
 *  - `stream` is a hipStream_t (NULL = the null stream). Device work is only
 *    enqueued; no call waits for the device.
 *  - Every device pointer is 16-byte aligned (checked: MOE_EINVAL); the
 *    kernels move rows as 16-byte vectors.
 *  - Data-type tensors (x, W1, b1, W2, b2, buf, pre, h, y, out, dout, dx, dy,
 *    dpre, dbuf, and Residual-MoE's W1r, b1r, W2r, b2r, pre_r, h_r, y_r,
 *    dpre_r, dx_r) are fp32 or bf16 as moe_shape.dtype says. logits, Wg,
 *    gates, dgates, dlogits, the auxiliary loss, the weight/bias gradients and
 *    the block-FP8 scales are fp32; MX and block-FP8 codes and MX scales are
 *    bytes. Index tables are int32.
 *  - Route tables are route-major [k, S]: entry r*S + s is route r of token s,
 *    r = 0 the largest gate.
 *  - The capacity C is computed on the device and written to capacity[0];
 *    later calls read it there. Row e*C + j of a flat [E*C, *] buffer is slot j
 *    of expert e. Buffers sized with the host bound cmax (moe_capacity_bound)
 *    always hold E*C rows.
 *  - Errors: arguments are checked before anything is enqueued; a failing
 *    check returns MOE_EINVAL, MOE_EUNSUPPORTED or MOE_EWORKSPACE and enqueues
 *    nothing. A failed launch returns MOE_EHIP. moe_last_error() gives the
 *    message of the last failure on the calling thread. Device faults surface
 *    at the caller's next synchronisation.
 *  - Preconditions not checked: logits are finite; device buffers have the
 *    sizes stated below; buffers that are written do not overlap inputs
 *    unless a call says so.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_EINVAL = -1,       /* bad argument: null pointer, size out of range */
    MOE_EUNSUPPORTED = -2, /* valid layer, but outside what the kernels support */
    MOE_EWORKSPACE = -3,   /* workspace smaller than moe_workspace_size() */
    MOE_EHIP = -4          /* a HIP runtime call or launch failed */
} moe_status;

enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1 };
enum { MOE_ACT_RELU = 0, MOE_ACT_GELU = 1 };
enum { MOE_MX_FP8 = 0, MOE_MX_FP4 = 1 };

/* The layer's sizes and options (Tutel catalogue page, "key configuration":
 * model_dim = M, number of experts = E, gate k and capacity_factor,
 * hidden_size_per_expert = H, has_fc1_bias / has_fc2_bias).
 * Supported: S >= 0; 1 <= k <= min(E, 32); E <= 512; M and H multiples of 64;
 * dtype MOE_DT_F32 or MOE_DT_BF16; act MOE_ACT_RELU (max(0,v)) or
 * MOE_ACT_GELU (0.5 v (1 + erf(v / sqrt 2))); capacity_factor finite. */
typedef struct moe_shape {
    int32_t S;   /* tokens */
    int32_t M;   /* model dim */
    int32_t E;   /* experts */
    int32_t k;   /* experts per token */
    int32_t H;   /* hidden size per expert */
    double capacity_factor;
    int32_t dtype;
    int32_t act;
    int32_t has_fc1_bias;
    int32_t has_fc2_bias;
} moe_shape;

/* Checks a shape on the host (no GPU needed). */
moe_status moe_validate(const moe_shape *shape);

/* Host upper bound of C (no GPU needed): for capacity_factor f > 0 the capacity
 * itself, ceil(k*S*f/E); for f == 0, S; for f < 0, min(ceil(k*S*|f|/E), S);
 * never below 1. Size every [E*C, *] buffer with E * (*cmax_host) rows. */
moe_status moe_capacity_bound(const moe_shape *shape, int32_t *cmax_host);

/* Bytes of device workspace moe_route, moe_layer_forward, the gate backward
 * calls and moe_layer_backward (with the gate backward) need (no GPU needed).
 * One buffer of this size serves all of them on one stream; calls that may run
 * at the same time need workspaces of their own. */
moe_status moe_workspace_size(const moe_shape *shape, size_t *bytes_host);

/* Gate projection (Tutel catalogue page, "key configuration": the top-k gate
 * scores each token against E experts): logits[s][e] = sum_m x[s][m] * Wg[m][e]
 * in fp32, within the fp32 summation bound of the exact sum (gamma_M *
 * sum_m |x[s][m] Wg[m][e]|, gamma_n = n 2^-24 / (1 - n 2^-24)). The summation
 * order is fixed, so the logits (on which routing decisions are taken) are
 * reproducible bit for bit from run to run; routing itself is exact given them.
 * x [S, M] data type, Wg [M, E] fp32 row-major, logits [S, E] fp32. */
moe_status moe_gate_project(const moe_shape *shape, const void *x, const float *Wg, float *logits,
                            void *stream);

/* Routing (Tutel catalogue page FAQ on k and capacity_factor; DeepSpeed PR
 * #8195 section 1: per-route index, location and gate from the top-k, int32):
 *   idx[r][s]   expert of route r of token s: experts ordered by logit, larger
 *               first, equal logits (+0 == -0) by lower index first;
 *   gates[r][s] softmax probability of that expert over all E logits (computed
 *               in fp64, rounded to fp32), not renormalised;
 *   loc[r][s]   number of earlier routes, in route-major then token order, to
 *               the same expert; the route is kept iff loc < C;
 *   needed[e]   routes to expert e;  capacity[0] = C;  fill[e] = min(needed, C);
 *   slot_route  (may be NULL) [E * cmax]: row e*C + loc gets r*S + s for every
 *               kept route; rows at or beyond fill[e] are not written.
 * logits [S, E] fp32; idx, loc [k, S] int32; gates [k, S] fp32; needed, fill [E]
 * int32; capacity [1] int32; ws: moe_workspace_size() bytes. */
moe_status moe_route(const moe_shape *shape, const float *logits, int32_t *idx, int32_t *loc,
                     float *gates, int32_t *needed, int32_t *fill, int32_t *capacity,
                     int32_t *slot_route, void *ws, size_t ws_bytes, void *stream);

/* Fast encode (blog part 3 section 3.5, "Encode"; DeepSpeed PR #8195 section 2,
 * the flat [e*c, m] buffer): buf[idx*C + loc] = x[s] (a bit copy) for every kept
 * route; every other row e*C + j with j < C is set to +0.
 * x [S, M]; buf [E * cmax, M]; the first E*C rows are written. */
moe_status moe_encode(const moe_shape *shape, const void *x, const int32_t *idx, const int32_t *loc,
                      const int32_t *fill, const int32_t *capacity, void *buf, void *stream);

/* Expert FFN (Tutel catalogue page, experts 'ffn'; blog part 3 section 3.5,
 * expert batch matrix multiply on the per-expert [E, C, M] layout), for the
 * filled rows j < fill[e] of each expert e:
 *   pre = buf[e*C+j] . W1[e]^T + b1[e]   (fp32 accumulation)
 *   h   = act(pre)                        stored in the data type
 *   y   = h . W2[e]^T + b2[e]             (fp32 accumulation), stored
 * W1 [E, H, M], b1 [E, H] (NULL iff !has_fc1_bias), W2 [E, M, H], b2 [E, M]
 * (NULL iff !has_fc2_bias); buf, y [E*cmax, M]; h, pre [E*cmax, H]; pre may be
 * NULL (it is needed by moe_layer_backward). Rows at or beyond fill[e] of
 * pre, h and y are not written. */
moe_status moe_expert_ffn(const moe_shape *shape, const void *buf, const void *W1, const void *b1,
                          const void *W2, const void *b2, const int32_t *fill,
                          const int32_t *capacity, void *pre, void *h, void *y, void *stream);

/* The two halves of moe_expert_ffn, for callers that schedule or time them
 * separately (same definitions, same row rules):
 *   moe_expert_fc1: pre = buf . W1[e]^T + b1[e]; h = act(pre)   (pre may be NULL)
 *   moe_expert_fc2: y = h . W2[e]^T + b2[e]                       */
moe_status moe_expert_fc1(const moe_shape *shape, const void *buf, const void *W1, const void *b1,
                          const int32_t *fill, const int32_t *capacity, void *pre, void *h, void *stream);
moe_status moe_expert_fc2(const moe_shape *shape, const void *h, const void *W2, const void *b2,
                          const int32_t *fill, const int32_t *capacity, void *y, void *stream);

/* moe_expert_ffn restricted to the capacity slots [slot_begin, slot_end) of
 * every expert: rows e*C + j with slot_begin <= j < min(fill[e], slot_end).
 * The rows of pre, h and y outside the window are left as they are. For
 * pipelining over the capacity dimension (MoE training blog, part 3 section
 * 3.4, adaptive pipelining: the capacity is cut into d chunks whose expert
 * computation runs as separate launches, here on caller streams; windows that
 * partition [0, cmax) compute exactly moe_expert_ffn). bf16 data only. */
moe_status moe_expert_ffn_window(const moe_shape *shape, const void *buf, const void *W1, const void *b1,
                                 const void *W2, const void *b2, const int32_t *fill,
                                 const int32_t *capacity, int32_t slot_begin, int32_t slot_end, void *pre,
                                 void *h, void *y, void *stream);

/* Fast decode (blog part 3 section 3.5, "Decode"; DeepSpeed PR #8195 section 3,
 * combine accumulated in fp32): out[s] = sum over kept routes r = 0..k-1, in
 * order, of gates[r][s] * y[idx*C + loc], accumulated in fp32 from +0 with
 * separately rounded multiply and add, then stored in the data type. A token
 * whose routes were all dropped gets 0. y [E*cmax, M]; out [S, M]. */
moe_status moe_decode(const moe_shape *shape, const void *y, const float *gates, const int32_t *idx,
                      const int32_t *loc, const int32_t *capacity, void *out, void *stream);

/* MX low-precision experts (Tutel catalogue page and its project summaries:
 * FP8 / MXFP4 quantised inference). Format: OCP Microscaling
 * (MX) -- 32 consecutive values along a row share one E8M0 scale byte b
 * (2^(b - 127)); elements are E4M3 (MOE_MX_FP8: one byte each, max 448) or
 * E2M1 (MOE_MX_FP4: two per byte, the even index in the low nibble, max 6).
 * Quantisation: e = floor(log2 max|v|) - (8 for E4M3, 2 for E2M1), clamped to
 * [-127, 127] (-127 for an all-zero block); elements = v / 2^e rounded to
 * nearest, ties to the even code, saturating, the sign kept (also of zero).
 *
 * moe_mx_quantize: a row-major [rows, K] matrix of dtype (fp32 or bf16), K a
 * multiple of 32 -> codes [rows, K] (fp8) or [rows, K/2] (fp4) bytes and
 * scales [rows, K/32] bytes. For the experts' weights: W1 [E*H, M] and W2
 * [E*M, H] rows, quantised along their input dimension. */
moe_status moe_mx_quantize(int32_t fmt, int64_t rows, int32_t K, int32_t dtype, const void *src,
                           void *codes, void *scales, void *stream);

/* moe_encode with the token rows quantised to MXFP8 on the way: buf_codes
 * [E*cmax, M] and buf_scales [E*cmax, M/32] bytes, the rows of moe_encode (a
 * token row quantised once, copied to each kept slot; padding rows are zero
 * codes with scale byte 0). bf16 x; M a multiple of 128. */
moe_status moe_encode_mx(const moe_shape *shape, const void *x, const int32_t *idx, const int32_t *loc,
                         const int32_t *fill, const int32_t *capacity, void *buf_codes, void *buf_scales,
                         void *stream);

/* Expert FFN on MX operands with gfx950's scaled MFMA, for the filled rows
 * j < fill[e] (padding rows are not written):
 *   pre = buf . W1[e]^T + b1[e]  (products of the MX values, fp32 accumulation)
 *   h   = act(pre) in fp32, quantised to MXFP8 along H: h_codes [E*cmax, H],
 *         h_scales [E*cmax, H/32]
 *   y   = h . W2[e]^T + b2[e]    (fp32 accumulation), stored bf16 [E*cmax, M]
 * W1 codes/scales from moe_mx_quantize of [E*H, M], W2 of [E*M, H], in format
 * wfmt (the tokens and h are always MXFP8); b1 [E, H], b2 [E, M] bf16 (NULL
 * iff the bias is off). dtype must be bf16; M and H multiples of 128. The
 * hardware's fp8 accumulation drops low-order bits of products far below the
 * largest in groups of eight (about 1e-4 of the sum of magnitudes). */
moe_status moe_expert_ffn_mx(const moe_shape *shape, int32_t wfmt, const void *buf_codes,
                             const void *buf_scales, const void *W1_codes, const void *W1_scales,
                             const void *b1, const void *W2_codes, const void *W2_scales, const void *b2,
                             const int32_t *fill, const int32_t *capacity, void *h_codes, void *h_scales,
                             void *y, void *stream);

/* The two halves of moe_expert_ffn_mx (same definitions and row rules):
 *   moe_expert_fc1_mx: h = MXFP8(act(buf . W1[e]^T + b1[e]))
 *   moe_expert_fc2_mx: y = h . W2[e]^T + b2[e]                 */
moe_status moe_expert_fc1_mx(const moe_shape *shape, int32_t wfmt, const void *buf_codes,
                             const void *buf_scales, const void *W1_codes, const void *W1_scales,
                             const void *b1, const int32_t *fill, const int32_t *capacity, void *h_codes,
                             void *h_scales, void *stream);
moe_status moe_expert_fc2_mx(const moe_shape *shape, int32_t wfmt, const void *h_codes, const void *h_scales,
                             const void *W2_codes, const void *W2_scales, const void *b2,
                             const int32_t *fill, const int32_t *capacity, void *y, void *stream);

/* The whole forward with MX experts: [gate projection] -> route ->
 * moe_encode_mx -> moe_expert_ffn_mx -> moe_decode (bf16 out), arguments as
 * in moe_layer_forward and the two calls above. */
moe_status moe_layer_forward_mx(const moe_shape *shape, int32_t wfmt, const void *x, const float *logits_in,
                                const float *Wg, float *logits_out, const void *W1_codes,
                                const void *W1_scales, const void *b1, const void *W2_codes,
                                const void *W2_scales, const void *b2, int32_t *idx, int32_t *loc,
                                float *gates, int32_t *needed, int32_t *fill, int32_t *capacity,
                                int32_t *slot_route, void *buf_codes, void *buf_scales, void *h_codes,
                                void *h_scales, void *y, void *out, void *ws, size_t ws_bytes, void *stream);

/* Block-wise FP8 experts (Tutel catalogue page and its project summaries:
 * BlockwiseFP8 quantised inference, named there without a definition; the
 * reading is the fine-grained scheme published with DeepSeek-V3, a model family
 * the project summary names). E4M3 elements (one byte each) with one fp32 scale
 * per block: 128 x 128 for the experts' weights (128 output features by 128
 * steps of the reduction dimension), 1 x 128 for token rows and h (128
 * consecutive features). A block is quantised as s = amax / 448 (fp32 division;
 * 448 is E4M3's largest value) and code = v / s (fp32 division) rounded to the
 * nearest E4M3 value, ties to the even code, saturating at +-448, the sign kept;
 * an all-zero block has s = 0 and codes 0. A code c of a block with scale s
 * stands for e4m3(c) * s. Scale arrays are fp32 [rows / brows][K / 128],
 * row-major.
 *
 * moe_blockfp8_quantize: a row-major [rows, K] matrix of dtype (fp32 or bf16),
 * K a multiple of 128, in blocks of brows x 128 (brows 1 or 128, rows a multiple
 * of brows) -> codes [rows, K] bytes, scales fp32 [rows / brows, K / 128]. For
 * the experts' weights (brows = 128): W1 [E*H, M] and W2 [E*M, H] rows,
 * quantised along their input dimension (H and M multiples of 128, so no block
 * straddles two experts). */
moe_status moe_blockfp8_quantize(int64_t rows, int32_t K, int32_t brows, int32_t dtype, const void *src,
                                 void *codes, float *scales, void *stream);

/* moe_encode with the token rows quantised to block-wise FP8 (1 x 128 blocks) on
 * the way: buf_codes [E*cmax, M] bytes and buf_scales fp32 [E*cmax, M/128], the
 * rows of moe_encode (a token row quantised once, copied to each kept slot;
 * padding rows have codes 0 and scale 0). bf16 x; M a multiple of 128. */
moe_status moe_encode_blockfp8(const moe_shape *shape, const void *x, const int32_t *idx, const int32_t *loc,
                               const int32_t *fill, const int32_t *capacity, void *buf_codes, float *buf_scales,
                               void *stream);

/* Expert FFN on block-wise FP8 operands with gfx950's fp8 MFMA, for the filled
 * rows j < fill[e] (padding rows are not written):
 *   pre = buf . W1[e]^T + b1[e]  (products of the dequantised values, fp32
 *         accumulation: each 128-deep block's partial sum times its two scales)
 *   h   = act(pre) in fp32, quantised in 1 x 128 blocks along H: h_codes
 *         [E*cmax, H], h_scales fp32 [E*cmax, H/128]
 *   y   = h . W2[e]^T + b2[e]    (fp32 accumulation), stored bf16 [E*cmax, M]
 * W1 codes/scales from moe_blockfp8_quantize(brows = 128) of [E*H, M], W2 of
 * [E*M, H]; b1 [E, H], b2 [E, M] bf16 (NULL iff the bias is off). dtype must be
 * bf16; M and H multiples of 128. The hardware's fp8 accumulation within a
 * block drops low-order bits of products far below the largest (about 1e-4 of
 * the sum of magnitudes). */
moe_status moe_expert_ffn_blockfp8(const moe_shape *shape, const void *buf_codes, const float *buf_scales,
                                   const void *W1_codes, const float *W1_scales, const void *b1,
                                   const void *W2_codes, const float *W2_scales, const void *b2,
                                   const int32_t *fill, const int32_t *capacity, void *h_codes, float *h_scales,
                                   void *y, void *stream);

/* The two halves of moe_expert_ffn_blockfp8 (same definitions and row rules):
 *   moe_expert_fc1_blockfp8: h = blockFP8(act(buf . W1[e]^T + b1[e]))
 *   moe_expert_fc2_blockfp8: y = h . W2[e]^T + b2[e]                 */
moe_status moe_expert_fc1_blockfp8(const moe_shape *shape, const void *buf_codes, const float *buf_scales,
                                   const void *W1_codes, const float *W1_scales, const void *b1,
                                   const int32_t *fill, const int32_t *capacity, void *h_codes, float *h_scales,
                                   void *stream);
moe_status moe_expert_fc2_blockfp8(const moe_shape *shape, const void *h_codes, const float *h_scales,
                                   const void *W2_codes, const float *W2_scales, const void *b2,
                                   const int32_t *fill, const int32_t *capacity, void *y, void *stream);

/* The whole forward with block-wise FP8 experts: [gate projection] -> route ->
 * moe_encode_blockfp8 -> moe_expert_ffn_blockfp8 -> moe_decode (bf16 out),
 * arguments as in moe_layer_forward and the calls above. */
moe_status moe_layer_forward_blockfp8(const moe_shape *shape, const void *x, const float *logits_in,
                                      const float *Wg, float *logits_out, const void *W1_codes,
                                      const float *W1_scales, const void *b1, const void *W2_codes,
                                      const float *W2_scales, const void *b2, int32_t *idx, int32_t *loc,
                                      float *gates, int32_t *needed, int32_t *fill, int32_t *capacity,
                                      int32_t *slot_route, void *buf_codes, float *buf_scales, void *h_codes,
                                      float *h_scales, void *y, void *out, void *ws, size_t ws_bytes,
                                      void *stream);

/* NVFP4 experts (Tutel catalogue page: the low-precision inference formats,
 * NVFP4 among them, listed for A100/A800/H100/MI300 hardware). NVFP4 is named,
 * not defined, there; the reading is NVIDIA's two-level 4-bit format: E2M1
 * elements (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives) in blocks of
 * 16 consecutive values along the reduction dimension, each block with an E4M3
 * scale, and one fp32 scale g per tensor (here one expert's weight matrix). None
 * of the listed GPUs multiplies 4-bit values, so the format is read as
 * weight-only: the experts' weights are stored NVFP4 and multiplied at their
 * exact values by bf16 tokens. Element c of a block with scale code q in a
 * tensor of scale g stands for e2m1(c) * e4m3(q) * g.
 *
 * moe_nvfp4_quantize: a row-major [rows, K] matrix of dtype (fp32 or bf16), K a
 * multiple of 16, taken as ntensor tensors of rows / ntensor consecutive rows
 * (the experts' weights: W1 [E*H, M] or W2 [E*M, H] with ntensor = E). Per
 * tensor, in fp32 arithmetic: g = amax / 2688 (448 * 6); per block of 16 values
 * d = (amax_b / 6) / g, q = the E4M3 code nearest d (ties to the even code,
 * saturating at 448); each value v -> the E2M1 code nearest v / (e4m3(q) * g)
 * (that product rounded to fp32, then the division; ties to the even code,
 * saturating at 6; the sign bit v's); codes 0 where e4m3(q) * g is 0. Outputs:
 * codes [rows, K/2] bytes (two per byte, the even index in the low nibble),
 * scales [rows, K/16] E4M3 bytes, g [ntensor] fp32. Two launches (the tensors'
 * amax first). */
moe_status moe_nvfp4_quantize(int64_t rows, int32_t K, int32_t ntensor, int32_t dtype, const void *src, void *codes,
                              void *scales, float *g, void *stream);

/* Expert FFN with NVFP4 weights and bf16 tokens, for the filled rows
 * j < fill[e] (padding rows are not written), the bf16 FFN's definitions on
 * the weights' values w = e2m1(c) * e4m3(q) * g:
 *   pre = buf . W1[e]^T + b1[e]   (fp32 accumulation), stored bf16 if pre != NULL
 *   h   = act(pre), stored bf16 [E*cmax, H]
 *   y   = h . W2[e]^T + b2[e]     (fp32 accumulation), stored bf16 [E*cmax, M]
 * W1 from moe_nvfp4_quantize of [E*H, M] with ntensor = E (codes [E*H, M/2],
 * scales [E*H, M/16], g [E]), W2 likewise of [E*M, H]; b1 [E, H], b2 [E, M]
 * bf16 (NULL iff the bias is off). Each weight value is a bf16 number, so the
 * products are exact and the sums run in fp32 as in the bf16 FFN; the expert's
 * g multiplies the fp32 sum before the bias is added. dtype must be bf16. */
moe_status moe_expert_ffn_nvfp4(const moe_shape *shape, const void *buf, const void *W1_codes, const void *W1_scales,
                                const float *W1_g, const void *b1, const void *W2_codes, const void *W2_scales,
                                const float *W2_g, const void *b2, const int32_t *fill, const int32_t *capacity,
                                void *pre, void *h, void *y, void *stream);

/* The two halves of moe_expert_ffn_nvfp4 (same definitions and row rules):
 *   moe_expert_fc1_nvfp4: pre (optional), h = act(buf . W1[e]^T + b1[e])
 *   moe_expert_fc2_nvfp4: y = h . W2[e]^T + b2[e]                     */
moe_status moe_expert_fc1_nvfp4(const moe_shape *shape, const void *buf, const void *W1_codes, const void *W1_scales,
                                const float *W1_g, const void *b1, const int32_t *fill, const int32_t *capacity,
                                void *pre, void *h, void *stream);
moe_status moe_expert_fc2_nvfp4(const moe_shape *shape, const void *h, const void *W2_codes, const void *W2_scales,
                                const float *W2_g, const void *b2, const int32_t *fill, const int32_t *capacity,
                                void *y, void *stream);

/* The whole forward (inference) with NVFP4 experts: [gate projection] -> route
 * -> encode -> moe_expert_ffn_nvfp4 -> moe_decode, arguments as in
 * moe_layer_forward (no pre-activation output) with the weights as above. */
moe_status moe_layer_forward_nvfp4(const moe_shape *shape, const void *x, const float *logits_in, const float *Wg,
                                   float *logits_out, const void *W1_codes, const void *W1_scales, const float *W1_g,
                                   const void *b1, const void *W2_codes, const void *W2_scales, const float *W2_g,
                                   const void *b2, int32_t *idx, int32_t *loc, float *gates, int32_t *needed,
                                   int32_t *fill, int32_t *capacity, int32_t *slot_route, void *buf, void *h, void *y,
                                   void *out, void *ws, size_t ws_bytes, void *stream);

/* Residual-MoE (MoE training blog, part 1 section 1.2, the residual half of
 * PR-MoE): every token also passes through one fixed dense MLP, and its output
 * is added to the MoE output. The dense branch has the experts' form with its
 * own weights over all S tokens:
 *   pre_r = x . W1r^T + b1r       (fp32 accumulation), stored if pre_r != NULL
 *   h_r   = act(pre_r)            stored in the data type
 *   y_r   = h_r . W2r^T + b2r      (fp32 accumulation), stored
 * W1r [H, M], b1r [H] (NULL iff !has_fc1_bias), W2r [M, H], b2r [M] (NULL iff
 * !has_fc2_bias); x, y_r [S, M]; pre_r, h_r [S, H] (pre_r is kept for the
 * backward; NULL for inference); ws: moe_workspace_size() bytes (8 bytes of it
 * hold the branch's row count for the grouped GEMMs). Supported for
 * S < 128 * 65535. */
moe_status moe_residual_ffn(const moe_shape *shape, const void *x, const void *W1r, const void *b1r,
                            const void *W2r, const void *b2r, void *pre_r, void *h_r, void *y_r, void *ws,
                            size_t ws_bytes, void *stream);

/* Backward of the dense branch for the layer's upstream gradient dout [S, M]
 * (the branch's output is added to the layer output, so its output gradient
 * is dout itself), the same definitions as the experts' backward with the
 * branch as one expert over all S rows:
 *   dpre_r = (dout . W2r) * act'(pre_r), stored, with pre_r the forward's
 *            stored pre-activation;       dx_r = dpre_r . W1r, stored
 *   dW2r = sum_s dout_s^T h_r,s, db2r = sum_s dout_s,
 *   dW1r = sum_s dpre_r,s^T x_s, db1r = sum_s dpre_r,s     (fp32)
 * dpre_r [S, H] and dx_r [S, M] are caller buffers in the data type; dW1r
 * [H, M], dW2r [M, H] fp32 (overwritten; zeros when S == 0); db1r [H], db2r
 * [M] fp32 or NULL (not computed). ws: moe_workspace_size() bytes. */
moe_status moe_residual_backward(const moe_shape *shape, const void *dout, const void *x, const void *pre_r,
                                 const void *h_r, const void *W1r, const void *W2r, void *dpre_r, void *dx_r,
                                 float *dW1r, float *db1r, float *dW2r, float *db2r, void *ws, size_t ws_bytes,
                                 void *stream);

/* moe_decode with the Residual-MoE add fused in: the fp32 sum over the kept
 * routes (as in moe_decode) gains y_r[s] after the last route, then is rounded
 * once to the data type. A token whose routes were all dropped gets y_r[s]. */
moe_status moe_decode_residual(const moe_shape *shape, const void *y, const float *gates,
                               const int32_t *idx, const int32_t *loc, const int32_t *capacity,
                               const void *y_r, void *out, void *stream);

/* Gate backward (the softmax gate is trained: MoE training blog, part 2 section
 * 2.1, training with top-1 gating and an auxiliary load-balance loss of
 * coefficient 0.01; DeepSpeed PR #8195, forward + backward step times). The
 * gates are unrenormalised softmax probabilities p of the logits (moe_route),
 * so with
 *   g[s][e] = sum of dgates[r][s] over the routes r with idx[r][s] == e
 *             + aux_coef * E * f_e / S,      f_e = needed[e] / (k S),
 *   dlogits[s][e] = p[s][e] * (g[s][e] - sum_j p[s][j] g[s][j])     (fp32)
 * and aux_loss[0] = aux_coef * E * sum_e f_e * (1/S) sum_s p[s][e] (fp32; 0
 * when S == 0): the load-balance loss in its usual routed-fraction times
 * mean-probability form, f held constant (it comes from an argmax). Every
 * route's dgates is used as given (moe_layer_backward passes 0 for dropped
 * routes). needed may be NULL only when aux_coef == 0 (no auxiliary term);
 * aux_loss may be NULL (not computed). logits [S,E] fp32 (the forward's);
 * idx [k,S] int32; dgates [k,S] fp32; needed [E] int32; dlogits [S,E] fp32;
 * ws: moe_workspace_size() bytes. Reductions run in a fixed order: results are
 * reproducible run to run. */
moe_status moe_gate_backward(const moe_shape *shape, const float *logits, const int32_t *idx,
                             const float *dgates, const int32_t *needed, double aux_coef,
                             float *dlogits, float *aux_loss, void *ws, size_t ws_bytes, void *stream);

/* Gradient of the gate projection's weights (logits = x . Wg, moe_gate_project):
 * dWg[m][e] = sum_s x[s][m] * dlogits[s][e], fp32 accumulation in a fixed
 * order, overwritten (all zeros when S == 0). x [S,M] data type; dlogits [S,E]
 * fp32; dWg [M,E] fp32; ws: moe_workspace_size() bytes. The projection's share
 * of dx, dlogits . Wg^T, is added inside moe_layer_backward. */
moe_status moe_gate_weight_grad(const moe_shape *shape, const void *x, const float *dlogits, float *dWg,
                                void *ws, size_t ws_bytes, void *stream);

/* The whole forward: [gate projection] -> route -> encode -> expert FFN ->
 * decode, on one stream, without a host synchronisation. Exactly one of
 * logits_in (given logits [S,E]) and Wg ([M,E], projected from x) is non-NULL;
 * with Wg, logits_out [S,E] receives the logits (it may be NULL only when
 * logits_in is given). Route outputs, buf, pre, h and y are kept for the
 * backward; pre may be NULL for inference. Sizes as in the calls above. */
moe_status moe_layer_forward(const moe_shape *shape, const void *x, const float *logits_in,
                             const float *Wg, float *logits_out, const void *W1, const void *b1,
                             const void *W2, const void *b2, int32_t *idx, int32_t *loc,
                             float *gates, int32_t *needed, int32_t *fill, int32_t *capacity,
                             int32_t *slot_route, void *buf, void *pre, void *h, void *y, void *out,
                             void *ws, size_t ws_bytes, void *stream);

/* moe_layer_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, results and kernels without the workspace.
 * Routing's counts go to a static scratch array of the library, 4 MiB per GPU
 * (held until the process ends), so shapes with E * k * ceil(S / 64) above
 * 1048576 counts return MOE_EUNSUPPORTED, enqueuing nothing. The call makes no
 * allocation of any kind. Every call on one GPU shares that GPU's scratch:
 * calls that may overlap on one GPU (different streams, or several host
 * threads) race and must be ordered by the caller; moe_layer_forward with
 * workspaces of their own does not have this limit. The first call on a
 * device looks up the scratch's address (not an allocation). */
moe_status moe_layer_forward_noalloc(const moe_shape *shape, const void *x, const float *logits_in,
                                     const float *Wg, float *logits_out, const void *W1, const void *b1,
                                     const void *W2, const void *b2, int32_t *idx, int32_t *loc, float *gates,
                                     int32_t *needed, int32_t *fill, int32_t *capacity, int32_t *slot_route,
                                     void *buf, void *pre, void *h, void *y, void *out, void *stream);

/* moe_layer_forward of a Residual-MoE layer: the same steps, plus the dense
 * branch (moe_residual_ffn: W1r, b1r, W2r, b2r -> pre_r, h_r, y_r; pre_r may
 * be NULL for inference) before decode, and decode as moe_decode_residual. */
moe_status moe_residual_layer_forward(const moe_shape *shape, const void *x, const float *logits_in,
                                      const float *Wg, float *logits_out, const void *W1, const void *b1,
                                      const void *W2, const void *b2, const void *W1r, const void *b1r,
                                      const void *W2r, const void *b2r, int32_t *idx, int32_t *loc,
                                      float *gates, int32_t *needed, int32_t *fill, int32_t *capacity,
                                      int32_t *slot_route, void *buf, void *pre, void *h, void *y,
                                      void *pre_r, void *h_r, void *y_r, void *out, void *ws, size_t ws_bytes,
                                      void *stream);

/* moe_layer_forward with the expert FFN pipelined over the capacity dimension
 * (MoE training blog, part 3 section 3.4, adaptive pipelining, its single-GPU
 * half): [gate projection], route and encode on `stream`; then the capacity
 * bound cmax is cut into `chunks` windows of ceil(cmax / chunks) slots, window
 * c computed by moe_expert_ffn_window on streams[c % nstreams]; decode on
 * `stream` after every chunk. events: nstreams + 1 caller-created hipEvent_t
 * (recorded and waited on, never destroyed). Same results as
 * moe_layer_forward. bf16 data only; 1 <= chunks, nstreams <= 64. */
moe_status moe_layer_forward_pipelined(const moe_shape *shape, const void *x, const float *logits_in,
                                       const float *Wg, float *logits_out, const void *W1, const void *b1,
                                       const void *W2, const void *b2, int32_t *idx, int32_t *loc,
                                       float *gates, int32_t *needed, int32_t *fill, int32_t *capacity,
                                       int32_t *slot_route, void *buf, void *pre, void *h, void *y,
                                       void *out, void *ws, size_t ws_bytes, int32_t chunks,
                                       void *const *streams, int32_t nstreams, void *const *events,
                                       void *stream);

/* The backward of decode, expert FFN and encode for upstream gradient dout
 * [S, M] (blog part 3 section 3.5: K1 is combine-backward, K2 the cross term,
 * K0 encode-backward), given the forward's saved tensors (buf, pre, h, y and
 * the route tables):
 *   dy[slot]     = gates[r][s] * dout[s] in fp32, stored (rows of kept routes only)
 *   dgates[r][s] = <dout[s], y[slot]> in fp32, 0 for dropped routes
 *   dpre = (dy . W2[e]) * act'(pre), stored, with pre the forward's stored
 *          pre-activation (in the data type);   dbuf = dpre . W1[e], stored
 *   dW2[e] = sum_j dy_j^T h_j, db2[e] = sum_j dy_j,
 *   dW1[e] = sum_j dpre_j^T buf_j, db1[e] = sum_j dpre_j   (fp32, over j < fill[e])
 *   dx[s] = sum over kept routes of dbuf[slot] (fp32 accumulation), stored;
 *           0 for a token whose routes were all dropped.
 * dy, dbuf [E*cmax, M] and dpre [E*cmax, H] are caller scratch; dy and dbuf
 * may be the same buffer. dW1 [E,H,M], dW2 [E,M,H] fp32; db1 [E,H], db2 [E,M]
 * fp32 or NULL (not computed); dgates [k,S] fp32; dx [S,M]. Gradients are
 * overwritten, not accumulated. pre must come from the forward.
 * Gate backward (moe_gate_backward, moe_gate_weight_grad), run when any of
 * logits, dlogits, dWg, aux_loss is non-NULL (all NULL: none of it, and Wg,
 * x, needed, ws are not read): from the forward's logits, needed and
 * aux_coef, dlogits and aux_loss (may be NULL) as in moe_gate_backward, from
 * the dgates just computed. With Wg (the projected gate; dWg then required,
 * x too), dWg = x^T . dlogits and dx[s] gains dlogits[s] . Wg^T, added in fp32
 * before dx's single rounding to the data type. ws: moe_workspace_size() bytes
 * (only with the gate backward). */
moe_status moe_layer_backward(const moe_shape *shape, const void *dout, const void *buf,
                              const void *pre, const void *h, const void *y, const float *gates,
                              const int32_t *idx, const int32_t *loc, const int32_t *fill,
                              const int32_t *capacity, const void *W1, const void *W2, void *dy,
                              void *dpre, void *dbuf, void *dx, float *dW1, float *db1, float *dW2,
                              float *db2, float *dgates, const float *logits, const int32_t *needed,
                              double aux_coef, const void *x, const float *Wg, float *dlogits,
                              float *dWg, float *aux_loss, void *ws, size_t ws_bytes, void *stream);

/* moe_layer_backward of a Residual-MoE layer (MoE training blog, part 1
 * section 1.2: out = MoE output + the dense branch's y_r): the same arguments
 * and results, plus the dense branch's backward (moe_residual_backward: W1r,
 * W2r, the forward's pre_r and h_r -> dpre_r, dx_r, dW1r, db1r, dW2r, db2r),
 * and dx[s] = the kept dbuf rows (+ the gate projection's share) + dx_r[s],
 * added in fp32 after the other terms, rounded once to the data type. x is
 * required; dx_r must not be dx. ws: moe_workspace_size() bytes (always). */
moe_status moe_residual_layer_backward(const moe_shape *shape, const void *dout, const void *buf,
                                       const void *pre, const void *h, const void *y, const float *gates,
                                       const int32_t *idx, const int32_t *loc, const int32_t *fill,
                                       const int32_t *capacity, const void *W1, const void *W2, void *dy,
                                       void *dpre, void *dbuf, void *dx, float *dW1, float *db1, float *dW2,
                                       float *db2, float *dgates, const float *logits, const int32_t *needed,
                                       double aux_coef, const void *x, const float *Wg, float *dlogits,
                                       float *dWg, float *aux_loss, const void *W1r, const void *W2r,
                                       const void *pre_r, const void *h_r, void *dpre_r, void *dx_r,
                                       float *dW1r, float *db1r, float *dW2r, float *db2r, void *ws,
                                       size_t ws_bytes, void *stream);

/* The stages of moe_layer_backward as calls of their own (same definitions,
 * same buffers), for callers that schedule or time them separately:
 *   moe_decode_backward           K1' and K2 (blog part 3 section 3.5): dy rows
 *                                 of kept routes and dgates [k,S];
 *   moe_expert_fc2_backward_data  dpre = (dy . W2[e]) * act'(pre), stored;
 *   moe_expert_fc2_weight_grad    dW2[e] = sum_j dy_j^T h_j, db2 (may be NULL);
 *   moe_expert_fc1_backward_data  dbuf = dpre . W1[e], stored;
 *   moe_expert_fc1_weight_grad    dW1[e] = sum_j dpre_j^T buf_j, db1 (may be NULL);
 *   moe_encode_backward           K0: dx[s] = sum of the token's kept dbuf rows
 *                                 (fp32, route order), stored (no gate share).
 * Every product covers the filled rows j < fill[e] of each expert. */
moe_status moe_decode_backward(const moe_shape *shape, const void *dout, const void *y, const float *gates,
                               const int32_t *idx, const int32_t *loc, const int32_t *capacity, void *dy,
                               float *dgates, void *stream);
moe_status moe_expert_fc2_backward_data(const moe_shape *shape, const void *dy, const void *W2, const void *pre,
                                        const int32_t *fill, const int32_t *capacity, void *dpre, void *stream);
moe_status moe_expert_fc2_weight_grad(const moe_shape *shape, const void *dy, const void *h, const int32_t *fill,
                                      const int32_t *capacity, float *dW2, float *db2, void *stream);
moe_status moe_expert_fc1_backward_data(const moe_shape *shape, const void *dpre, const void *W1,
                                        const int32_t *fill, const int32_t *capacity, void *dbuf, void *stream);
moe_status moe_expert_fc1_weight_grad(const moe_shape *shape, const void *dpre, const void *buf,
                                      const int32_t *fill, const int32_t *capacity, float *dW1, float *db1,
                                      void *stream);
moe_status moe_encode_backward(const moe_shape *shape, const void *dbuf, const int32_t *idx, const int32_t *loc,
                               const int32_t *capacity, void *dx, void *stream);

/* Message of the last failing call on this thread ("" if none). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
