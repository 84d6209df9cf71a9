/*
 * dsq.h -- C ABI of libdsq: group-quantized fused-dequant GEMV / GEMM and the
 * top-k routed mixture-of-experts SwiGLU FFN on AMD MI355X (gfx950).
 *
 * The method (all citations name the page and its section):
 *   "Hand-writing a DeepSeek inference engine in pure C" (hnwysp.cn/news/134870)
 *     §2.3  weights quantized group-wise (groups of 64 or 128 along the
 *           reduction axis), asymmetric, dequantized as (q - zero_point) *
 *           scale; the stored layout must suit the matmul kernel;
 *     §3.2  scale = (max - min) / (2^bits - 1), zero_point = round(-min /
 *           scale), q = clamp(round(v / scale) + zero_point, 0, 2^bits - 1);
 *           INT4 stores two values per byte; scale and zero point are fp32;
 *           dequantization is fused into the matmul's inner loop;
 *     §3.3  the matmul;
 *     §3.4  softmax with the maximum subtracted;
 *     §3.5  MoE: router = linear layer + softmax, top-k experts, tokens
 *           grouped by expert so each expert's weights are read once, outputs
 *           combined by a weighted sum;
 *     §5.1  a zero scale is an error.
 *   "ds4 code walkthrough" (ds4-learning.pages.dev), Part 1: every shape is
 *     validated before use, errors are reported rather than fatal inside
 *     the library, no allocation inside the token loop.
 *
 * Conventions shared by every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing, keeps no state between calls (the expert cache keeps
 *     its state in caller-owned tables) and never synchronises (except
 *     dsq_moe_ffn_cached, whose host must see the routing); every call only
 *     enqueues kernels on `stream` (a hipStream_t, NULL = the default
 *     stream): no memset, copy or synchronisation, so a call can be captured
 *     into a HIP graph and replayed (dsq_moe_ffn_cached excepted).  Calls are
 *     re-entrant; two calls that share a workspace must be ordered on one
 *     stream.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     failed check returns a negative dsq_status and enqueues nothing, so no
 *     output is written.  Launch failures return DSQ_ERR_HIP.
 *   - Results are deterministic for given inputs on a given device: no
 *     floating-point atomics anywhere.
 *   - fp32 tensors are row-major and 16-byte aligned.
 */
#ifndef DSQ_H
#define DSQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t dsq_status;
#define DSQ_OK 0
#define DSQ_ERR_INVALID_ARG (-1) /* NULL pointer, value out of range      */
#define DSQ_ERR_SHAPE (-2)       /* K % group != 0, sizes <= 0, k > E ... */
#define DSQ_ERR_ALIGN (-3)       /* pointer not aligned as required      */
#define DSQ_ERR_WORKSPACE (-4)   /* workspace NULL or too small          */
#define DSQ_ERR_UNSUPPORTED (-5) /* valid but not implemented (limits)   */
#define DSQ_ERR_NO_DEVICE (-6)   /* no HIP device visible                */
#define DSQ_ERR_HIP (-7)         /* a HIP runtime call or launch failed  */
#define DSQ_ERR_OVERFLOW (-8)    /* a size computation overflows         */
#define DSQ_ERR_LAYOUT (-9)      /* packed buffer has an unknown layout  */

/* Arithmetic of the matmuls. */
#define DSQ_MATH_FP32 0      /* fp32 products and sums (VALU FMA)              */
#define DSQ_MATH_BF16_MFMA 1 /* activations and dequantized weights rounded to  */
                             /* bf16, products summed in fp32 on MFMA           */
#define DSQ_MATH_AUTO 2      /* BF16_MFMA when the token count M >= 64, else    */
                             /* FP32                                            */

/* Flags written (OR-ed) into the packer's status word. */
#define DSQ_FLAG_DEGENERATE 1 /* a group with max == min (scale 0), a scale   */
                              /* that is not finite, or |zero point| > 2^24   */
#define DSQ_FLAG_NONFINITE 2  /* a group holding NaN or +-inf                 */

/*
 * Device layout, version 1 (DSQ_LAYOUT_VERSION).  For a weight W[batch][N][K]
 * quantized with `bits` and `group`, RB = K * bits / 8 bytes per row:
 *   per batch entry b, at byte offset b * stride:
 *     payload : N rows of RB bytes, row-major.
 *               INT8: byte k of row n is q[n][k] (0..255).
 *               INT4: the 32-bit little-endian word j of a row holds
 *                     k = 8j .. 8j+7; its byte i (0..3) holds q[n][8j+i] in
 *                     the low nibble and q[n][8j+4+i] in the high nibble, so
 *                     masking the word with 0x0F0F0F0F yields four
 *                     consecutive codes and shifting by 4 first the next four.
 *     meta    : at offset align256(N * RB): N rows of K/group pairs
 *               (float scale, float zero_point); the zero point is an exact
 *               integer held in fp32.
 *   stride = align256(N * RB) + align256(N * (K/group) * 8).
 * A flagged group has all its codes 0 and scale = zero point = 0.
 *
 * group = 256 (bits = 4 only) selects the two-level super-block format, the
 * block of "ds4 code walkthrough", trace 4 (quant block struct sizes): fp16 d,
 * fp16 dmin, 12 bytes of scales, 128 bytes of nibbles per 256 weights.  Its
 * arithmetic is read from those fields: 8 sub-blocks of 32 weights; sub-block
 * j has a 6-bit scale sc_j and a 6-bit min m_j; a weight dequantizes to
 * d*sc_j*q - dmin*m_j.  Quantizer, in fp32 with roundf:
 *   off_j = max(0, -min_j), step_j = (max_j + off_j) / 15,
 *   d = fp16(max step / 63), dmin = fp16(max off / 63) (nearest even),
 *   sc_j = clamp(round(step_j / d), 0, 63), m_j = clamp(round(off_j / dmin), 0, 63),
 *   q = clamp(round((w + dmin*m_j) / (d*sc_j)), 0, 15)  (0 when a divisor is 0).
 * Layout: the payload as the 4-bit group format (a 16-byte chunk is one
 * sub-block); the metadata holds per row K/256 16-byte block headers:
 * word 0 = d | dmin << 16 (fp16 bits), words 1..3 = a little-endian 96-bit
 * field stream with sc_0..sc_7 then m_0..m_7, field f at bits 6f..6f+5.
 *   stride = align256(N * K/2) + align256(N * (K/256) * 16)
 * A block holding a NaN or infinity (DSQ_FLAG_NONFINITE), or whose d or dmin
 * overflows fp16 (DSQ_FLAG_DEGENERATE), is stored as zeros.  This format is
 * read by dsq_gemv and dsq_gemv_topk; dsq_gemm with M >= 2, dsq_moe_ffn and
 * dsq_moe_block return DSQ_ERR_UNSUPPORTED for it.
 */
#define DSQ_LAYOUT_VERSION 1u

typedef struct dsq_qweight {
  int32_t bits;            /* 8 or 4                                          */
  int32_t group;           /* 64 or 128 along K; 256 = super-block (4-bit)    */
  int64_t K;               /* reduction length (columns of W)                 */
  int64_t N;               /* outputs (rows of W)                             */
  int64_t batch;           /* number of matrices (experts); 1 for dense       */
  uint32_t layout_version; /* written by dsq_pack_weights                     */
  uint32_t reserved;       /* must be 0                                       */
  void* data;              /* device buffer of dsq_packed_bytes() bytes,      */
                           /* 256-byte aligned, owned by the caller           */
} dsq_qweight;

/* Human-readable name of a status code (static string, never NULL). */
const char* dsq_status_string(dsq_status s);

/* Bytes of the packed buffer for W[batch][N][K]; 0 if the arguments are
   invalid (bits, group, K % group, non-positive sizes) or overflow. */
size_t dsq_packed_bytes(int32_t bits, int32_t group, int64_t K, int64_t N, int64_t batch);

/* Fill a descriptor (layout_version = DSQ_LAYOUT_VERSION, reserved = 0).
   Validates like dsq_packed_bytes and the 256-byte alignment of data. */
dsq_status dsq_qweight_init(dsq_qweight* w, int32_t bits, int32_t group, int64_t K, int64_t N,
                            int64_t batch, void* data);

/*
 * dsq_pack_weights -- quantize and lay out weights ("quantize once at model
 * conversion time", hnwysp.cn/news/134870 §3.2 and §2.3).
 *   src        : fp32 [count][N][K] device, the weights of batch entries
 *                first .. first+count-1 of `out`.
 *   out        : descriptor from dsq_qweight_init; out->data receives the
 *                codes and (scale, zero point) of those entries.
 *   dev_flags  : optional device int32; DSQ_FLAG_* bits of every flagged
 *                group of this call are OR-ed into it (the caller zeroes it).
 *                NULL = do not report.
 * Quantization per group of `group` consecutive weights along K, in IEEE fp32
 * with correctly rounded division and round-half-away-from-zero:
 *   scale = (max - min) / (2^bits - 1); zp = round(-min / scale);
 *   q = clamp(round(v / scale) + zp, 0, 2^bits - 1).
 * Errors: DSQ_ERR_INVALID_ARG (NULL src/out/data, first/count out of range),
 * DSQ_ERR_SHAPE, DSQ_ERR_ALIGN (src not 16-byte or data not 256-byte
 * aligned), DSQ_ERR_LAYOUT (descriptor version), DSQ_ERR_NO_DEVICE,
 * DSQ_ERR_HIP.
 */
dsq_status dsq_pack_weights(const float* src, const dsq_qweight* out, int64_t first,
                            int64_t count, int32_t* dev_flags, void* stream);

/*
 * dsq_gemv -- y = dequant(W[expert]) x for one activation vector (decode,
 * M = 1), dequantization fused into the reduction (hnwysp.cn/news/134870
 * §3.2, §3.3):  y[n] = sum_k x[k] * (q[n][k] - zp[n][g]) * scale[n][g].
 *   W : packed weight (layout 1); expert in [0, W->batch).
 *   x : fp32 [K] device.   y : fp32 [N] device (written).
 * fp32 arithmetic; per output |y - exact| <= 1e-5 * sum_k |x[k] w[n][k]|.
 * Errors: DSQ_ERR_INVALID_ARG, DSQ_ERR_SHAPE, DSQ_ERR_ALIGN, DSQ_ERR_LAYOUT,
 * DSQ_ERR_NO_DEVICE, DSQ_ERR_HIP.
 */
dsq_status dsq_gemv(const dsq_qweight* W, int64_t expert, const float* x, float* y,
                    void* stream);

/*
 * dsq_gemm -- Y = X dequant(W[expert])^T for M activation rows (batched
 * decode and prefill): the matmul of "Hand-writing a DeepSeek inference
 * engine in pure C" (hnwysp.cn/news/134870) §3.3 with the dequantization
 * (q - zero_point) * scale of §3.2 fused into its inner loop; many rows at
 * once are the batched prompt processing that "Running a 284B-parameter LLM
 * from 3.2 GB of RAM in plain C" (feinterview.poetries.top) names as the
 * missing piece (one weight read reused by every prompt token).
 *   X : fp32 [M][K] device.   Y : fp32 [M][N] device (written).
 *   math : DSQ_MATH_FP32, DSQ_MATH_BF16_MFMA or DSQ_MATH_AUTO.
 *   workspace : device scratch of dsq_gemm_workspace_bytes(M, N, K, math)
 *               bytes (NULL allowed when that is 0, as for FP32 with M = 1),
 *               256-byte aligned; its contents on entry are ignored.
 *               BF16_MFMA: when K is split across workgroups, the fp32
 *               partial tiles, added in a fixed order (deterministic).
 *               FP32: X split into two bf16 parts in matrix-core operand
 *               order.
 * FP32: |err| <= 1e-5 * sum|x w| per output (M = 1 runs the GEMV; M >= 2
 * multiplies exact integer codes by x = hi + lo, |x - hi - lo| <= 2^-17 |x|,
 * on the matrix cores and applies zero point and scale per group in fp32:
 * the split leaves at most 2^-17 = 7.6e-6 of sum|x w|, the fp32 group sums
 * and scaling the rest of the 1e-5; worst-case inputs -- every activation at
 * the significand that maximises the split residual, every product of one
 * sign -- are among the tests).
 * BF16_MFMA: X and the dequantized weights are rounded to bf16 and products
 * are summed in fp32: |err| <= 1e-2 * sum|x w| per output.
 * A workspace query of 0 for M >= 2 (or for BF16_MFMA) means the shape is
 * beyond the limits (dsq_gemm then returns DSQ_ERR_UNSUPPORTED); BF16_MFMA
 * needs M*K*4 and N*K below 2^31; FP32 with M >= 2 needs one packed entry
 * (dsq_packed_bytes(bits, group, K, N, 1)) below 2^31 bytes, else
 * DSQ_ERR_UNSUPPORTED.
 */
size_t dsq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t math);
dsq_status dsq_gemm(const dsq_qweight* W, int64_t expert, const float* X, float* Y, int64_t M,
                    int32_t math, void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsq_moe_route_topk -- router softmax + top-k + renormalisation
 * (hnwysp.cn/news/134870 §3.4, §3.5).
 *   logits : fp32 [T][E] device;  bias : fp32 [E] device or NULL, added to
 *            every logit before anything else.
 *   idx    : int32 [T][top_k] device: the top_k experts by score, highest
 *            first; equal scores rank the higher expert index first.
 *   weights: fp32 [T][top_k] device: softmax probabilities of the selected
 *            experts divided by their sum (so they sum to 1); computed from
 *            the max-subtracted scores.
 * Scores must be finite (a NaN is ranked as -infinity).
 * Limits: 1 <= top_k <= min(E, 32), E <= 4096.
 */
dsq_status dsq_moe_route_topk(const float* logits, const float* bias, int64_t T, int32_t E,
                              int32_t top_k, int32_t* idx, float* weights, void* stream);

/*
 * dsq_moe_group -- group the T*top_k routing entries by expert
 * ("Hand-writing a DeepSeek inference engine in pure C",
 * hnwysp.cn/news/134870, §3.5: the tokens routed to one expert are gathered
 * so that the expert's weights are read once).  A stable counting sort,
 * integer only, so the result is exact:
 *   counts[e]  = number of entries j = t*top_k + i with idx[j] == e
 *   offsets[e] = counts[0] + ... + counts[e-1];  offsets[E] = their total
 *   perm[p]    = the entries j in ascending (expert, j) order
 *   pos[j]     = the p with perm[p] == j
 *   idx       : int32 [T][top_k] device; the experts of one token are
 *               distinct (as dsq_moe_route_topk returns them).  An entry
 *               outside [0, E) is grouped nowhere (pos = -1); a repeated
 *               expert within a token gives unspecified values, every
 *               write still inside the outputs.
 *   counts    : int32 [E];  offsets : int32 [E+1];  perm, pos : int32
 *               [T*top_k] (perm's first offsets[E] entries written); device.
 *   workspace : dsq_moe_group_workspace_bytes(T, E, top_k) bytes, 256-byte
 *               aligned (contents on entry ignored).
 * These are the grouping kernels dsq_moe_ffn runs.  Up to 256 tokens one
 * workgroup does the work; beyond, every entry is ranked in O(1) from
 * per-expert prefixes of bitmap popcounts.
 * Limits: T <= 65536, 1 <= E <= 4096, 1 <= top_k <= min(E, 32).
 * Errors: DSQ_ERR_INVALID_ARG (NULL), DSQ_ERR_SHAPE, DSQ_ERR_UNSUPPORTED,
 * DSQ_ERR_ALIGN, DSQ_ERR_WORKSPACE, DSQ_ERR_NO_DEVICE, DSQ_ERR_HIP.
 */
size_t dsq_moe_group_workspace_bytes(int64_t T, int32_t E, int32_t top_k);
dsq_status dsq_moe_group(const int32_t* idx, int64_t T, int32_t E, int32_t top_k,
                         int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsq_topk -- output-head selection: the k largest logits, which choose the
 * next token (hnwysp.cn/news/134870 §2.1: the pipeline ends in the output
 * projection, logits and sampling; "ds4 code walkthrough": the session
 * API's argmax / sample step; "Running a 284B-parameter LLM from 3.2 GB of
 * RAM in plain C": the end-to-end check compares the argmax at every
 * position).
 *   y      : fp32 [N] device, read only.
 *   idx    : int32 [k] device: the k largest in rank order -- larger value
 *            first; equal values (-0 equals +0) rank the smaller index
 *            first (the first maximum a greater-than scan keeps); NaN ranks
 *            below every number.  k = 1 is the argmax.
 *   values : fp32 [k] device: y[idx[r]].
 *   workspace : dsq_topk_workspace_bytes(N, k) bytes, 256-byte aligned
 *            (contents on entry ignored).
 * Exact: the selection compares the fp32 values themselves.
 * Limits: 1 <= k <= min(N, 256), N < 2^31.  Errors: DSQ_ERR_INVALID_ARG,
 * DSQ_ERR_SHAPE (k out of 1..N), DSQ_ERR_UNSUPPORTED (k > 256),
 * DSQ_ERR_ALIGN, DSQ_ERR_WORKSPACE, DSQ_ERR_NO_DEVICE, DSQ_ERR_HIP.
 */
size_t dsq_topk_workspace_bytes(int64_t N, int32_t k);
dsq_status dsq_topk(const float* y, int64_t N, int32_t k, int32_t* idx, float* values,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * dsq_gemv_topk -- the output head: y = dequant(W[expert]) x (as dsq_gemv,
 * written to y) followed by dsq_topk(y, W->N, k, ...) on the same stream.
 * Arguments, limits and errors as the two calls; workspace:
 * dsq_topk_workspace_bytes(W->N, k).  The result is the same as the two
 * calls'; for k = 1 and the group formats with K * bits / 8 <= 4096 the
 * GEMV ranks its own outputs and one small selection follows (no second
 * pass over y).
 */
dsq_status dsq_gemv_topk(const dsq_qweight* W, int64_t expert, const float* x, float* y,
                         int32_t k, int32_t* idx, float* values, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * dsq_moe_ffn -- one routed MoE layer ("Hand-writing a DeepSeek inference
 * engine in pure C", hnwysp.cn/news/134870, §3.5: the router is a linear
 * layer followed by softmax and top-k; the tokens routed to one expert are
 * grouped so that its weights are read once; the expert outputs are summed
 * with the routing weights; §3.4: softmax with the maximum subtracted; §3.2:
 * the experts' weights dequantized inside the matmuls; the SwiGLU expert form
 * and the renormalised weights are the workload's definition):
 *   l = X Wr^T (+ bias)                    router logits, fp32
 *   (idx, w) = route_topk(l)               as dsq_moe_route_topk
 *   group the T*top_k entries by expert    stable, ascending token order
 *   h = silu(X Wg_e^T) * (X Wu_e^T)        per expert, its tokens only
 *   Y[t] = sum_i w[t][i] * (h Wd_e^T)[t]   summed in slot order i = 0..k-1
 *   X        : fp32 [T][H] device.     router_w : fp32 [E][H] device.
 *   bias     : fp32 [E] device or NULL.
 *   gate, up : packed, batch = E, N = I, K = H.  down : batch = E, N = H,
 *              K = I.  All three share bits and group.
 *   math     : as dsq_gemm, choosing by T.  The router is always fp32.  The
 *              expert GEMMs run on the matrix cores with the weights as exact
 *              integer codes; FP32 splits the activations (X, then h) into two
 *              bf16 parts, BF16_MFMA rounds them to bf16.
 *   Y        : fp32 [T][H] device (written).
 *   workspace: dsq_moe_workspace_bytes(T, E, top_k, H, I, math) bytes,
 *              256-byte aligned; contents on entry are ignored.
 *   Optional outputs (NULL to skip): logits_out fp32 [T][E] (including the
 *   bias), idx_out int32 [T][k], w_out fp32 [T][k], expert_counts_out int32
 *   [E] (tokens routed to each expert; the pages log overloaded experts).
 * Limits: T <= 65536, E <= 4096, 1 <= top_k <= min(E, 32); the activation
 * tiles of the grouped GEMM must stay below 2 GiB (about T * top_k * max(H, I)
 * * 4 bytes for FP32): dsq_moe_workspace_bytes returns 0 beyond that; one
 * expert's packed gate (and down) matrix (dsq_packed_bytes(bits, group, K, N,
 * 1)) must stay below 2^31 bytes, else DSQ_ERR_UNSUPPORTED.
 */
size_t dsq_moe_workspace_bytes(int64_t T, int32_t E, int32_t top_k, int64_t H, int64_t I,
                               int32_t math);
dsq_status dsq_moe_ffn(const float* X, const float* router_w, const float* bias,
                       const dsq_qweight* gate, const dsq_qweight* up, const dsq_qweight* down,
                       int64_t T, int32_t top_k, int32_t math, float* Y, void* workspace,
                       size_t workspace_bytes, float* logits_out, int32_t* idx_out,
                       float* w_out, int32_t* expert_counts_out, void* stream);

/*
 * dsq_moe_ffn_noalloc -- dsq_moe_ffn for callers that cannot allocate or pass
 * device memory of their own: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  The same kernels and results as
 * dsq_moe_ffn (bitwise), with the workspace taken from a fixed scratch array
 * of DSQ_NOALLOC_SCRATCH_BYTES that the library's code object holds on every
 * device it runs on, until the process ends.  The call allocates nothing.
 *   Arguments as dsq_moe_ffn without workspace / workspace_bytes.
 *   Limit: dsq_moe_workspace_bytes(T, E, top_k, H, I, math) <=
 *   DSQ_NOALLOC_SCRATCH_BYTES (64 MiB: up to 64 tokens of the 4096-hidden,
 *   2048-intermediate, 256-expert top-6 layer); larger calls return
 *   DSQ_ERR_WORKSPACE and enqueue nothing.
 *   Every call on a device shares that device's scratch: calls that may
 *   overlap on one device (several streams, several host threads) race and
 *   must be ordered by the caller.  The scratch keeps the last call's
 *   contents; the kernels read none of it before writing it.
 * Errors as dsq_moe_ffn, plus DSQ_ERR_WORKSPACE for sizes beyond the scratch.
 */
#define DSQ_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
dsq_status dsq_moe_ffn_noalloc(const float* X, const float* router_w, const float* bias,
                               const dsq_qweight* gate, const dsq_qweight* up,
                               const dsq_qweight* down, int64_t T, int32_t top_k, int32_t math,
                               float* Y, float* logits_out, int32_t* idx_out, float* w_out,
                               int32_t* expert_counts_out, void* stream);

/*
 * dsq_moe_block -- the MoE step of a transformer block with its norm and
 * residual ("Hand-writing a DeepSeek inference engine in pure C",
 * hnwysp.cn/news/134870, §2.1: each block normalises with RMSNorm before the
 * feed-forward / MoE step and adds the residual after it; the epsilon of the
 * "ds4 code walkthrough" model constants is 1e-6):
 *   xn[t] = X[t] / sqrt(mean_h X[t][h]^2 + eps) * norm_w      fp32
 *   Y     = X + moe_ffn(xn)                                    as dsq_moe_ffn
 *   X       : fp32 [T][H] device, the residual stream.  Y may be X itself
 *             (in-place update); any other overlap of Y with an input is
 *             undefined.
 *   norm_w  : fp32 [H] device, 16-byte aligned, the RMSNorm weight.
 *   eps     : finite, > 0 (the pages use 1e-6).
 *   router_w, bias, gate, up, down, T, top_k, math : as dsq_moe_ffn; the
 *             router and the experts see xn.
 *   workspace : dsq_moe_block_workspace_bytes(T, E, top_k, H, I, math)
 *             bytes, 256-byte aligned (contents on entry ignored).
 *   Optional outputs (NULL to skip): xn_out fp32 [T][H] (16-byte aligned,
 *   the normalised rows), and logits_out, idx_out, w_out, expert_counts_out
 *   as dsq_moe_ffn.
 * Limits as dsq_moe_ffn.  Errors as dsq_moe_ffn, plus DSQ_ERR_INVALID_ARG
 * for a NULL norm_w or an eps that is not finite and positive.
 */
size_t dsq_moe_block_workspace_bytes(int64_t T, int32_t E, int32_t top_k, int64_t H, int64_t I,
                                     int32_t math);
dsq_status dsq_moe_block(const float* X, const float* norm_w, float eps, const float* router_w,
                         const float* bias, const dsq_qweight* gate, const dsq_qweight* up,
                         const dsq_qweight* down, int64_t T, int32_t top_k, int32_t math,
                         float* Y, void* workspace, size_t workspace_bytes, float* xn_out,
                         float* logits_out, int32_t* idx_out, float* w_out,
                         int32_t* expert_counts_out, void* stream);

/*
 * Expert cache: host-resident experts streamed into HBM slots, least
 * recently used first out ("Running a 284B-parameter LLM from 3.2 GB of RAM
 * in plain C": per token the router decides which experts are needed and
 * only those are read into an LRU cache; a larger cache hits more often, and
 * a cache smaller than one step's set of experts never hits).  Here the
 * store is host memory and the cache lives in HBM; a miss is one host-to-
 * device copy of the expert's three packed matrices.
 *
 * All state sits in caller-owned memory; the library allocates nothing.
 *   gate, up, down : the device slots, descriptors of packed weights with
 *                    batch = slots (as for dsq_moe_ffn: N = I, K = H for
 *                    gate/up, N = H, K = I for down; shared bits and group).
 *   host_gate, host_up, host_down : host stores of E packed entries each,
 *                    entry e at e * (the matrix's per-entry stride, i.e.
 *                    dsq_packed_bytes(bits, group, K, N, 1)), bytes exactly
 *                    as dsq_pack_weights lays out one entry.  Pinned memory
 *                    (hipHostMalloc) makes the copies asynchronous.
 *   slot_of [E], expert_of [slots], last_use [slots] : host tables.
 * Counters: hits and misses count requests (one per routing entry);
 * bytes_copied the host-to-device bytes of the misses.
 */
typedef struct dsq_expert_cache {
  dsq_qweight gate, up, down;  /* device slots (batch = slots)                */
  const void* host_gate;       /* host stores, E entries each                 */
  const void* host_up;
  const void* host_down;
  int32_t E;                   /* experts in the stores                       */
  int32_t slots;               /* = gate.batch                                */
  int32_t* slot_of;            /* [E]: slot holding expert e, or -1           */
  int32_t* expert_of;          /* [slots]: expert in slot s, or -1            */
  uint64_t* last_use;          /* [slots]: request stamp of the last use      */
  uint64_t clock;              /* requests so far                             */
  uint64_t hits, misses, bytes_copied;
} dsq_expert_cache;

/* Fill a cache over the given slots, stores and tables; every slot starts
   empty.  Errors: DSQ_ERR_INVALID_ARG (NULL pointer, E < 1), DSQ_ERR_SHAPE
   (slot descriptors that do not form one MoE layer), and the descriptor
   errors of dsq_moe_ffn. */
dsq_status dsq_expert_cache_init(dsq_expert_cache* cache, const dsq_qweight* gate,
                                 const dsq_qweight* up, const dsq_qweight* down,
                                 const void* host_gate, const void* host_up,
                                 const void* host_down, int32_t E, int32_t* slot_of,
                                 int32_t* expert_of, uint64_t* last_use);

/*
 * dsq_expert_cache_plan -- host only, no GPU call: map n requested experts
 * (host [n]) to slots (slot_out host [n]) as one call.  A requested expert
 * already in a slot is a hit; a miss takes an empty slot (lowest index)
 * or else the least recently used slot not used in this call; every request,
 * hit or miss, stamps its slot in request order.  Misses are reported in
 * fill_expert/fill_slot (host [n] each, *n_fill
 * entries written, in request order).  Errors: DSQ_ERR_INVALID_ARG (NULL,
 * n < 0, an expert out of 0..E-1), DSQ_ERR_UNSUPPORTED (one call needs more
 * distinct experts than there are slots; the tables stay consistent, the
 * entries before the failing one are mapped).
 */
dsq_status dsq_expert_cache_plan(dsq_expert_cache* cache, const int32_t* experts, int64_t n,
                                 int32_t* slot_out, int32_t* fill_expert, int32_t* fill_slot,
                                 int64_t* n_fill);

/* Bytes of workspace for dsq_moe_ffn_cached: 0 if the arguments are invalid. */
size_t dsq_moe_cached_workspace_bytes(int64_t T, int32_t E, int32_t slots, int32_t top_k,
                                      int64_t H, int64_t I, int32_t math);

/*
 * dsq_moe_ffn_cached -- dsq_moe_ffn with the experts behind an expert cache:
 *   route on the GPU (fp32 router logits with the bias, softmax + top-k +
 *   renormalisation as dsq_moe_route_topk), copy the routing to the host and
 *   SYNCHRONISE the stream (the one call of the library that does: the host
 *   must see the routing to fetch experts), map the requested experts to
 *   slots as dsq_expert_cache_plan and enqueue the copies of the misses,
 *   then run the expert FFN of dsq_moe_ffn on the slots.
 *   router_w : fp32 [E][H] device (E = cache->E); bias fp32 [E] or NULL.
 *   host_idx, host_slots : host [T][k] int32 scratch (the routing and its
 *            slots); host_slots must stay valid until the stream reaches
 *            this call's end.
 *   workspace: dsq_moe_cached_workspace_bytes(T, E, slots, top_k, H, I, math).
 *   Optional outputs: logits_out fp32 [T][E], idx_out int32 [T][k] (expert
 *   ids), w_out fp32 [T][k], all device.
 * Limits as dsq_moe_ffn, plus T*top_k distinct experts fit the slots.
 * Errors as dsq_moe_ffn and dsq_expert_cache_plan.
 */
dsq_status dsq_moe_ffn_cached(const float* X, const float* router_w, const float* bias,
                              dsq_expert_cache* cache, int64_t T, int32_t top_k, int32_t math,
                              float* Y, void* workspace, size_t workspace_bytes,
                              int32_t* host_idx, int32_t* host_slots, float* logits_out,
                              int32_t* idx_out, float* w_out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DSQ_H */
