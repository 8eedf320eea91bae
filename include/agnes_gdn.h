/*
 * agnes_gdn — gated delta-rule layer on AMD Instinct MI355X (gfx950).
 *
 * The layer, as the pages describe it (model card "Agnes-3.0-Flash Preview",
 * section 架构, delta-rule row; discosf article "Agnes 3.0 Flash 刚上线就刷屏…",
 * section 二.1): a depth-wise causal convolution of kernel 4 in front, the gated
 * delta-rule recurrence with 16 key / 48 value heads of dimension 128 and an
 * fp32 recurrent state, a gated RMS-norm behind; prefill runs chunked (chunk 64)
 * and decode runs one token at a time.  The recurrence is the gated delta rule
 * of Yang, Kautz & Hatamizadeh ("Gated Delta Networks", ICLR 2025):
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = scale * S_t q_t,         alpha_t = exp(g_t),
 *
 * per value head h, reading key head h / (Hv / Hk) for q and k.  The state S is
 * stored [value dim][key dim] (the shape of v k^T).
 *
 * Conventions shared by every call:
 *   - Every tensor pointer is a DEVICE pointer, row-major, with the head
 *     dimension contiguous.  Tensor base pointers must be 16-byte aligned and
 *     element strides multiples of 8 elements (vector loads of 16 bytes).
 *   - The caller owns every buffer, including the prefill workspace.  The
 *     library never allocates, frees or synchronises (the status query
 *     agnes_gdn_workspace_status aside); every call is enqueued on `stream` (a
 *     hipStream_t; NULL = the default stream) and returns before the GPU work
 *     ends.
 *   - All argument checks happen before anything is launched.  On a failed
 *     check the call returns a negative agnes_status, launches nothing and
 *     leaves every output untouched.  A launch failure returns AGNES_ERR_HIP and
 *     records the hipError_t, readable with agnes_gdn_last_hip_error() on the
 *     same thread.  Faults inside kernels surface at the caller's next sync.
 *   - Device-side index arrays (cu_seqlens) cannot be checked on the host
 *     without a sync: they must hold cu[0] = 0, be nondecreasing and end at
 *     total_tokens.  Kernels clamp every index to [0, total_tokens], so a
 *     malformed array cannot make them access memory outside the buffers, but
 *     the results are then unspecified.
 *   - Functions keep no state between calls and may be called concurrently
 *     from several threads on disjoint buffers.
 *   - Supported set: head_dim 128, conv kernel_size 4, Hv a multiple of Hk.
 *     Anything else returns AGNES_ERR_UNSUPPORTED.  So does a problem so large
 *     that one of its launches would exceed the device's grid (a launch counts
 *     its work-items in 32 bits).  In round numbers: a prefill of 2^21 or more
 *     (sequence, value head) pairs or of more than about 2^28.4 / Hk tokens (22M
 *     at Hk = 16); from 2^24 (entry, value head) pairs of a decode step or a
 *     fused decode step, 2^31 rows of a gated
 *     RMS-norm or 2^26 / Hkv tokens of an attention prefill on.
 *   - Sizes: a call takes at most INT32_MAX tokens (cu_seqlens are int32); more
 *     is AGNES_ERR_INVALID_ARG.  A buffer whose extent, from its size and
 *     stride, runs past the end of the address space is AGNES_ERR_INVALID_ARG
 *     too (it overlaps everything).  The workspace size queries return 0 for
 *     every problem the matching call rejects.
 */
#ifndef AGNES_GDN_H
#define AGNES_GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum agnes_status {
  AGNES_OK = 0,
  AGNES_ERR_INVALID_ARG = -1, /* NULL / misaligned pointer, bad size, stride or overlap */
  AGNES_ERR_UNSUPPORTED = -2, /* valid request outside the supported set       */
  AGNES_ERR_WORKSPACE = -3,   /* workspace smaller than the size query returned */
  AGNES_ERR_HIP = -4          /* a HIP launch failed; see agnes_gdn_last_hip_error */
} agnes_status;

typedef enum agnes_dtype {
  AGNES_F32 = 0,  /* IEEE binary32 */
  AGNES_BF16 = 1, /* bfloat16 (top half of binary32); stores round to nearest even */
  /* Not a type.  It widens the enum to every value from 0 to INT32_MAX, so that any such
   * value a caller passes is a valid object of this type (C++ leaves values beyond an enum's
   * range undefined); the calls reject everything but the two types above. */
  AGNES_DTYPE_MAX_ENUM = 0x7fffffff
} agnes_dtype;

/*
 * agnes_gdn_conv — depth-wise causal convolution + SiLU, then optional per-head
 * L2 normalisation (model card 架构 table, delta-rule row: causal conv of
 * kernel 4 in front of the recurrence).
 *
 *   y[t, c] = SiLU(bias[c] + sum_{j=0}^{K-1} w[c, j] * xh[t - (K-1) + j, c])
 *
 * with xh = x inside the token's sequence and, before the sequence's first
 * token, the sequence's conv history (conv_state, oldest first; zeros when
 * conv_state is NULL).  w[c, K-1] multiplies the current token.  Nothing
 * crosses a sequence boundary.  Then each of the first `l2norm_heads` groups of
 * `head_dim` channels (the q and k heads: 32 for the 16+16 q/k heads) is
 * divided by sqrt(sum of squares + l2norm_eps).  Arithmetic is fp32.
 *
 *   x           [total_tokens rows, channels], row stride x_token_stride elems, `dtype`
 *   y           [total_tokens rows, channels], row stride y_token_stride elems, `dtype`;
 *               must not overlap x
 *   weight      [channels, kernel_size], `dtype`, contiguous
 *   bias        [channels], `dtype`, or NULL (no bias)
 *   cu_seqlens  device int32 [num_seqs + 1] (prefill mode), or NULL for DECODE
 *               mode: num_seqs sequences of exactly one token (total_tokens ==
 *               num_seqs), whose history is conv_state (required).
 *   conv_state  [num_seqs, channels, kernel_size - 1], `dtype`, oldest first, or
 *               NULL (prefill only: zero history, final history not written).
 *               In: each sequence's history.  Out: the last kernel_size-1 inputs
 *               of each sequence (history included for sequences shorter than
 *               kernel_size-1), written after every read of the old contents.
 *   head_dim    channels per head for the L2 step (128); channels must be a
 *               multiple of 8 and l2norm_heads*head_dim <= channels.
 *
 * weight, bias and conv_state need only be 4-byte aligned (x and y 16-byte).
 * When all three that are given are 16-byte aligned, the taps, biases and
 * history are read, and the history written, as 16-byte vectors (measured:
 * decode mode at 256 x 10240 channels 27.5 -> 14.1 us, prefill at 8192 tokens
 * 70.7 -> 59.4 us); otherwise element by element, with the same results.
 */
int agnes_gdn_conv(const void* x, int64_t x_token_stride, void* y, int64_t y_token_stride,
                   agnes_dtype dtype, const void* weight, const void* bias,
                   const int32_t* cu_seqlens, int num_seqs, int64_t total_tokens,
                   int channels, int kernel_size, void* conv_state, int l2norm_heads,
                   int head_dim, float l2norm_eps, void* stream);

/*
 * agnes_gdn_prefill_workspace_size — bytes of device workspace that
 * agnes_gdn_prefill_chunked needs for this problem (may be 0).  Returns 0 and
 * sets nothing for arguments outside the supported set (the call then fails
 * with the matching status).
 */
size_t agnes_gdn_prefill_workspace_size(int num_seqs, int64_t total_tokens, int num_k_heads,
                                        int num_v_heads, int head_dim, agnes_dtype in_dtype);

/*
 * agnes_gdn_prefill_chunked — chunked prefill of the gated delta rule over a
 * packed batch of sequences (discosf article, section 二.1: chunked prefill
 * with chunk 64; model card 架构 table: fp32 state).  Exactly the token
 * recurrence above, re-associated per chunk of 64 tokens (the WY/UT form of
 * Yang et al., "Parallelizing Linear Transformers with the Delta Rule over
 * Sequence Length", NeurIPS 2024, with the gate of Gated Delta Networks).
 *
 *   q, k          [total_tokens, num_k_heads, head_dim], row stride qk_token_stride
 *                 elems (views into the conv output are fine), `in_dtype`
 *   v             [total_tokens, num_v_heads, head_dim], row stride v_token_stride
 *   g, beta       fp32 [total_tokens, num_v_heads] contiguous: log-decay and write strength
 *   cu_seqlens    device int32 [num_seqs + 1] (see conventions)
 *   scale         output multiplier (1.0 = o_t = S_t q_t)
 *   initial_state fp32 [num_seqs, num_v_heads, head_dim(v), head_dim(k)] or NULL (zeros)
 *   final_state   same shape, or NULL (not written).  May alias initial_state
 *                 exactly (in-place update); any other overlap is rejected.
 *   o             [total_tokens, num_v_heads, head_dim] contiguous, `o_dtype`
 *   workspace     device buffer of >= agnes_gdn_prefill_workspace_size() bytes
 *                 (may be NULL when that size is 0)
 *
 * in_dtype BF16 computes the chunk products on fp16 matrix cores with fp32
 * accumulation and an fp32 state; in_dtype F32 computes everything in fp32.
 * Sequences of length 0 pass their initial state (or zeros) to final_state.
 *
 * With bf16 inputs, where the scan leaves a quarter of the device's compute
 * units free and the sequences average at least 512 tokens, the call runs in
 * two stages: the precomputation of the second part of every sequence runs
 * on a side stream of the library's own beside the scan of the first part,
 * and is joined back into `stream` before the second scan; work enqueued on
 * `stream` afterwards sees every result.  Each caller stream gets its own side
 * stream (created with its events on first use, default priority, up to 4 per
 * device; a fifth caller stream shares the least recently used one), so calls
 * on different streams prepare side by side.  Calls enqueue under a lock; the
 * side stream joins a graph capture of `stream`.  Results are bit-identical to
 * the one-stage run.
 */
int agnes_gdn_prefill_chunked(const void* q, const void* k, const void* v, agnes_dtype in_dtype,
                              int64_t qk_token_stride, int64_t v_token_stride,
                              const float* g, const float* beta, const int32_t* cu_seqlens,
                              int num_seqs, int64_t total_tokens, int num_k_heads,
                              int num_v_heads, int head_dim, float scale,
                              const float* initial_state, float* final_state, void* o,
                              agnes_dtype o_dtype, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * agnes_gdn_prefill_fused — agnes_gdn_conv (prefill mode, L2 on the q and k
 * heads) followed by agnes_gdn_prefill_chunked, as one call that never stores
 * the conv output (model card 架构 table, delta-rule row: the kernel-4 causal
 * conv in front of the recurrence; discosf article, section 二.1: chunked
 * prefill, chunk 64).  The conv runs inside the prefill kernels; q, k and v
 * go to the matrix cores as fp16 straight from the fp32 conv result (the
 * separate calls round them to bf16 in between).
 *
 *   x            [total_tokens, C] bf16, C = (2 Hk + Hv) * head_dim channels q (Hk
 *                heads) | k (Hk heads) | v (Hv heads); row stride x_token_stride
 *   conv_weight  [C, 4] bf16 contiguous;  conv_bias [C] bf16 or NULL
 *   conv_state   [num_seqs, C, 3] bf16 contiguous, oldest first, or NULL (zero
 *                history, final history not written).  In: each sequence's
 *                history.  Out: the last 3 inputs of each sequence (history
 *                included for sequences shorter than 3), written after every read
 *                of the old contents.
 *   l2norm_eps   the q/k L2 norm divides by sqrt(sum of squares + l2norm_eps)
 *   the rest     as agnes_gdn_prefill_chunked (same workspace size query with
 *                in_dtype AGNES_BF16; the same two-stage execution).
 * Supported: bf16 x (AGNES_ERR_UNSUPPORTED otherwise), head_dim 128, Hv a multiple of Hk.
 */
int agnes_gdn_prefill_fused(const void* x, int64_t x_token_stride, agnes_dtype dtype,
                            const void* conv_weight, const void* conv_bias, void* conv_state,
                            const float* g, const float* beta, const int32_t* cu_seqlens,
                            int num_seqs, int64_t total_tokens, int num_k_heads, int num_v_heads,
                            int head_dim, float scale, float l2norm_eps,
                            const float* initial_state, float* final_state, void* o,
                            agnes_dtype o_dtype, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * agnes_gdn_decode_step — one stepwise decode token for each of `batch`
 * independent sequences (discosf article, section 二.1: stepwise decode path),
 * updating each fp32 state in place with one read and one write:
 *
 *   d_i = beta (v_i - alpha (S k)_i);  o_i = scale (alpha (S q)_i + d_i (k . q));
 *   S_i <- alpha S_i + d_i k^T       (row i = value dim)
 *
 *   q, k   [batch, num_k_heads, head_dim], row stride qk_token_stride elems, `in_dtype`
 *   v      [batch, num_v_heads, head_dim], row stride v_token_stride elems
 *   g, beta fp32 [batch, num_v_heads] contiguous
 *   state  fp32 [batch, num_v_heads, head_dim(v), head_dim(k)], updated in place
 *   o      [batch, num_v_heads, head_dim] contiguous, `o_dtype`
 */
int agnes_gdn_decode_step(const void* q, const void* k, const void* v, agnes_dtype in_dtype,
                          int64_t qk_token_stride, int64_t v_token_stride,
                          const float* g, const float* beta, int batch, int num_k_heads,
                          int num_v_heads, int head_dim, float scale, float* state,
                          void* o, agnes_dtype o_dtype, void* stream);

/*
 * agnes_gdn_gated_rmsnorm — gated RMS-norm after the recurrence (model card
 * 架构 table, delta-rule row), per row of `dim` values:
 *
 *   y = o / sqrt(mean(o^2) + eps) * weight * z * sigmoid(z)
 *
 *   o       [rows, dim] contiguous, `o_dtype`   (rows = tokens * value heads)
 *   z       [rows, dim] contiguous, `zw_dtype`  (the gate)
 *   weight  [dim], `zw_dtype`, shared by all rows
 *   y       [rows, dim] contiguous, `y_dtype`; may alias o exactly when o_dtype == y_dtype
 *   dim     128
 */
int agnes_gdn_gated_rmsnorm(const void* o, agnes_dtype o_dtype, const void* z,
                            const void* weight, agnes_dtype zw_dtype, float eps, int64_t rows,
                            int dim, void* y, agnes_dtype y_dtype, void* stream);

/*
 * agnes_gdn_decode_fused — one decode token per batch entry through the whole
 * delta layer in two launches (discosf article, section 二.1: stepwise
 * decode; model card 架构 table, delta-rule row: kernel-4 causal conv in front,
 * gated RMS-norm behind, fp32 state).  For each entry b with slot s:
 *
 *   u = SiLU(conv(x[b], conv_state[s]))   over the q | k | v channels, and the
 *       conv history of slot s advanced by x[b] (oldest first);
 *   q, k = the q and k heads of u, each divided by sqrt(sum of squares + l2norm_eps);
 *   the gated delta-rule step of agnes_gdn_decode_step on state[s] (in place),
 *       giving o (o = scale * S q);
 *   y = o / sqrt(mean(o^2) + norm_eps) * norm_weight * SiLU(z[b])  per value head.
 *
 * The same arithmetic as agnes_gdn_conv (decode mode, l2norm_heads = 2 Hk) ->
 * agnes_gdn_decode_step -> agnes_gdn_gated_rmsnorm, except that q, k, v and o
 * stay fp32 between the steps instead of being stored in `dtype`.
 *
 *   x            [batch, C] with C = (2 Hk + Hv) * head_dim: channels q (Hk heads),
 *                k (Hk heads), v (Hv heads); row stride x_token_stride elems, `dtype`
 *   conv_weight  [C, 4] contiguous, `dtype`;  conv_bias [C] `dtype` or NULL
 *   conv_state   [num_slots, C, 3] contiguous, `dtype`, oldest first; in place
 *   g, beta      fp32 [batch, Hv] contiguous
 *   z            [batch, Hv, head_dim] contiguous, `dtype` (the norm's gate)
 *   norm_weight  [head_dim], `dtype`
 *   state        fp32 [num_slots, Hv, head_dim(v), head_dim(k)] contiguous; in place
 *   slots        device int32 [batch]: the state / conv-history slot of each
 *                entry, or NULL (slot = entry index; then num_slots >= batch).
 *                An entry whose slot is negative or >= num_slots is padding: its
 *                y (and o) rows are written as zeros and nothing else is touched.
 *                Two entries naming the same slot race (unspecified results).
 *   y            [batch, Hv, head_dim] contiguous, `o_dtype`
 *   o            [batch, Hv, head_dim] contiguous, `o_dtype`, or NULL: the
 *                recurrence output before the norm
 * Supported: head_dim 128, Hv a multiple of Hk.
 * Slots exist for a serving pool in which a sequence keeps its caches at a
 * fixed slot while the batch composition changes from step to step.
 */
int agnes_gdn_decode_fused(const void* x, int64_t x_token_stride, agnes_dtype dtype,
                           const void* conv_weight, const void* conv_bias, void* conv_state,
                           const float* g, const float* beta, const void* z,
                           const void* norm_weight, float* state, const int32_t* slots,
                           int num_slots, int batch, int num_k_heads, int num_v_heads,
                           int head_dim, float scale, float l2norm_eps, float norm_eps,
                           void* y, void* o, agnes_dtype o_dtype, void* stream);

/* Human-readable name of an agnes_status value (static string). */
/*
 * agnes_gdn_layer_prefill_workspace_size — bytes of device workspace
 * agnes_gdn_layer_prefill needs (0 for an empty batch or arguments outside the
 * supported set).
 */
size_t agnes_gdn_layer_prefill_workspace_size(int num_seqs, int64_t total_tokens, int num_k_heads,
                                              int num_v_heads, int head_dim);

/*
 * agnes_gdn_layer_prefill — the whole delta-rule layer in prefill mode: the
 * causal conv + SiLU + L2 of q, k, the chunked gated delta rule and the gated
 * RMSNorm (model card "Agnes-3.0-Flash Preview", 架构 table, delta-rule row:
 * conv in front, gated RMS-norm behind; discosf article, section 二.1: chunked
 * prefill, chunk 64), with the recurrence output normalised inside the prefill:
 * o need not go to memory.
 *
 *   x ... final_state   as agnes_gdn_prefill_fused
 *   z             bf16 [total_tokens, num_v_heads, head_dim], row stride z_token_stride
 *   norm_weight   bf16 [head_dim];  norm_eps as agnes_gdn_gated_rmsnorm
 *   y             [total_tokens, num_v_heads, head_dim] contiguous, out_dtype:
 *                 y = o / sqrt(mean(o^2) + norm_eps) * w * silu(z) per head row
 *   o             the same shape and out_dtype, or NULL (not written)
 *   workspace     >= agnes_gdn_layer_prefill_workspace_size() bytes, 256-byte aligned
 *
 * The four workgroups that share a value head exchange per-token partial sums
 * of squares through the workspace; they take their roles in the order they
 * start, so any batch size runs (no co-residency of the grid is assumed).
 * Errors as agnes_gdn_prefill_fused; the workspace is cleared by the call.
 *
 * Runs in two stages where agnes_gdn_prefill_chunked does (same side stream,
 * same guarantees).
 */
int agnes_gdn_layer_prefill(const void* x, int64_t x_token_stride, agnes_dtype dtype,
                            const void* conv_weight, const void* conv_bias, void* conv_state,
                            const float* g, const float* beta, const int32_t* cu_seqlens,
                            int num_seqs, int64_t total_tokens, int num_k_heads, int num_v_heads,
                            int head_dim, float scale, float l2norm_eps,
                            const float* initial_state, float* final_state, const void* z,
                            int64_t z_token_stride, const void* norm_weight, float norm_eps,
                            void* y, void* o, agnes_dtype out_dtype, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * agnes_gdn_layer_prefill_noalloc — agnes_gdn_layer_prefill for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments and results without the workspace, which is instead a fixed
 * 64 MiB array in device memory that the library's code object brings with it, one per device
 * (held until the process ends).  The call allocates, frees and creates nothing: it always runs
 * in one stage (no side stream) and looks the array's address up on its first call on a device.
 *
 *   Supported: problems whose agnes_gdn_layer_prefill_workspace_size is at most 64 MiB (one
 *   sequence of up to about 2400 tokens of the 16 / 48-head layer); larger ones return
 *   AGNES_ERR_UNSUPPORTED and launch nothing.
 *   Every call on a device uses that device's one array: calls that may overlap in time on one
 *   device (on different streams, or from several threads) race and give unspecified results.
 *   Each call clears what it needs cleared; the array keeps the last call's contents.
 */
int agnes_gdn_layer_prefill_noalloc(const void* x, int64_t x_token_stride, agnes_dtype dtype,
                                    const void* conv_weight, const void* conv_bias, void* conv_state,
                                    const float* g, const float* beta, const int32_t* cu_seqlens,
                                    int num_seqs, int64_t total_tokens, int num_k_heads,
                                    int num_v_heads, int head_dim, float scale, float l2norm_eps,
                                    const float* initial_state, float* final_state, const void* z,
                                    int64_t z_token_stride, const void* norm_weight, float norm_eps,
                                    void* y, void* o, agnes_dtype out_dtype, void* stream);

/*
 * agnes_attn_prefill_workspace_size — bytes of device workspace agnes_attn_prefill
 * needs (0 for an empty batch or more than INT32_MAX tokens).
 */
size_t agnes_attn_prefill_workspace_size(int num_seqs, int64_t total_tokens);

/*
 * agnes_attn_prefill — the global attention layer over a packed batch (model card
 * "Agnes-3.0-Flash Preview", 架构 table, rows 全局注意力 and 位置编码; discosf
 * article, section 二.1): RMS-norm of every q and k head, three-axis rotary on
 * their first rot_dim dims, causal softmax attention inside each sequence
 * (query head h reads KV head h / (num_q_heads / num_kv_heads)), and the output
 * times sigmoid(gate).
 *
 *   q, gate        bf16 [total_tokens, num_q_heads, head_dim], row strides
 *                  q_token_stride, gate_token_stride (elements, multiples of 8)
 *   k, v           bf16 [total_tokens, num_kv_heads, head_dim], row strides
 *                  k_token_stride, v_token_stride
 *   q_norm_weight, k_norm_weight   bf16 [head_dim]: x / sqrt(mean(x^2) + norm_eps) * w
 *   positions      device int32 [3][positions_stride] (text, height, width) per
 *                  token, or NULL for text (the index in the sequence on all
 *                  three axes).  Frequency j < rot_dim/2 turns dims j and
 *                  j + rot_dim/2 by position(axis j mod 3) * rope_base^(-2j/rot_dim);
 *                  the angles are formed in fp64.
 *   cu_seqlens     device int32 [num_seqs + 1], cu[0] = 0, nondecreasing
 *   scale          softmax scale; <= 0 selects 1/sqrt(head_dim)
 *   k_out          bf16 [total_tokens, num_kv_heads, head_dim], row stride
 *                  k_out_token_stride: receives the normalised, rotated k (the KV
 *                  cache rows); the attention reads it, so it is required
 *   v_out          optional bf16 copy of v (row stride v_out_token_stride), or NULL
 *   o              [total_tokens, num_q_heads, head_dim] contiguous, o_dtype
 *   workspace      >= agnes_attn_prefill_workspace_size() bytes, 256-byte aligned
 *
 * Supported: head_dim 256, rot_dim 64, num_q_heads % num_kv_heads == 0, token
 * strides of q, k, v and k_out up to 2^24 elements.  The
 * products run on bf16 matrix cores with fp32 accumulation: q after norm and
 * rotary, k as stored in k_out, v, and the softmax weights are bf16 operands;
 * the softmax statistics are fp32.  k_out, v_out and o must not overlap any
 * input or each other.
 */
int agnes_attn_prefill(const void* q, int64_t q_token_stride, const void* k, int64_t k_token_stride,
                       const void* v, int64_t v_token_stride, const void* gate,
                       int64_t gate_token_stride, const void* q_norm_weight,
                       const void* k_norm_weight, const int32_t* positions,
                       int64_t positions_stride, const int32_t* cu_seqlens, int num_seqs,
                       int64_t total_tokens, int num_q_heads, int num_kv_heads, int head_dim,
                       int rot_dim, float rope_base, float norm_eps, float scale, void* k_out,
                       int64_t k_out_token_stride, void* v_out, int64_t v_out_token_stride,
                       void* o, agnes_dtype o_dtype, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * agnes_attn_decode_workspace_size — bytes of device workspace agnes_attn_decode
 * needs for this batch, head count and cache length (0 for an empty batch and
 * for counts outside the supported set).
 */
size_t agnes_attn_decode_workspace_size(int batch, int num_q_heads, int num_kv_heads,
                                        int64_t max_len);

/*
 * agnes_attn_decode — one decode step of the global attention layer (model card
 * "Agnes-3.0-Flash Preview", 架构 table, rows 全局注意力 and 位置编码; discosf
 * article, section 二.1: only these layers keep a KV cache).  For each batch
 * entry b with L = cache_lens[b] tokens cached: the new token's q and k are
 * RMS-normed and rotated at position L (or positions[.][b]), its k and v are
 * written into the caches at index L, and its output is the softmax attention
 * over the L + 1 cached keys, times sigmoid(gate).
 *
 *   q, gate        bf16 [batch, num_q_heads, head_dim], row strides in elements
 *   k, v           bf16 [batch, num_kv_heads, head_dim], row strides in elements
 *   q_norm_weight, k_norm_weight, rope_base, norm_eps, scale   as agnes_attn_prefill
 *   positions      device int32 [3][positions_stride] per entry, or NULL (L on
 *                  all three axes)
 *   k_cache, v_cache  bf16 [batch, max_len, num_kv_heads, head_dim] contiguous;
 *                  row L of entry b is written (k normalised and rotated, v as given)
 *   cache_lens     device int32 [batch]; an entry with a length outside
 *                  [0, max_len) is padding: its o is zero and no cache row changes
 *   o              [batch, num_q_heads, head_dim] contiguous, o_dtype
 *   workspace      >= agnes_attn_decode_workspace_size() bytes, 256-byte aligned
 *
 * The caller advances cache_lens after the call.  Same supported set and number
 * formats as agnes_attn_prefill.  o, the caches and the inputs must not overlap.
 */
int agnes_attn_decode(const void* q, int64_t q_stride, const void* k, int64_t k_stride,
                      const void* v, int64_t v_stride, const void* gate, int64_t gate_stride,
                      const void* q_norm_weight, const void* k_norm_weight,
                      const int32_t* positions, int64_t positions_stride, void* k_cache,
                      void* v_cache, int64_t max_len, const int32_t* cache_lens, int batch,
                      int num_q_heads, int num_kv_heads, int head_dim, int rot_dim,
                      float rope_base, float norm_eps, float scale, void* o, agnes_dtype o_dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Status of a bf16 prefill call (agnes_gdn_prefill_chunked with in_dtype BF16,
 * agnes_gdn_prefill_fused, agnes_gdn_layer_prefill): the call clears a status word at the start
 * of its workspace and its kernels set these sticky bits in it.
 *
 *   AGNES_WS_WAIT_LDS       a bounded wait for another wave of the same workgroup gave up
 *   AGNES_WS_WAIT_EXCHANGE  (whole-layer call) a bounded wait for the partial sums of squares of
 *                           another workgroup of the same value head gave up
 *   AGNES_WS_WAIT_ROLE      (whole-layer call) a workgroup found no role to take and returned
 *                           without touching any buffer
 *   AGNES_WS_RANGE          a value on the fp16 matrix-core path was outside +-65504 or not
 *                           finite: a bf16 q/k input of magnitude >= 65536 (plain call), an
 *                           entry of the chunk-local factors P = exp(gamma_r - gamma_s) q_r.k_s
 *                           or X = (I + A)^-1 (checked where they are formed: positive log-decays
 *                           whose sum within a chunk exceeds ~11 overflow P), or the state of a
 *                           sequence at its end (an fp16 state or U operand out of range anywhere
 *                           in the sequence leaves the fp32 state non-finite there).  Inputs that
 *                           are not finite also set it.
 *
 * A wait gives up only after its bound (about 10^6..10^7 polls of ~30 ns): with a correct
 * workspace and grid it never does.  Any bit set means the outputs of that call are not
 * reliable.  The fp16 domain in which every bit stays clear: |q|, |k| < 65504 (the layer's q
 * and k are unit vectors), |v|, |state| and |U| (the delta-corrected values) < 65504, and
 * log-decays g <= 0 or small enough that no chunk's in-chunk decay sum exceeds ~11.
 */
enum {
  AGNES_WS_WAIT_LDS = 1,
  AGNES_WS_WAIT_EXCHANGE = 2,
  AGNES_WS_WAIT_ROLE = 4,
  AGNES_WS_RANGE = 8
};

/*
 * agnes_gdn_workspace_status — waits for the work enqueued on `stream` to finish (this call
 * synchronises `stream`, unlike every other call), then stores the status word of a bf16
 * prefill workspace (the first 4 bytes of `workspace`, device memory) in *flags (host).  Call it
 * after the prefill call whose workspace it is; another call on the same workspace clears it.
 * Returns AGNES_ERR_INVALID_ARG for a NULL or misaligned pointer, AGNES_ERR_HIP if the copy
 * fails.
 */
int agnes_gdn_workspace_status(const void* workspace, uint32_t* flags, void* stream);

/*
 * agnes_gdn_set_wait_limit — process-wide bound on the polls of every bounded wait of the bf16
 * prefill calls launched after it (0: each wait's own bound, the default).  For tests and
 * debugging of the status bits: a small bound makes the waits give up, the kernels still end
 * normally, and the results are then unreliable.  Not meant to change while calls are being
 * launched from other threads.  Returns AGNES_OK.
 */
int agnes_gdn_set_wait_limit(uint32_t polls);

/*
 * agnes_gdn_set_prefill_stages — process-wide stage cuts of the bf16 prefill calls launched
 * after it (agnes_gdn_prefill_chunked, agnes_gdn_prefill_fused and the whole-layer calls).  When
 * the scan of a call leaves a quarter of the compute units free and its sequences average at
 * least 8 chunks, the call runs in n_cuts + 1 stages: stage k covers chunks
 * [cuts[k-1], cuts[k]) in 1/40ths of each sequence's chunk count (cuts[-1] = 0, cuts[n_cuts] =
 * 40), the preparation of stage k + 1 overlapping the scan of stage k on a side stream and the
 * state carried between stages in the workspace.  The stages change the schedule only: the
 * results are the same bit for bit.  `cuts` (host, n_cuts values) must increase strictly inside
 * (0, 40), 0 <= n_cuts <= 7; n_cuts = 0 runs every call in one stage; once set, the cuts apply
 * to every kind of call.  n_cuts = -1 (`cuts` not read) restores the defaults: one cut at 26 for
 * the whole-layer calls (two stages, the first 13/20 of the chunks) and at 28 for the two prefill
 * calls (7/10).  Not meant to change while calls are being launched from other threads.  Returns
 * AGNES_OK, or AGNES_ERR_INVALID_ARG (nothing changed) for any other list.
 */
int agnes_gdn_set_prefill_stages(const int32_t* cuts, int n_cuts);

/*
 * Measurement kernels: the two ceilings the benchmark reports its roofline fractions against,
 * measured on the machine itself beside the vendor's peaks.
 *
 * agnes_gdn_ceiling_rmw_stream — every 16-byte vector of `buf` (device, `bytes` a multiple of
 * 16, 16-byte aligned) read once and written back once (multiplied by 1.0, so the contents are
 * unchanged): the access pattern of the decode step's in-place state update.  Bytes moved per
 * call: 2 * bytes.
 *
 * agnes_gdn_ceiling_mfma — `blocks` workgroups of four waves, each wave issuing `iters` rounds of
 * 8 independent bf16 16x16x32 matrix-core products on operands held in registers (each
 * accumulator reused 8 products later).  FLOPs per call: blocks * 4 * iters * 8 * 16384.  One
 * float per wave is written to `sink` (device, blocks * 4 floats).
 *
 * Both return AGNES_ERR_INVALID_ARG for a NULL or misaligned buffer, a size that is not a
 * multiple of 16, or blocks / iters outside [1, 2^20]; AGNES_ERR_HIP if the launch fails.
 */
int agnes_gdn_ceiling_rmw_stream(void* buf, size_t bytes, void* stream);
int agnes_gdn_ceiling_mfma(float* sink, int blocks, int iters, void* stream);

/*
 * agnes_gdn_release — destroys the HIP objects the library keeps between calls: the side streams
 * and their events that the calls in stages create on first use (after waiting for the work on
 * each stream).  A later call in stages creates them again.  Call it when no
 * call of the library is in flight, e.g. before the process exits, so that no library handle is
 * left for the runtime's own teardown; it makes no HIP call when nothing was created.  Returns
 * AGNES_OK, or AGNES_ERR_HIP if a destroy fails.
 */
int agnes_gdn_release(void);

const char* agnes_gdn_status_string(int status);

/* hipError_t of the last AGNES_ERR_HIP returned on the calling thread (0 if none). */
int agnes_gdn_last_hip_error(void);

/* Library version string, e.g. "0.1.0". */
const char* agnes_gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* AGNES_GDN_H */
