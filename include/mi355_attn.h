/* mi355_attn.h - C ABI of the MI355X (gfx950) scaled dot-product / multi-head attention library (attention forward
 * and backward, multi-head attention forward, the encoder layer around it).
 *
 * What is computed (sources are web pages about "Attention Is All You Need"):
 *   Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V
 *     - "Attention Is All You Need" (lettle.cn translation), section 3.2.1 Scaled Dot-Product Attention, the
 *       Attention(Q,K,V) equation: dot products of each query with all keys, each divided by sqrt(d_k), a softmax
 *       over the keys, and the weighted sum of the values.
 *   Causal mask: for decoder self-attention the score of key j for query i is set to -inf before the softmax when
 *   j > i, so its weight is exactly 0; position i sees itself and everything before it.
 *     - "Transformer：抛弃循环与卷积的序列建模" (jiashun-ye.github.io), section "Transformer 中的三种 Attention", and the
 *       mask matrix M of its training example (section "训练样本").
 *   MultiHead(Q, K, V) = Concat(head_1, ..., head_h) W^O,  head_i = Attention(Xq W_i^Q, Xkv W_i^K, Xkv W_i^V)
 *     - same page, section "Multi-Head Attention"; lettle.cn translation section 3.2.2. Queries come from Xq, keys and
 *       values from Xkv: Xkv == Xq for self-attention, the encoder output for encoder-decoder attention (section
 *       "Transformer 中的三种 Attention").
 *   Backward pass: the gradients of a loss L with respect to Q, K and V given dL/dO, by the chain rule through the
 *   forward computation (the step of training that carries the loss back through attention).
 *     - "Transformer：抛弃循环与卷积的序列建模", section "训练样本", subsection "反向传播".
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library never allocates, frees or copies
 *     caller memory and never synchronises the stream. Work is enqueued on `stream` (a hipStream_t; NULL means the
 *     default stream) and the call returns before it finishes.
 *   - Tensors are dense, row-major, in the element type `dtype` (ATTN_F32: IEEE float32; ATTN_BF16: bfloat16 bit
 *     patterns, accumulation in float32). Every pointer must be 16-byte aligned.
 *   - A non-zero return is an attn_status. Argument errors are detected before any HIP call, and nothing has been
 *     enqueued or written when they are returned. ATTN_ERR_HIP means a HIP call (the launch) failed; faults while the
 *     kernels run show up at the caller's next synchronisation, as for any asynchronous HIP work.
 *   - attn_last_error() gives a thread-local, human-readable detail for the most recent non-OK return.
 *   - No C++ exception crosses this interface. The library keeps no state besides that thread-local string.
 */
#ifndef MI355_ATTN_H
#define MI355_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID = 1,     /* null pointer, non-positive size, misaligned pointer, output overlapping an input,
                               unknown mask kind, workspace too small */
  ATTN_ERR_UNSUPPORTED = 2, /* valid request this library does not implement: dtype other than F32/BF16, head dims
                               other than those an entry point lists, causal mask with n_q != n_k, sizes beyond the
                               limits below */
  ATTN_ERR_HIP = 3          /* a HIP runtime call failed */
} attn_status;

typedef enum { ATTN_MASK_NONE = 0, ATTN_MASK_CAUSAL = 1 } attn_mask_kind;
typedef enum {
  ATTN_F32 = 0,
  ATTN_BF16 = 1,
  ATTN_BF16_F32O = 2 /* sdpa_backward only: bf16 tensors except O, which is the float32 forward output (out_f32 of
                        sdpa_forward_train) */
} attn_dtype;

/* Size limits (ATTN_ERR_UNSUPPORTED beyond them). */
#define ATTN_MAX_SEQ   (1 << 24) /* n_q, n_k */
#define ATTN_MAX_HEADS 65536     /* B * h */

/* sdpa_forward: scaled dot-product attention of every (batch, head) pair.
 *   Q   [B, h, n_q, d_k]   queries
 *   K   [B, h, n_k, d_k]   keys
 *   V   [B, h, n_k, d_v]   values
 *   out [B, h, n_q, d_v]   out[b,h,i,:] = sum_j softmax_j(Q[b,h,i,:] . K[b,h,j,:] / sqrt(d_k)) V[b,h,j,:]
 *   mask_kind: ATTN_MASK_NONE, or ATTN_MASK_CAUSAL (keys j > i excluded; requires n_q == n_k).
 *   dtype: ATTN_BF16 (bf16 in/out, float32 scores, softmax and accumulation; the softmax weights are rounded to
 *          bf16 before they multiply V) or ATTN_F32 (float32 throughout).
 *   Head widths: d_k = d_v, one of 32, 64, 128: d_model = 512 split over h = 16, 8 or 4 heads, the head-count
 *   variants that keep the total work about constant ("Transformer：抛弃循环与卷积的序列建模", section
 *   "模型变体与消融实验"); the base model uses 64. `out` must not overlap Q, K or V. */
int sdpa_forward(const void* Q, const void* K, const void* V, int mask_kind, void* out, int dtype,
                 int64_t B, int64_t h, int64_t n_q, int64_t n_k, int64_t d_k, int64_t d_v, void* stream);

/* sdpa_forward_lse: sdpa_forward that also writes the row log-sum-exp of the scaled scores,
 *   lse [B, h, n_q] float32 (natural log): lse[b,h,i] = log sum_j exp(Q[b,h,i,:] . K[b,h,j,:] / sqrt(d_k)) over the
 *   keys row i may see, so that the weights are exp(score - lse). It is the statistic sdpa_backward needs.
 *   For ATTN_BF16 the sum is that of the bf16-rounded weights the kernel multiplies V with, so that the weights the
 *   backward pass recomputes are those of the forward output.
 *   Other arguments, requirements and errors as sdpa_forward; `lse` must not overlap any other tensor. */
int sdpa_forward_lse(const void* Q, const void* K, const void* V, int mask_kind, void* out, float* lse, int dtype,
                     int64_t B, int64_t h, int64_t n_q, int64_t n_k, int64_t d_k, int64_t d_v, void* stream);

/* sdpa_forward_padded: sdpa_forward with a key padding mask, for batches of sequences of different lengths padded to
 * n_k ("Transformer：抛弃循环与卷积的序列建模", section "训练样本": <PAD> positions that fill a batch are excluded by
 * a padding mask; section "训练配置": batches group sequences of similar length).
 *   kv_len [B] int32, device: batch entry b has min(max(kv_len[b], 0), n_k) real keys; keys j >= kv_len[b] get weight
 *          exactly 0, their K and V rows are never read (any contents, NaN included, are fine) and key tiles wholly
 *          past the length cost nothing. A row left with no key (kv_len[b] <= 0) gets output 0 (and lse -inf).
 *          Query rows are not masked: every row's output is computed over its batch entry's real keys.
 *   lse: optional (NULL: not written); as for sdpa_forward_lse.
 *   Combined with ATTN_MASK_CAUSAL, query i sees keys j <= i with j < kv_len[b].
 *   Other arguments, requirements and errors as sdpa_forward_lse; kv_len must not overlap out or lse. */
int sdpa_forward_padded(const void* Q, const void* K, const void* V, const int32_t* kv_len, int mask_kind, void* out,
                        float* lse, int dtype, int64_t B, int64_t h, int64_t n_q, int64_t n_k, int64_t d_k,
                        int64_t d_v, void* stream);

/* sdpa_forward_window: restricted self-attention ("Transformer：抛弃循环与卷积的序列建模", section "Self-Attention的优势":
 * each position attends only to a neighbourhood of size r, at cost O(r n d); section "总结": proposed for very long
 * sequences). Query i sees keys j with |i - j| <= window (a band of 2 window + 1 keys centred on i, clipped at the
 * ends); with ATTN_MASK_CAUSAL also j <= i, i.e. keys i - window .. i. Key tiles outside every band of a workgroup
 * are never read.
 *   window >= 0 (ATTN_ERR_INVALID otherwise); requires n_q == n_k (ATTN_ERR_UNSUPPORTED otherwise).
 *   lse: optional (NULL: not written), as for sdpa_forward_lse.
 *   Other arguments, requirements and errors as sdpa_forward. */
int sdpa_forward_window(const void* Q, const void* K, const void* V, int64_t window, int mask_kind, void* out,
                        float* lse, int dtype, int64_t B, int64_t h, int64_t n_q, int64_t n_k, int64_t d_k,
                        int64_t d_v, void* stream);

/* sdpa_forward_train: the forward pass of training, in one entry point for every mask: sdpa_forward_lse,
 * sdpa_forward_padded (kv_len != NULL) or sdpa_forward_window (window >= 0), which can also keep the output before
 * its rounding to bf16 for the backward pass ("Transformer：抛弃循环与卷积的序列建模", section "训练样本", subsection
 * "反向传播": the loss is carried back through the forward computation, which needs what the forward pass produced).
 *   kv_len: NULL or the key padding, as for sdpa_forward_padded.
 *   window: -1 for none, or the radius of restricted self-attention as for sdpa_forward_window (requires n_q == n_k
 *           and kv_len == NULL: ATTN_ERR_UNSUPPORTED otherwise).
 *   out [B, h, n_q, d_v] in dtype, and lse [B, h, n_q] float32 (required), as for sdpa_forward_lse.
 *   out_f32: NULL, or for ATTN_BF16 a float32 [B, h, n_q, d_v] tensor that receives the output before it is rounded
 *            to bf16 (out is exactly its round-to-nearest-even). Passing it to sdpa_backward with dtype
 *            ATTN_BF16_F32O lets the backward pass form D_i = dO_i . O_i from the unrounded output: where the weights
 *            are nearly one-hot, dP - D is a small difference of two nearly equal numbers and the bf16 rounding of
 *            O would dominate it. ATTN_F32 with out_f32 != NULL: ATTN_ERR_INVALID.
 *   Other arguments, requirements and errors as sdpa_forward_lse; out_f32 must not overlap any other tensor. */
int sdpa_forward_train(const void* Q, const void* K, const void* V, const int32_t* kv_len, int64_t window,
                       int mask_kind, void* out, float* out_f32, float* lse, int dtype, int64_t B, int64_t h,
                       int64_t n_q, int64_t n_k, int64_t d_k, int64_t d_v, void* stream);

/* sdpa_backward: gradients of attention.
 *   Q, K, V      the forward inputs, as for sdpa_forward
 *   O   [B, h, n_q, d_v]  the forward output and lse [B, h, n_q] float32 its row log-sum-exp (sdpa_forward_lse, or
 *                         sdpa_forward_padded with the same kv_len, on the same Q, K, V and mask_kind)
 *   kv_len [B] int32 or NULL: the key padding of the forward pass (NULL: none); gradients of padding keys' K and V
 *          rows are written as 0, and rows that saw no key pass no gradient
 *   window: the radius of a restricted self-attention forward pass (sdpa_forward_window), or -1 for none; >= 0
 *          requires n_q == n_k and kv_len == NULL (ATTN_ERR_UNSUPPORTED otherwise)
 *   dO  [B, h, n_q, d_v]  dL/dO, the upstream gradient
 *   dQ  [B, h, n_q, d_k], dK [B, h, n_k, d_k], dV [B, h, n_k, d_v]: written with dL/dQ, dL/dK, dL/dV:
 *       P = exp(Q K^T / sqrt(d_k) - lse) (0 where masked), dV = P^T dO, dP = dO V^T,
 *       dS = P o (dP - D) with D_i = dO_i . O_i, dQ = dS K / sqrt(d_k), dK = dS^T Q / sqrt(d_k).
 *   workspace: device scratch of at least sdpa_backward_workspace_size(...) bytes, 16-byte aligned, owned by the
 *              caller (it holds per-row lse and D between the three launches).
 *   dtype: ATTN_BF16 (bf16 tensors, float32 accumulation, P and dS rounded to bf16 where they enter the matrix core,
 *          outputs rounded to nearest even), ATTN_BF16_F32O (the same, but O is the float32 out_f32 of
 *          sdpa_forward_train, so D is formed from the unrounded output) or ATTN_F32 (float32 throughout). lse is
 *          float32 in all three.
 *   Requirements as sdpa_forward (d_k = d_v in {32, 64, 128}). dQ, dK, dV and the
 *   workspace must not overlap each other or any input. Every element of dQ, dK and dV is written. */
int sdpa_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* lse,
                  const int32_t* kv_len, int64_t window, int mask_kind, void* dQ, void* dK, void* dV, void* workspace,
                  size_t workspace_bytes, int dtype, int64_t B, int64_t h, int64_t n_q, int64_t n_k, int64_t d_k,
                  int64_t d_v, void* stream);

/* Bytes of workspace sdpa_backward needs for these sizes (0 if the sizes are invalid). */
size_t sdpa_backward_workspace_size(int dtype, int64_t B, int64_t h, int64_t n_q, int64_t n_k, int64_t d_k,
                                    int64_t d_v);

/* mha_forward: multi-head attention with learned projections and no biases.
 *   Xq  [B, n_q, d_model]  query-side input; Xkv [B, n_k, d_model] key/value-side input (may be the same pointer
 *                          as Xq for self-attention)
 *   Wq  [d_model, h*d_k]   column block i (columns i*d_k .. i*d_k+d_k-1) is W_i^Q; Wk likewise is W_i^K
 *   Wv  [d_model, h*d_v]   column block i is W_i^V
 *   Wo  [h*d_v, d_model]   output projection W^O; the concat orders head 1..h along its rows' index
 *   out [B, n_q, d_model]  Concat(head_1..head_h) W^O
 *   workspace: device scratch of at least mha_workspace_size(...) bytes, 16-byte aligned, owned by the caller; it
 *              holds the projected Q/K/V (head-major) and the concatenated heads, in `dtype`.
 *   dtype: ATTN_BF16 only (the projections accumulate in float32 and round to bf16).
 *   Requirements: d_k = d_v in {32, 64, 128} with h * d_k a multiple of 64 (the head-count variants of
 *   "Transformer：抛弃循环与卷积的序列建模", section "模型变体与消融实验"), d_model a positive multiple of 64, causal
 *   only with n_q == n_k. `out` must not overlap any input or the workspace, and the workspace must not overlap any
 *   input. */
int mha_forward(const void* Xq, const void* Xkv, const void* Wq, const void* Wk, const void* Wv, const void* Wo,
                int mask_kind, void* out, void* workspace, size_t workspace_bytes, int dtype,
                int64_t B, int64_t n_q, int64_t n_k, int64_t d_model, int64_t h, int64_t d_k, int64_t d_v,
                void* stream);

/* Bytes of workspace mha_forward needs for these sizes (0 if the sizes are invalid). */
size_t mha_workspace_size(int dtype, int64_t B, int64_t n_q, int64_t n_k, int64_t h, int64_t d_k, int64_t d_v);

/* mha_forward_noalloc: mha_forward without a caller workspace, for callers that cannot allocate device memory
 * (code being captured into a HIP graph, tight serving loops, harnesses that forbid allocation). The projected
 * Q/K/V and the concatenated heads go to a scratch array the library holds in device memory: one array of
 * ATTN_NOALLOC_SCRATCH_BYTES per GPU it runs on, kept until the process ends. The call allocates nothing and
 * frees nothing.
 *   Arguments, layouts and requirements as mha_forward, without workspace and workspace_bytes. The sizes must need
 *   at most ATTN_NOALLOC_SCRATCH_BYTES of workspace (mha_workspace_size(...) <= ATTN_NOALLOC_SCRATCH_BYTES; the
 *   base model's B = 32, n = 128, d_model = 512 needs 16 MiB); larger sizes return ATTN_ERR_INVALID before any HIP
 *   call. The scratch of the current device is used, so `stream` must belong to the current device.
 *   Calls on one GPU share its scratch: calls that overlap in time on one GPU (on different streams, or from
 *   different threads) race and must be ordered by the caller. Every byte of scratch a call reads is written earlier
 *   in the same call, so nothing needs clearing between calls.
 *   Errors: as mha_forward; ATTN_ERR_HIP also when the scratch's device address cannot be obtained. */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20) /* 32 MiB */
int mha_forward_noalloc(const void* Xq, const void* Xkv, const void* Wq, const void* Wk, const void* Wv,
                        const void* Wo, int mask_kind, void* out, int dtype, int64_t B, int64_t n_q, int64_t n_k,
                        int64_t d_model, int64_t h, int64_t d_k, int64_t d_v, void* stream);

/* encoder_layer_forward: one Transformer encoder layer in the pages' post-norm form (each sub-layer's output is
 * LayerNorm(x + Sublayer(x)): "Attention Is All You Need", lettle.cn translation, section 3.1; "Transformer：抛弃循环与
 * 卷积的序列建模", sections "FFN" and "Residual Connection 与 LayerNorm"):
 *     H1  = LayerNorm_1(X + MultiHead(X, X, X))            (MultiHead as mha_forward: no biases)
 *     out = LayerNorm_2(H1 + max(0, H1 W1 + b1) W2 + b2)   (the position-wise FFN)
 *   X   [B, n, d_model]; Wq, Wk, Wv, Wo [d_model, d_model] (head i = column block i, as mha_forward)
 *   W1  [d_model, d_ff], b1 [d_ff], W2 [d_ff, d_model], b2 [d_model]
 *   ln1_gamma, ln1_beta, ln2_gamma, ln2_beta [d_model]: LayerNorm(r) = (r - mean) / sqrt(var + eps) * gamma + beta
 *       over the d_model features of each position, var the biased variance (mean squared deviation), eps >= 0
 *   kv_len [B] int32 or NULL: key padding of the self-attention, as sdpa_forward_padded (NULL: none)
 *   mask_kind: ATTN_MASK_NONE (encoder) or ATTN_MASK_CAUSAL (masked self-attention, a decoder-only layer)
 *   out [B, n, d_model]
 *   workspace: at least encoder_layer_workspace_size(...) bytes, 16-byte aligned (per-head Q/K/V, the concatenated
 *              heads, the residual sums, H1 and the FFN hidden activations, all bf16).
 *   dtype: ATTN_BF16 only: every tensor above is bf16; products accumulate in float32, the LayerNorm statistics are
 *          float32, and every intermediate listed for the workspace is rounded to bf16.
 *   Requirements: d_model = d h <= 1024 with head width d in {32, 64, 128} and d_model a multiple of 64, d_ff a
 *   positive multiple of 64. `out` must not overlap any input or the workspace; the workspace must not overlap any
 *   input. */
int encoder_layer_forward(const void* X, const int32_t* kv_len, const void* Wq, const void* Wk, const void* Wv,
                          const void* Wo, const void* ln1_gamma, const void* ln1_beta, const void* W1, const void* b1,
                          const void* W2, const void* b2, const void* ln2_gamma, const void* ln2_beta, float eps,
                          int mask_kind, void* out, void* workspace, size_t workspace_bytes, int dtype, int64_t B,
                          int64_t n, int64_t d_model, int64_t h, int64_t d_ff, void* stream);

/* Bytes of workspace encoder_layer_forward needs for these sizes (0 if the sizes are invalid). */
size_t encoder_layer_workspace_size(int dtype, int64_t B, int64_t n, int64_t d_model, int64_t h, int64_t d_ff);

/* Static string naming an attn_status value. */
const char* attn_status_string(int status);

/* Thread-local detail of the last non-OK return on this thread ("" if none). Valid until the next call on it. */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MI355_ATTN_H */
