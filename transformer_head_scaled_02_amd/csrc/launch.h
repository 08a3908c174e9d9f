// Internal (C++) launch interface between the C-ABI host layer and the kernels. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355 {

// One attention problem over [B, H] heads of width 64. Q/K/V rows are dense (64 elements); the output row of query i
// of head (b, h) starts at O + b*o_stride_b + h*o_stride_h + i*o_stride_row (elements), which covers both the
// [B,h,n_q,64] layout and the concatenated [B,n_q,h*64] layout.
struct AttnArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  int B, H, n_q, n_k;
  int64_t q_stride_bh, k_stride_bh;   // elements between consecutive (b,h) heads of Q and of K/V
  int64_t o_stride_b, o_stride_h, o_stride_row;
  int causal;
  float* lse;  // optional (nullptr: not written): row log-sum-exp of query i of head bh at lse[bh*n_q + i]
  // optional (nullptr: none) key padding: batch entry b has min(max(kv_len[b], 0), n_k) real keys; later keys get
  // weight 0 and are never read; a row with no key to see gets output 0 and lse -inf
  const int* kv_len;
  // restricted self-attention (windowed != 0, n_q == n_k): query i sees keys j with |i - j| <= window only
  int windowed, window;
  // optional (nullptr: not written), bf16 kernels only: the output before its rounding to bf16, float32, dense
  // [B, H, n_q, D] whatever the strides of O (the operand from which the backward pass forms D = dO . O)
  float* o32;
};

// d: the head width d_k = d_v, 32, 64 or 128 (every other value: hipErrorInvalidValue, nothing launched)
hipError_t launch_attn_fwd_bf16(const AttnArgs& a, int d, hipStream_t stream);
hipError_t launch_attn_fwd_f32(const AttnArgs& a, int d, hipStream_t stream);
// Unmasked (optionally key-padded) attention at width 64 with eight-wave ping-pong workgroups of 512 queries
// (causal or windowed arguments: hipErrorInvalidValue, nothing launched)
hipError_t launch_attn_fwd_pp_bf16(const AttnArgs& a, hipStream_t stream);

// Backward pass of attention over [B, H] heads of width d (32, 64 or 128), every tensor dense [B, H, n, d] in the element
// type.
// `aux` is the workspace: per head and per 64-row query tile, 256 floats = [log2(e)*lse of the 64 rows | D of the 64
// rows | per row 8 bytes: -D as three bf16 parts and a zero], where D_i = dO_i . O_i; rows past n_q hold lse = +inf
// and D = 0 (their weights come out 0).
struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* lse;  // [B, H, n_q], natural log
  float* aux;
  void* dQ;
  void* dK;
  void* dV;
  int B, H, n_q, n_k;
  int causal;
  const int* kv_len;  // optional key padding, as in AttnArgs; dK and dV rows of padding keys are written as 0
  int windowed, window;  // optional restricted self-attention, as in AttnArgs
  int o_f32;             // bf16 tensors with O in float32 (AttnArgs::o32 of the forward pass)
};
constexpr int kAuxFloatsPerTile = 256;

// Real keys of batch entry b: n_k, or the clamped padding length.
__device__ __forceinline__ int real_keys(const int* kv_len, int b, int n_k) {
  return kv_len == nullptr ? n_k : min(max(kv_len[b], 0), n_k);
}
// d: the head width, 32, 64 or 128 (every other value: hipErrorInvalidValue, nothing launched)
hipError_t launch_attn_bwd_pre(const BwdArgs& a, bool f32, int d, hipStream_t stream);  // fills `aux`
hipError_t launch_attn_bwd_bf16(const BwdArgs& a, int d, hipStream_t stream);  // pre-pass, dK/dV, dQ
hipError_t launch_attn_bwd_f32(const BwdArgs& a, int d, hipStream_t stream);

// Multi-head self-attention of short sequences in one launch (bf16, head width 64): for every (batch entry b, head i)
// the projections Q_i = X_b W_i^Q, K_i = X_b W_i^K, V_i = X_b W_i^V and head_i = softmax(Q_i K_i^T / 8) V_i (causal
// and key padding as in AttnArgs), written to columns 64i .. 64i+63 of C [B, n, H*64]. X [B, n, dm], Wq/Wk/Wv
// [dm, H*64] row-major bf16. Requires 1 <= n <= 128 and dm a positive multiple of 64 (hipErrorInvalidValue
// otherwise, nothing launched).
struct FusedMhaArgs {
  const void* X;
  const void* Wq;
  const void* Wk;
  const void* Wv;
  void* C;
  const int* kv_len;  // optional key padding (nullptr: none), as in AttnArgs
  int B, H, n, dm;
  int causal;
};
constexpr int kFusedMhaMaxSeq = 128;
hipError_t launch_mha_self_fused_bf16(const FusedMhaArgs& a, hipStream_t stream);

// C = A[M,K] * W[K,N] in bf16 with fp32 accumulation, up to three independent problems in one launch.
// Row-major C (ldc = N) when head_seq == 0; otherwise "head-major" with heads of w = 2^head_shift columns (w in
// {32, 64, 128}): column n of row m goes to C[((m / head_seq) * (N / w) + n / w) * head_seq + m % head_seq][n % w],
// i.e. [B, N/w, head_seq, w].
// Optional row-major epilogue (head_seq == 0 only): v = acc + bias[n]; if relu: v = max(v, 0); v += residual[m][n];
// then rounded to bf16. bias [N] and residual [M, N] are bf16; nullptr skips the step.
struct GemmProblem {
  const void* A;
  const void* W;
  void* C;
  int M, N, K;
  int head_seq;
  const void* bias;
  const void* residual;
  int relu;
  int head_shift;  // head-major only: log2 of the head width
};
hipError_t launch_gemm_bf16(const GemmProblem* probs, int nprobs, hipStream_t stream);

// y = LayerNorm(x) * gamma + beta over rows of D bf16 values (fp32 statistics, biased variance), M rows;
// D a multiple of 64, at most 1024; gamma, beta bf16 [D].
hipError_t launch_layer_norm_bf16(const void* x, const void* gamma, const void* beta, void* y, int M, int D, float eps,
                                  hipStream_t stream);

// Records a printf-style detail as the calling thread's last error (attn_last_error) and returns `code`.
int fail_status(int code, const char* fmt, ...);

}  // namespace mi355
