// C-ABI host layer: argument validation, workspace carving and kernel dispatch on the caller's stream.
//
// sdpa_forward -> one fused attention launch (bf16 MFMA kernel or fp32 VALU kernel); sdpa_forward_lse also writes
//                 the row log-sum-exp.
// encoder_layer_forward -> projections, attention, W^O + residual, LayerNorm, FFN W1 + bias + ReLU, FFN W2 + bias +
//                 residual, LayerNorm: seven launches (six for short sequences at head width 64, where the
//                 projections and the attention are one launch), no host sync.
// sdpa_forward_window -> the same launch restricted to a band of keys around each query.
// sdpa_forward_padded -> the same launch with per-batch key counts (key padding mask).
// sdpa_backward -> three launches: the per-row pre-pass (D = dO . O and lse into the workspace), dK/dV, dQ.
// mha_forward  -> Q/K/V projections (one grouped GEMM launch writing per-head layout into the workspace), the fused
//                 attention writing the concatenated heads, and the W^O GEMM into `out`: three launches, no host sync
//                 (two for short self-attention at head width 64: projections and attention in one launch).
// Every argument error is returned before the first HIP call; nothing is enqueued in that case.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/mi355_attn.h"
#include "launch.h"

#define ATTN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {
thread_local char g_err[512] = "";
}  // namespace

int mi355::fail_status(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

namespace {

using mi355::fail_status;

// (a null pointer counts as aligned: optional arguments are checked for null by the caller)
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// byte ranges [a, a+na) and [b, b+nb) intersect
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

constexpr size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Largest grid any attention launch would use for these sizes (8 queries per workgroup, the fp32 kernel at width 128,
// is the smallest block).
bool grid_fits(int64_t B, int64_t h, int64_t n_q) { return ((n_q + 7) / 8) * B * h <= 0x7fffffffLL; }
// The backward launches use blocks of as few as 32 rows of either side.
bool grid_fits32(int64_t B, int64_t h, int64_t n) { return ((n + 31) / 32) * B * h <= 0x7fffffffLL; }

struct MhaLayout {
  size_t q_off, k_off, v_off, c_off, total;
};

MhaLayout mha_layout(int64_t B, int64_t n_q, int64_t n_k, int64_t h, int64_t d) {
  const size_t q = (size_t)B * h * n_q * d * 2, kv = (size_t)B * h * n_k * d * 2;
  MhaLayout L;
  L.q_off = 0;
  L.k_off = round_up(L.q_off + q, 256);
  L.v_off = round_up(L.k_off + kv, 256);
  L.c_off = round_up(L.v_off + kv, 256);
  L.total = round_up(L.c_off + q, 256);
  return L;
}

// x is finite and >= 0 (checked on the bit pattern: the library is built assuming no NaN in arithmetic, so a float
// comparison could be folded away)
bool finite_nonneg(float x) {
  uint32_t b;
  memcpy(&b, &x, sizeof b);
  if ((b & 0x7f800000u) == 0x7f800000u) return false;  // inf or NaN
  return (b >> 31) == 0 || b == 0x80000000u;             // positive, +0 or -0
}

struct EncLayout {
  size_t q_off, k_off, v_off, c_off, r_off, h_off, f_off, total;
};

// Workspace of encoder_layer_forward: per-head Q/K/V, the concatenated heads, the residual sums (R1, then R2), H1
// and the FFN hidden activations, each region 256-byte aligned.
EncLayout enc_layout(int64_t B, int64_t n, int64_t d_model, int64_t d_ff) {
  const size_t act = (size_t)B * n * d_model * 2;
  EncLayout L;
  L.q_off = 0;
  L.k_off = round_up(L.q_off + act, 256);
  L.v_off = round_up(L.k_off + act, 256);
  L.c_off = round_up(L.v_off + act, 256);
  L.r_off = round_up(L.c_off + act, 256);
  L.h_off = round_up(L.r_off + act, 256);
  L.f_off = round_up(L.h_off + act, 256);
  L.total = round_up(L.f_off + (size_t)B * n * d_ff * 2, 256);
  return L;
}

// Head widths of the multi-head paths: 32, 64 or 128 (the attention kernels' widths), with h * d a multiple of 64
// (the GEMM's column granule); log2 of the width, or -1.
int head_shift(int64_t h, int64_t d) {
  if (h <= 0 || (h * d) % 64) return -1;
  return d == 32 ? 5 : d == 64 ? 6 : d == 128 ? 7 : -1;
}

bool enc_sizes_ok(int64_t B, int64_t n, int64_t d_model, int64_t h, int64_t d_ff) {
  return B > 0 && n > 0 && h > 0 && d_model % h == 0 && head_shift(h, d_model / h) >= 0 && d_model <= 1024 &&
         d_ff > 0 && d_ff % 64 == 0 &&
         d_ff <= 65536 && n <= ATTN_MAX_SEQ && B * h <= ATTN_MAX_HEADS && B * n <= 0x7fffffffLL && grid_fits(B, h, n);
}

}  // namespace

ATTN_EXPORT const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID: return "ATTN_ERR_INVALID";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    default: return "ATTN_UNKNOWN_STATUS";
  }
}

ATTN_EXPORT const char* attn_last_error(void) { return g_err; }

namespace {

// Shared checks of sdpa_forward / sdpa_forward_lse / sdpa_backward on the tensor sizes; 0 when they pass.
int check_sdpa_sizes(const char* fn, int dtype, int mask_kind, int64_t B, int64_t h, int64_t n_q, int64_t n_k,
                     int64_t d_k, int64_t d_v, bool backward) {
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail_status(ATTN_ERR_UNSUPPORTED, "%s: dtype %d", fn, dtype);
  if (mask_kind != ATTN_MASK_NONE && mask_kind != ATTN_MASK_CAUSAL)
    return fail_status(ATTN_ERR_INVALID, "%s: mask_kind %d", fn, mask_kind);
  if (B <= 0 || h <= 0 || n_q <= 0 || n_k <= 0 || d_k <= 0 || d_v <= 0)
    return fail_status(ATTN_ERR_INVALID, "%s: sizes must be positive (B=%lld h=%lld n_q=%lld n_k=%lld d_k=%lld "
                       "d_v=%lld)", fn, (long long)B, (long long)h, (long long)n_q, (long long)n_k, (long long)d_k,
                       (long long)d_v);
  // the forward and backward kernels take d_k = d_v in {32, 64, 128}
  if (d_k != d_v || (d_k != 32 && d_k != 64 && d_k != 128))
    return fail_status(ATTN_ERR_UNSUPPORTED, "%s: head dims d_k=%lld d_v=%lld (implemented: d_k = d_v in {32, 64, "
                       "128})", fn, (long long)d_k, (long long)d_v);
  if (mask_kind == ATTN_MASK_CAUSAL && n_q != n_k)
    return fail_status(ATTN_ERR_UNSUPPORTED, "%s: causal mask needs n_q == n_k (got %lld, %lld)", fn,
                       (long long)n_q, (long long)n_k);
  if (n_q > ATTN_MAX_SEQ || n_k > ATTN_MAX_SEQ || B > ATTN_MAX_HEADS || h > ATTN_MAX_HEADS ||
      B * h > ATTN_MAX_HEADS || !grid_fits(B, h, n_q) ||
      (backward && (!grid_fits32(B, h, n_q) || !grid_fits32(B, h, n_k))))
    return fail_status(ATTN_ERR_UNSUPPORTED, "%s: sizes beyond the library limits", fn);
  return ATTN_OK;
}

int sdpa_forward_impl(const char* fn, const void* Q, const void* K, const void* V, const int32_t* kv_len,
                      int mask_kind, void* out, float* lse, int dtype, int64_t B, int64_t h, int64_t n_q, int64_t n_k,
                      int64_t d_k, int64_t d_v, void* stream, int64_t window = -1, float* out32 = nullptr) {
  if (int st = check_sdpa_sizes(fn, dtype, mask_kind, B, h, n_q, n_k, d_k, d_v, false)) return st;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(out) || !aligned16(lse) || !aligned16(kv_len) ||
      !aligned16(out32))
    return fail_status(ATTN_ERR_INVALID, "%s: pointers must be 16-byte aligned", fn);
  if (out32 && dtype != ATTN_BF16)
    return fail_status(ATTN_ERR_INVALID, "%s: out_f32 is for ATTN_BF16 (the ATTN_F32 output is already float32)", fn);
  const size_t es = dtype == ATTN_BF16 ? 2 : 4;
  const size_t q_bytes = (size_t)B * h * n_q * d_k * es, kv_bytes = (size_t)B * h * n_k * d_k * es;
  if (overlaps(out, q_bytes, Q, q_bytes) || overlaps(out, q_bytes, K, kv_bytes) || overlaps(out, q_bytes, V, kv_bytes))
    return fail_status(ATTN_ERR_INVALID, "%s: out overlaps an input", fn);
  if (lse) {
    const size_t lse_bytes = (size_t)B * h * n_q * 4;
    if (overlaps(lse, lse_bytes, Q, q_bytes) || overlaps(lse, lse_bytes, K, kv_bytes) ||
        overlaps(lse, lse_bytes, V, kv_bytes) || overlaps(lse, lse_bytes, out, q_bytes))
      return fail_status(ATTN_ERR_INVALID, "%s: lse overlaps another tensor", fn);
  }
  if (kv_len) {
    const size_t len_bytes = (size_t)B * 4;
    if (overlaps(kv_len, len_bytes, out, q_bytes) || (lse && overlaps(kv_len, len_bytes, lse, (size_t)B * h * n_q * 4)))
      return fail_status(ATTN_ERR_INVALID, "%s: kv_len overlaps an output", fn);
  }
  if (out32) {
    const size_t o32_bytes = (size_t)B * h * n_q * d_v * 4;
    if (overlaps(out32, o32_bytes, Q, q_bytes) || overlaps(out32, o32_bytes, K, kv_bytes) ||
        overlaps(out32, o32_bytes, V, kv_bytes) || overlaps(out32, o32_bytes, out, q_bytes) ||
        (lse && overlaps(out32, o32_bytes, lse, (size_t)B * h * n_q * 4)) ||
        (kv_len && overlaps(out32, o32_bytes, kv_len, (size_t)B * 4)))
      return fail_status(ATTN_ERR_INVALID, "%s: out_f32 overlaps another tensor", fn);
  }

  mi355::AttnArgs a{};
  a.Q = Q; a.K = K; a.V = V; a.O = out;
  a.B = (int)B; a.H = (int)h; a.n_q = (int)n_q; a.n_k = (int)n_k;
  a.q_stride_bh = n_q * d_k;
  a.k_stride_bh = n_k * d_k;
  a.o_stride_b = h * n_q * d_k;
  a.o_stride_h = n_q * d_k;
  a.o_stride_row = d_k;
  a.causal = mask_kind == ATTN_MASK_CAUSAL;
  a.lse = lse;
  a.kv_len = kv_len;
  a.o32 = out32;
  if (window >= 0) {
    a.windowed = 1;
    a.window = (int)(window < n_k ? window : n_k);
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      dtype == ATTN_BF16 ? mi355::launch_attn_fwd_bf16(a, (int)d_k, s) : mi355::launch_attn_fwd_f32(a, (int)d_k, s);
  if (e != hipSuccess) return fail_status(ATTN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ATTN_OK;
}

size_t bwd_workspace_bytes(int64_t B, int64_t h, int64_t n_q) {
  return (size_t)B * h * ((n_q + 63) / 64) * mi355::kAuxFloatsPerTile * sizeof(float);
}

}  // namespace

ATTN_EXPORT int sdpa_forward(const void* Q, const void* K, const void* V, int mask_kind, void* out, int dtype,
                             int64_t B, int64_t h, int64_t n_q, int64_t n_k, int64_t d_k, int64_t d_v, void* stream) {
  if (!Q || !K || !V || !out) return fail_status(ATTN_ERR_INVALID, "sdpa_forward: null tensor pointer");
  return sdpa_forward_impl("sdpa_forward", Q, K, V, nullptr, mask_kind, out, nullptr, dtype, B, h, n_q, n_k, d_k, d_v,
                           stream);
}

ATTN_EXPORT int sdpa_forward_padded(const void* Q, const void* K, const void* V, const int32_t* kv_len, int mask_kind,
                                    void* out, float* lse, int dtype, int64_t B, int64_t h, int64_t n_q, int64_t n_k,
                                    int64_t d_k, int64_t d_v, void* stream) {
  if (!Q || !K || !V || !kv_len || !out)
    return fail_status(ATTN_ERR_INVALID, "sdpa_forward_padded: null tensor pointer");
  return sdpa_forward_impl("sdpa_forward_padded", Q, K, V, kv_len, mask_kind, out, lse, dtype, B, h, n_q, n_k, d_k, d_v,
                           stream);
}

ATTN_EXPORT int sdpa_forward_window(const void* Q, const void* K, const void* V, int64_t window, int mask_kind,
                                    void* out, float* lse, int dtype, int64_t B, int64_t h, int64_t n_q, int64_t n_k,
                                    int64_t d_k, int64_t d_v, void* stream) {
  if (!Q || !K || !V || !out) return fail_status(ATTN_ERR_INVALID, "sdpa_forward_window: null tensor pointer");
  if (window < 0) return fail_status(ATTN_ERR_INVALID, "sdpa_forward_window: window %lld < 0", (long long)window);
  if (n_q != n_k)
    return fail_status(ATTN_ERR_UNSUPPORTED, "sdpa_forward_window: restricted self-attention needs n_q == n_k (got "
                       "%lld, %lld)", (long long)n_q, (long long)n_k);
  return sdpa_forward_impl("sdpa_forward_window", Q, K, V, nullptr, mask_kind, out, lse, dtype, B, h, n_q, n_k, d_k,
                           d_v, stream, window);
}

ATTN_EXPORT int sdpa_forward_lse(const void* Q, const void* K, const void* V, int mask_kind, void* out, float* lse,
                                 int dtype, int64_t B, int64_t h, int64_t n_q, int64_t n_k, int64_t d_k, int64_t d_v,
                                 void* stream) {
  if (!Q || !K || !V || !out || !lse) return fail_status(ATTN_ERR_INVALID, "sdpa_forward_lse: null tensor pointer");
  return sdpa_forward_impl("sdpa_forward_lse", Q, K, V, nullptr, mask_kind, out, lse, dtype, B, h, n_q, n_k, d_k, d_v,
                           stream);
}

ATTN_EXPORT int sdpa_forward_train(const void* Q, const void* K, const void* V, const int32_t* kv_len, int64_t window,
                                   int mask_kind, void* out, float* out_f32, float* lse, int dtype, int64_t B,
                                   int64_t h, int64_t n_q, int64_t n_k, int64_t d_k, int64_t d_v, void* stream) {
  static const char* fn = "sdpa_forward_train";
  if (!Q || !K || !V || !out || !lse) return fail_status(ATTN_ERR_INVALID, "%s: null tensor pointer", fn);
  if (window >= 0 && n_q != n_k)
    return fail_status(ATTN_ERR_UNSUPPORTED, "%s: restricted self-attention needs n_q == n_k (got %lld, %lld)", fn,
                       (long long)n_q, (long long)n_k);
  if (window >= 0 && kv_len)
    return fail_status(ATTN_ERR_UNSUPPORTED, "%s: a window together with key padding is not implemented", fn);
  return sdpa_forward_impl(fn, Q, K, V, kv_len, mask_kind, out, lse, dtype, B, h, n_q, n_k, d_k, d_v, stream,
                           window < 0 ? -1 : window, out_f32);
}

ATTN_EXPORT size_t sdpa_backward_workspace_size(int dtype, int64_t B, int64_t h, int64_t n_q, int64_t n_k,
                                                int64_t d_k, int64_t d_v) {
  if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_BF16_F32O) return 0;
  if (B <= 0 || h <= 0 || n_q <= 0 || n_k <= 0 || d_k != d_v || (d_k != 32 && d_k != 64 && d_k != 128)) return 0;
  if (n_q > ATTN_MAX_SEQ || n_k > ATTN_MAX_SEQ || B > ATTN_MAX_HEADS || h > ATTN_MAX_HEADS || B * h > ATTN_MAX_HEADS)
    return 0;
  return bwd_workspace_bytes(B, h, n_q);
}

ATTN_EXPORT int sdpa_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                              const float* lse, const int32_t* kv_len, int64_t window, int mask_kind, void* dQ,
                              void* dK, void* dV, void* workspace,
                              size_t workspace_bytes, int dtype, int64_t B, int64_t h, int64_t n_q, int64_t n_k,
                              int64_t d_k, int64_t d_v, void* stream) {
  static const char* fn = "sdpa_backward";
  if (!Q || !K || !V || !O || !dO || !lse || !dQ || !dK || !dV || !workspace)
    return fail_status(ATTN_ERR_INVALID, "%s: null pointer", fn);
  const bool o32 = dtype == ATTN_BF16_F32O;  // bf16 tensors, O float32
  if (o32) dtype = ATTN_BF16;
  if (int st = check_sdpa_sizes(fn, dtype, mask_kind, B, h, n_q, n_k, d_k, d_v, true)) return st;
  if (window >= 0 && n_q != n_k)
    return fail_status(ATTN_ERR_UNSUPPORTED, "%s: a window needs n_q == n_k (got %lld, %lld)", fn, (long long)n_q,
                       (long long)n_k);
  if (window >= 0 && kv_len)
    return fail_status(ATTN_ERR_UNSUPPORTED, "%s: a window with key padding has no forward entry point", fn);
  const size_t need = bwd_workspace_bytes(B, h, n_q);
  if (workspace_bytes < need)
    return fail_status(ATTN_ERR_INVALID, "%s: workspace %zu bytes, need %zu", fn, workspace_bytes, need);
  const void* ptrs[] = {Q, K, V, O, dO, lse, dQ, dK, dV, workspace, kv_len};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail_status(ATTN_ERR_INVALID, "%s: pointers must be 16-byte aligned", fn);
  const size_t es = dtype == ATTN_BF16 ? 2 : 4;
  const size_t q_b = (size_t)B * h * n_q * d_k * es, kv_b = (size_t)B * h * n_k * d_k * es;
  const size_t lse_b = (size_t)B * h * n_q * 4;
  const void* ins[] = {Q, K, V, O, dO, lse, kv_len};
  const size_t in_b[] = {q_b, kv_b, kv_b, o32 ? 2 * q_b : q_b, q_b, lse_b, kv_len ? (size_t)B * 4 : 0};
  void* outs[] = {dQ, dK, dV, workspace};
  const size_t out_b[] = {q_b, kv_b, kv_b, need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 7; ++j)
      if (overlaps(outs[i], out_b[i], ins[j], in_b[j]))
        return fail_status(ATTN_ERR_INVALID, "%s: an output or the workspace overlaps an input", fn);
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_b[i], outs[j], out_b[j]))
        return fail_status(ATTN_ERR_INVALID, "%s: outputs and workspace must not overlap", fn);
  }

  mi355::BwdArgs a{};
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.dO = dO; a.lse = lse;
  a.aux = static_cast<float*>(workspace);
  a.dQ = dQ; a.dK = dK; a.dV = dV;
  a.B = (int)B; a.H = (int)h; a.n_q = (int)n_q; a.n_k = (int)n_k;
  a.causal = mask_kind == ATTN_MASK_CAUSAL;
  a.kv_len = kv_len;
  a.o_f32 = o32;
  if (window >= 0) {
    a.windowed = 1;
    a.window = (int)(window < n_k ? window : n_k);
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = dtype == ATTN_BF16 ? mi355::launch_attn_bwd_bf16(a, (int)d_k, s)
                                          : mi355::launch_attn_bwd_f32(a, (int)d_k, s);
  if (e != hipSuccess) return fail_status(ATTN_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ATTN_OK;
}

ATTN_EXPORT size_t mha_workspace_size(int dtype, int64_t B, int64_t n_q, int64_t n_k, int64_t h, int64_t d_k,
                                      int64_t d_v) {
  if (dtype != ATTN_BF16 || B <= 0 || n_q <= 0 || n_k <= 0 || h <= 0 || d_k != d_v || head_shift(h, d_k) < 0) return 0;
  if (n_q > ATTN_MAX_SEQ || n_k > ATTN_MAX_SEQ || B > ATTN_MAX_HEADS || h > ATTN_MAX_HEADS) return 0;
  return mha_layout(B, n_q, n_k, h, d_k).total;
}

namespace {

// Argument checks of mha_forward and its allocation-free variant (no HIP call). `name` prefixes the error detail.
// `workspace` may be null when `check_ws` is false (the variant's scratch is the library's own).
int mha_check(const char* name, const void* Xq, const void* Xkv, const void* Wq, const void* Wk, const void* Wv,
              const void* Wo, int mask_kind, const void* out, const void* workspace, size_t workspace_bytes,
              bool check_ws, int dtype, int64_t B, int64_t n_q, int64_t n_k, int64_t d_model, int64_t h,
              int64_t d_k, int64_t d_v, MhaLayout* layout, int* hshift) {
  if (!Xq || !Xkv || !Wq || !Wk || !Wv || !Wo || !out || (check_ws && !workspace))
    return fail_status(ATTN_ERR_INVALID, "%s: null pointer", name);
  if (dtype != ATTN_BF16) return fail_status(ATTN_ERR_UNSUPPORTED, "%s: dtype %d (only ATTN_BF16)", name, dtype);
  if (mask_kind != ATTN_MASK_NONE && mask_kind != ATTN_MASK_CAUSAL)
    return fail_status(ATTN_ERR_INVALID, "%s: mask_kind %d", name, mask_kind);
  if (B <= 0 || n_q <= 0 || n_k <= 0 || d_model <= 0 || h <= 0 || d_k <= 0 || d_v <= 0)
    return fail_status(ATTN_ERR_INVALID, "%s: sizes must be positive", name);
  const int hsh = d_k == d_v ? head_shift(h, d_k) : -1;
  if (hsh < 0)
    return fail_status(ATTN_ERR_UNSUPPORTED, "%s: head dims d_k=%lld d_v=%lld with h=%lld (implemented: d_k = "
                       "d_v in {32, 64, 128}, h*d_k a multiple of 64)", name, (long long)d_k, (long long)d_v,
                       (long long)h);
  if (d_model % 64)
    return fail_status(ATTN_ERR_UNSUPPORTED, "%s: d_model=%lld is not a multiple of 64", name, (long long)d_model);
  if (mask_kind == ATTN_MASK_CAUSAL && n_q != n_k)
    return fail_status(ATTN_ERR_UNSUPPORTED, "%s: causal mask needs n_q == n_k", name);
  if (n_q > ATTN_MAX_SEQ || n_k > ATTN_MAX_SEQ || B > ATTN_MAX_HEADS || h > ATTN_MAX_HEADS ||
      B * h > ATTN_MAX_HEADS || d_model > 65536 || B * n_q > 0x7fffffffLL || B * n_k > 0x7fffffffLL ||
      !grid_fits(B, h, n_q))
    return fail_status(ATTN_ERR_UNSUPPORTED, "%s: sizes beyond the library limits", name);
  const MhaLayout L = mha_layout(B, n_q, n_k, h, d_k);
  if (!check_ws && workspace_bytes < L.total)
    return fail_status(ATTN_ERR_INVALID, "%s: these sizes need %zu bytes of scratch; the library's scratch holds %zu "
                       "(mha_forward takes a caller workspace of any size)", name, L.total, workspace_bytes);
  if (workspace_bytes < L.total)
    return fail_status(ATTN_ERR_INVALID, "%s: workspace %zu bytes, need %zu", name, workspace_bytes, L.total);
  const void* ptrs[] = {Xq, Xkv, Wq, Wk, Wv, Wo, out, check_ws ? workspace : out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail_status(ATTN_ERR_INVALID, "%s: pointers must be 16-byte aligned", name);
  const size_t xq_b = (size_t)B * n_q * d_model * 2, xkv_b = (size_t)B * n_k * d_model * 2;
  const size_t w_b = (size_t)d_model * h * d_k * 2;
  const void* ins[] = {Xq, Xkv, Wq, Wk, Wv, Wo};
  const size_t in_b[] = {xq_b, xkv_b, w_b, w_b, w_b, w_b};
  for (int i = 0; i < 6; ++i) {
    if (overlaps(out, xq_b, ins[i], in_b[i])) return fail_status(ATTN_ERR_INVALID, "%s: out overlaps an input", name);
    if (check_ws && overlaps(workspace, L.total, ins[i], in_b[i]))
      return fail_status(ATTN_ERR_INVALID, "%s: workspace overlaps an input", name);
  }
  if (check_ws && overlaps(out, xq_b, workspace, L.total))
    return fail_status(ATTN_ERR_INVALID, "%s: out overlaps workspace", name);
  *layout = L;
  *hshift = hsh;
  return ATTN_OK;
}

// The three launches of mha_forward (arguments already checked): projections into the workspace, attention into the
// concatenated heads, W^O into `out`.
int mha_run(const char* name, const void* Xq, const void* Xkv, const void* Wq, const void* Wk, const void* Wv,
            const void* Wo, int mask_kind, void* out, void* workspace, const MhaLayout& L, int hsh, int64_t B,
            int64_t n_q, int64_t n_k, int64_t d_model, int64_t h, int64_t d_k, hipStream_t s) {
  char* ws = static_cast<char*>(workspace);
  void* Qh = ws + L.q_off;
  void* Kh = ws + L.k_off;
  void* Vh = ws + L.v_off;
  void* Ch = ws + L.c_off;
  const int hd = (int)(h * d_k);

  // Short self-attention at head width 64: projections and attention in one launch per (batch entry, head), the
  // heads written straight into the concatenated layout; then the output projection.
  if (Xq == Xkv && n_q == n_k && n_q <= mi355::kFusedMhaMaxSeq && d_k == 64 && d_model % 64 == 0) {
    mi355::FusedMhaArgs f{};
    f.X = Xq; f.Wq = Wq; f.Wk = Wk; f.Wv = Wv; f.C = Ch;
    f.B = (int)B; f.H = (int)h; f.n = (int)n_q; f.dm = (int)d_model;
    f.causal = mask_kind == ATTN_MASK_CAUSAL;
    hipError_t e = mi355::launch_mha_self_fused_bf16(f, s);
    if (e != hipSuccess)
      return fail_status(ATTN_ERR_HIP, "%s: projection/attention launch failed: %s", name, hipGetErrorString(e));
    mi355::GemmProblem outp = {Ch, Wo, out, (int)(B * n_q), (int)d_model, hd, 0};
    e = mi355::launch_gemm_bf16(&outp, 1, s);
    if (e != hipSuccess) return fail_status(ATTN_ERR_HIP, "%s: W^O launch failed: %s", name, hipGetErrorString(e));
    return ATTN_OK;
  }

  // 1. projections, written per head: Qh [B,h,n_q,d], Kh/Vh [B,h,n_k,d]
  mi355::GemmProblem proj[3] = {
      {Xq, Wq, Qh, (int)(B * n_q), hd, (int)d_model, (int)n_q, nullptr, nullptr, 0, hsh},
      {Xkv, Wk, Kh, (int)(B * n_k), hd, (int)d_model, (int)n_k, nullptr, nullptr, 0, hsh},
      {Xkv, Wv, Vh, (int)(B * n_k), hd, (int)d_model, (int)n_k, nullptr, nullptr, 0, hsh},
  };
  hipError_t e = mi355::launch_gemm_bf16(proj, 3, s);
  if (e != hipSuccess) return fail_status(ATTN_ERR_HIP, "%s: projection launch failed: %s", name, hipGetErrorString(e));

  // 2. attention per head, output written into the concatenated layout [B, n_q, h*d]
  mi355::AttnArgs a{};
  a.Q = Qh; a.K = Kh; a.V = Vh; a.O = Ch;
  a.B = (int)B; a.H = (int)h; a.n_q = (int)n_q; a.n_k = (int)n_k;
  a.q_stride_bh = n_q * d_k;
  a.k_stride_bh = n_k * d_k;
  a.o_stride_b = n_q * hd;
  a.o_stride_h = d_k;
  a.o_stride_row = hd;
  a.causal = mask_kind == ATTN_MASK_CAUSAL;
  e = mi355::launch_attn_fwd_bf16(a, (int)d_k, s);
  if (e != hipSuccess) return fail_status(ATTN_ERR_HIP, "%s: attention launch failed: %s", name, hipGetErrorString(e));

  // 3. output projection: out [B*n_q, d_model] = concat [B*n_q, h*d] x Wo [h*d, d_model]
  mi355::GemmProblem outp = {Ch, Wo, out, (int)(B * n_q), (int)d_model, hd, 0};
  e = mi355::launch_gemm_bf16(&outp, 1, s);
  if (e != hipSuccess) return fail_status(ATTN_ERR_HIP, "%s: W^O launch failed: %s", name, hipGetErrorString(e));
  return ATTN_OK;
}

// The allocation-free variant's scratch: one array per GPU the library runs on, held until the process ends. In
// host code `scratch` names a host-side stand-in, not device memory: its device address is taken once per device
// with hipGetSymbolAddress (with that device current) and only that address is used.
constexpr size_t kNoAllocScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// This device's scratch address (the current device's), looked up on its first use.
int scratch_address(const char* name, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_status(ATTN_ERR_HIP, "%s: hipGetDevice failed: %s", name, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail_status(ATTN_ERR_UNSUPPORTED, "%s: device index %d", name, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail_status(ATTN_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed: %s", name, hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *ptr = g_scratch_dev[dev];
  return ATTN_OK;
}

}  // namespace

ATTN_EXPORT int mha_forward(const void* Xq, const void* Xkv, const void* Wq, const void* Wk, const void* Wv,
                            const void* Wo, int mask_kind, void* out, void* workspace, size_t workspace_bytes,
                            int dtype, int64_t B, int64_t n_q, int64_t n_k, int64_t d_model, int64_t h, int64_t d_k,
                            int64_t d_v, void* stream) {
  MhaLayout L;
  int hsh = 0;
  const int st = mha_check("mha_forward", Xq, Xkv, Wq, Wk, Wv, Wo, mask_kind, out, workspace, workspace_bytes, true,
                           dtype, B, n_q, n_k, d_model, h, d_k, d_v, &L, &hsh);
  if (st != ATTN_OK) return st;
  return mha_run("mha_forward", Xq, Xkv, Wq, Wk, Wv, Wo, mask_kind, out, workspace, L, hsh, B, n_q, n_k, d_model, h,
                 d_k, static_cast<hipStream_t>(stream));
}

ATTN_EXPORT int mha_forward_noalloc(const void* Xq, const void* Xkv, const void* Wq, const void* Wk, const void* Wv,
                                    const void* Wo, int mask_kind, void* out, int dtype, int64_t B, int64_t n_q,
                                    int64_t n_k, int64_t d_model, int64_t h, int64_t d_k, int64_t d_v, void* stream) {
  MhaLayout L;
  int hsh = 0;
  const int st = mha_check("mha_forward_noalloc", Xq, Xkv, Wq, Wk, Wv, Wo, mask_kind, out, nullptr,
                           kNoAllocScratchBytes, false, dtype, B, n_q, n_k, d_model, h, d_k, d_v, &L, &hsh);
  if (st != ATTN_OK) return st;
  void* ws = nullptr;
  const int sa = scratch_address("mha_forward_noalloc", &ws);
  if (sa != ATTN_OK) return sa;
  return mha_run("mha_forward_noalloc", Xq, Xkv, Wq, Wk, Wv, Wo, mask_kind, out, ws, L, hsh, B, n_q, n_k, d_model,
                 h, d_k, static_cast<hipStream_t>(stream));
}

ATTN_EXPORT size_t encoder_layer_workspace_size(int dtype, int64_t B, int64_t n, int64_t d_model, int64_t h,
                                                int64_t d_ff) {
  if (dtype != ATTN_BF16 || !enc_sizes_ok(B, n, d_model, h, d_ff)) return 0;
  return enc_layout(B, n, d_model, d_ff).total;
}

ATTN_EXPORT int encoder_layer_forward(const void* X, const int32_t* kv_len, const void* Wq, const void* Wk,
                                      const void* Wv, const void* Wo, const void* ln1_gamma, const void* ln1_beta,
                                      const void* W1, const void* b1, const void* W2, const void* b2,
                                      const void* ln2_gamma, const void* ln2_beta, float eps, int mask_kind, void* out,
                                      void* workspace, size_t workspace_bytes, int dtype, int64_t B, int64_t n,
                                      int64_t d_model, int64_t h, int64_t d_ff, void* stream) {
  static const char* fn = "encoder_layer_forward";
  const void* ins[] = {X, Wq, Wk, Wv, Wo, ln1_gamma, ln1_beta, W1, b1, W2, b2, ln2_gamma, ln2_beta};
  for (const void* p : ins)
    if (!p) return fail_status(ATTN_ERR_INVALID, "%s: null pointer", fn);
  if (!out || !workspace) return fail_status(ATTN_ERR_INVALID, "%s: null pointer", fn);
  if (dtype != ATTN_BF16) return fail_status(ATTN_ERR_UNSUPPORTED, "%s: dtype %d (only ATTN_BF16)", fn, dtype);
  if (mask_kind != ATTN_MASK_NONE && mask_kind != ATTN_MASK_CAUSAL)
    return fail_status(ATTN_ERR_INVALID, "%s: mask_kind %d", fn, mask_kind);
  if (B <= 0 || n <= 0 || d_model <= 0 || h <= 0 || d_ff <= 0)
    return fail_status(ATTN_ERR_INVALID, "%s: sizes must be positive", fn);
  if (!finite_nonneg(eps)) return fail_status(ATTN_ERR_INVALID, "%s: eps must be finite and >= 0", fn);
  if (!enc_sizes_ok(B, n, d_model, h, d_ff))
    return fail_status(ATTN_ERR_UNSUPPORTED, "%s: needs d_model = d h <= 1024 with d in {32, 64, 128}, d_model a "
                       "multiple of 64 and d_ff a multiple of 64 (got "
                       "d_model=%lld h=%lld d_ff=%lld), sizes within the library limits", fn, (long long)d_model,
                       (long long)h, (long long)d_ff);
  const EncLayout L = enc_layout(B, n, d_model, d_ff);
  if (workspace_bytes < L.total)
    return fail_status(ATTN_ERR_INVALID, "%s: workspace %zu bytes, need %zu", fn, workspace_bytes, L.total);
  for (const void* p : ins)
    if (!aligned16(p)) return fail_status(ATTN_ERR_INVALID, "%s: pointers must be 16-byte aligned", fn);
  if (!aligned16(out) || !aligned16(workspace) || !aligned16(kv_len))
    return fail_status(ATTN_ERR_INVALID, "%s: pointers must be 16-byte aligned", fn);
  const size_t act_b = (size_t)B * n * d_model * 2, wsq = (size_t)d_model * d_model * 2;
  const size_t vec_b = (size_t)d_model * 2;
  const size_t in_b[] = {act_b, wsq, wsq, wsq, wsq, vec_b, vec_b, (size_t)d_model * d_ff * 2, (size_t)d_ff * 2,
                         (size_t)d_ff * d_model * 2, vec_b, vec_b, vec_b};
  for (int i = 0; i < 13; ++i) {
    if (overlaps(out, act_b, ins[i], in_b[i])) return fail_status(ATTN_ERR_INVALID, "%s: out overlaps an input", fn);
    if (overlaps(workspace, L.total, ins[i], in_b[i]))
      return fail_status(ATTN_ERR_INVALID, "%s: workspace overlaps an input", fn);
  }
  if (kv_len && (overlaps(kv_len, (size_t)B * 4, out, act_b) || overlaps(kv_len, (size_t)B * 4, workspace, L.total)))
    return fail_status(ATTN_ERR_INVALID, "%s: kv_len overlaps an output or the workspace", fn);
  if (overlaps(out, act_b, workspace, L.total)) return fail_status(ATTN_ERR_INVALID, "%s: out overlaps workspace", fn);

  char* ws = static_cast<char*>(workspace);
  void *Qh = ws + L.q_off, *Kh = ws + L.k_off, *Vh = ws + L.v_off, *Ch = ws + L.c_off;
  void *R = ws + L.r_off, *H1 = ws + L.h_off, *F = ws + L.f_off;
  const int M = (int)(B * n), dm = (int)d_model, ff = (int)d_ff;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
#define ENC_STEP(call, what)                                                                          \
  e = (call);                                                                                        \
  if (e != hipSuccess) return fail_status(ATTN_ERR_HIP, "%s: %s launch failed: %s", fn, what, hipGetErrorString(e));

  // 1. Q/K/V projections into the per-head layout, 2. attention into the concatenated heads (short sequences at head
  // width 64: both in one launch per (batch entry, head))
  const int dh = (int)(d_model / h), hsh = head_shift(h, dh);
  if (n <= mi355::kFusedMhaMaxSeq && dh == 64) {
    mi355::FusedMhaArgs f{};
    f.X = X; f.Wq = Wq; f.Wk = Wk; f.Wv = Wv; f.C = Ch; f.kv_len = kv_len;
    f.B = (int)B; f.H = (int)h; f.n = (int)n; f.dm = dm;
    f.causal = mask_kind == ATTN_MASK_CAUSAL;
    ENC_STEP(mi355::launch_mha_self_fused_bf16(f, s), "projection/attention");
  } else {
    mi355::GemmProblem proj[3] = {{X, Wq, Qh, M, dm, dm, (int)n, nullptr, nullptr, 0, hsh},
                                  {X, Wk, Kh, M, dm, dm, (int)n, nullptr, nullptr, 0, hsh},
                                  {X, Wv, Vh, M, dm, dm, (int)n, nullptr, nullptr, 0, hsh}};
    ENC_STEP(mi355::launch_gemm_bf16(proj, 3, s), "projection");
    mi355::AttnArgs a{};
    a.Q = Qh; a.K = Kh; a.V = Vh; a.O = Ch;
    a.B = (int)B; a.H = (int)h; a.n_q = (int)n; a.n_k = (int)n;
    a.q_stride_bh = n * dh;
    a.k_stride_bh = n * dh;
    a.o_stride_b = n * d_model;
    a.o_stride_h = dh;
    a.o_stride_row = d_model;
    a.causal = mask_kind == ATTN_MASK_CAUSAL;
    a.kv_len = kv_len;
    ENC_STEP(mi355::launch_attn_fwd_bf16(a, dh, s), "attention");
  }
  // 3. R1 = X + Concat W^O (residual in the GEMM epilogue), H1 = LayerNorm(R1)
  mi355::GemmProblem wo = {Ch, Wo, R, M, dm, dm, 0, nullptr, X, 0};
  ENC_STEP(mi355::launch_gemm_bf16(&wo, 1, s), "W^O");
  ENC_STEP(mi355::launch_layer_norm_bf16(R, ln1_gamma, ln1_beta, H1, M, dm, eps, s), "LayerNorm 1");
  // 4. F = max(0, H1 W1 + b1), R2 = H1 + F W2 + b2 (bias, ReLU and residual in the GEMM epilogues), out = LayerNorm(R2)
  mi355::GemmProblem f1 = {H1, W1, F, M, ff, dm, 0, b1, nullptr, 1};
  ENC_STEP(mi355::launch_gemm_bf16(&f1, 1, s), "FFN W1");
  mi355::GemmProblem f2 = {F, W2, R, M, dm, ff, 0, b2, H1, 0};
  ENC_STEP(mi355::launch_gemm_bf16(&f2, 1, s), "FFN W2");
  ENC_STEP(mi355::launch_layer_norm_bf16(R, ln2_gamma, ln2_beta, out, M, dm, eps, s), "LayerNorm 2");
#undef ENC_STEP
  return ATTN_OK;
}
