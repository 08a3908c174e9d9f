// Backward pass of scaled dot-product attention in fp32 throughout, d_k = d_v = D in {32, 64, 128}, for gfx950.
//
// Same mathematics as the bf16 backward (the chain rule through O = P V, the row softmax and S = Q K^T / sqrt(D):
// "Transformer：抛弃循环与卷积的序列建模", section "训练样本", subsection "反向传播"; forward definition "Attention Is
// All You Need", lettle.cn translation, section 3.2.1), with every value in fp32, P and dS included. This path serves
// small fp32 problems, so it is plain VALU code: two threads per row (four at D = 128), each holding one part of the
// row's vectors, partial dot products combined by lane exchanges; the other side's rows are staged in LDS in tiles
// of 32 and read as broadcasts. The per-row lse and D come from the shared pre-pass (workspace tiles of 64 rows).
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace mi355 {
namespace {

constexpr int kRows = 32;  // rows per workgroup (two threads each) and per staged tile

// the width-dependent constants: row width, threads per row, the part of a row one thread holds, log2(e) / sqrt(D)
// and 1 / sqrt(D)
template <int D>
struct Width {
  static_assert(D == 32 || D == 64 || D == 128, "head width of the backward kernels");
  static constexpr int kD = D, kParts = D == 128 ? 4 : 2, kHalf = D / kParts;
  static constexpr double kSqrtD = D == 64 ? 8.0 : D == 32 ? 5.656854249492381 : 11.313708498984761;
  static constexpr float kC = (float)(1.4426950408889634 / kSqrtD);
  static constexpr float kInvSqrtD = (float)(1.0 / kSqrtD);
};

// sum of a partial dot product over the kParts threads of a row
template <int kParts>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int off = 1; off < kParts; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

// lse2 (= log2(e) * lse) and D of query row i of head bh, from the workspace tiles
__device__ __forceinline__ float2 aux_row(const float* aux, int n_tiles, int bh, int i) {
  const float* at = aux + ((int64_t)bh * n_tiles + i / 64) * kAuxFloatsPerTile;
  return float2{at[i % 64], at[64 + i % 64]};
}

// dK and dV: a workgroup owns 32 keys; query rows stream through LDS.
template <int D>
__global__ __launch_bounds__(Width<D>::kParts * kRows) void attn_bwd_dkdv_f32(BwdArgs a) {
  constexpr int kD = Width<D>::kD, kHalf = Width<D>::kHalf, kParts = Width<D>::kParts;
  constexpr float kC = Width<D>::kC, kInvSqrtD = Width<D>::kInvSqrtD;
  __shared__ float Qs[kRows][kD], dOs[kRows][kD], Ls[kRows], Ds[kRows];
  const int tid = threadIdx.x, h = tid % kParts;
  const int n_q = a.n_q, n_k = a.n_k, n_tiles = (n_q + 63) / 64;
  const int nkb = (n_k + kRows - 1) / kRows;
  const int bh = blockIdx.x / nkb, k0 = (blockIdx.x % nkb) * kRows;
  const int key = k0 + tid / kParts;
  const int n_real = real_keys(a.kv_len, bh / a.H, n_k);  // keys from n_real on are padding: gradient 0
  const float* Qp = static_cast<const float*>(a.Q) + (int64_t)bh * n_q * kD;
  const float* dOp = static_cast<const float*>(a.dO) + (int64_t)bh * n_q * kD;
  const float* Kp = static_cast<const float*>(a.K) + (int64_t)bh * n_k * kD;
  const float* Vp = static_cast<const float*>(a.V) + (int64_t)bh * n_k * kD;

  float k[kHalf], v[kHalf], dk[kHalf], dv[kHalf];
#pragma unroll
  for (int d = 0; d < kHalf; ++d) {
    k[d] = key < n_real ? Kp[(int64_t)key * kD + kHalf * h + d] : 0.f;
    v[d] = key < n_real ? Vp[(int64_t)key * kD + kHalf * h + d] : 0.f;
    dk[d] = dv[d] = 0.f;
  }
  // causal: rows before k0 see none of these keys; a workgroup of padding keys only writes zeros
  int q_begin = a.causal ? k0 : 0, q_end = k0 < n_real ? n_q : 0;
  if (a.windowed) {  // restricted self-attention: rows within a.window of some key of the block
    if (!a.causal) q_begin = max(0, k0 - a.window) / kRows * kRows;
    q_end = min(q_end, k0 + kRows + a.window);
  }
  for (int q0 = q_begin; q0 < q_end; q0 += kRows) {
    __syncthreads();
    for (int e = tid; e < kRows * kD; e += kParts * kRows) {
      const int r = e / kD, c = e % kD;
      const bool ok = q0 + r < n_q;
      Qs[r][c] = ok ? Qp[(int64_t)(q0 + r) * kD + c] : 0.f;
      dOs[r][c] = ok ? dOp[(int64_t)(q0 + r) * kD + c] : 0.f;
    }
    if (tid < kRows) {
      const bool ok = q0 + tid < n_q;
      const float2 ld = ok ? aux_row(a.aux, n_tiles, bh, q0 + tid) : float2{INFINITY, 0.f};
      Ls[tid] = ld.x;
      Ds[tid] = ld.y;
    }
    __syncthreads();
    for (int i = 0; i < kRows; ++i) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < kHalf; ++d) {
        s = fmaf(k[d], Qs[i][kHalf * h + d], s);
        dp = fmaf(v[d], dOs[i][kHalf * h + d], dp);
      }
      s = row_sum<kParts>(s);
      dp = row_sum<kParts>(dp);
      const int row = q0 + i;
      float p = fast_exp2(fmaf(s, kC, -Ls[i]));  // 0 for rows past n_q and rows that saw no key (lse2 = +inf)
      if ((a.causal && key > row) || key >= n_real || (a.windowed && (key > row + a.window || key < row - a.window)))
        p = 0.f;
      const float ds = p * (dp - Ds[i]);
#pragma unroll
      for (int d = 0; d < kHalf; ++d) {
        dv[d] = fmaf(p, dOs[i][kHalf * h + d], dv[d]);
        dk[d] = fmaf(ds, Qs[i][kHalf * h + d], dk[d]);
      }
    }
  }
  if (key < n_k) {
    float* dkr = static_cast<float*>(a.dK) + ((int64_t)bh * n_k + key) * kD + kHalf * h;
    float* dvr = static_cast<float*>(a.dV) + ((int64_t)bh * n_k + key) * kD + kHalf * h;
#pragma unroll
    for (int d = 0; d < kHalf; d += 4) {
      *reinterpret_cast<float4*>(dvr + d) = float4{dv[d], dv[d + 1], dv[d + 2], dv[d + 3]};
      *reinterpret_cast<float4*>(dkr + d) =
          float4{dk[d] * kInvSqrtD, dk[d + 1] * kInvSqrtD, dk[d + 2] * kInvSqrtD, dk[d + 3] * kInvSqrtD};
    }
  }
}

// dQ: a workgroup owns 32 queries; key/value rows stream through LDS.
template <int D>
__global__ __launch_bounds__(Width<D>::kParts * kRows) void attn_bwd_dq_f32(BwdArgs a) {
  constexpr int kD = Width<D>::kD, kHalf = Width<D>::kHalf, kParts = Width<D>::kParts;
  constexpr float kC = Width<D>::kC, kInvSqrtD = Width<D>::kInvSqrtD;
  __shared__ float Ks[kRows][kD], Vs[kRows][kD];
  const int tid = threadIdx.x, h = tid % kParts;
  const int n_q = a.n_q, n_k = a.n_k, n_tiles = (n_q + 63) / 64;
  const int nqb = (n_q + kRows - 1) / kRows;
  const int bh = blockIdx.x / nqb, qb0 = (blockIdx.x % nqb) * kRows;
  const int qi = qb0 + tid / kParts;
  const int n_real = real_keys(a.kv_len, bh / a.H, n_k);  // keys from n_real on (padding) are never read
  const float* Qp = static_cast<const float*>(a.Q) + (int64_t)bh * n_q * kD;
  const float* dOp = static_cast<const float*>(a.dO) + (int64_t)bh * n_q * kD;
  const float* Kp = static_cast<const float*>(a.K) + (int64_t)bh * n_k * kD;
  const float* Vp = static_cast<const float*>(a.V) + (int64_t)bh * n_k * kD;

  float q[kHalf], o[kHalf], dq[kHalf];
#pragma unroll
  for (int d = 0; d < kHalf; ++d) {
    q[d] = qi < n_q ? Qp[(int64_t)qi * kD + kHalf * h + d] : 0.f;
    o[d] = qi < n_q ? dOp[(int64_t)qi * kD + kHalf * h + d] : 0.f;
    dq[d] = 0.f;
  }
  const float2 ld = qi < n_q ? aux_row(a.aux, n_tiles, bh, qi) : float2{INFINITY, 0.f};
  int k_end = a.causal ? min(n_real, qb0 + kRows) : n_real;  // keys after the last query are never needed
  int k_begin = 0;
  if (a.windowed) {  // restricted self-attention: keys within a.window of some query of the block
    k_end = min(k_end, qb0 + kRows + a.window);
    k_begin = max(0, qb0 - a.window) / kRows * kRows;
  }
  for (int k0 = k_begin; k0 < k_end; k0 += kRows) {
    __syncthreads();
    for (int e = tid; e < kRows * kD; e += kParts * kRows) {
      const int r = e / kD, c = e % kD;
      const bool ok = k0 + r < n_real;
      Ks[r][c] = ok ? Kp[(int64_t)(k0 + r) * kD + c] : 0.f;
      Vs[r][c] = ok ? Vp[(int64_t)(k0 + r) * kD + c] : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < kRows; ++j) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < kHalf; ++d) {
        s = fmaf(q[d], Ks[j][kHalf * h + d], s);
        dp = fmaf(o[d], Vs[j][kHalf * h + d], dp);
      }
      s = row_sum<kParts>(s);
      dp = row_sum<kParts>(dp);
      const int key = k0 + j;
      float p = fast_exp2(fmaf(s, kC, -ld.x));
      if (key >= n_real || (a.causal && key > qi) || (a.windowed && (key > qi + a.window || key < qi - a.window)))
        p = 0.f;
      const float ds = p * (dp - ld.y);
#pragma unroll
      for (int d = 0; d < kHalf; ++d) dq[d] = fmaf(ds, Ks[j][kHalf * h + d], dq[d]);
    }
  }
  if (qi < n_q) {
    float* r = static_cast<float*>(a.dQ) + ((int64_t)bh * n_q + qi) * kD + kHalf * h;
#pragma unroll
    for (int d = 0; d < kHalf; d += 4)
      *reinterpret_cast<float4*>(r + d) =
          float4{dq[d] * kInvSqrtD, dq[d + 1] * kInvSqrtD, dq[d + 2] * kInvSqrtD, dq[d + 3] * kInvSqrtD};
  }
}

}  // namespace

namespace {

template <int D>
hipError_t launch_bwd_f32_d(const BwdArgs& a, int64_t nb_kv, int64_t nb_q, hipStream_t stream) {
  constexpr int kThreads = Width<D>::kParts * kRows;
  hipLaunchKernelGGL(attn_bwd_dkdv_f32<D>, dim3((unsigned)nb_kv), dim3(kThreads), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dq_f32<D>, dim3((unsigned)nb_q), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_f32(const BwdArgs& a, int d, hipStream_t stream) {
  const int64_t nb_kv = (int64_t)((a.n_k + kRows - 1) / kRows) * a.B * a.H;
  const int64_t nb_q = (int64_t)((a.n_q + kRows - 1) / kRows) * a.B * a.H;
  if (nb_kv <= 0 || nb_kv > 0x7fffffff || nb_q <= 0 || nb_q > 0x7fffffff || (d != 32 && d != 64 && d != 128))
    return hipErrorInvalidValue;
  const hipError_t e = launch_attn_bwd_pre(a, true, d, stream);
  if (e != hipSuccess) return e;
  if (d == 64) return launch_bwd_f32_d<64>(a, nb_kv, nb_q, stream);
  if (d == 32) return launch_bwd_f32_d<32>(a, nb_kv, nb_q, stream);
  return launch_bwd_f32_d<128>(a, nb_kv, nb_q, stream);
}

}  // namespace mi355
