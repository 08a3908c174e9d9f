// Scaled dot-product attention forward in fp32 throughout, d_k = d_v = D in {32, 64, 128}, for gfx950.
//
// Same mathematics as the bf16 kernel (softmax(Q K^T / sqrt(D)) V per head, optional causal mask; "Attention Is All
// You Need" (lettle.cn translation), section 3.2.1), but every value stays fp32, including the softmax weights that
// multiply V. This path serves small fp32 problems, so it is a plain VALU kernel: D/8 threads per query row, each
// with eight of the row's dimensions in registers (q and its share of the output accumulator; the partial dot
// products are added across the row's lanes), key/value tiles staged in LDS and read as broadcasts, and the softmax
// streamed tile by tile (running max, rescaled running sum). A workgroup is one wave of 64 / (D/8) query rows; a tile's
// key loop stops at the last key any row of the workgroup may see.
#include "device_common.h"
#include "launch.h"

#include <math.h>

namespace mi355 {
namespace {

constexpr int kThreads = 64;  // one wave per workgroup
constexpr int kBK = 32;       // keys per tile
constexpr int kDT = 8;        // dimensions of a row per thread

// threads per query row (D / 8): a thread's share of every K and V row is two 16-byte LDS reads, and the short
// problems this kernel serves (a handful of query rows) spread over more waves
template <int D>
constexpr int threads_per_row() { return D / kDT; }
// queries per workgroup
template <int D>
constexpr int rows_per_block() { return kThreads / threads_per_row<D>(); }

template <int D>
__global__ __launch_bounds__(kThreads) void attn_fwd_f32(AttnArgs a, int n_qblocks, float c) {
  constexpr int kD = D;
  constexpr int kTPR = threads_per_row<D>();
  constexpr int kBQ = rows_per_block<D>();
  __shared__ __attribute__((aligned(16))) float Ks[kBK * kD];
  __shared__ __attribute__((aligned(16))) float Vs[kBK * kD];

  const int tid = threadIdx.x;
  const int part = tid % kTPR;  // this thread's dimensions: part*kDT .. part*kDT + kDT-1
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  int qb = blk % n_qblocks;
  const int bh = blk / n_qblocks;
  if (a.causal) qb = n_qblocks - 1 - qb;
  const int b = bh / a.H, hh = bh % a.H;
  const int n_q = a.n_q, n_k = real_keys(a.kv_len, b, a.n_k);  // keys from n_k on (padding) are never read
  const float* Qp = static_cast<const float*>(a.Q) + (int64_t)bh * a.q_stride_bh;
  const float* Kp = static_cast<const float*>(a.K) + (int64_t)bh * a.k_stride_bh;
  const float* Vp = static_cast<const float*>(a.V) + (int64_t)bh * a.k_stride_bh;
  float* Op = static_cast<float*>(a.O) + b * a.o_stride_b + hh * a.o_stride_h;

  const int q0 = qb * kBQ;
  const int qi = q0 + tid / kTPR;
  float q[kDT], o[kDT];
#pragma unroll
  for (int d = 0; d < kDT; d += 4) {
    const float4 v =
        qi < n_q ? *reinterpret_cast<const float4*>(Qp + (int64_t)qi * kD + part * kDT + d) : float4{0, 0, 0, 0};
    q[d] = v.x; q[d + 1] = v.y; q[d + 2] = v.z; q[d + 3] = v.w;
    o[d] = o[d + 1] = o[d + 2] = o[d + 3] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  int n_end = n_k, k_begin = 0;
  if (a.causal) n_end = min(n_k, q0 + kBQ);  // keys after the block's last query are never needed
  if (a.windowed) {  // restricted self-attention: keys within a.window of some query of the block
    n_end = min(n_end, q0 + kBQ + a.window);
    k_begin = max(0, q0 - a.window) / kBK * kBK;
  }
  for (int k0 = k_begin; k0 < n_end; k0 += kBK) {
    __syncthreads();
    // 32 rows x D floats per tensor in float4 chunks; rows past n_k load as zeros
    for (int ch = tid; ch < kBK * kD / 4; ch += kThreads) {
      const int r = ch / (kD / 4), col = (ch % (kD / 4)) * 4;
      // (a branch, not a select between a global row and a zero constant: the select became a flat load from a
      // private copy of the constant)
      float4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (k0 + r < n_k) {
        kv = *reinterpret_cast<const float4*>(Kp + (int64_t)(k0 + r) * kD + col);
        vv = *reinterpret_cast<const float4*>(Vp + (int64_t)(k0 + r) * kD + col);
      }
      *reinterpret_cast<float4*>(&Ks[r * kD + col]) = kv;
      *reinterpret_cast<float4*>(&Vs[r * kD + col]) = vv;
    }
    __syncthreads();

    float s[kBK];
#pragma unroll
    for (int j = 0; j < kBK; ++j) s[j] = -INFINITY;
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kBK; ++j) {
      // four partial sums over d mod 4: four independent fma chains of D/4 (one chain of D would serialise on the
      // fma latency)
      if (k0 + j >= n_end) continue;  // (uniform) no row of the workgroup sees a later key of this tile
      float acc4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int d = 0; d < kDT; ++d) acc4[d & 3] = fmaf(q[d], Ks[j * kD + part * kDT + d], acc4[d & 3]);
      float acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
#pragma unroll
      for (int off = 1; off < kTPR; off <<= 1) acc += __shfl_xor(acc, off);  // (the same sum in every lane of the row)
      const int key = k0 + j;
      if (key >= n_k || (a.causal && key > qi) || (a.windowed && (key > qi + a.window || key < qi - a.window)))
        acc = -INFINITY;
      s[j] = acc;
      mx = fmaxf(mx, acc);
    }
    const float m_new = fmaxf(m, mx * c);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int d = 0; d < kDT; ++d) o[d] *= alpha;
#pragma unroll
    for (int j = 0; j < kBK; ++j) {
      if (k0 + j >= n_end) continue;
      const float p = fast_exp2(fmaf(s[j], c, -m_use));
      l += p;
#pragma unroll
      for (int d = 0; d < kDT; ++d) o[d] = fmaf(p, Vs[j * kD + part * kDT + d], o[d]);
    }
  }
  if (qi < n_q) {
    const bool seen = l > 0.f;  // false only for a row with no real key (all padding): output 0, lse -inf
    const float inv = seen ? 1.0f / l : 0.f;
    // row log-sum-exp of the scaled scores, natural log: log2(sum_j exp2(s_j c)) = m + log2(l)
    if (a.lse != nullptr && part == 0)
      a.lse[(int64_t)bh * n_q + qi] = seen ? (m + __builtin_amdgcn_logf(l)) * 0.6931471805599453f : -INFINITY;
    float* orow = Op + (int64_t)qi * a.o_stride_row + part * kDT;
#pragma unroll
    for (int d = 0; d < kDT; d += 4)
      *reinterpret_cast<float4*>(orow + d) = float4{o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv};
  }
}

}  // namespace

hipError_t launch_attn_fwd_f32(const AttnArgs& a, int d, hipStream_t stream) {
  if (d != 32 && d != 64 && d != 128) return hipErrorInvalidValue;
  const int rows = kThreads / (d / kDT);
  const int n_qblocks = (a.n_q + rows - 1) / rows;
  const int64_t nblocks = (int64_t)n_qblocks * a.B * a.H;
  if (nblocks <= 0 || nblocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nblocks);
  // c = log2(e) / sqrt(d)
  switch (d) {
    case 32:
      hipLaunchKernelGGL(attn_fwd_f32<32>, grid, dim3(kThreads), 0, stream, a, n_qblocks,
                         (float)(1.4426950408889634 / 5.656854249492381));
      break;
    case 64:
      hipLaunchKernelGGL(attn_fwd_f32<64>, grid, dim3(kThreads), 0, stream, a, n_qblocks,
                         (float)(1.4426950408889634 / 8.0));
      break;
    default:
      hipLaunchKernelGGL(attn_fwd_f32<128>, grid, dim3(kThreads), 0, stream, a, n_qblocks,
                         (float)(1.4426950408889634 / 11.313708498984761));
      break;
  }
  return hipGetLastError();
}

}  // namespace mi355
