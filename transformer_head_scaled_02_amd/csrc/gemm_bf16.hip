// bf16 GEMM C = A W with fp32 accumulation on gfx950 MFMA, for the multi-head attention projections.
//
// Q_i = Xq W_i^Q, K_i = Xkv W_i^K, V_i = Xkv W_i^V for all heads at once (W_i is the column block i of the packed
// [d_model, h*64] matrix), and Concat(head_1..head_h) W^O: "Transformer：抛弃循环与卷积的序列建模"
// (jiashun-ye.github.io), section "Multi-Head Attention"; no bias appears in these formulas.
//
// Tile 128 x 64 x 64 per workgroup of 4 waves; each wave owns 32 rows x 64 columns (two 32x32 MFMA accumulators).
// A tiles are staged row-major in LDS; W tiles (k-major in memory) are transposed on the way into LDS so that both
// MFMA operands are 16-byte LDS reads. Up to three independent problems share one launch (the Q, K and V projections).
// The "head-major" epilogue writes column block n/64 of row (b, i) straight to [b][n/64][i][n%64], which is the
// per-head layout the attention kernel reads, so no separate reshape pass exists. The row-major epilogue can add a
// bias, apply ReLU and add a residual before the rounding to bf16: the position-wise FFN max(0, x W1 + b1) W2 + b2 and
// the residual connection x + Sublayer(x) of the encoder layer ("Transformer：抛弃循环与卷积的序列建模", sections
// "FFN" and "Residual Connection 与 LayerNorm") then cost no extra pass over memory.
#include "device_common.h"
#include "launch.h"

namespace mi355 {
namespace {

constexpr int kBM = 128, kBN = 64, kBK = 64;
constexpr int kLds = 72;  // LDS row stride (bf16 elements)
constexpr int kThreads = 256;
constexpr int kMaxProbs = 3;

struct GemmBatch {
  GemmProblem p[kMaxProbs];
  int tiles_n[kMaxProbs];
  int tile_start[kMaxProbs + 1];
  int nprobs;
};

__global__ __launch_bounds__(kThreads) void gemm_bf16_mfma(GemmBatch batch) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t Wt[kBN * kLds];

  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  int pi = 0;
  while (pi + 1 < batch.nprobs && blk >= batch.tile_start[pi + 1]) ++pi;
  const GemmProblem& P = batch.p[pi];
  const int local = blk - batch.tile_start[pi];
  const int tm = local / batch.tiles_n[pi], tn = local % batch.tiles_n[pi];
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int M = P.M, N = P.N, K = P.K;
  const uint16_t* A = static_cast<const uint16_t*>(P.A);
  const uint16_t* W = static_cast<const uint16_t*>(P.W);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;

  // loaders: A chunk c = tid + 256i -> row c/8, cols 8*(c%8); W rows k0 + 2*(tid/8) (+1), cols n0 + 8*(tid%8)
  uint4 ar[4], wr0, wr1;
  const int wkp = tid >> 3, wnc = (tid & 7) * 8;
  auto gload = [&](int k0) {
    const uint4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i, r = c >> 3, col = (c & 7) * 8;
      ar[i] = (m0 + r < M) ? *reinterpret_cast<const uint4*>(A + (int64_t)(m0 + r) * K + k0 + col) : z;
    }
    wr0 = *reinterpret_cast<const uint4*>(W + (int64_t)(k0 + 2 * wkp) * N + n0 + wnc);
    wr1 = *reinterpret_cast<const uint4*>(W + (int64_t)(k0 + 2 * wkp + 1) * N + n0 + wnc);
  };
  auto lds_store = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i, r = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<uint4*>(&As[r * kLds + col]) = ar[i];
    }
    const uint32_t wa[4] = {wr0.x, wr0.y, wr0.z, wr0.w};
    const uint32_t wb[4] = {wr1.x, wr1.y, wr1.z, wr1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t lo = (e & 1) ? (wa[e >> 1] >> 16) : (wa[e >> 1] & 0xffffu);
      const uint32_t hi = (e & 1) ? (wb[e >> 1] & 0xffff0000u) : (wb[e >> 1] << 16);
      *reinterpret_cast<uint32_t*>(&Wt[(wnc + e) * kLds + 2 * wkp]) = lo | hi;
    }
  };

  f32x16 acc0 = {}, acc1 = {};
  const uint16_t* arow = &As[(32 * wave + li) * kLds + 8 * g];
  const uint16_t* brow = &Wt[li * kLds + 8 * g];
  gload(0);
  for (int k0 = 0; k0 < K; k0 += kBK) {
    __syncthreads();
    lds_store();
    __syncthreads();
    if (k0 + kBK < K) gload(k0 + kBK);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + 16 * kk);
      const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(brow + 16 * kk);
      const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(brow + 32 * kLds + 16 * kk);
      acc0 = mfma32x32x16(a, b0, acc0);
      acc1 = mfma32x32x16(a, b1, acc1);
    }
  }

  // accumulator register r: row m0 + 32*wave + 8(r/4) + 4g + r%4, column n0 + 32nb + li
  uint16_t* C = static_cast<uint16_t*>(P.C);
  const uint16_t* bias = static_cast<const uint16_t*>(P.bias);
  const uint16_t* res = static_cast<const uint16_t*>(P.residual);
  const int hs = P.head_seq;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const f32x16& acc = nb ? acc1 : acc0;
    const int n = n0 + 32 * nb + li;
    const float bn = bias != nullptr ? bf16_bits_to_f32(bias[n]) : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int mm = m0 + 32 * wave + 8 * (r >> 2) + 4 * g + (r & 3);
      if (mm >= M) continue;
      int64_t off;
      float v = acc[r];
      if (hs == 0) {
        off = (int64_t)mm * N + n;
        v += bn;
        if (P.relu) v = fmaxf(v, 0.f);
        if (res != nullptr) v += bf16_bits_to_f32(res[off]);
      } else {
        const int bb = mm / hs, i = mm % hs;
        off = (((int64_t)bb * (N / 64) + n / 64) * hs + i) * 64 + (n & 63);
      }
      C[off] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu);
    }
  }
}

// LayerNorm of rows of D bf16 values, one wave per row: each lane takes 16-byte chunks l and l + 64; the mean and then
// the mean squared deviation are reduced across the wave in fp32 (two passes over registers, no cancellation).
__global__ __launch_bounds__(256) void layer_norm_bf16(const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma,
                                                      const uint16_t* __restrict__ beta, uint16_t* __restrict__ y,
                                                      int M, int D, float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= M) return;  // (uniform per wave)
  const int nchunk = D / 8;
  const uint16_t* xr = x + (int64_t)row * D;
  float v[2][8];
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int ch = lane + 64 * c;
    uint4 w = {0u, 0u, 0u, 0u};
    if (ch < nchunk) w = *reinterpret_cast<const uint4*>(xr + 8 * ch);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[c][2 * j] = __uint_as_float(ws[j] << 16);
      v[c][2 * j + 1] = __uint_as_float(ws[j] & 0xffff0000u);
      sum += v[c][2 * j] + v[c][2 * j + 1];
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
  const float mean = sum / (float)D;
  float sq = 0.f;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (lane + 64 * c >= nchunk) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float d = v[c][j] - mean;
      sq = fmaf(d, d, sq);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sq += __shfl_xor(sq, o);
  const float rstd = 1.0f / sqrtf(sq / (float)D + eps);
  uint16_t* yr = y + (int64_t)row * D;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int ch = lane + 64 * c;
    if (ch >= nchunk) continue;
    const uint4 gw = *reinterpret_cast<const uint4*>(gamma + 8 * ch);
    const uint4 bw = *reinterpret_cast<const uint4*>(beta + 8 * ch);
    const uint32_t gs[4] = {gw.x, gw.y, gw.z, gw.w}, bs[4] = {bw.x, bw.y, bw.z, bw.w};
    uint32_t out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float y0 = fmaf((v[c][2 * j] - mean) * rstd, __uint_as_float(gs[j] << 16), __uint_as_float(bs[j] << 16));
      const float y1 = fmaf((v[c][2 * j + 1] - mean) * rstd, __uint_as_float(gs[j] & 0xffff0000u),
                            __uint_as_float(bs[j] & 0xffff0000u));
      out[j] = pack_bf16x2(y0, y1);
    }
    *reinterpret_cast<uint4*>(yr + 8 * ch) = uint4{out[0], out[1], out[2], out[3]};
  }
}

}  // namespace

hipError_t launch_layer_norm_bf16(const void* x, const void* gamma, const void* beta, void* y, int M, int D, float eps,
                                  hipStream_t stream) {
  if (M <= 0 || D <= 0 || D % 64 || D > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(layer_norm_bf16, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(gamma),
                     static_cast<const uint16_t*>(beta), static_cast<uint16_t*>(y), M, D, eps);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmProblem* probs, int nprobs, hipStream_t stream) {
  if (nprobs < 1 || nprobs > kMaxProbs) return hipErrorInvalidValue;
  GemmBatch batch{};
  batch.nprobs = nprobs;
  int64_t total = 0;
  for (int i = 0; i < nprobs; ++i) {
    const GemmProblem& p = probs[i];
    if (p.M <= 0 || p.N <= 0 || p.K <= 0 || p.N % kBN || p.K % kBK) return hipErrorInvalidValue;
    batch.p[i] = p;
    batch.tiles_n[i] = p.N / kBN;
    batch.tile_start[i] = (int)total;
    total += (int64_t)((p.M + kBM - 1) / kBM) * batch.tiles_n[i];
    if (total > 0x7fffffff) return hipErrorInvalidValue;
  }
  batch.tile_start[nprobs] = (int)total;
  hipLaunchKernelGGL(gemm_bf16_mfma, dim3((unsigned)total), dim3(kThreads), 0, stream, batch);
  return hipGetLastError();
}

}  // namespace mi355
