// bf16 GEMM C = A W with fp32 accumulation on gfx950 MFMA, for the multi-head attention projections and the FFN.
//
// Q_i = Xq W_i^Q, K_i = Xkv W_i^K, V_i = Xkv W_i^V for all heads at once (W_i is the column block i of the packed
// [d_model, h*64] matrix), and Concat(head_1..head_h) W^O: "Transformer：抛弃循环与卷积的序列建模"
// (jiashun-ye.github.io), section "Multi-Head Attention"; no bias appears in these formulas.
//
// A workgroup of 4 waves computes a 128 x 128 tile of C, each wave a 64 x 64 quarter as 2 x 2 blocks of
// v_mfma_f32_32x32x16_bf16. The product is formed transposed, C^T = W^T A^T: the MFMA's first operand is a 32-column
// strip of W read from LDS with ds_read_b64_tr_b16 (8 consecutive k of one column per lane, the operand layout W's
// row-major [K, N] storage does not give directly), its second a 32-row strip of A read row-wise, and each lane ends
// up with 4 consecutive columns of one row of C, stored 8 bytes at a time. A (128 x 64) and W (64 x 128) k-tiles go
// HBM -> LDS by global_load_lds_dwordx4 into a two-stage ring (64 KB: two workgroups per CU), as four 64 x 64
// sub-tiles with 128-byte rows and the XOR chunk swizzle of attn_tile.h, which keeps both the row reads and the
// transposed reads free of bank conflicts. Up to three independent problems share one launch (the Q, K and V
// projections).
// The "head-major" epilogue writes column block n/w of row (b, i) straight to [b][n/w][i][n%w] (w the head width),
// which is the per-head layout the attention kernel reads, so no separate reshape pass exists. The row-major epilogue
// can add a bias, apply ReLU and add a residual before the rounding to bf16: the position-wise FFN
// max(0, x W1 + b1) W2 + b2 and the residual connection x + Sublayer(x) of the encoder layer
// ("Transformer：抛弃循环与卷积的序列建模", sections "FFN" and "Residual Connection 与 LayerNorm") then cost no extra
// pass over memory.
#include "attn_tile.h"
#include "launch.h"

namespace mi355 {
namespace {

constexpr int kTN = 128, kTK = 64;             // workgroup tile columns and k-tile (rows: TM = 128 or 64)
constexpr int kSub = 64 * 64;                  // one 64 x 64 bf16 sub-tile, rows of 128 bytes (8 KB)
// a stage: [A rows 0..TM-1 (TM/64 sub-tiles) | W cols 0-63 | W cols 64-127]
constexpr int kMaxProbs = 3;
constexpr int kGemmStages = 2;  // ring depth of the launch
constexpr int kGemmWaves = 8;   // waves per workgroup (2 x kGemmWaves/2 over the tile)

struct GemmBatch {
  GemmProblem p[kMaxProbs];
  int tiles_n[kMaxProbs];
  int tile_start[kMaxProbs + 1];
  int nprobs;
};

template <int kStagesG, int TM, int NWV>
__global__ __launch_bounds__(64 * NWV, 1) void gemm_bf16_mfma(GemmBatch batch) {
  constexpr int kStageElemsG = (TM / 64 + 2) * kSub;
  constexpr int WN = NWV / 2;          // waves across the 128 columns (2 down the rows)
  constexpr int MB = TM / 64;          // 32-row blocks per wave
  constexpr int NB = 4 / WN;           // 32-column blocks per wave
  constexpr int kACopies = TM / 8;     // one-kilobyte copies of A rows per stage (W: 16)
  constexpr int kCPW = (kACopies + 16) / NWV;  // copies per wave
  static_assert((kACopies + 16) % NWV == 0, "copies split evenly over the waves");
  __shared__ __attribute__((aligned(16))) uint16_t smem[kStagesG * kStageElemsG];

  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  int pi = 0;
  while (pi + 1 < batch.nprobs && blk >= batch.tile_start[pi + 1]) ++pi;
  const GemmProblem& P = batch.p[pi];
  const int local = blk - batch.tile_start[pi];
  const int tm = local / batch.tiles_n[pi], tn = local % batch.tiles_n[pi];
  const int m0 = tm * TM, n0 = tn * kTN;
  const int M = P.M, N = P.N, K = P.K;
  const uint16_t* A = static_cast<const uint16_t*>(P.A);
  const uint16_t* W = static_cast<const uint16_t*>(P.W);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int rows_left = M - m0;            // rows of A (and C) in this tile, >= 1
  const bool half_n = n0 + 64 >= N;        // only the first 64 columns exist (N is a multiple of 64)

  // Copies: wave w issues copies 8w .. 8w+7 of a stage; copies 0-15 bring A rows 8c .. 8c+7, copies 16-31 W rows
  // (k) 8c .. 8c+7 of sub-tile c/8. Lane l brings the logical chunk that belongs at physical chunk l%8 of row l/8 of
  // its eight rows; the two per-lane offsets (first or second eight rows of a 16-row swizzle period) serve all copies.
  const uint32_t smem_lds = (uint32_t)(uintptr_t)smem;
  const int lr = lane >> 3;
  uint32_t a_voff[2], w_voff[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const uint32_t chunk = (uint32_t)(((lane & 7) ^ swz(8 * c + lr)) << 4);
    a_voff[c] = (uint32_t)lr * (uint32_t)K * 2u + chunk;
    w_voff[c] = (uint32_t)lr * (uint32_t)N * 2u + chunk;
  }
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int k0 = t * kTK;
    const uint32_t stage = smem_lds + (uint32_t)((t % kStagesG) * kStageElemsG * 2);
#pragma unroll
    for (int i = 0; i < kCPW; ++i) {
      const int gi = kCPW * wave + i;  // (uniform)
      if (gi < kACopies) {
        // A rows 8gi .. 8gi+7 of the tile
        const uint32_t dst = stage + (uint32_t)(gi >> 3) * kSub * 2u + (uint32_t)(gi & 7) * 1024u;
        if (rows_left >= TM) {
          lds_dma16(A + (int64_t)(m0 + 8 * gi) * K + k0, a_voff[gi & 1], dst);
        } else {
          // rows past M read row M-1 (their results are not stored); offsets from the unshifted tile base
          int l8 = lr;
          asm volatile("" : "+v"(l8));
          const int row = 8 * gi + l8;
          const uint32_t chunk = (uint32_t)(((lane & 7) ^ swz(row)) << 4);
          lds_dma16(A + (int64_t)m0 * K + k0, (uint32_t)min(row, rows_left - 1) * (uint32_t)K * 2u + chunk, dst);
        }
      } else {
        // W k-rows 8c .. 8c+7 of sub-tile s (columns n0 + 64s ..); a missing second half re-reads the first (its
        // results are not stored)
        const int gw = gi - kACopies, sub = gw >> 3, c = gw & 7;
        const int src_sub = half_n ? 0 : sub;
        const uint32_t dst = stage + (uint32_t)(MB + sub) * kSub * 2u + (uint32_t)c * 1024u;
        lds_dma16(W + (int64_t)(k0 + 8 * c) * N + n0 + 64 * src_sub, w_voff[c & 1], dst);
      }
    }
  };

  // Operand offsets. Second operand (A^T, 16 k x 32 rows of A): lane reads row 32mb + li of its A sub-tile, k =
  // 16ks + 8g .. +7 (logical chunk 2ks + g). First operand (W^T, 32 columns x 16 k): two transposed reads give column
  // 32nb + l%32 of its W sub-tile at k-rows 16ks + 8g + (0..3) and 16ks + 8g + 4 + (0..3); within each 16-lane group
  // source lane 4j + t addresses row r0 + j, columns c0 + 4t .. +3.
  int aoff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) aoff[ks] = li * kD + (((2 * ks + g) ^ swz(li)) << 3);
  int toff[2][2];
  {
    const int jj = (lane & 15) >> 2;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int row = 8 * g + jj + 4 * hi;
        const int lchunk = 4 * nb + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        toff[nb][hi] = row * kD + ((lchunk ^ swz(row)) << 3) + 4 * (lane & 1);
      }
  }

  f32x16 acc[NB][MB];  // [nb][mb]: register r = C[row 32mb + li][column 32nb + 8(r/4) + 4g + r%4] of this wave's part
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x16{};

  const int nk = K / kTK;
#pragma unroll
  for (int i = 0; i < kStagesG - 1; ++i)
    if (i < nk) issue(i);
  for (int t = 0; t < nk; ++t) {
    // this wave's copies of k-tile t (8 per tile; the later tiles' may stay in flight), then everyone's; everyone is
    // also done with t-1, whose stage tile t + kStagesG - 1 now takes
    const int ahead = min(kStagesG - 2, nk - 1 - t);
    if (kStagesG >= 4 && ahead >= 2) wait_vmcnt<(kStagesG >= 4 ? 2 * kCPW : 0)>();
    else if (kStagesG >= 3 && ahead >= 1) wait_vmcnt<(kStagesG >= 3 ? kCPW : 0)>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (t + kStagesG - 1 < nk) issue(t + kStagesG - 1);
    const uint16_t* st = smem + (t % kStagesG) * kStageElemsG;
    const uint16_t* As = st + (wave / WN) * (TM / 2) * kD;  // this wave's TM/2 rows of A
    // this wave's 32 NB columns: sub-tile (wn * NB) / 2, 32-column blocks cb0 .. cb0 + NB - 1 within it
    const int wn = wave % WN, cb0 = (wn * NB) % 2;
    const uint16_t* Ws = st + (MB + (wn * NB) / 2) * kSub;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 bo[MB], ao[NB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) bo[mb] = *reinterpret_cast<const bf16x8*>(As + mb * 32 * kD + aoff[ks]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x4 lo = lds_read_tr16x4(Ws + ks * 16 * kD + toff[cb0 + nb][0]);
        const bf16x4 hi = lds_read_tr16x4(Ws + ks * 16 * kD + toff[cb0 + nb][1]);
        ao[nb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = mfma32x32x16(ao[nb], bo[mb], acc[nb][mb]);
    }
  }

  // Epilogue: lane writes columns n .. n+3 of row m for each (nb, mb, r/4).
  const int mw = m0 + (TM / 2) * (wave / WN), nw = n0 + (128 / WN) * (wave % WN);
  if (nw >= N) return;  // (uniform) the missing half of a 64-column-wide problem
  uint16_t* C = static_cast<uint16_t*>(P.C);
  const uint16_t* bias = static_cast<const uint16_t*>(P.bias);
  const uint16_t* res = static_cast<const uint16_t*>(P.residual);
  const int hs = P.head_seq;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = mw + 32 * mb + li;
    if (m >= M) continue;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int n = nw + 32 * nb + 8 * rg + 4 * g;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = acc[nb][mb][4 * rg + i];
        int64_t off;
        if (hs == 0) {
          off = (int64_t)m * N + n;
          if (bias != nullptr) {
            const uint2 bw = *reinterpret_cast<const uint2*>(bias + n);
            v[0] += __uint_as_float(bw.x << 16);
            v[1] += __uint_as_float(bw.x & 0xffff0000u);
            v[2] += __uint_as_float(bw.y << 16);
            v[3] += __uint_as_float(bw.y & 0xffff0000u);
          }
          if (P.relu) {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = fmaxf(v[i], 0.f);
          }
          if (res != nullptr) {
            const uint2 rw = *reinterpret_cast<const uint2*>(res + off);
            v[0] += __uint_as_float(rw.x << 16);
            v[1] += __uint_as_float(rw.x & 0xffff0000u);
            v[2] += __uint_as_float(rw.y << 16);
            v[3] += __uint_as_float(rw.y & 0xffff0000u);
          }
        } else {
          // (a lane's four columns n .. n+3 lie in one head: n is a multiple of 4 and the width of 32 or more)
          const int bb = m / hs, i = m % hs, hsh = P.head_shift;
          off = ((((int64_t)bb * (N >> hsh) + (n >> hsh)) * hs + i) << hsh) + (n & ((1 << hsh) - 1));
        }
        *reinterpret_cast<uint2*>(C + off) = uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
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
  // 128-row tiles when they already give at least two workgroups per CU, else 64-row tiles (twice the workgroups)
  int64_t tiles128 = 0;
  for (int i = 0; i < nprobs; ++i)
    tiles128 += (int64_t)((probs[i].M + 127) / 128) * ((probs[i].N + kTN - 1) / kTN);
  const int tm = tiles128 >= 512 ? 128 : 64;
  GemmBatch batch{};
  batch.nprobs = nprobs;
  int64_t total = 0;
  for (int i = 0; i < nprobs; ++i) {
    const GemmProblem& p = probs[i];
    if (p.M <= 0 || p.N <= 0 || p.K <= 0 || p.N % 64 || p.K % kTK) return hipErrorInvalidValue;
    // the copies' per-lane byte offsets are 32-bit: up to 128 rows of A (a ragged tile's rows are addressed from its
    // first row) and eight k-rows of W must stay below 4 GiB
    if ((int64_t)128 * p.K * 2 > 0xffffffffLL || (int64_t)8 * p.N * 2 > 0xffffffffLL) return hipErrorInvalidValue;
    batch.p[i] = p;
    batch.tiles_n[i] = (p.N + kTN - 1) / kTN;
    batch.tile_start[i] = (int)total;
    total += (int64_t)((p.M + tm - 1) / tm) * batch.tiles_n[i];
    if (total > 0x7fffffff) return hipErrorInvalidValue;
  }
  batch.tile_start[nprobs] = (int)total;
  if (tm == 128)
    hipLaunchKernelGGL((gemm_bf16_mfma<kGemmStages, 128, kGemmWaves>), dim3((unsigned)total), dim3(64 * kGemmWaves), 0,
                       stream, batch);
  else
    hipLaunchKernelGGL((gemm_bf16_mfma<kGemmStages, 64, kGemmWaves>), dim3((unsigned)total), dim3(64 * kGemmWaves), 0,
                       stream, batch);
  return hipGetLastError();
}

}  // namespace mi355
