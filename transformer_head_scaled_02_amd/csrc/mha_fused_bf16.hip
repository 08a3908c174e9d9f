// Multi-head self-attention for short sequences, bf16, head width 64, for gfx950 (MI355X): one workgroup per
// (batch entry, head) computes the head's projections and its attention without leaving the CU.
//
// For batch entry b and head i (no biases, row-vector convention X W):
//   Q_i = X_b W_i^Q,  K_i = X_b W_i^K,  V_i = X_b W_i^V      (W_i = column block i of the packed [d_model, h*64])
//   head_i = softmax(Q_i K_i^T / sqrt(64)) V_i                (optional causal mask, optional key padding)
// and head_i is written to columns 64i .. 64i+63 of Concat(head_1..head_h) [B, n, h*64], which the W^O product then
// reads. Definitions: "Transformer：抛弃循环与卷积的序列建模" (jiashun-ye.github.io), section "Multi-Head Attention";
// "Attention Is All You Need" (lettle.cn translation), sections 3.2.1 (equation Attention(Q,K,V)) and 3.2.2.
//
// Why: at n <= 128 the projection GEMM and the attention kernel are each a few microseconds of fixed cost (launch,
// pipeline fill, one HBM round trip of Q/K/V written and read back). Here the 128 x 192 block [Q_i | K_i | V_i] is
// formed in the workgroup (X rows and the three 64-column weight blocks stream through a four-stage LDS ring by
// global_load_lds_dwordx4, up to three k-tiles in flight behind the one in use; the product is formed transposed,
// C^T = W^T X^T, exactly as in the projection GEMM, so the bf16 Q_i, K_i, V_i are the same numbers), rounded to bf16
// into LDS over the ring's space, and the attention runs on them from there: with
// every key in LDS the softmax is the plain one (row max over all keys, exp2, row sums on the matrix core from the
// same bf16 weights that multiply V), no online rescaling. Eight waves share the projection (wave w forms rows
// 32(w/2) .. +31 against three 32-column blocks of the weights over the whole of d_model, so no partial sums have to
// meet) and the attention (waves w and w + 4 take the same 32 queries against the first and the second 64 keys,
// merged through LDS).
#include "attn_tile.h"
#include "launch.h"

namespace mi355 {
namespace {

constexpr int kFWaves = 8;
constexpr int kFMaxN = 128;                   // sequence length limit (rows of X, queries and keys)
constexpr int kFTK = 64;                      // k-tile of the projections
constexpr int kFSub = 64 * 64;                // one 64 x 64 bf16 sub-tile, rows of 128 bytes (8 KB)
constexpr int kFStageElems = 5 * kFSub;       // a stage: [X rows 0-63 | X rows 64-127 | W^Q_i | W^K_i | W^V_i]
constexpr int kFStages = 4;                  // the whole 160 KB of LDS; Q/K/V reuse it after the last k-tile
constexpr int kFCPW = (16 + 24) / kFWaves;    // one-kilobyte copies per wave per stage (16 of X, 8 per weight)

__global__ __launch_bounds__(64 * kFWaves, 1) void mha_self_fused_bf16(FusedMhaArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[kFStages * kFStageElems];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 5, li = lane & 31;
  // consecutive logical blocks are the heads of one batch entry, so an XCD's heads share X_b in its L2
  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int b = blk / a.H, hh = blk % a.H;
  const int n = a.n, dm = a.dm, N = a.H * kD;
  const uint16_t* X = static_cast<const uint16_t*>(a.X) + (int64_t)b * n * dm;
  const uint16_t* Wm[3] = {static_cast<const uint16_t*>(a.Wq) + kD * hh, static_cast<const uint16_t*>(a.Wk) + kD * hh,
                           static_cast<const uint16_t*>(a.Wv) + kD * hh};

  // Copies of one stage (k-tile t): copy gi = kFCPW*wave + i; gi < 16 brings X rows 8gi .. 8gi+7 (rows past n read
  // row n-1: their results are never used), gi >= 16 brings k-rows 8c .. 8c+7 of weight block (gi-16)/8. Lane l
  // brings the logical 16-byte chunk that belongs at physical chunk l%8 of row l/8 of its eight rows (the XOR swizzle
  // of attn_tile.h, which repeats every 16 rows: two per-lane offsets serve every full copy).
  const uint32_t smem_lds = (uint32_t)(uintptr_t)smem;
  const int lr = lane >> 3;
  uint32_t x_voff[2], w_voff[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const uint32_t chunk = (uint32_t)(((lane & 7) ^ swz(8 * c + lr)) << 4);
    x_voff[c] = (uint32_t)lr * (uint32_t)dm * 2u + chunk;
    w_voff[c] = (uint32_t)lr * (uint32_t)N * 2u + chunk;
  }
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int k0 = t * kFTK;
    const uint32_t stage = smem_lds + (uint32_t)((t % kFStages) * kFStageElems * 2);
#pragma unroll
    for (int i = 0; i < kFCPW; ++i) {
      const int gi = kFCPW * wave + i;  // (uniform)
      if (gi < 16) {
        const uint32_t dst = stage + (uint32_t)(gi >> 3) * kFSub * 2u + (uint32_t)(gi & 7) * 1024u;
        if (8 * gi + 8 <= n) {
          lds_dma16(X + (int64_t)(8 * gi) * dm + k0, x_voff[gi & 1], dst);
        } else {
          int l8 = lr;
          asm volatile("" : "+v"(l8));
          const int row = 8 * gi + l8;
          const uint32_t chunk = (uint32_t)(((lane & 7) ^ swz(row)) << 4);
          lds_dma16(X + k0, (uint32_t)min(row, n - 1) * (uint32_t)dm * 2u + chunk, dst);
        }
      } else {
        const int gw = gi - 16, m = gw >> 3, c = gw & 7;
        const uint32_t dst = stage + (uint32_t)(2 + m) * kFSub * 2u + (uint32_t)c * 1024u;
        lds_dma16(Wm[m] + (int64_t)(k0 + 8 * c) * N, w_voff[c & 1], dst);
      }
    }
  };

  // Projection operands, as in the projection GEMM. Second operand (X^T): row 32rb + li of X, k = 16ks + 8g .. +7
  // (logical chunk 2ks + g). First operand (W^T): two transposed reads give column 32nb + l%32 of a weight block at
  // k-rows 16ks + 8g + (0..3) and 16ks + 8g + 4 + (0..3).
  // Wave w covers 32 rows of X against three 32-column blocks, over every k-step of every k-tile. (Splitting the
  // k-steps between waves w and w + 4, each on 64 rows, reads fewer operands from LDS per product but leaves two
  // partial sums per output to meet in LDS: measured 6 % slower over the whole mha_forward call.)
  const int rb = wave >> 1;          // this wave's 32 rows of X: 32rb .. 32rb + 31
  const int cb0 = 3 * (wave & 1);    // and its three 32-column blocks of [W^Q_i | W^K_i | W^V_i]
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
  // acc[c]: register r = C[row 32rb + li][column 32(cb % 2) + 8(r/4) + 4g + r%4] of block cb = cb0 + c
  f32x16 acc[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) acc[c] = f32x16{};

  const int nk = dm / kFTK;
#pragma unroll
  for (int i = 0; i < kFStages - 1; ++i)
    if (i < nk) issue(i);
  for (int t = 0; t < nk; ++t) {
    // this wave's copies of k-tile t (those of up to two later tiles may stay in flight), then everyone's; everyone
    // is also done with k-tile t - 1, whose stage the copies of t + 3 now refill
    const int ahead = min(kFStages - 2, nk - 1 - t);
    if (ahead >= 2) wait_vmcnt<2 * kFCPW>();
    else if (ahead == 1) wait_vmcnt<kFCPW>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (t + kFStages - 1 < nk) issue(t + kFStages - 1);
    const uint16_t* st = smem + (t % kFStages) * kFStageElems;
    const uint16_t* Xs = st + (rb >> 1) * kFSub + (rb & 1) * 32 * kD;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 ao[3];
      const bf16x8 bo = *reinterpret_cast<const bf16x8*>(Xs + aoff[ks]);
#pragma unroll
      for (int c = 0; c < 3; ++c) {
        const int cb = cb0 + c;
        const uint16_t* Ws = st + (2 + (cb >> 1)) * kFSub + ks * 16 * kD;
        const bf16x4 lo = lds_read_tr16x4(Ws + toff[cb & 1][0]);
        const bf16x4 hi = lds_read_tr16x4(Ws + toff[cb & 1][1]);
        ao[c] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int c = 0; c < 3; ++c) acc[c] = mfma32x32x16(ao[c], bo, acc[c]);
    }
  }
  lds_barrier();  // every wave is done with the ring before its space is reused

  // [Q_i | K_i | V_i] rounded to bf16 at qkv: row r of matrix m at qkv + m*128*64 + r*64, logical chunk c of the row
  // at physical chunk c ^ swz(r) (a lane's four columns are half a chunk). The ring's space is free now: qkv takes
  // 48 KB from its 96 KB mark, and the attention step's merge buffer (4 x 34 x 64 floats) its start.
  float* const red = reinterpret_cast<float*>(smem);
  uint16_t* const qkv = smem + 4 * 6 * 16 * 64 * 2;
  static_assert(4 * 34 * 64 * 2 <= 4 * 6 * 16 * 64 * 2, "the merge buffer ends before qkv");
  static_assert(4 * 6 * 16 * 64 * 2 + 3 * kFMaxN * kD <= kFStages * kFStageElems, "Q/K/V fit in the ring's space");
  {
    const int row = 32 * rb + li;
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      const int cb = cb0 + c, m = cb >> 1;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int chunk = 4 * (cb & 1) + rg;
        uint16_t* dst = qkv + m * kFMaxN * kD + row * kD + ((chunk ^ swz(row)) << 3) + 4 * g;
        *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(acc[c][4 * rg], acc[c][4 * rg + 1]),
                                               pack_bf16x2(acc[c][4 * rg + 2], acc[c][4 * rg + 3])};
      }
    }
  }
  lds_barrier();

  // Attention, transposed as in the attention kernels: S^T = K Q^T with a wave's 32 queries in the lane index (B
  // operand: lane supplies Q[q][32g + 8ks + j]) and keys in the registers. Waves w and w + 4 take queries
  // 32(w%4) .. +31 against keys 0-63 and 64-127 respectively; each forms its part with its own row max, and wave w
  // merges the two parts through LDS.
  const int kh = wave >> 2, r4 = wave & 3;  // key half, query block
  const uint16_t* Qs = qkv;
  const uint16_t* Ks = qkv + kFMaxN * kD;
  const uint16_t* Vs = qkv + 2 * kFMaxN * kD;
  const int q = 32 * r4 + li;
  const int n_real = real_keys(a.kv_len, b, n);  // keys from n_real on are padding: weight 0
  const int nkb = (n_real + 31) / 32;             // 32-key blocks holding a real key (uniform)
  const int kb0 = 2 * kh;                         // this wave's key blocks kb0, kb0 + 1
  bf16x8 qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(Qs + q * kD + (((4 * g + ks) ^ swz(q)) << 3));
  f32x16 s[2];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int kb = kb0 + j;
    s[j] = f32x16{};
    if (kb >= nkb) continue;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 kr = *reinterpret_cast<const bf16x8*>(Ks + (32 * kb + li) * kD + (((4 * g + ks) ^ swz(li)) << 3));
      s[j] = mfma32x32x16(kr, qf[ks], s[j]);
    }
    // register r holds key 32kb + 8(r/4) + 4g + r%4: padding keys and (causal) keys after the query get -inf
    if (a.causal || 32 * kb + 32 > n_real) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
        if (key >= n_real || (a.causal && key > q)) s[j][r] = -INFINITY;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[j][r]);
  }
  mx = max_with_partner32(mx);  // the other half of this query's keys of the block sits in lane li +- 32
  // exp2(s c - max c); a part with no key to see (all -inf) keeps offset 0, so its weights are exactly 0
  const float neg_m = mx == -INFINITY ? 0.f : -mx * kScaleLog2;

  // P in bf16 as the B operands of O^T = V^T P^T: k-step kk holds registers 8(kk%2) .. +7 of key block kb0 + kk/2
  bf16x8 pf[4];
  f32x4 ts = {};
  const bf16x8 lsel = lsum_selector(lane);
  const int nks = 2 * min(max(nkb - kb0, 0), 2);  // this wave's 16-key steps holding a real key
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if (kk >= nks) continue;
    const f32x16& sk = s[kk >> 1];
    const int base = 8 * (kk & 1);
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = pack_bf16x2(fast_exp2(scaled_minus(sk[base + 2 * j], neg_m)),
                         fast_exp2(scaled_minus(sk[base + 2 * j + 1], neg_m)));
    pf[kk] = __builtin_bit_cast(bf16x8, (uint4){w[0], w[1], w[2], w[3]});
    ts = mfma16x16x32(lsel, pf[kk], ts);  // row sums of the same bf16 weights
  }
  // V^T operands: transposed reads of V rows 16ks + 4g + (lane%16)/4 (+8), logical chunk 4mb2 + 2((lane/16)%2) +
  // (lane%4)/2, element 4(lane%2)
  int voff[2][2];
  {
    const int jj = (lane & 15) >> 2;
#pragma unroll
    for (int mb2 = 0; mb2 < 2; ++mb2)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int row = 4 * g + jj + 8 * hi;
        const int lchunk = 4 * mb2 + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        voff[mb2][hi] = row * kD + ((lchunk ^ swz(row)) << 3) + 4 * (lane & 1);
      }
  }
  f32x16 o[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    if (kk >= nks) continue;
    const uint16_t* vt = Vs + (2 * kb0 + kk) * 16 * kD;  // keys 32kb0 + 16kk .. +15
#pragma unroll
    for (int mb2 = 0; mb2 < 2; ++mb2) {
      const bf16x4 lo = lds_read_tr16x4(vt + voff[mb2][0]);
      const bf16x4 hi = lds_read_tr16x4(vt + voff[mb2][1]);
      o[mb2] = mfma32x32x16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pf[kk], o[mb2]);
    }
  }

  // merge: wave w + 4 hands over its part (offset, row sum, O) through LDS (the partial-sum space, free again)
  float* const part = red + r4 * 34 * 64;  // per wave pair: [O^T registers 0..31 | -offset | row sum] x 64 lanes
  if (kh == 1) {
#pragma unroll
    for (int mb2 = 0; mb2 < 2; ++mb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) part[(16 * mb2 + r) * 64 + lane] = o[mb2][r];
    part[32 * 64 + lane] = neg_m;
    part[33 * 64 + lane] = ts[0];
  }
  lds_barrier();
  if (kh == 1) return;
  const float neg_m2 = part[32 * 64 + lane], l2 = part[33 * 64 + lane];
  const float l1 = ts[0];
  // scale each part to the larger of the two offsets; a part without keys (row sum 0) contributes nothing
  const float neg_mm = l1 > 0.f ? (l2 > 0.f ? fminf(neg_m, neg_m2) : neg_m) : neg_m2;
  const float a1 = l1 > 0.f ? fast_exp2(neg_mm - neg_m) : 0.f;
  const float a2 = l2 > 0.f ? fast_exp2(neg_mm - neg_m2) : 0.f;
  const float l = a1 * l1 + a2 * l2;

  // O = O^T / l; lane holds d = 32mb2 + 8(r/4) + 4g + r%4 of query q
  if (q < n) {
    const float inv = l > 0.f ? 1.0f / l : 0.f;  // a row with no real key: output 0
    uint16_t* orow = static_cast<uint16_t*>(a.C) + ((int64_t)b * n + q) * N + kD * hh;
#pragma unroll
    for (int mb2 = 0; mb2 < 2; ++mb2)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (a1 * o[mb2][4 * rg + i] + a2 * part[(16 * mb2 + 4 * rg + i) * 64 + lane]) * inv;
        *reinterpret_cast<uint2*>(orow + 32 * mb2 + 8 * rg + 4 * g) =
            uint2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
  }
}

}  // namespace

hipError_t launch_mha_self_fused_bf16(const FusedMhaArgs& a, hipStream_t stream) {
  if (a.n < 1 || a.n > kFMaxN || a.dm < kFTK || a.dm % kFTK || a.H < 1) return hipErrorInvalidValue;
  // the copies' per-lane byte offsets are 32-bit: the 128 rows of X (a short sequence's rows are addressed from row 0)
  // and eight k-rows of the weights must stay below 4 GiB
  if ((int64_t)kFMaxN * a.dm * 2 > 0xffffffffLL || (int64_t)8 * a.H * kD * 2 > 0xffffffffLL) return hipErrorInvalidValue;
  const int64_t nblocks = (int64_t)a.B * a.H;
  if (nblocks <= 0 || nblocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mha_self_fused_bf16, dim3((unsigned)nblocks), dim3(64 * kFWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mi355
