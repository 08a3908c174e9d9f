// Backward pass of scaled dot-product attention, bf16 in/out, d_k = d_v = D in {32, 64, 128}, for gfx950 (MI355X).
//
// The forward pass is O = P V with P = softmax(Q K^T / sqrt(64)) row by row ("Attention Is All You Need", lettle.cn
// translation, section 3.2.1, equation Attention(Q,K,V)); training carries the loss back through it by the chain
// rule ("Transformer：抛弃循环与卷积的序列建模", jiashun-ye.github.io, section "训练样本", subsection "反向传播").
// Given Q, K, V, the forward output O, the forward's row log-sum-exp lse and the upstream gradient dO:
//   P  = exp(Q K^T / sqrt(D) - lse)      (recomputed tile by tile from the saved lse, never stored)
//   dV = P^T dO,   dP = dO V^T,   dS = P o (dP - Dg) with Dg_i = dO_i . O_i = sum_j P_ij dP_ij,
//   dQ = dS K / sqrt(D),   dK = dS^T Q / sqrt(D).
// Masked weights (causal: key after query) are exactly 0 and pass no gradient. fp32 accumulation throughout; P and
// dS are rounded to bf16 where they enter the matrix core; outputs are rounded to bf16 (nearest even).
//
// Three launches:
//  1. attn_bwd_pre: D = dO . O per query row (fp32) and log2(e) * lse, written to the workspace in 64-row tiles;
//     rows past n_q get lse = +inf and D = 0, so their recomputed weights are exactly 0 wherever they are read.
//     Each row's -D is also stored as three bf16 parts whose sum is -D to float32 precision: one extra k-step of the
//     dP product (those parts against a column of ones) then yields dP - D straight from the matrix core, which
//     saves a VALU subtraction per score in both gradient kernels (widths 32 and 64; at 128, where a wave's
//     registers are already full, the subtraction measured faster and stays on the VALU).
//  2. attn_bwd_dkdv (widths 32 and 128, and the window at every width; width 64 otherwise runs the same arithmetic
//     in attn_bwd_dkdv_pp_bf16, eight waves in ping-pong, described at that kernel):
//     a workgroup of NW waves owns NW*32 keys of one head; each wave keeps the K and V rows of its 32
//     keys in registers as MFMA B operands. 64-row query tiles (Q rows, dO rows and the tile's lse/D, 17 KB) stream
//     through a 3-stage LDS ring by global_load_lds_dwordx4. Per tile and 32-row half, S = Q K^T and dP = dO V^T
//     come out of v_mfma_f32_32x32x16_bf16 with the wave's keys in the lane index and queries in the accumulator
//     registers; P and dS are formed on the VALU and packed to bf16, which is directly the B operand of
//     dV^T += dO^T P and dK^T += Q^T dS, whose A operands are transposed LDS reads (ds_read_b64_tr_b16) of the dO
//     and Q tiles. Four products per tile, no cross-wave reduction, no atomics.
//  3. attn_bwd_dq (widths 32 and 128, and the window at every width; width 64 otherwise runs the same arithmetic in
//     attn_bwd_dq_pp_bf16, eight waves in ping-pong): a workgroup of NW waves owns NW*32 queries; each wave keeps its
//     Q and dO rows in registers as B operands and its rows' lse and D in lanes. K/V tiles stream through the ring;
//     per tile S^T = K Q^T and dP^T = V dO^T (keys in registers, queries in lanes), dS^T on the VALU packed to bf16
//     as the B operand of dQ^T += K^T dS^T, whose A operand is a transposed read of the K tile. Three products per
//     tile.
// Splitting dQ from dK/dV costs one recomputation of S and dP (seven products per score instead of five) but needs
// neither atomics nor a transpose of dS, and every output is written once, deterministically.
// Causal: query tiles wholly before a wave's keys (dK/dV) and key tiles wholly after a wave's queries (dQ) are
// skipped (in the ping-pong kernels, whose eight waves step through the tiles together, such a tile is masked whole
// and adds exactly 0); the tiles that straddle the diagonal set the future scores to -inf before the exponential.
#include <math.h>

#include <type_traits>

#include "attn_tile.h"
#include "launch.h"

namespace mi355 {
namespace {

constexpr int kAuxElems = kAuxFloatsPerTile * 2;            // one tile's lse/D block in 16-bit LDS elements (1 KB)
constexpr float kLog2e = 1.4426950408889634f;

// 1 / sqrt(D), the scale of dQ and dK (exact for D = 64)
template <int D>
constexpr float inv_sqrt_d() {
  static_assert(D == 32 || D == 64 || D == 128, "head width of the backward kernels");
  return D == 64 ? 0.125f : D == 32 ? (float)(1.0 / 5.656854249492381) : (float)(1.0 / 11.313708498984761);
}

// LDS element offset of lane (li, g)'s operand row read in k-step ks: row li of a 32-row block, logical 16-byte
// chunk (D/16)g + ks (the d order every product here uses: k-step ks holds d = 8((D/16)g + ks) .. +7 of lane group g).
template <int D>
__device__ __forceinline__ int row_off(int li, int g, int ks) {
  return li * D + ((((D / 16) * g + ks) ^ swz_d<D>(li)) << 3);
}

// Offsets of the two transposed reads that give the A operand of a product contracting over the 64 rows of an LDS
// tile: for output rows 32mb + (0..31) (tile columns) and k-step ks, lane l needs tile rows 16ks + 4g + (0..3) and
// 16ks + 8 + 4g + (0..3) of column 32mb + l%32, which is the k order of a 32x32 accumulator's registers 8(ks%2) ..
// +7 read as a B operand.
template <int D>
__device__ __forceinline__ int tr_off(int lane, int mb, int hi) {
  const int g = lane >> 5, jj = (lane & 15) >> 2;
  const int row = 4 * g + jj + 8 * hi;
  const int lchunk = 4 * mb + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  return row * D + ((lchunk ^ swz_d<D>(row)) << 3) + 4 * (lane & 1);
}
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* tile, int ks, const int (&off)[D / 32][2], int mb) {
  const bf16x4 lo = lds_read_tr16x4(tile + ks * 16 * D + off[mb][0]);
  const bf16x4 hi = lds_read_tr16x4(tile + ks * 16 * D + off[mb][1]);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ void settle_f(float& v) { asm volatile("" : "+v"(v)); }

// -x as three bf16 parts, packed {hi | mid << 16, lo}: hi = bf16(-x), mid = bf16(-x - hi), lo = bf16(-x - hi - mid)
// (each remainder exact in float32), so hi + mid + lo equals -x to about 2^-24 relative. As an extra k-step of an
// MFMA against a column of ones, they subtract x from every accumulator of the row in float32.
__device__ __forceinline__ uint2 neg_bf16_split3(float x) {
  const float nx = -x;
  const uint32_t h = pack_bf16x2(nx, 0.f) & 0xffffu;
  const float r1 = nx - __uint_as_float(h << 16);
  const uint32_t m = pack_bf16x2(r1, 0.f) & 0xffffu;
  const float r2 = r1 - __uint_as_float(m << 16);
  const uint32_t l = pack_bf16x2(r2, 0.f) & 0xffffu;
  return uint2{h | (m << 16), l};
}

// The matching column of ones: k = 0, 1, 2 of a k-step are 1 in the lanes that supply k = 0..7 (g = 0), all else 0.
__device__ __forceinline__ bf16x8 ones3_operand(int g) {
  const uint32_t one2 = 0x3f803f80u, one1 = 0x00003f80u;  // bf16 1.0 = 0x3f80
  return __builtin_bit_cast(bf16x8, g == 0 ? uint4{one2, one1, 0u, 0u} : uint4{0u, 0u, 0u, 0u});
}

// Copies of one ring stage: 64 rows of D elements of tensor `ta` (the first 128 D bytes of the stage) and of `tb`
// (the next), each wave moving its share of the 2 D/8 one-kilobyte pieces; rows at or past `rows_left` read row
// rows_left-1 instead. Copy gi moves R = 512/D rows from row R (gi mod D/8); lane l brings the logical chunk that
// belongs at physical chunk l mod D/8 of its row (the XOR swizzle of swz_d). D/32 per-lane offsets (one per copy of
// a 16-row swizzle period) serve every copy; the rest of the row offset goes into the scalar base.
template <int NW, int D>
__device__ __forceinline__ void issue_rows(const uint16_t* ta, const uint16_t* tb, int rows_left, uint32_t stage,
                                           int wave, int lrow, const uint32_t (&ld_voff)[D / 32]) {
  constexpr int kCPT = D / 8, kRPC = 512 / D, kNOff = D / 32, kTileElemsD = kBN * D;
  constexpr int kLPW = 2 * kCPT / NW;
  static_assert((2 * kCPT) % NW == 0 && kLPW % kNOff == 0, "copies split evenly over the waves");
  if (rows_left >= kBN) {
#pragma unroll
    for (int i = 0; i < kLPW; ++i) {
      const int gi = wave * kLPW + i;
      const int c = gi & (kCPT - 1);
      lds_dma16((gi < kCPT ? ta : tb) + (c / kNOff) * 16 * D, ld_voff[c & (kNOff - 1)],
                stage + (gi < kCPT ? 0u : kTileElemsD * 2u) + (uint32_t)c * 1024u);
    }
  } else {
    // from the unshifted tile base: lane offset = row min(row, last) with the swizzle of destination row `row` (the
    // 16-row shift is folded back in, so the 32-bit offset stays non-negative)
    const int last = rows_left - 1;
    int lr = lrow;
    asm volatile("" : "+v"(lr));  // computed here, on this rare path, rather than kept live in registers
#pragma unroll
    for (int i = 0; i < kLPW; ++i) {
      const int gi = wave * kLPW + i;
      const int c = gi & (kCPT - 1);
      const int row = kRPC * c + lr;
      lds_dma16(gi < kCPT ? ta : tb,
                ld_voff[c & (kNOff - 1)] + (uint32_t)((min(row, last) - (kRPC * (c & (kNOff - 1)) + lr)) * D * 2),
                stage + (gi < kCPT ? 0u : kTileElemsD * 2u) + (uint32_t)c * 1024u);
    }
  }
}

// Wait until at most `ahead` tiles of this wave's copies (kPer vector-memory operations each) are still in flight.
template <int kPer, int kStages>
__device__ __forceinline__ void wait_copies(int ahead) {
  static_assert(kStages >= 2 && kStages <= 4 && kPer * (kStages - 2) < 64, "ring depth");
  if (kStages >= 4 && ahead >= 2) wait_vmcnt<(kStages >= 4 ? 2 * kPer : 0)>();
  else if (kStages >= 3 && ahead >= 1) wait_vmcnt<(kStages >= 3 ? kPer : 0)>();
  else wait_vmcnt<0>();
}

// D_i = dO_i . O_i and log2(e) * lse_i for one 64-row query tile of one head (rows of D elements); 4 threads per row.
// kO32: bf16 dO with the float32 (unrounded) forward output O. The tile's block of 256 floats holds [log2(e) lse of
// the 64 rows | D of the 64 rows | per row 8 bytes: bf16 {-D_hi, -D_mid, -D_lo, 0}] (neg_bf16_split3).
template <class T, int D, bool kO32 = false>
__global__ __launch_bounds__(256) void attn_bwd_pre(BwdArgs a, int n_tiles) {
  const int bh = blockIdx.x / n_tiles, t = blockIdx.x % n_tiles;
  const int r = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int n_q = a.n_q;
  const int row = t * kBN + r;
  float dot = 0.f;
  if (row < n_q) {
    const int64_t base = ((int64_t)bh * n_q + row) * D + (D / 4) * part;
    if constexpr (sizeof(T) == 2 && kO32) {
      const float4* o = reinterpret_cast<const float4*>(static_cast<const float*>(a.O) + base);
      const uint4* d = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.dO) + base);
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const uint4 dv = d[c];
        const float4 o0 = o[2 * c], o1 = o[2 * c + 1];
        const float of[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
        const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dot = fmaf(of[2 * j], __uint_as_float(dw[j] << 16), dot);
          dot = fmaf(of[2 * j + 1], __uint_as_float(dw[j] & 0xffff0000u), dot);
        }
      }
    } else if constexpr (sizeof(T) == 2) {
      const uint4* o = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.O) + base);
      const uint4* d = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.dO) + base);
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const uint4 ov = o[c], dv = d[c];
        const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w}, dw[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dot = fmaf(__uint_as_float(ow[j] << 16), __uint_as_float(dw[j] << 16), dot);
          dot = fmaf(__uint_as_float(ow[j] & 0xffff0000u), __uint_as_float(dw[j] & 0xffff0000u), dot);
        }
      }
    } else {
      const float4* o = reinterpret_cast<const float4*>(static_cast<const float*>(a.O) + base);
      const float4* d = reinterpret_cast<const float4*>(static_cast<const float*>(a.dO) + base);
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const float4 ov = o[c], dv = d[c];
        dot = fmaf(ov.x, dv.x, dot);
        dot = fmaf(ov.y, dv.y, dot);
        dot = fmaf(ov.z, dv.z, dot);
        dot = fmaf(ov.w, dv.w, dot);
      }
    }
  }
  dot += __shfl_xor(dot, 1);
  dot += __shfl_xor(dot, 2);
  float* at = a.aux + ((int64_t)bh * n_tiles + t) * kAuxFloatsPerTile;
  if (part == 0) {
    // +inf for padding rows and for rows that saw no key (lse = -inf): their weights come out exactly 0
    const float lse = row < n_q ? a.lse[(int64_t)bh * n_q + row] : -INFINITY;
    at[r] = lse == -INFINITY ? INFINITY : lse * kLog2e;
  } else {
    const float dv = row < n_q ? dot : 0.f;
    if (part == 1) {
      at[kBN + r] = dv;
    } else {
      const uint2 w = neg_bf16_split3(dv);
      at[2 * kBN + 2 * r + (part - 2)] = __uint_as_float(part == 2 ? w.x : w.y);
    }
  }
}

// dK and dV: see the file comment (launch 2).
template <int D, int NW, int kStages, bool WIN>
__global__ __launch_bounds__(64 * NW, D == 128 ? 1 : 2) void attn_bwd_dkdv_bf16(BwdArgs a, int n_kblocks) {
  constexpr int kD = D;                           // (shadows the 64 of the shared tile header)
  constexpr int kTileElems = kBN * D;             // one 64-row tile of D elements
  constexpr int kKS = D / 16, kMB = D / 32;       // k-steps over d; 32-wide blocks of d
  constexpr int kCPT = D / 8, kRPC = 512 / D, kNOff = D / 32;  // tile copies: per tensor, rows each, offsets
  constexpr int kBK = 32 * NW;                    // keys per workgroup
  constexpr int kLPW = 2 * kCPT / NW;             // Q/dO copies per wave per tile (wave 0 also copies lse/D)
  constexpr int kStageElems = 2 * kTileElems + kAuxElems;
  static_assert((2 * kCPT) % NW == 0, "tile copies split evenly over the waves");
  __shared__ __attribute__((aligned(16))) uint16_t smem[kStages * kStageElems];  // [stage][Q | dO | lse, D]

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 5, li = lane & 31;
  const int n_q = a.n_q, n_k = a.n_k;
  const bool causal = a.causal != 0;
  const int n_tiles = (n_q + kBN - 1) / kBN;

  int kb, slot;  // causal: key block 0 sees the most query tiles, so it goes first
  if (causal) {
    causal_order(blockIdx.x, gridDim.x, n_kblocks, slot, kb);
  } else {
    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    kb = blk % n_kblocks;
    slot = blk / n_kblocks;
  }
  int bh;
  const int b = head_of_slot(slot, a.B, a.H, bh);
  const int n_real = real_keys(a.kv_len, b, n_k);  // keys from n_real on are padding: gradient 0
  const uint16_t* Qp = static_cast<const uint16_t*>(a.Q) + (int64_t)bh * n_q * kD;
  const uint16_t* dOp = static_cast<const uint16_t*>(a.dO) + (int64_t)bh * n_q * kD;
  const uint16_t* Kp = static_cast<const uint16_t*>(a.K) + (int64_t)bh * n_k * kD;
  const uint16_t* Vp = static_cast<const uint16_t*>(a.V) + (int64_t)bh * n_k * kD;
  const float* auxp = a.aux + (int64_t)bh * n_tiles * kAuxFloatsPerTile;

  const int k_blk0 = kb * kBK;
  const int kw0 = k_blk0 + 32 * wave;  // this wave's keys: kw0 .. kw0+31; lane's key kw0 + li
  const int key = kw0 + li;
  const bool wave_real = kw0 < n_real;  // (uniform) the wave has at least one real key

  // K and V rows as B operands of S = Q K^T and dP = dO V^T: lane supplies row `key`, d = 8(4g + ks) .. +7.
  bf16x8 kf[kKS], vf[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    const int64_t off = (int64_t)key * kD + 8 * ((kD / 16) * g + ks);
    kf[ks] = key < n_real ? *reinterpret_cast<const bf16x8*>(Kp + off) : bf16x8{};
    vf[ks] = key < n_real ? *reinterpret_cast<const bf16x8*>(Vp + off) : bf16x8{};
  }
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    settle(kf[ks]);
    settle(vf[ks]);
  }

  // Query tiles: causal work starts at the tile holding the workgroup's first key. Per wave, tiles before t_first
  // hold only rows before all its keys (all weights 0) and tiles from t_nomask on only rows at or after all of them.
  constexpr bool win = WIN;  // restricted self-attention (a separate instantiation)
  const int wr = a.window;
  int t0 = causal ? k_blk0 / kBN : 0;
  int t_first = causal ? kw0 / kBN : 0;
  const int t_nomask = causal ? (kw0 + 31) / kBN + 1 : 0;
  int t_last = n_tiles - 1;  // this wave's last query tile
  if (win) {  // restricted self-attention: rows key - window .. key + window (.. key when causal)
    if (!causal) {
      t0 = max(0, k_blk0 - wr) / kBN;
      t_first = max(0, kw0 - wr) / kBN;
    }
    t_last = min(t_last, (kw0 + 31 + wr) / kBN);
  }
  // a query row may see this lane's key when lo_off <= key - row <= hi_off
  const int hi_off = causal ? 0 : (win ? wr : (1 << 30));
  const int lo_off = win ? -wr : -(1 << 30);

  const uint32_t smem_lds = (uint32_t)(uintptr_t)smem;
  const int lrow = lane / kCPT;
  uint32_t ld_voff[kNOff];
#pragma unroll
  for (int c = 0; c < kNOff; ++c) {
    const int row = kRPC * c + lrow;
    ld_voff[c] = (uint32_t)(row * kD + (((lane % kCPT) ^ swz_d<D>(row)) << 3)) * 2u;
  }
  auto issue = [&](int t) __attribute__((always_inline)) {
    const uint32_t stage = smem_lds + (uint32_t)(((t - t0) % kStages) * kStageElems * 2);
    issue_rows<NW, D>(Qp + (int64_t)t * kBN * kD, dOp + (int64_t)t * kBN * kD, n_q - t * kBN, stage, wave, lrow,
                   ld_voff);
    if (wave == 0) lds_dma16(auxp + (int64_t)t * kAuxFloatsPerTile, (uint32_t)lane * 16u, stage + kTileElems * 4u);
  };

  int roff[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) roff[ks] = row_off<D>(li, g, ks);
  int toff[kMB][2];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) toff[mb][hi] = tr_off<D>(lane, mb, hi);

  f32x16 dv[kMB], dk[kMB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) dv[mb] = dk[mb] = f32x16{};
  constexpr bool kFoldD = D != 128;  // D subtracted by an extra k-step of dP (see the file comment)
  const bf16x8 ones3 = ones3_operand(g);  // B operand of the k-step that subtracts each query row's D from dP

  // a workgroup of padding keys only writes zeros
  int nt = k_blk0 < n_real ? n_tiles : 0;
  if (win) nt = min(nt, (k_blk0 + kBK - 1 + wr) / kBN + 1);
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i)
    if (t0 + i < nt) issue(t0 + i);
  for (int t = t0; t < nt; ++t) {
    // wait for this wave's copies of tile t (the later tiles' may stay in flight), then for every wave's
    const int ahead = min(kStages - 2, nt - 1 - t);
    if (wave == 0) wait_copies<kLPW + 1, kStages>(ahead);
    else wait_copies<kLPW, kStages>(ahead);
    lds_barrier();  // also: every wave is done with tile t-1, whose stage tile t + kStages - 1 now takes
    if (t + kStages - 1 < nt) issue(t + kStages - 1);
    if (t < t_first || t > t_last || !wave_real) continue;
    const bool masked = win || t < t_nomask;
    const uint16_t* st = smem + ((t - t0) % kStages) * kStageElems;
    const float* aux = reinterpret_cast<const float*>(st + 2 * kTileElems);

    bf16x8 pp[4], ps[4];  // P and dS in bf16, B operands for k-steps (16 query rows) 0..3 of the tile
#pragma unroll
    for (int mq = 0; mq < 2; ++mq) {
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
        s = mfma32x32x16(*reinterpret_cast<const bf16x8*>(st + mq * 32 * kD + roff[ks]), kf[ks], s);
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
        dp = mfma32x32x16(*reinterpret_cast<const bf16x8*>(st + kTileElems + mq * 32 * kD + roff[ks]), vf[ks], dp);
      if constexpr (kFoldD) {
        // dP - D: A operand row li = query 32mq + li with k = 0..2 the parts of its -D (the lanes of g = 1 supply
        // k = 8..15, which meet zeros in ones3)
        const uint2 nd = *reinterpret_cast<const uint2*>(aux + 2 * kBN + 2 * (32 * mq + li));
        dp = mfma32x32x16(__builtin_bit_cast(bf16x8, uint4{nd.x, nd.y, 0u, 0u}), ones3, dp);
      }
      // register r holds query row 32mq + 8(r/4) + 4g + r%4 of the tile: its lse (and D) come in fours
      f32x4 lq[4], dq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lq[i] = *reinterpret_cast<const f32x4*>(aux + 32 * mq + 8 * i + 4 * g);
        if constexpr (!kFoldD) dq[i] = *reinterpret_cast<const f32x4*>(aux + kBN + 32 * mq + 8 * i + 4 * g);
      }
      if (masked) {  // uniform: tiles that straddle the wave's keys, and every tile of the window
        const int base = key - t * kBN - 32 * mq - 4 * g;
        const int ub = base - hi_off, lb = base - lo_off;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          // key - row = base - (8(r/4) + r%4); allowed when lo_off <= key - row <= hi_off
          if (8 * (r >> 2) + (r & 3) < ub || (WIN && 8 * (r >> 2) + (r & 3) > lb)) s[r] = -INFINITY;
      }
      float p[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(__builtin_fmaf(s[r], scale_log2<D>(), -lq[r >> 2][r & 3]));
        ds[r] = kFoldD ? p[r] * dp[r] : p[r] * (dp[r] - dq[r >> 2][r & 3]);  // folded: dp holds dP - D
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        uint32_t wp[4], wd[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          wp[j] = pack_bf16x2(p[8 * hf + 2 * j], p[8 * hf + 2 * j + 1]);
          wd[j] = pack_bf16x2(ds[8 * hf + 2 * j], ds[8 * hf + 2 * j + 1]);
        }
        pp[2 * mq + hf] = __builtin_bit_cast(bf16x8, (uint4){wp[0], wp[1], wp[2], wp[3]});
        ps[2 * mq + hf] = __builtin_bit_cast(bf16x8, (uint4){wd[0], wd[1], wd[2], wd[3]});
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS, contracting over the tile's 64 query rows
#pragma unroll
    for (int kq = 0; kq < 4; ++kq)
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        dv[mb] = mfma32x32x16(tr_operand<D>(st + kTileElems, kq, toff, mb), pp[kq], dv[mb]);
        dk[mb] = mfma32x32x16(tr_operand<D>(st, kq, toff, mb), ps[kq], dk[mb]);
      }
  }

  // lane holds d = 32mb + 8(r/4) + 4g + r%4 of its key's dV and dK rows; padding keys get 0
  if (key >= n_real) {
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) dv[mb] = dk[mb] = f32x16{};
  }
  if (key < n_k) {
    uint16_t* dvrow = static_cast<uint16_t*>(a.dV) + ((int64_t)bh * n_k + key) * kD;
    uint16_t* dkrow = static_cast<uint16_t*>(a.dK) + ((int64_t)bh * n_k + key) * kD;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d = 32 * mb + 8 * rg + 4 * g;
        const uint2 wv = {pack_bf16x2(dv[mb][4 * rg], dv[mb][4 * rg + 1]),
                          pack_bf16x2(dv[mb][4 * rg + 2], dv[mb][4 * rg + 3])};
        const uint2 wk = {pack_bf16x2(dk[mb][4 * rg] * inv_sqrt_d<D>(), dk[mb][4 * rg + 1] * inv_sqrt_d<D>()),
                          pack_bf16x2(dk[mb][4 * rg + 2] * inv_sqrt_d<D>(), dk[mb][4 * rg + 3] * inv_sqrt_d<D>())};
        *reinterpret_cast<uint2*>(dvrow + d) = wv;
        *reinterpret_cast<uint2*>(dkrow + d) = wk;
      }
  }
}

// dK and dV at width 64 with the eight waves of a workgroup in ping-pong, as in the forward's attn_fwd_pp_bf16:
// waves w and w + 4 share a SIMD, and the two groups of four are held half a query tile apart by the barrier that
// ends every slot, so that in every slot one wave of each SIMD feeds the matrix core while the other runs the
// exponentials and the dS products on the VALU. Per query tile u a wave's work splits into
//   M(u):  dV^T += dO^T P(u-1), dK^T += Q^T dS(u-1) (transposed reads of tile u-1), then S(u) = Q K^T and
//          dP(u) - D = dO V^T (- D by the extra k-step) from row reads of tile u: 34 products;
//   V(u):  P(u) = exp2(S c - log2(e) lse), dS(u) = P o (dP - D), both packed to bf16.
// Slot schedule:   slot  0     1     2     3    ...  2n-1    2n
//                  g0:   M(0)  V(0)  M(1)  V(1) ...  V(n-1)  M(n)
//                  g1:   -     M(0)  V(0)  M(1) ...  M(n-1)  V(n-1) M(n)
// Tile u is read in slots 2u .. 2u+3; the group in its V slot (whose vector-memory issue is otherwise idle) copies
// the tiles: tile u + 3 in group 1's V(u) (slot 2u + 2), into the stage of tile u - 1, last read in slot 2u + 1.
// Each wave owns 32 keys (the workgroup 256); the arithmetic per key is exactly that of attn_bwd_dkdv_bf16.
// Unlike the forward, the matrix-core slot sets the pace here (the VALU slot ends well before its barrier), so the
// matrix-core wave holds the higher issue priority.
constexpr int kPPBwdStages = 4;

__global__ __launch_bounds__(512, 1) void attn_bwd_dkdv_pp_bf16(BwdArgs a, int n_kblocks) {
  constexpr int D = 64;
  constexpr int kStageElems = 2 * kTileElems + kAuxElems;  // [Q | dO | lse, D]
  constexpr int kBK = 32 * 8;                              // keys per workgroup
  constexpr int kLPW = 4;                                  // Q/dO copies per copying wave per tile
  __shared__ __attribute__((aligned(16))) uint16_t smem[kPPBwdStages * kStageElems];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, gw = wave & 3;
  const int lane = tid & 63;
  const int g = lane >> 5, li = lane & 31;
  const int n_q = a.n_q, n_k = a.n_k;
  const bool causal = a.causal != 0;
  const int n_tiles = (n_q + kBN - 1) / kBN;

  int kb, slot;  // causal: key block 0 sees the most query tiles, so it goes first
  if (causal) {
    causal_order(blockIdx.x, gridDim.x, n_kblocks, slot, kb);
  } else {
    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    kb = blk % n_kblocks;
    slot = blk / n_kblocks;
  }
  int bh;
  const int b = head_of_slot(slot, a.B, a.H, bh);
  const int n_real = real_keys(a.kv_len, b, n_k);  // keys from n_real on are padding: gradient 0
  const uint16_t* Qp = static_cast<const uint16_t*>(a.Q) + (int64_t)bh * n_q * D;
  const uint16_t* dOp = static_cast<const uint16_t*>(a.dO) + (int64_t)bh * n_q * D;
  const uint16_t* Kp = static_cast<const uint16_t*>(a.K) + (int64_t)bh * n_k * D;
  const uint16_t* Vp = static_cast<const uint16_t*>(a.V) + (int64_t)bh * n_k * D;
  const float* auxp = a.aux + (int64_t)bh * n_tiles * kAuxFloatsPerTile;

  const int k_blk0 = kb * kBK;
  const int kw0 = k_blk0 + 32 * wave;  // this wave's keys: kw0 .. kw0+31; lane's key kw0 + li
  const int key = kw0 + li;

  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int64_t off = (int64_t)key * D + 8 * (4 * g + ks);
    kf[ks] = key < n_real ? *reinterpret_cast<const bf16x8*>(Kp + off) : bf16x8{};
    vf[ks] = key < n_real ? *reinterpret_cast<const bf16x8*>(Vp + off) : bf16x8{};
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    settle(kf[ks]);
    settle(vf[ks]);
  }

  // Query tiles t0 .. nt-1 (local index u = t - t0). Causal: the workgroup starts at the tile holding its first key,
  // and tiles from t_nomask on need no mask for this wave.
  const int t0 = causal ? k_blk0 / kBN : 0;
  const int t_nomask = causal ? (kw0 + 31) / kBN + 1 : 0;
  const int nt = k_blk0 < n_real ? n_tiles : 0;  // a workgroup of padding keys only writes zeros
  const int nu = nt - t0;

  const uint32_t smem_lds = (uint32_t)(uintptr_t)smem;
  const int lrow = lane / 8;
  uint32_t ld_voff[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int row = 8 * c + lrow;
    ld_voff[c] = (uint32_t)(row * D + (((lane % 8) ^ swz_d<D>(row)) << 3)) * 2u;
  }
  // group 1 copies: wave 4 + gw moves Q/dO pieces 4gw .. 4gw+3 of the tile, and wave 4 also the tile's lse/D block
  auto issue = [&](int u) __attribute__((always_inline)) {
    const int t = t0 + u;
    const uint32_t stage = smem_lds + (uint32_t)((u % kPPBwdStages) * kStageElems * 2);
    issue_rows<4, D>(Qp + (int64_t)t * kBN * D, dOp + (int64_t)t * kBN * D, n_q - t * kBN, stage, gw, lrow, ld_voff);
    if (gw == 0) lds_dma16(auxp + (int64_t)t * kAuxFloatsPerTile, (uint32_t)lane * 16u, stage + kTileElems * 4u);
  };

  int roff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) roff[ks] = row_off<D>(li, g, ks);
  int toff[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) toff[mb][hi] = tr_off<D>(lane, mb, hi);
  const bf16x8 ones3 = ones3_operand(g);

  f32x16 dv[2], dk[2];
  bf16x8 pp[4], ps[4];  // P and dS in bf16, B operands for k-steps (16 query rows) 0..3 of the tile
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) dv[mb] = dk[mb] = f32x16{};

  // M(u): the gradient products of tile u - 1, then S and dP - D of tile u (either part may be absent). The operand
  // reads run ahead of the products: the update's transposed reads two k-steps ahead (double-buffered), and every
  // S / dP operand of tile u issued while the update's last products run; the four S / dP accumulators are
  // interleaved, so that no product waits for the one before it. A fence after each operand keeps the reads in the
  // order the products use them (the compiler would group them by base register).
  auto mslot = [&](int u, auto upd_c, auto sdp_c, f32x16(&s)[2], f32x16(&dp)[2]) __attribute__((always_inline)) {
    constexpr bool upd = decltype(upd_c)::value, sdp = decltype(sdp_c)::value;
    __builtin_amdgcn_s_setprio(3);
    const uint16_t* stc = smem + (u % kPPBwdStages) * kStageElems;
    const float* auxc = reinterpret_cast<const float*>(stc + 2 * kTileElems);
    bf16x8 qr[2][2], dr[2][2];  // [k-step % 2][mq]: S / dP operands, two k-steps ahead of their products
    uint2 nd[2];
    auto read_ks = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
      for (int mq = 0; mq < 2; ++mq) {
        qr[ks & 1][mq] = *reinterpret_cast<const bf16x8*>(stc + mq * 32 * D + roff[ks]);
        __builtin_amdgcn_sched_barrier(0);
        dr[ks & 1][mq] = *reinterpret_cast<const bf16x8*>(stc + kTileElems + mq * 32 * D + roff[ks]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto read_sdp = [&]() __attribute__((always_inline)) {
      read_ks(0);
      read_ks(1);
#pragma unroll
      for (int mq = 0; mq < 2; ++mq) nd[mq] = *reinterpret_cast<const uint2*>(auxc + 2 * kBN + 2 * (32 * mq + li));
    };
    if constexpr (upd) {
      const uint16_t* st = smem + ((u - 1) % kPPBwdStages) * kStageElems;
      bf16x8 ot[2][2], qt[2][2];
#pragma unroll
      for (int kq = 0; kq < 2; ++kq)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          ot[kq][mb] = tr_operand<D>(st + kTileElems, kq, toff, mb);
          __builtin_amdgcn_sched_barrier(0);
          qt[kq][mb] = tr_operand<D>(st, kq, toff, mb);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          dv[mb] = mfma32x32x16(ot[kq & 1][mb], pp[kq], dv[mb]);
          dk[mb] = mfma32x32x16(qt[kq & 1][mb], ps[kq], dk[mb]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (kq + 2 < 4) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            ot[kq & 1][mb] = tr_operand<D>(st + kTileElems, kq + 2, toff, mb);
            __builtin_amdgcn_sched_barrier(0);
            qt[kq & 1][mb] = tr_operand<D>(st, kq + 2, toff, mb);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // the first S / dP operands go into the registers the update's k-steps 0 and 1 have released
        if constexpr (sdp) {
          if (kq == 2) read_ks(0);
          if (kq == 3) {
            read_ks(1);
#pragma unroll
            for (int mq = 0; mq < 2; ++mq)
              nd[mq] = *reinterpret_cast<const uint2*>(auxc + 2 * kBN + 2 * (32 * mq + li));
          }
        }
      }
    } else if constexpr (sdp) {
      read_sdp();
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (sdp) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mq = 0; mq < 2; ++mq) {
          s[mq] = mfma32x32x16(qr[ks & 1][mq], kf[ks], ks == 0 ? f32x16{} : s[mq]);
          dp[mq] = mfma32x32x16(dr[ks & 1][mq], vf[ks], ks == 0 ? f32x16{} : dp[mq]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (ks + 2 < 4) read_ks(ks + 2);
      }
#pragma unroll
      for (int mq = 0; mq < 2; ++mq)
        dp[mq] = mfma32x32x16(__builtin_bit_cast(bf16x8, uint4{nd[mq].x, nd[mq].y, 0u, 0u}), ones3, dp[mq]);
    }
  };

  // V(u): P and dS of tile u in bf16
  auto vslot = [&](int u, f32x16(&s)[2], const f32x16(&dp)[2]) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(0);
    const int t = t0 + u;
    const uint16_t* st = smem + (u % kPPBwdStages) * kStageElems;
    const float* aux = reinterpret_cast<const float*>(st + 2 * kTileElems);
    const bool masked = t < t_nomask;  // (uniform) causal tiles that straddle the wave's keys
#pragma unroll
    for (int mq = 0; mq < 2; ++mq) {
      // register r holds query row 32mq + 8(r/4) + 4g + r%4 of the tile: its log2(e) lse come in fours
      f32x4 lq[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) lq[i] = *reinterpret_cast<const f32x4*>(aux + 32 * mq + 8 * i + 4 * g);
      if (masked) {
        const int base = key - t * kBN - 32 * mq - 4 * g;  // key - row = base - (8(r/4) + r%4); allowed when <= 0
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + (r & 3) < base) s[mq][r] = -INFINITY;
      }
      float p[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(__builtin_fmaf(s[mq][r], scale_log2<D>(), -lq[r >> 2][r & 3]));
        ds[r] = p[r] * dp[mq][r];
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        uint32_t wp[4], wd[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          wp[j] = pack_bf16x2(p[8 * hf + 2 * j], p[8 * hf + 2 * j + 1]);
          wd[j] = pack_bf16x2(ds[8 * hf + 2 * j], ds[8 * hf + 2 * j + 1]);
        }
        pp[2 * mq + hf] = __builtin_bit_cast(bf16x8, (uint4){wp[0], wp[1], wp[2], wp[3]});
        ps[2 * mq + hf] = __builtin_bit_cast(bf16x8, (uint4){wd[0], wd[1], wd[2], wd[3]});
      }
    }
    // P and dS are only used by the next M slot: without this the compiler sinks their arithmetic past the slot's
    // barrier into that slot, and the two waves of a SIMD would take turns again instead of overlapping
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      settle(pp[k]);
      settle(ps[k]);
    }
  };

  if (nu > 0) {  // (uniform over the workgroup)
    // prologue: group 1 brings tiles 0..2 and waits for tile 0
    if (grp == 1) {
#pragma unroll
      for (int u = 0; u < 3; ++u)
        if (u < nu) issue(u);
      if (gw == 0) wait_copies<kLPW + 1, 4>(min(2, nu - 1));
      else wait_copies<kLPW, 4>(min(2, nu - 1));
    }
    lds_barrier();
    // Group 1 enters one slot later (an extra barrier first) and group 0 leaves with an extra barrier, so every wave
    // passes the same number of barriers. Before the barrier that ends its M slot 2u + 1, group 1 waits until its
    // copies of tile u + 1 have landed (tile u + 2 may stay in flight).
    auto after_m = [&](int u) __attribute__((always_inline)) {
      if (grp == 1) {
        const int ahead = min(1, nu - 2 - u);  // tiles after u + 1 still in flight: u + 2 if it exists
        if (ahead >= 0) {
          if (gw == 0) {
            if (ahead >= 1) wait_vmcnt<kLPW + 1>();
            else wait_vmcnt<0>();
          } else {
            if (ahead >= 1) wait_vmcnt<kLPW>();
            else wait_vmcnt<0>();
          }
        }
      }
      lds_barrier();
    };
    auto after_v = [&](int u) __attribute__((always_inline)) {
      if (grp == 1 && u + 3 < nu) issue(u + 3);
      lds_barrier();
    };
    if (grp == 1) lds_barrier();  // slot 0 of group 1: nothing
    const std::true_type yes;
    const std::false_type no;
    // Every wave runs every tile of the loop through one code path (a single copy of the slots keeps the register
    // allocation inside 256): a causal tile wholly before a wave's keys has all its weights masked to exactly 0 and
    // adds exactly 0 to dV and dK. S and dP live from a tile's M slot to its V slot only.
    {
      f32x16 s[2], dp[2];
      mslot(0, no, yes, s, dp);
      after_m(0);
      vslot(0, s, dp);
      after_v(0);
    }
    for (int u = 1; u < nu; ++u) {
      f32x16 s[2], dp[2];
      mslot(u, yes, yes, s, dp);
      after_m(u);
      vslot(u, s, dp);
      after_v(u);
    }
    {
      f32x16 s[2], dp[2];
      mslot(nu, yes, no, s, dp);
    }
    lds_barrier();
    if (grp == 0) lds_barrier();  // slot 2nu + 1 of group 0: nothing
  }

  // lane holds d = 32mb + 8(r/4) + 4g + r%4 of its key's dV and dK rows; padding keys get 0
  if (key >= n_real) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) dv[mb] = dk[mb] = f32x16{};
  }
  if (key < n_k) {
    uint16_t* dvrow = static_cast<uint16_t*>(a.dV) + ((int64_t)bh * n_k + key) * D;
    uint16_t* dkrow = static_cast<uint16_t*>(a.dK) + ((int64_t)bh * n_k + key) * D;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d = 32 * mb + 8 * rg + 4 * g;
        const uint2 wv = {pack_bf16x2(dv[mb][4 * rg], dv[mb][4 * rg + 1]),
                          pack_bf16x2(dv[mb][4 * rg + 2], dv[mb][4 * rg + 3])};
        const uint2 wk = {pack_bf16x2(dk[mb][4 * rg] * inv_sqrt_d<D>(), dk[mb][4 * rg + 1] * inv_sqrt_d<D>()),
                          pack_bf16x2(dk[mb][4 * rg + 2] * inv_sqrt_d<D>(), dk[mb][4 * rg + 3] * inv_sqrt_d<D>())};
        *reinterpret_cast<uint2*>(dvrow + d) = wv;
        *reinterpret_cast<uint2*>(dkrow + d) = wk;
      }
  }
}

// dQ: see the file comment (launch 3).
template <int D, int NW, int kStages, bool WIN>
__global__ __launch_bounds__(64 * NW, D == 128 ? 1 : 2) void attn_bwd_dq_bf16(BwdArgs a, int n_qblocks) {
  constexpr int kD = D;                           // (shadows the 64 of the shared tile header)
  constexpr int kTileElems = kBN * D;             // one 64-row tile of D elements
  constexpr int kKS = D / 16, kMB = D / 32;       // k-steps over d; 32-wide blocks of d
  constexpr int kCPT = D / 8, kRPC = 512 / D, kNOff = D / 32;  // tile copies: per tensor, rows each, offsets
  constexpr int kBM = 32 * NW;  // queries per workgroup
  static_assert((2 * kCPT) % NW == 0, "tile copies split evenly over the waves");
  __shared__ __attribute__((aligned(16))) uint16_t smem[kStages * 2 * kTileElems];  // [stage][K | V]

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 5, li = lane & 31;
  const bool causal = a.causal != 0;
  const int n_q = a.n_q;
  const int n_tiles_q = (n_q + kBN - 1) / kBN;

  int qb, slot;
  if (causal) {
    causal_order(blockIdx.x, gridDim.x, n_qblocks, slot, qb);
    qb = n_qblocks - 1 - qb;  // heaviest query blocks first
  } else {
    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    qb = blk % n_qblocks;
    slot = blk / n_qblocks;
  }
  int bh;
  const int b = head_of_slot(slot, a.B, a.H, bh);
  const int n_k = real_keys(a.kv_len, b, a.n_k);  // keys from n_k on (padding) are never read
  const uint16_t* Qp = static_cast<const uint16_t*>(a.Q) + (int64_t)bh * n_q * kD;
  const uint16_t* dOp = static_cast<const uint16_t*>(a.dO) + (int64_t)bh * n_q * kD;
  const uint16_t* Kp = static_cast<const uint16_t*>(a.K) + (int64_t)bh * a.n_k * kD;
  const uint16_t* Vp = static_cast<const uint16_t*>(a.V) + (int64_t)bh * a.n_k * kD;
  const float* auxp = a.aux + (int64_t)bh * n_tiles_q * kAuxFloatsPerTile;

  const int q_blk0 = qb * kBM;
  const int qw0 = q_blk0 + 32 * wave;
  const int q = qw0 + li;

  // Q and dO rows as B operands of S^T = K Q^T and dP^T = V dO^T (d = 8(4g + ks) .. +7); zero past n_q
  bf16x8 qf[kKS], df[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    const int64_t off = (int64_t)q * kD + 8 * ((kD / 16) * g + ks);
    qf[ks] = q < n_q ? *reinterpret_cast<const bf16x8*>(Qp + off) : bf16x8{};
    df[ks] = q < n_q ? *reinterpret_cast<const bf16x8*>(dOp + off) : bf16x8{};
  }
  constexpr bool kFoldD = D != 128;  // D subtracted by an extra k-step of dP^T (see the file comment)
  float lse2 = INFINITY, dq_d = 0.f;  // rows past n_q: weights 0
  uint2 nd = {0u, 0u};                 // the query's -D as three bf16 parts (0 past n_q)
  if (q < n_q) {
    const float* at = auxp + (int64_t)(q / kBN) * kAuxFloatsPerTile;
    lse2 = at[q % kBN];
    if constexpr (kFoldD) nd = *reinterpret_cast<const uint2*>(at + 2 * kBN + 2 * (q % kBN));
    else dq_d = at[kBN + q % kBN];
  }
  // the extra k-step of dP^T = V dO^T that subtracts D: A = a column of ones (keys x k), B = the query's -D parts
  const bf16x8 ones3 = ones3_operand(g);
  const bf16x8 ndop = __builtin_bit_cast(bf16x8, uint4{nd.x, nd.y, 0u, 0u});
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    settle(qf[ks]);
    settle(df[ks]);
  }
  settle_f(lse2);
  if constexpr (!kFoldD) settle_f(dq_d);

  int nt = (n_k + kBN - 1) / kBN;
  if (causal) nt = min(nt, (q_blk0 + kBM - 1) / kBN + 1);
  // tiles before t_mask need no mask for any query of this wave; tiles from t_skip on lie entirely in its future
  int t_mask = min(causal ? qw0 / kBN : nt, n_k / kBN);
  int t_skip = causal ? min(nt, (qw0 + 31) / kBN + 1) : nt;
  int key_lim = (causal ? min(q, n_k - 1) : n_k - 1) - 4 * g;  // keys past it (from the lane's first) masked
  // restricted self-attention: key tiles from the workgroup's first band start on; keys before key_lo also masked
  constexpr bool win = WIN;  // restricted self-attention (a separate instantiation)
  int t_begin = 0, t_first = 0, key_lo = -(1 << 30);
  if (win) {
    const int wr = a.window;
    t_begin = max(0, q_blk0 - wr) / kBN;
    t_first = max(0, qw0 - wr) / kBN;
    nt = min(nt, (q_blk0 + kBM - 1 + wr) / kBN + 1);
    t_skip = min(t_skip, (qw0 + 31 + wr) / kBN + 1);
    t_mask = 0;
    key_lim = min(key_lim, q + wr - 4 * g);
    key_lo = q - wr - 4 * g;
  }

  const uint32_t smem_lds = (uint32_t)(uintptr_t)smem;
  const int lrow = lane / kCPT;
  uint32_t ld_voff[kNOff];
#pragma unroll
  for (int c = 0; c < kNOff; ++c) {
    const int row = kRPC * c + lrow;
    ld_voff[c] = (uint32_t)(row * kD + (((lane % kCPT) ^ swz_d<D>(row)) << 3)) * 2u;
  }
  auto issue = [&](int t) __attribute__((always_inline)) {
    const uint32_t stage = smem_lds + (uint32_t)((t % kStages) * 2 * kTileElems * 2);
    issue_rows<NW, D>(Kp + (int64_t)t * kBN * kD, Vp + (int64_t)t * kBN * kD, n_k - t * kBN, stage, wave, lrow, ld_voff);
  };

  int roff[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) roff[ks] = row_off<D>(li, g, ks);
  int toff[kMB][2];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) toff[mb][hi] = tr_off<D>(lane, mb, hi);

  f32x16 dq[kMB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) dq[mb] = f32x16{};

  constexpr int kLPW = 2 * kCPT / NW;
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i)
    if (t_begin + i < nt) issue(t_begin + i);
  for (int t = t_begin; t < nt; ++t) {
    wait_copies<kLPW, kStages>(min(kStages - 2, nt - 1 - t));
    lds_barrier();
    if (t + kStages - 1 < nt) issue(t + kStages - 1);
    if (t >= t_skip || (WIN && t < t_first)) continue;
    const bool masked = t >= t_mask;
    const uint16_t* st = smem + (t % kStages) * 2 * kTileElems;

    // S^T and dP^T: register r of block kb holds key 32kb + 8(r/4) + 4g + r%4 of the tile, query = lane's
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = dp[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
        s[kb] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(st + kb * 32 * kD + roff[ks]), qf[ks], s[kb]);
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
        dp[kb] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(st + kTileElems + kb * 32 * kD + roff[ks]), df[ks],
                              dp[kb]);
      if constexpr (kFoldD) dp[kb] = mfma32x32x16(ones3, ndop, dp[kb]);  // dP^T - D
    }
    if (masked) {
      const int lim = key_lim - t * kBN, lo = key_lo - t * kBN;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + 8 * (r >> 2) + (r & 3) > lim || (WIN && 32 * kb + 8 * (r >> 2) + (r & 3) < lo))
            s[kb][r] = -INFINITY;
    }
    // dS^T in bf16, B operand of k-step ks: registers 8(ks%2) .. +7 of key block ks/2
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kb = ks >> 1, base = 8 * (ks & 1);
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = fast_exp2(__builtin_fmaf(s[kb][base + 2 * j], scale_log2<D>(), -lse2));
        const float p1 = fast_exp2(__builtin_fmaf(s[kb][base + 2 * j + 1], scale_log2<D>(), -lse2));
        w[j] = kFoldD ? pack_bf16x2(p0 * dp[kb][base + 2 * j], p1 * dp[kb][base + 2 * j + 1])
                      : pack_bf16x2(p0 * (dp[kb][base + 2 * j] - dq_d), p1 * (dp[kb][base + 2 * j + 1] - dq_d));
      }
      const bf16x8 pds = __builtin_bit_cast(bf16x8, (uint4){w[0], w[1], w[2], w[3]});
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) dq[mb] = mfma32x32x16(tr_operand<D>(st, ks, toff, mb), pds, dq[mb]);
    }
  }

  // dQ = dQ^T / sqrt(D); lane holds d = 32mb + 8(r/4) + 4g + r%4 of its query
  if (q < n_q) {
    uint16_t* row = static_cast<uint16_t*>(a.dQ) + ((int64_t)bh * n_q + q) * kD;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const uint2 w = {pack_bf16x2(dq[mb][4 * rg] * inv_sqrt_d<D>(), dq[mb][4 * rg + 1] * inv_sqrt_d<D>()),
                         pack_bf16x2(dq[mb][4 * rg + 2] * inv_sqrt_d<D>(), dq[mb][4 * rg + 3] * inv_sqrt_d<D>())};
        *reinterpret_cast<uint2*>(row + 32 * mb + 8 * rg + 4 * g) = w;
      }
  }
}

// dQ at width 64 with the eight waves of a workgroup in ping-pong, as attn_bwd_dkdv_pp_bf16: waves w and w + 4 share
// a SIMD and run half a key tile apart, so that in every slot one wave of each SIMD feeds the matrix core while the
// other forms dS on the VALU. Per key tile u a wave's work splits into
//   M(u):  dQ^T += K^T dS^T(u-1) (transposed reads of tile u-1), then S^T(u) = K Q^T and dP^T(u) - D = V dO^T (- D by
//          the extra k-step) from row reads of tile u: 26 products;
//   V(u):  P = exp2(S^T c - log2(e) lse) (masked where the tile needs it), dS^T = P o (dP^T - D), packed to bf16.
// Slot schedule and copies as in attn_bwd_dkdv_pp_bf16, with K/V tiles (16 KB) in a four-stage ring. Each wave owns
// 32 queries (the workgroup 256); the arithmetic per query is exactly that of attn_bwd_dq_bf16.
__global__ __launch_bounds__(512, 1) void attn_bwd_dq_pp_bf16(BwdArgs a, int n_qblocks) {
  constexpr int D = 64;
  constexpr int kStageElems = 2 * kTileElems;  // [K | V]
  constexpr int kBM = 32 * 8;                  // queries per workgroup
  constexpr int kLPW = 4;                      // K/V copies per copying wave per tile
  __shared__ __attribute__((aligned(16))) uint16_t smem[kPPBwdStages * kStageElems];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, gw = wave & 3;
  const int lane = tid & 63;
  const int g = lane >> 5, li = lane & 31;
  const bool causal = a.causal != 0;
  const int n_q = a.n_q;
  const int n_tiles_q = (n_q + kBN - 1) / kBN;

  int qb, slot;
  if (causal) {
    causal_order(blockIdx.x, gridDim.x, n_qblocks, slot, qb);
    qb = n_qblocks - 1 - qb;  // heaviest query blocks first
  } else {
    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    qb = blk % n_qblocks;
    slot = blk / n_qblocks;
  }
  int bh;
  const int b = head_of_slot(slot, a.B, a.H, bh);
  const int n_k = real_keys(a.kv_len, b, a.n_k);  // keys from n_k on (padding) are never read
  const uint16_t* Qp = static_cast<const uint16_t*>(a.Q) + (int64_t)bh * n_q * D;
  const uint16_t* dOp = static_cast<const uint16_t*>(a.dO) + (int64_t)bh * n_q * D;
  const uint16_t* Kp = static_cast<const uint16_t*>(a.K) + (int64_t)bh * a.n_k * D;
  const uint16_t* Vp = static_cast<const uint16_t*>(a.V) + (int64_t)bh * a.n_k * D;
  const float* auxp = a.aux + (int64_t)bh * n_tiles_q * kAuxFloatsPerTile;

  const int q_blk0 = qb * kBM;
  const int qw0 = q_blk0 + 32 * wave;
  const int q = qw0 + li;

  // Q and dO rows as B operands of S^T = K Q^T and dP^T = V dO^T; zero past n_q
  bf16x8 qf[4], df[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int64_t off = (int64_t)q * D + 8 * (4 * g + ks);
    qf[ks] = q < n_q ? *reinterpret_cast<const bf16x8*>(Qp + off) : bf16x8{};
    df[ks] = q < n_q ? *reinterpret_cast<const bf16x8*>(dOp + off) : bf16x8{};
  }
  float lse2 = INFINITY;  // rows past n_q: weights 0
  uint2 nd = {0u, 0u};    // the query's -D as three bf16 parts (0 past n_q)
  if (q < n_q) {
    const float* at = auxp + (int64_t)(q / kBN) * kAuxFloatsPerTile;
    lse2 = at[q % kBN];
    nd = *reinterpret_cast<const uint2*>(at + 2 * kBN + 2 * (q % kBN));
  }
  const bf16x8 ones3 = ones3_operand(g);
  const bf16x8 ndop = __builtin_bit_cast(bf16x8, uint4{nd.x, nd.y, 0u, 0u});
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    settle(qf[ks]);
    settle(df[ks]);
  }
  settle_f(lse2);

  // Key tiles 0 .. nt-1 (causal: up to the workgroup's last query). Tiles from t_mask on hold keys past some query of
  // this wave (or past n_k) and are masked; a tile wholly after the wave's queries is masked entirely and adds 0.
  int nt = (n_k + kBN - 1) / kBN;
  if (causal) nt = min(nt, (q_blk0 + kBM - 1) / kBN + 1);
  const int t_mask = min(causal ? qw0 / kBN : nt, n_k / kBN);
  const int key_lim = (causal ? min(q, n_k - 1) : n_k - 1) - 4 * g;  // keys past it (from the lane's first) masked
  const int nu = nt;

  const uint32_t smem_lds = (uint32_t)(uintptr_t)smem;
  const int lrow = lane / 8;
  uint32_t ld_voff[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int row = 8 * c + lrow;
    ld_voff[c] = (uint32_t)(row * D + (((lane % 8) ^ swz_d<D>(row)) << 3)) * 2u;
  }
  // group 1 copies: wave 4 + gw moves K/V pieces 4gw .. 4gw+3 of the tile
  auto issue = [&](int u) __attribute__((always_inline)) {
    const uint32_t stage = smem_lds + (uint32_t)((u % kPPBwdStages) * kStageElems * 2);
    issue_rows<4, D>(Kp + (int64_t)u * kBN * D, Vp + (int64_t)u * kBN * D, n_k - u * kBN, stage, gw, lrow, ld_voff);
  };

  int roff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) roff[ks] = row_off<D>(li, g, ks);
  int toff[2][2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) toff[mb][hi] = tr_off<D>(lane, mb, hi);

  f32x16 dq[2];
  bf16x8 pds[4];  // dS^T in bf16, B operands for k-steps (16 keys) 0..3 of the tile
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) dq[mb] = f32x16{};

  // M(u): the dQ product of tile u - 1, then S^T and dP^T - D of tile u (either part may be absent), operand reads
  // two k-steps ahead of their products and fenced in the order the products use them.
  auto mslot = [&](int u, auto upd_c, auto sdp_c, f32x16(&s)[2], f32x16(&dp)[2]) __attribute__((always_inline)) {
    constexpr bool upd = decltype(upd_c)::value, sdp = decltype(sdp_c)::value;
    __builtin_amdgcn_s_setprio(3);
    const uint16_t* stc = smem + (u % kPPBwdStages) * kStageElems;
    bf16x8 kr[2][2], vr[2][2];  // [k-step % 2][kb]: S^T / dP^T operands
    auto read_ks = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        kr[ks & 1][kb] = *reinterpret_cast<const bf16x8*>(stc + kb * 32 * D + roff[ks]);
        __builtin_amdgcn_sched_barrier(0);
        vr[ks & 1][kb] = *reinterpret_cast<const bf16x8*>(stc + kTileElems + kb * 32 * D + roff[ks]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if constexpr (upd) {
      const uint16_t* st = smem + ((u - 1) % kPPBwdStages) * kStageElems;
      bf16x8 kt[2][2];  // [k-step % 2][mb]: transposed K operands of the dQ product
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          kt[ks][mb] = tr_operand<D>(st, ks, toff, mb);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) dq[mb] = mfma32x32x16(kt[ks & 1][mb], pds[ks], dq[mb]);
        __builtin_amdgcn_sched_barrier(0);
        if (ks + 2 < 4) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            kt[ks & 1][mb] = tr_operand<D>(st, ks + 2, toff, mb);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if constexpr (sdp) {
          if (ks == 2) read_ks(0);
          if (ks == 3) read_ks(1);
        }
      }
    } else if constexpr (sdp) {
      read_ks(0);
      read_ks(1);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (sdp) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          s[kb] = mfma32x32x16(kr[ks & 1][kb], qf[ks], ks == 0 ? f32x16{} : s[kb]);
          dp[kb] = mfma32x32x16(vr[ks & 1][kb], df[ks], ks == 0 ? f32x16{} : dp[kb]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (ks + 2 < 4) read_ks(ks + 2);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) dp[kb] = mfma32x32x16(ones3, ndop, dp[kb]);  // dP^T - D
    }
  };

  // V(u): dS^T of tile u in bf16
  auto vslot = [&](int u, f32x16(&s)[2], const f32x16(&dp)[2]) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(0);
    if (u >= t_mask) {  // (uniform) register r of block kb holds key 32kb + 8(r/4) + 4g + r%4 of the tile
      const int lim = key_lim - u * kBN;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) s[kb][r] = -INFINITY;
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kb = ks >> 1, base = 8 * (ks & 1);
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = fast_exp2(__builtin_fmaf(s[kb][base + 2 * j], scale_log2<D>(), -lse2));
        const float p1 = fast_exp2(__builtin_fmaf(s[kb][base + 2 * j + 1], scale_log2<D>(), -lse2));
        w[j] = pack_bf16x2(p0 * dp[kb][base + 2 * j], p1 * dp[kb][base + 2 * j + 1]);
      }
      pds[ks] = __builtin_bit_cast(bf16x8, (uint4){w[0], w[1], w[2], w[3]});
    }
    // dS is only used by the next M slot: pinned here so that its arithmetic is not sunk past the slot's barrier
#pragma unroll
    for (int k = 0; k < 4; ++k) settle(pds[k]);
  };

  if (nu > 0) {  // (uniform over the workgroup; no real key: dQ = 0)
    // prologue: group 1 brings tiles 0..2 and waits for tile 0
    if (grp == 1) {
#pragma unroll
      for (int u = 0; u < 3; ++u)
        if (u < nu) issue(u);
      wait_copies<kLPW, 4>(min(2, nu - 1));
    }
    lds_barrier();
    // Group 1 enters one slot later and group 0 leaves with an extra barrier, so every wave passes the same number
    // of barriers. Before the barrier that ends its M slot 2u + 1, group 1 waits until its copies of tile u + 1 have
    // landed (tile u + 2 may stay in flight).
    auto after_m = [&](int u) __attribute__((always_inline)) {
      if (grp == 1 && u + 1 < nu) {
        if (u + 2 < nu) wait_vmcnt<kLPW>();
        else wait_vmcnt<0>();
      }
      lds_barrier();
    };
    auto after_v = [&](int u) __attribute__((always_inline)) {
      if (grp == 1 && u + 3 < nu) issue(u + 3);
      lds_barrier();
    };
    if (grp == 1) lds_barrier();  // slot 0 of group 1: nothing
    const std::true_type yes;
    const std::false_type no;
    {
      f32x16 s[2], dp[2];
      mslot(0, no, yes, s, dp);
      after_m(0);
      vslot(0, s, dp);
      after_v(0);
    }
    for (int u = 1; u < nu; ++u) {
      f32x16 s[2], dp[2];
      mslot(u, yes, yes, s, dp);
      after_m(u);
      vslot(u, s, dp);
      after_v(u);
    }
    {
      f32x16 s[2], dp[2];
      mslot(nu, yes, no, s, dp);
    }
    lds_barrier();
    if (grp == 0) lds_barrier();  // slot 2nu + 1 of group 0: nothing
  }

  // dQ = dQ^T / sqrt(D); lane holds d = 32mb + 8(r/4) + 4g + r%4 of its query
  if (q < n_q) {
    uint16_t* row = static_cast<uint16_t*>(a.dQ) + ((int64_t)bh * n_q + q) * D;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const uint2 w = {pack_bf16x2(dq[mb][4 * rg] * inv_sqrt_d<D>(), dq[mb][4 * rg + 1] * inv_sqrt_d<D>()),
                         pack_bf16x2(dq[mb][4 * rg + 2] * inv_sqrt_d<D>(), dq[mb][4 * rg + 3] * inv_sqrt_d<D>())};
        *reinterpret_cast<uint2*>(row + 32 * mb + 8 * rg + 4 * g) = w;
      }
  }
}

bool grid_ok(int64_t n) { return n > 0 && n <= 0x7fffffff; }

}  // namespace

namespace {

template <int D>
void launch_pre_d(const BwdArgs& a, bool f32, dim3 grid, int n_tiles, hipStream_t stream) {
  if (f32) hipLaunchKernelGGL((attn_bwd_pre<float, D>), grid, dim3(256), 0, stream, a, n_tiles);
  else if (a.o_f32) hipLaunchKernelGGL((attn_bwd_pre<uint16_t, D, true>), grid, dim3(256), 0, stream, a, n_tiles);
  else hipLaunchKernelGGL((attn_bwd_pre<uint16_t, D>), grid, dim3(256), 0, stream, a, n_tiles);
}

}  // namespace

hipError_t launch_attn_bwd_pre(const BwdArgs& a, bool f32, int d, hipStream_t stream) {
  const int n_tiles = (a.n_q + kBN - 1) / kBN;
  const int64_t nb = (int64_t)n_tiles * a.B * a.H;
  if (!grid_ok(nb) || (d != 32 && d != 64 && d != 128)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nb);
  if (d == 64) launch_pre_d<64>(a, f32, grid, n_tiles, stream);
  else if (d == 32) launch_pre_d<32>(a, f32, grid, n_tiles, stream);
  else launch_pre_d<128>(a, f32, grid, n_tiles, stream);
  return hipGetLastError();
}

namespace {

template <int D>
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  constexpr int NW = 4, kStagesKV = 3, kStagesQ = 3;
  const int n_kblocks = (a.n_k + 32 * NW - 1) / (32 * NW);
  const int n_qblocks = (a.n_q + 32 * NW - 1) / (32 * NW);
  const int64_t nb_kv = (int64_t)n_kblocks * a.B * a.H, nb_q = (int64_t)n_qblocks * a.B * a.H;
  // width 64 without a window: the eight-wave ping-pong dK/dV kernel, 256 keys a workgroup
  const int n_kb_pp = (a.n_k + 255) / 256, n_qb_pp = (a.n_q + 255) / 256;
  const int64_t nb_pp = (int64_t)n_kb_pp * a.B * a.H, nbq_pp = (int64_t)n_qb_pp * a.B * a.H;
  if (!grid_ok(nb_kv) || !grid_ok(nb_q) || !grid_ok(nb_pp) || !grid_ok(nbq_pp)) return hipErrorInvalidValue;
  hipError_t e = launch_attn_bwd_pre(a, false, D, stream);
  if (e != hipSuccess) return e;
  if (a.windowed) {
    hipLaunchKernelGGL((attn_bwd_dkdv_bf16<D, NW, kStagesKV, true>), dim3((unsigned)nb_kv), dim3(64 * NW), 0, stream,
                       a, n_kblocks);
  } else {
    if constexpr (D == 64)
      hipLaunchKernelGGL(attn_bwd_dkdv_pp_bf16, dim3((unsigned)nb_pp), dim3(512), 0, stream, a, n_kb_pp);
    else
      hipLaunchKernelGGL((attn_bwd_dkdv_bf16<D, NW, kStagesKV, false>), dim3((unsigned)nb_kv), dim3(64 * NW), 0,
                         stream, a, n_kblocks);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.windowed) {
    hipLaunchKernelGGL((attn_bwd_dq_bf16<D, NW, kStagesQ, true>), dim3((unsigned)nb_q), dim3(64 * NW), 0, stream, a,
                       n_qblocks);
  } else {
    if constexpr (D == 64)
      hipLaunchKernelGGL(attn_bwd_dq_pp_bf16, dim3((unsigned)nbq_pp), dim3(512), 0, stream, a, n_qb_pp);
    else
      hipLaunchKernelGGL((attn_bwd_dq_bf16<D, NW, kStagesQ, false>), dim3((unsigned)nb_q), dim3(64 * NW), 0, stream,
                         a, n_qblocks);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const BwdArgs& a, int d, hipStream_t stream) {
  if (d == 64) return launch_bwd_bf16<64>(a, stream);
  if (d == 32) return launch_bwd_bf16<32>(a, stream);
  if (d == 128) return launch_bwd_bf16<128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace mi355
