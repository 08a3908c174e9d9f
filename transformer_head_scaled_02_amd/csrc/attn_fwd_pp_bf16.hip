// Fused scaled dot-product attention forward, bf16 in/out, d_k = d_v = 64, unmasked (optionally with key padding),
// for gfx950 (MI355X): the two waves that share a SIMD run in ping-pong.
//
// Computes, for every (batch, head) and query i:  O_i = sum_j softmax_j(Q_i . K_j / sqrt(64)) V_j. Definition:
// "Attention Is All You Need" (lettle.cn translation), section 3.2.1, equation Attention(Q,K,V).
//
// Why a second kernel for the same arithmetic: per 64-query x 64-key tile a wave spends about as many SIMD cycles
// on the softmax (an fma, an exp2 and half a pack per score on the VALU, the exp2 being limited to one
// instruction per ~8.6 cycles per SIMD) as on its two products (32 cycles per v_mfma_f32_32x32x16_bf16, 16 of
// them per product). The matrix core and the VALU of a SIMD can execute at the same time, but only for
// instructions of different waves that happen to be ready at the same time; left to the hardware, the two waves
// of a SIMD drift into step and mostly take turns. Here the workgroup has eight waves, and waves w and w + 4 share
// a SIMD; the two groups of four are held half a tile apart by the barrier that ends every slot:
//
//      slot:      0        1        2        3       ...   2n       2n+1
//      group 0:   M(0)     S(0)     M(1)     S(1)    ...   M(n)     -
//      group 1:   -        M(0)     S(0)     M(1)    ...   S(n-1)   M(n)
//
// where M(j) is the matrix-core work  O += V(j-1)^T P(j-1)  and  S(j) = K(j) Q^T  (32 products, operands read
// from LDS), and S(j) in the softmax slot is  P(j) = exp2(S(j) c - m)  packed to bf16, its row sums on the matrix
// core, the offset check and its rare slow path (all VALU but eight small products). In every slot one wave of
// each SIMD feeds the matrix core while the other runs the softmax.
//
// The arithmetic is exactly that of the lockstep kernel (attn_fwd_bf16.hip): S^T = K Q^T with the wave's queries
// in the lane index, the exponent argument s*c - m as one fma on the fp32 score (c = log2(e)/8), P rounded to bf16
// and summed on the matrix core from the very values that multiply V, and the lazy offset m (set by the first
// tile's row max, raised only when a tile's row sum of P exceeds 2^20, per row). K/V tiles go HBM -> LDS by
// global_load_lds_dwordx4 into a four-tile ring that all eight waves read (one copy per tile serves 512 queries);
// the copies are issued by the group that runs the softmax, whose VMEM issue is otherwise idle.
#include <math.h>

#include <type_traits>

#include "attn_tile.h"
#include "launch.h"

namespace mi355 {
namespace {

constexpr int kPPWaves = 8;                // two groups of four; waves w and w + 4 share a SIMD
constexpr int kPPQW = 64;                  // queries per wave: halves of 32
constexpr int kPPBM = kPPWaves * kPPQW;    // queries per workgroup
constexpr int kPPStages = 4;               // ring depth (tile t is read in slots 2t .. 2t+3)
constexpr int kPPLPW = 4;                  // one-kilobyte copies per copying wave per tile (16 per tile, 4 waves)

__global__ __launch_bounds__(64 * kPPWaves, 1) void attn_fwd_pp_bf16(AttnArgs a, int n_qblocks) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[kPPStages * 2 * kTileElems];  // [stage][K | V]

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, gw = wave & 3;
  const int lane = tid & 63;
  const int g = lane >> 5, li = lane & 31;

  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int qb = blk % n_qblocks, slot = blk / n_qblocks;
  int bh;
  const int b = head_of_slot(slot, a.B, a.H, bh), hh = bh - b * a.H;
  const int n_q = a.n_q;
  const int n_k = real_keys(a.kv_len, b, a.n_k);  // keys from n_k on (padding) are never read
  const uint16_t* Qp = static_cast<const uint16_t*>(a.Q) + (int64_t)bh * a.q_stride_bh;
  const uint16_t* Kp = static_cast<const uint16_t*>(a.K) + (int64_t)bh * a.k_stride_bh;
  const uint16_t* Vp = static_cast<const uint16_t*>(a.V) + (int64_t)bh * a.k_stride_bh;
  uint16_t* Op = static_cast<uint16_t*>(a.O) + b * a.o_stride_b + hh * a.o_stride_h;
  const int qw0 = qb * kPPBM + wave * kPPQW;  // half h owns queries qw0 + 32h + (0..31)

  // Q as the B operand of S^T = K Q^T (lane supplies Q[q][32g + 8ks + j]); rows at or past n_q are zero.
  bf16x8 qf[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = qw0 + 32 * h + li;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[h][ks] = q < n_q ? *reinterpret_cast<const bf16x8*>(Qp + (int64_t)q * kD + 32 * g + 8 * ks) : bf16x8{};
  }
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) settle(qf[h][ks]);

  const int nt = (n_k + kBN - 1) / kBN;
  const int nt_full = n_k / kBN;
  const int key_lim = n_k - 1 - 4 * g;  // (only the last tile can hold keys past it)

  // Tile copies (group 1 only): copy gi = 4*gw + i (0..15) of a tile moves rows 8c .. 8c+7 (c = gi mod 8) of K
  // (gi < 8) or V; lane l brings the logical chunk that belongs at physical chunk l mod 8 of row 8c + l/8. The
  // swizzle repeats every 16 rows: two per-lane offsets serve every copy. Rows past n_k read row n_k - 1.
  const uint32_t smem_lds = (uint32_t)(uintptr_t)smem;
  const int lrow = lane >> 3;
  uint32_t ld_voff[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int row = 8 * c + lrow;
    ld_voff[c] = (uint32_t)(row * kD + (((lane & 7) ^ swz(row)) << 3)) * 2u;
  }
  auto issue_tile = [&](int t) __attribute__((always_inline)) {
    const uint32_t stage = smem_lds + (uint32_t)((t % kPPStages) * 2 * kTileElems * 2);
    const uint16_t* kt = Kp + (int64_t)t * kBN * kD;
    const uint16_t* vt = Vp + (int64_t)t * kBN * kD;
    if (t < nt_full) {
#pragma unroll
      for (int i = 0; i < kPPLPW; ++i) {
        const int gi = gw * kPPLPW + i;
        const int c = gi & 7;
        lds_dma16((gi < 8 ? kt : vt) + (c / 2) * 16 * kD, ld_voff[i & 1],
                  stage + (gi < 8 ? 0u : kTileElems * 2u) + (uint32_t)c * 1024u);
      }
    } else {
      const int last_row = n_k - 1 - t * kBN;  // last valid row of this partial tile, >= 0
      int lr = lrow;
      asm volatile("" : "+v"(lr));
#pragma unroll
      for (int i = 0; i < kPPLPW; ++i) {
        const int gi = gw * kPPLPW + i;
        const int c = gi & 7;
        const int row = 8 * c + lr;
        lds_dma16(gi < 8 ? kt : vt, ld_voff[i & 1] + (uint32_t)((min(row, last_row) - (8 * (c & 1) + lr)) * kD * 2),
                  stage + (gi < 8 ? 0u : kTileElems * 2u) + (uint32_t)c * 1024u);
      }
    }
  };

  // per-lane LDS element offsets (as in the lockstep kernel): K operand row li, logical chunk 4g + ks; V transpose
  // reads of rows 4g + (lane%16)/4 (+8), logical chunk 4mb + 2*((lane/16)%2) + (lane%4)/2, element 4*(lane%2)
  int koff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) koff[ks] = li * kD + (((4 * g + ks) ^ swz(li)) << 3);
  int voff[2][2];
  const int jj = (lane & 15) >> 2;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int row = 4 * g + jj + 8 * hi;
      const int lchunk = 4 * mb + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
      voff[mb][hi] = kTileElems + row * kD + ((lchunk ^ swz(row)) << 3) + 4 * (lane & 1);
    }
  const bf16x8 lsel = lsum_selector(lane);

  f32x16 o[2][2], s[2][2];
  bf16x8 pf[2][4];
  float neg_m[2], l[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    o[h][0] = o[h][1] = f32x16{};
    neg_m[h] = 0.f;
    l[h] = 0.f;
  }

  // Matrix-core slot M(j): O += V(j-1)^T P(j-1) (j >= 1), then S(j) = K(j) Q^T (j < nt). The V operands are read
  // first (the products that need them go first), then the K operands.
  auto mslot = [&](int j, auto pv_c, auto qk_c) __attribute__((always_inline)) {
    constexpr bool pv = decltype(pv_c)::value, qk = decltype(qk_c)::value;
    __builtin_amdgcn_s_setprio(0);
    bf16x8 va[4][2], kr[4][2];
    if (pv) {
      const uint16_t* st = smem + ((j - 1) % kPPStages) * 2 * kTileElems;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x4 lo = lds_read_tr16x4(st + ks * 16 * kD + voff[mb][0]);
          const bf16x4 hi = lds_read_tr16x4(st + ks * 16 * kD + voff[mb][1]);
          va[ks][mb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    }
    if (qk) {
      const uint16_t* st = smem + (j % kPPStages) * 2 * kTileElems;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) kr[ks][kb] = *reinterpret_cast<const bf16x8*>(st + kb * 32 * kD + koff[ks]);
    }
    // (every operand read is issued before the first product; the output products go first, and the score
    // products after them: interleaved, S, P and both operand sets would be live at once)
    __builtin_amdgcn_sched_barrier(0);
    if (pv) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int h = 0; h < 2; ++h) o[h][mb] = mfma32x32x16(va[ks][mb], pf[h][ks], o[h][mb]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (qk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) s[h][kb] = mfma32x32x16(kr[0][kb], qf[h][0], f32x16{});
#pragma unroll
      for (int ks = 1; ks < 4; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h) s[h][kb] = mfma32x32x16(kr[ks][kb], qf[h][ks], s[h][kb]);
    }
  };

  f32x4 ts[2];
  // P = exp2(s*c - m) of half h in bf16, and its row sums on the matrix core
  auto exponentiate = [&](int h) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const f32x16& sk = s[h][ks >> 1];
      const int base = 8 * (ks & 1);
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = pack_bf16x2(fast_exp2(scaled_minus(sk[base + 2 * j], neg_m[h])),
                           fast_exp2(scaled_minus(sk[base + 2 * j + 1], neg_m[h])));
      pf[h][ks] = __builtin_bit_cast(bf16x8, (uint4){w[0], w[1], w[2], w[3]});
    }
    f32x4 t = mfma16x16x32(lsel, pf[h][0], f32x4{});
#pragma unroll
    for (int ks = 1; ks < 4; ++ks) t = mfma16x16x32(lsel, pf[h][ks], t);
    ts[h] = t;
  };
  // this row's max of s*c over the tile (both lanes of the row), half h
  auto row_max = [&](int h) __attribute__((always_inline)) {
    float mx[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      mx[j] = fmaxf(fmaxf(fmaxf(s[h][0][4 * j], s[h][0][4 * j + 1]), fmaxf(s[h][0][4 * j + 2], s[h][0][4 * j + 3])),
                    fmaxf(fmaxf(s[h][1][4 * j], s[h][1][4 * j + 1]), fmaxf(s[h][1][4 * j + 2], s[h][1][4 * j + 3])));
    return max_with_partner32(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]))) * kScaleLog2;
  };

  // Softmax slot S(j): mask (last, partial tile only), P and its row sums for both halves, then the per-row offset
  // check with its slow path, and the row sums added to l. S(j) stays in registers until the next M slot
  // overwrites it, so the slow path recomputes P from it directly.
  auto sslot = [&](int j) __attribute__((always_inline)) {
    // The softmax wave needs an issue slot every few cycles, the matrix-core wave one per 32-cycle product: issue
    // priority goes to the softmax while both are ready.
    __builtin_amdgcn_s_setprio(3);
    if (j >= nt_full) {
      const int lim = key_lim - j * kBN;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) s[h][kb][r] = -INFINITY;
    }
    if (j == 0) {
      // the first tile sets the offset to its row max (O and l are still zero: nothing to rescale)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        neg_m[h] = -row_max(h);
        exponentiate(h);
      }
    } else {
      exponentiate(0);
      exponentiate(1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // accepted when 0 <= sum <= limit; as unsigned bit patterns this also rejects inf and NaN
        const bool need = __float_as_uint(ts[h][0]) > __float_as_uint(kTileSumLimit);
        if (__builtin_amdgcn_ballot_w64(need)) {
          // slow path: raise the offset of the rows that need it to the tile's row max (never lowering it), rescale
          // O and l, and recompute P. The same decision for both lanes of a row (computed in every lane).
          const float rmax = row_max(h);
          const bool partner = partner32_any(need);
          const bool raise = need || partner;
          const float d = raise ? fmaxf(rmax + neg_m[h], 0.f) : 0.f;
          const float alpha = fast_exp2(-d);
          l[h] *= alpha;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            o[h][0][r] *= alpha;
            o[h][1][r] *= alpha;
          }
          neg_m[h] -= d;
          exponentiate(h);
        }
      }
    }
    l[0] += ts[0][0];
    l[1] += ts[1][0];
  };

  if (nt > 0) {  // (no real key: every row's output is 0; the whole workgroup skips the loop)
    // prologue: group 1 brings tiles 0..2 and waits for tile 0
    if (grp == 1) {
#pragma unroll
      for (int t = 0; t < 3; ++t)
        if (t < nt) issue_tile(t);
      if (nt >= 3) wait_vmcnt<2 * kPPLPW>();
      else if (nt == 2) wait_vmcnt<kPPLPW>();
      else wait_vmcnt<0>();
    }
    lds_barrier();
    const std::true_type yes;
    const std::false_type no;
    // Both groups run the same loop; group 1 enters it one slot later (an extra barrier first) and group 0 leaves
    // it with an extra barrier, so every wave passes the same number of barriers. Group 1 copies the tiles: tile t
    // in its softmax slot 2t - 4 (t >= 3; tiles 0..2 in the prologue), and before the barrier that ends its M slot
    // 2t - 1 it waits until its copies of tile t have landed. Tile t is read in slots 2t .. 2t + 3 and its stage
    // is refilled with tile t + 4 in slot 2t + 4. The first and the last M slot are peeled off the loop, so that S
    // is overwritten in every M slot of the loop and never live across one.
    auto after_m = [&](int j) __attribute__((always_inline)) {
      if (grp == 1) {
        if (j + 2 < nt) wait_vmcnt<kPPLPW>();  // (tile j + 2 may stay in flight)
        else wait_vmcnt<0>();
      }
      lds_barrier();
    };
    auto after_s = [&](int j) __attribute__((always_inline)) {
      if (grp == 1 && j + 3 < nt) issue_tile(j + 3);
      lds_barrier();
    };
    if (grp == 1) lds_barrier();  // slot 0 of group 1: nothing
    mslot(0, no, yes);
    after_m(0);
    sslot(0);
    after_s(0);
    for (int j = 1; j < nt; ++j) {
      mslot(j, yes, yes);
      after_m(j);
      sslot(j);
      after_s(j);
    }
    mslot(nt, yes, no);
    lds_barrier();
    if (grp == 0) lds_barrier();  // slot 2nt + 1 of group 0: nothing
  }

  // O = O^T / l; lane holds d = 32mb + 8(r/4) + 4g + r%4 of its query.
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = qw0 + 32 * h + li;
    if (q < n_q) {
      const bool seen = l[h] > 0.f;  // false only for a row with no real key (all padding): output 0, lse -inf
      const float inv = seen ? 1.0f / l[h] : 0.f;
      if (a.lse != nullptr && g == 0)
        a.lse[(int64_t)bh * n_q + q] = seen ? (__builtin_amdgcn_logf(l[h]) - neg_m[h]) * kLn2 : -INFINITY;
      uint16_t* orow = Op + (int64_t)q * a.o_stride_row;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const uint2 w = {pack_bf16x2(o[h][mb][4 * rg] * inv, o[h][mb][4 * rg + 1] * inv),
                           pack_bf16x2(o[h][mb][4 * rg + 2] * inv, o[h][mb][4 * rg + 3] * inv)};
          *reinterpret_cast<uint2*>(orow + 32 * mb + 8 * rg + 4 * g) = w;
        }
      if (a.o32 != nullptr) {
        float* frow = a.o32 + ((int64_t)bh * n_q + q) * 64;
#pragma unroll
        for (int mb = 0; mb < 64 / 32; ++mb)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg)
            *reinterpret_cast<float4*>(frow + 32 * mb + 8 * rg + 4 * g) =
                float4{o[h][mb][4 * rg] * inv, o[h][mb][4 * rg + 1] * inv, o[h][mb][4 * rg + 2] * inv,
                       o[h][mb][4 * rg + 3] * inv};
      }
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd_pp_bf16(const AttnArgs& a, hipStream_t stream) {
  if (a.causal || a.windowed) return hipErrorInvalidValue;
  const int n_qblocks = (a.n_q + kPPBM - 1) / kPPBM;
  const int64_t nblocks = (int64_t)n_qblocks * a.B * a.H;
  if (nblocks <= 0 || nblocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_fwd_pp_bf16, dim3((unsigned)nblocks), dim3(64 * kPPWaves), 0, stream, a, n_qblocks);
  return hipGetLastError();
}

}  // namespace mi355
