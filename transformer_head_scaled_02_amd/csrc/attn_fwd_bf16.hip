// Fused scaled dot-product attention forward, bf16 in/out, d_k = d_v = D in {32, 64, 128}, for gfx950 (MI355X).
//
// Computes, for every (batch, head) and query i:  O_i = sum_j softmax_j(Q_i . K_j / sqrt(D)) V_j, with the optional
// causal mask (keys j > i get score -inf, i.e. weight 0). Definition: "Attention Is All You Need" (lettle.cn
// translation), section 3.2.1, equation Attention(Q,K,V); mask: "Transformer：抛弃循环与卷积的序列建模"
// (jiashun-ye.github.io), section "Transformer 中的三种 Attention".
//
// Design (a workgroup of NW waves owns NW*32 queries of one head; keys are streamed in tiles of 64):
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: a wave's 32 queries sit in the
//    lane index (lanes l and l+32 both own query l%32), keys in the accumulator registers. The fp32 exponentials
//    packed to bf16 are directly the B operand of the second product O^T = V^T P^T: the n x n score matrix never
//    leaves registers.
//  * K and V tiles go HBM -> LDS with global_load_lds_dwordx4 (no register staging, no LDS store instructions) into
//    a STAGES-deep ring; one barrier per tile, placed before the last half's P V^T product of tile t: it publishes
//    tile t+1, whose K operands are then read into registers while those products run (so the next tile's score
//    products never wait on LDS), and it frees tile t's stage for the copy of tile t + STAGES. Each wave issues
//    16/NW of the 16 one-kilobyte copies of a tile from a scalar tile base and fixed per-lane offsets. Rows are
//    unpadded (128 B) with an XOR chunk swizzle that keeps the K row reads and the V transpose reads
//    (ds_read_b64_tr_b16) free of bank conflicts.
//  * The softmax runs on the VALU, which on this chip is busier than the matrix core at d = 64 (one v_exp_f32 per
//    score costs about as many SIMD cycles as the score's share of both products), so the steady-state tile spends
//    only an exp2 and half a v_cvt_pk_bf16_f32 per score:
//      - the exponent argument s*c - m (c = log2(e)/sqrt(64), m the row's offset) is one v_fmamk_f32 on the fp32
//        score: the scale is applied to the accumulated score, never to the bf16 inputs, where its rounding would
//        grow with the size of the scores;
//      - the row sum of P is accumulated on the matrix core (v_mfma_f32_16x16x32_bf16 with a 0/1 selector operand)
//        from the very bf16 P that multiplies V, and that per-tile sum also guards the offset: while it stays at
//        most 2^20 every p of the tile is at most 2^20 and the tile is accepted; otherwise (a rare slow path, and
//        always on a row's first tile) the row's offset is raised to the tile's row max, the accumulated O and l
//        are rescaled and the tile's P is recomputed before it touches O. The decision is per row, so a row never
//        depends on another row's keys.
//  * With H = 2 a wave owns two independent halves of 32 queries: every K and V operand read from LDS feeds two
//    products, and one half's MFMAs fill the gaps of the other half's softmax chain within the same wave. This
//    configuration serves unmasked attention only; its one masked tile (a ragged last tile) runs the halves one after
//    the other, which needs fewer registers than the interleaved order and keeps the kernel within the
//    two-waves-per-SIMD budget.
//  * The steady-state loop is unrolled over the ring so every LDS address is a per-lane base plus an immediate
//    offset (the few remaining tiles compute their stage at run time); two workgroups per CU (two waves per SIMD)
//    let one wave's MFMAs overlap the other's VALU work.
//  * Key tiles entirely after a wave's last query are skipped (causal), and query blocks run heaviest first.
#include <math.h>

#include "attn_tile.h"
#include "launch.h"

namespace mi355 {
namespace {

// a ring stage given at compile time (integral_constant) or at run time (int)
template <class T>
__device__ __forceinline__ constexpr int stage_index(T s) { return (int)s; }

template <int D, int NW, int H, int MINB, int STAGES, bool WIN>
__global__ __launch_bounds__(64 * NW, MINB) void attn_fwd_bf16(AttnArgs a, int n_qblocks) {
  static_assert(D == 32 || D == 64 || D == 128, "head width");
  constexpr int kD = D;                   // (shadows the 64 of the shared tile header)
  constexpr int kTileElems = kBN * D;     // one 64-key tile of K or V
  constexpr int kKS = D / 16;             // k-steps of S^T = K Q^T
  constexpr int kMB = D / 32;             // 32-row blocks of O^T
  constexpr int kCPT = D / 8;             // one-kilobyte copies per K (or V) tile
  constexpr int kRPC = 512 / D;           // tile rows per copy
  constexpr int kNOff = D / 32;           // copies per 16 rows (one swizzle period): distinct per-lane copy offsets
  constexpr int kQW = 32 * H;             // queries per wave: H independent halves of 32
  constexpr int kBM = kQW * NW;           // queries per workgroup
  constexpr int kLPW = 2 * kCPT / NW;     // one-kilobyte tile copies per wave per tile
  // Wide heads (D = 128) read each tile's K operands at the start of its step and V's per output block, and take
  // the ring barrier after the tile's last product: holding the next tile's K and all of V in registers as well
  // would not fit two waves per SIMD.
  constexpr bool kLate = D >= 128;
  static_assert((2 * kCPT) % NW == 0 && kLPW % kNOff == 0,
                "tile copies split evenly over the waves, each wave's copies a whole number of swizzle periods");
  static_assert(STAGES >= 2 && STAGES <= 4, "ring depth");
  static_assert(H == 1 || H == 2, "one or two query halves per wave");
  static_assert(!kLate || H == 1, "wide heads have one query half per wave");
  __shared__ __attribute__((aligned(16))) uint16_t smem[STAGES * 2 * kTileElems];  // [stage][K | V]

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 5, li = lane & 31;
  const bool causal = H == 1 && a.causal != 0;  // the two-half kernel serves unmasked attention only

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
  const int b = head_of_slot(slot, a.B, a.H, bh), hh = bh - b * a.H;
  const int n_q = a.n_q;
  int n_k = real_keys(a.kv_len, b, a.n_k);  // keys from n_k on (padding) are never read
  const uint16_t* Qp = static_cast<const uint16_t*>(a.Q) + (int64_t)bh * a.q_stride_bh;
  const uint16_t* Kp = static_cast<const uint16_t*>(a.K) + (int64_t)bh * a.k_stride_bh;
  const uint16_t* Vp = static_cast<const uint16_t*>(a.V) + (int64_t)bh * a.k_stride_bh;
  uint16_t* Op = static_cast<uint16_t*>(a.O) + b * a.o_stride_b + hh * a.o_stride_h;

  const int q_blk0 = qb * kBM;
  const int qw0 = q_blk0 + wave * kQW;  // first query of this wave; half h owns queries qw0 + 32h + (0..31)
  static_assert(!WIN || H == 1, "the windowed kernel has one query half per wave");
  // Restricted self-attention: tiles are counted from the tile of the first key any query of the workgroup may see
  // (key kb0); from here on n_k and every key bound are relative to it.
  int kb0 = 0;
  if constexpr (WIN) {
    kb0 = max(0, q_blk0 - a.window) / kBN * kBN;
    Kp += (int64_t)kb0 * kD;
    Vp += (int64_t)kb0 * kD;
    n_k = max(n_k - kb0, 0);
  }

  // Q as the B operand of S^T = K Q^T: lane supplies Q[q][(D/2)g + 8ks + j], ks = 0..D/16-1 (the same d order as
  // the K operand). Rows at or past n_q are zero.
  bf16x8 qf[H][kKS];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const int q = qw0 + 32 * h + li;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      qf[h][ks] = q < n_q ? *reinterpret_cast<const bf16x8*>(Qp + (int64_t)q * kD + (kD / 2) * g + 8 * ks) : bf16x8{};
  }
#pragma unroll
  for (int h = 0; h < H; ++h)
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) settle(qf[h][ks]);

  int nt = (n_k + kBN - 1) / kBN;
  if (causal) nt = min(nt, (q_blk0 + kBM - 1 - kb0) / kBN + 1);
  // tiles before t_mask need no mask for any query of this wave; tiles from t_skip on lie entirely in its future
  int t_mask = min(causal ? (qw0 - kb0) / kBN : nt, n_k / kBN);
  int t_skip = causal ? min(nt, (qw0 + kQW - 1 - kb0) / kBN + 1) : nt;
  const int nt_full = n_k / kBN;  // tiles with no row past n_k
  // keys past this bound, counted from the lane's first key 4g of tile 0, are masked
  int key_lim[H];
#pragma unroll
  for (int h = 0; h < H; ++h) key_lim[h] = (causal ? min(qw0 + 32 * h + li - kb0, n_k - 1) : n_k - 1) - 4 * g;
  // window: keys before key_lo (same counting) are masked too, the workgroup's tiles end after its last query's
  // window, and every tile takes the masked path
  int key_lo = 0;
  if constexpr (WIN) {
    const int w = a.window;
    key_lo = qw0 + li - w - kb0 - 4 * g;
    key_lim[0] = min(key_lim[0], qw0 + li + w - kb0 - 4 * g);
    nt = min(nt, (q_blk0 + kBM - 1 + w - kb0) / kBN + 1);
    t_mask = 0;
    t_skip = min(t_skip, (qw0 + kQW - 1 + w - kb0) / kBN + 1);
  }

  // Tile copies: copy gi (0 .. 2*D/8 - 1) of a tile moves rows R*c .. R*c + R-1 (R = 512/D rows of a kilobyte,
  // c = gi mod D/8) of K (gi < D/8) or V; lane l brings the logical chunk that belongs at physical chunk l mod D/8 of
  // row R*c + l/(D/8). The swizzle repeats every 16 rows, so D/32 per-lane offsets (rows R*i + l/(D/8)) serve every
  // copy, the rest of the row offset going into the scalar base. Rows past n_k read row n_k-1 (their scores are
  // masked and their weights are zero).
  const uint32_t smem_lds = (uint32_t)(uintptr_t)smem;  // LDS byte address of the ring
  const int lrow = lane / kCPT;
  uint32_t ld_voff[kNOff];
#pragma unroll
  for (int c = 0; c < kNOff; ++c) {
    const int row = kRPC * c + lrow;
    ld_voff[c] = (uint32_t)(row * kD + (((lane % kCPT) ^ swz_d<D>(row)) << 3)) * 2u;
  }
  auto issue_tile = [&](int t) __attribute__((always_inline)) {
    const uint32_t stage = smem_lds + (uint32_t)((t % STAGES) * 2 * kTileElems * 2);
    const uint16_t* kt = Kp + (int64_t)t * kBN * kD;
    const uint16_t* vt = Vp + (int64_t)t * kBN * kD;
    if (t < nt_full) {
#pragma unroll
      for (int i = 0; i < kLPW; ++i) {
        const int gi = wave * kLPW + i;
        const int c = gi & (kCPT - 1);  // this copy moves rows R*c .. R*c + R-1
        lds_dma16((gi < kCPT ? kt : vt) + (c / kNOff) * 16 * kD, ld_voff[i % kNOff],
                  stage + (gi < kCPT ? 0u : kTileElems * 2u) + (uint32_t)c * 1024u);
      }
    } else {
      // Partial tile: from the unshifted tile base, lane offset = row min(row, last_row) with the chunk swizzle of
      // destination row `row` (the 16-row shift is folded back in, so the 32-bit offset is never negative).
      const int last_row = n_k - 1 - t * kBN;  // last valid row of this partial tile, >= 0
      // (lrow passes through an empty asm so these rare-path rows are computed here, not kept in registers)
      int lr = lrow;
      asm volatile("" : "+v"(lr));
#pragma unroll
      for (int i = 0; i < kLPW; ++i) {
        const int gi = wave * kLPW + i;
        const int c = gi & (kCPT - 1);
        const int row = kRPC * c + lr;
        lds_dma16(gi < kCPT ? kt : vt,
                  ld_voff[i % kNOff] + (uint32_t)((min(row, last_row) - (kRPC * (c & (kNOff - 1)) + lr)) * kD * 2),
                  stage + (gi < kCPT ? 0u : kTileElems * 2u) + (uint32_t)c * 1024u);
      }
    }
  };

  // per-lane LDS element offsets: K operand row li, logical chunk (D/16)g + ks; V transpose-read row 4g +
  // (lane%16)/4 (+8 for the second half), logical chunk 4mb + 2*((lane/16)%2) + (lane%4)/2, element 4*(lane%2) of
  // the chunk
  int koff[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) koff[ks] = li * kD + ((((kD / 16) * g + ks) ^ swz_d<D>(li)) << 3);
  int voff[kMB][2];
  const int jj = (lane & 15) >> 2;
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int row = 4 * g + jj + 8 * hi;
      const int lchunk = 4 * mb + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
      voff[mb][hi] = kTileElems + row * kD + ((lchunk ^ swz_d<D>(row)) << 3) + 4 * (lane & 1);
    }
  const bf16x8 lsel = lsum_selector(lane);

  f32x16 o[H][kMB];
  float neg_m[H], l[H];  // -m (m = the row's exponent offset, log2 units, set by the first tile) and the row sum
#pragma unroll
  for (int h = 0; h < H; ++h) {
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) o[h][mb] = f32x16{};
    // (window: a finite "unset" offset far above any score, so that the first tile a row can see overflows its
    // tile sum and takes the slow path, which sets the offset to that tile's row max; tiles the row cannot see leave
    // it alone)
    neg_m[h] = WIN ? 1024.f : 0.f;
    l[h] = 0.f;
  }

  // One tile: S^T = K Q^T, P = exp2(s*c - m) packed to bf16 with its row sums, the offset check, O^T += V^T P^T,
  // for each query half. The K and V operands are read from LDS once and serve every half; while one half's softmax
  // runs on the VALU, the other half's products keep the matrix core busy. Masked tiles give keys past the row's
  // bound the score -inf. The first tile sets the offset to its row max.
  auto step = [&](int t, auto stage_c, auto masked_c, auto first_c, bf16x8(&kreg)[kKS][2], auto&& mid)
                  __attribute__((always_inline)) {
    constexpr bool kM = decltype(masked_c)::value;
    constexpr bool kFirst = decltype(first_c)::value;
    const uint16_t* stage = smem + stage_index(stage_c) * 2 * kTileElems;

    auto load_k = [&](bf16x8(&ka)[kKS][2]) __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) ka[ks][kb] = *reinterpret_cast<const bf16x8*>(stage + kb * 32 * kD + koff[ks]);
    };
    f32x16 s[H][2];
    // S^T = K Q^T for half h; s[h][kb] register r holds key 32kb + 8(r/4) + 4g + r%4 of the tile
    auto scores = [&](auto h_c, const bf16x8(&ka)[kKS][2]) __attribute__((always_inline)) {
      constexpr int h = decltype(h_c)::value;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[h][kb] = mfma32x32x16(ka[0][kb], qf[h][0], f32x16{});
#pragma unroll
      for (int ks = 1; ks < kKS; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[h][kb] = mfma32x32x16(ka[ks][kb], qf[h][ks], s[h][kb]);
      if (kM) {
        const int lim = key_lim[h] - t * kBN, lo = key_lo - t * kBN;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kb + 8 * (r >> 2) + (r & 3) > lim || (WIN && 32 * kb + 8 * (r >> 2) + (r & 3) < lo))
              s[h][kb][r] = -INFINITY;
      }
    };

    bf16x8 pf[H][4];
    f32x4 ts[H];
    // P = exp2(s*c - m) in bf16 and the tile's row sum of P, for half h
    auto exponentiate = [&](auto h_c) __attribute__((always_inline)) {
      constexpr int h = decltype(h_c)::value;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f32x16& sk = s[h][ks >> 1];
        const int base = 8 * (ks & 1);
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w[j] = pack_bf16x2(fast_exp2(scaled_minus<D>(sk[base + 2 * j], neg_m[h])),
                             fast_exp2(scaled_minus<D>(sk[base + 2 * j + 1], neg_m[h])));
        pf[h][ks] = __builtin_bit_cast(bf16x8, (uint4){w[0], w[1], w[2], w[3]});
      }
      ts[h] = mfma16x16x32(lsel, pf[h][0], f32x4{});
#pragma unroll
      for (int ks = 1; ks < 4; ++ks) ts[h] = mfma16x16x32(lsel, pf[h][ks], ts[h]);
    };
    // this row's max of s*c over the tile (both lanes of the row), for half h
    auto row_max = [&](auto h_c) __attribute__((always_inline)) {
      constexpr int h = decltype(h_c)::value;
      float mx[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        mx[j] = fmaxf(fmaxf(fmaxf(s[h][0][4 * j], s[h][0][4 * j + 1]), fmaxf(s[h][0][4 * j + 2], s[h][0][4 * j + 3])),
                      fmaxf(fmaxf(s[h][1][4 * j], s[h][1][4 * j + 1]), fmaxf(s[h][1][4 * j + 2], s[h][1][4 * j + 3])));
      return max_with_partner32(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]))) * scale_log2<D>();
    };
    // the softmax of half h, ending with its row sums added to l
    auto softmax = [&](auto h_c) __attribute__((always_inline)) {
      constexpr int h = decltype(h_c)::value;
      if (kFirst) {
        // the first tile sets the offset to its row max (o and l are still zero: nothing to rescale)
        neg_m[h] = -row_max(h_c);
        exponentiate(h_c);
      } else {
        exponentiate(h_c);
        // accepted when 0 <= sum <= limit; as unsigned bit patterns this also rejects inf and NaN (a NaN sum comes
        // from 0 * inf when another row's p overflowed)
        const bool need = __float_as_uint(ts[h][0]) > __float_as_uint(kTileSumLimit);
        if (__builtin_amdgcn_ballot_w64(need)) {
          // Slow path: S was overwritten by P; recompute it (the tile is still in LDS), raise the offset of the rows
          // that need it to the tile's row max (never lowering it), rescale O and l, and recompute P. The empty asm
          // with a memory clobber makes the compiler read the K operands from LDS again instead of keeping them
          // alive across the fast path.
          asm volatile("" ::: "memory");
          {
            bf16x8 ka[kKS][2];
            load_k(ka);
            scores(h_c, ka);
          }
          const float rmax = row_max(h_c);
          // the same decision for both lanes of a row (computed in every lane: a cross-lane read must not sit
          // behind a branch on the lane's own flag)
          const bool partner = partner32_any(need);
          const bool raise = need || partner;
          const float d = raise ? fmaxf(rmax + neg_m[h], 0.f) : 0.f;  // how far m rises
          const float alpha = fast_exp2(-d);
          l[h] *= alpha;
#pragma unroll
          for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb) o[h][mb][r] *= alpha;
          neg_m[h] -= d;
          exponentiate(h_c);
        }
      }
      l[h] += ts[h][0];
    };

    // Masked tiles of the two-half kernel (only a ragged last tile: it serves unmasked attention) run the halves one
    // after the other, which needs fewer registers than the interleaved order.
    constexpr bool kSeq = kM && H == 2;
    if constexpr (kLate) {
      bf16x8 ka[kKS][2];
      load_k(ka);
      scores(std::integral_constant<int, 0>{}, ka);
    } else if (!kSeq) {
      unroll<H>([&](auto h_c) __attribute__((always_inline)) { scores(h_c, kreg); });
    }
    // V^T operands, read once for every half: k-step ks pairs P registers 8(ks%2) .. +7 of key block ks/2 with keys
    // 16ks + 4g + (0..3) and 16ks + 8 + 4g + (0..3); two transpose reads of V rows give the matching operand.
    if constexpr (kLate) {
      // one half; each 32-row block of V^T is read just before its products, and the ring barrier follows the
      // tile's last read of V
      softmax(std::integral_constant<int, 0>{});
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        bf16x8 vm[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x4 lo = lds_read_tr16x4(stage + ks * 16 * kD + voff[mb][0]);
          const bf16x4 hi = lds_read_tr16x4(stage + ks * 16 * kD + voff[mb][1]);
          vm[ks] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) o[0][mb] = mfma32x32x16(vm[ks], pf[0][ks], o[0][mb]);
      }
      mid();
    } else {
      bf16x8 va[4][kMB];
      unroll<H>([&](auto h_c) __attribute__((always_inline)) {
        constexpr int h = decltype(h_c)::value;
        if (kSeq) scores(h_c, kreg);
        softmax(h_c);
        if (h == 0) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb) {
              const bf16x4 lo = lds_read_tr16x4(stage + ks * 16 * kD + voff[mb][0]);
              const bf16x4 hi = lds_read_tr16x4(stage + ks * 16 * kD + voff[mb][1]);
              va[ks][mb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        }
        if (h == H - 1) mid();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb) o[h][mb] = mfma32x32x16(va[ks][mb], pf[h][ks], o[h][mb]);
      });
    }
  };

  // K operands of a tile, read from its ring stage
  auto read_k = [&](const uint16_t* st, bf16x8(&kr)[kKS][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) kr[ks][kb] = *reinterpret_cast<const bf16x8*>(st + kb * 32 * kD + koff[ks]);
  };
  // Between the last half's softmax and its P V^T product of tile t: wait until this wave's copies of tile t+1 have
  // landed (later tiles may stay in flight), then for every wave's (the barrier, which also certifies that every
  // wave has read V of tile t and K of every tile up to t+1, so tile t's stage is free), read K of tile t+1 into
  // registers while the products run, and issue tile t + STAGES into the freed stage.
  // (Wide heads: the same, after the tile's last product, and without the K read.)
  bf16x8 kr[kKS][2];
  auto mid = [&](int t, auto next_stage_c) __attribute__((always_inline)) {
    if (t + 1 >= nt) return;
    const int ahead = min(STAGES - 2, nt - 2 - t);  // tiles issued after t+1
    if (ahead >= 2) wait_vmcnt<2 * kLPW>();
    else if (ahead == 1) wait_vmcnt<kLPW>();
    else wait_vmcnt<0>();
    lds_barrier();
    if constexpr (!kLate) read_k(smem + stage_index(next_stage_c) * 2 * kTileElems, kr);
    if (t + STAGES < nt) issue_tile(t + STAGES);
  };

  const std::false_type no;
  const std::true_type yes;
  if (nt > 0) {  // (no real key: every row's output is 0)
#pragma unroll
    for (int t = 0; t < STAGES; ++t)
      if (t < nt) issue_tile(t);
    {
      const int ahead = min(STAGES - 1, nt - 1);
      if (ahead >= 3) wait_vmcnt<3 * kLPW>();
      else if (ahead == 2) wait_vmcnt<2 * kLPW>();
      else if (ahead == 1) wait_vmcnt<kLPW>();
      else wait_vmcnt<0>();
      lds_barrier();
      if constexpr (!kLate) read_k(smem, kr);
    }
    // tile 0 (every row has at least one key it may see there)
    {
      auto m0 = [&]() __attribute__((always_inline)) { mid(0, std::integral_constant<int, 1 % STAGES>{}); };
      if constexpr (WIN) step(0, std::integral_constant<int, 0>{}, yes, no, kr, m0);
      else if (t_mask > 0) step(0, std::integral_constant<int, 0>{}, no, yes, kr, m0);
      else step(0, std::integral_constant<int, 0>{}, yes, yes, kr, m0);
    }
    int t = 1;
    // steady state: groups of STAGES unmasked tiles starting at t = 1 (mod STAGES), so each tile's ring stage is a
    // compile-time constant
    for (; t + STAGES <= t_mask; t += STAGES)
      unroll<STAGES>([&](auto u) __attribute__((always_inline)) {
        constexpr int kU = decltype(u)::value;
        auto mu = [&]() __attribute__((always_inline)) {
          mid(t + kU, std::integral_constant<int, (2 + kU) % STAGES>{});
        };
        step(t + kU, std::integral_constant<int, (1 + kU) % STAGES>{}, no, no, kr, mu);
      });
    // the remaining tiles, with the ring stage computed at run time
    for (; t < t_mask; ++t) {
      auto md = [&]() __attribute__((always_inline)) { mid(t, (t + 1) % STAGES); };
      step(t, t % STAGES, no, no, kr, md);
    }
    for (; t < nt; ++t) {
      auto md = [&]() __attribute__((always_inline)) { mid(t, (t + 1) % STAGES); };
      if (t < t_skip) step(t, t % STAGES, yes, no, kr, md);
      else md();
    }
  }

  // O = O^T / l; lane holds d = 32mb + 8(r/4) + 4g + r%4 of its query.
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const int q = qw0 + 32 * h + li;
    if (q < n_q) {
      const bool seen = l[h] > 0.f;  // false only for a row with no real key (all padding): output 0, lse -inf
      const float inv = seen ? 1.0f / l[h] : 0.f;
      // row log-sum-exp of the scaled scores, natural log: log2(sum_j exp2(s_j c)) = m + log2(l)
      if (a.lse != nullptr && g == 0)
        a.lse[(int64_t)bh * n_q + q] = seen ? (__builtin_amdgcn_logf(l[h]) - neg_m[h]) * kLn2 : -INFINITY;
      uint16_t* orow = Op + (int64_t)q * a.o_stride_row;
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const uint2 w = {pack_bf16x2(o[h][mb][4 * rg] * inv, o[h][mb][4 * rg + 1] * inv),
                           pack_bf16x2(o[h][mb][4 * rg + 2] * inv, o[h][mb][4 * rg + 3] * inv)};
          *reinterpret_cast<uint2*>(orow + 32 * mb + 8 * rg + 4 * g) = w;
        }
      if (a.o32 != nullptr) {
        float* frow = a.o32 + ((int64_t)bh * n_q + q) * kD;
#pragma unroll
        for (int mb = 0; mb < kD / 32; ++mb)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg)
            *reinterpret_cast<float4*>(frow + 32 * mb + 8 * rg + 4 * g) =
                float4{o[h][mb][4 * rg] * inv, o[h][mb][4 * rg + 1] * inv, o[h][mb][4 * rg + 2] * inv,
                       o[h][mb][4 * rg + 3] * inv};
      }
    }
  }
}

template <int D, int NW, int H, int MINB, int STAGES, bool WIN = false>
hipError_t launch(const AttnArgs& a, hipStream_t stream) {
  constexpr int kBM = 32 * H * NW;
  const int n_qblocks = (a.n_q + kBM - 1) / kBM;
  const int64_t nblocks = (int64_t)n_qblocks * a.B * a.H;
  if (nblocks <= 0 || nblocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_fwd_bf16<D, NW, H, MINB, STAGES, WIN>), dim3((unsigned)nblocks), dim3(64 * NW), 0, stream,
                     a, n_qblocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, int d, hipStream_t stream) {
  // Unmasked: from 512 queries on, the eight-wave ping-pong kernel; below, 4-wave workgroups of 256 queries (two
  // halves of 32 per wave), two per CU (two waves per SIMD, 256 registers each), a 3-tile ring; up to 256 queries
  // (short sequences, where a call is bound by latency), 128-query workgroups with one half per wave and a 2-tile
  // ring, so that no wave runs with queries all past n_q at 128 queries and more workgroups share the work.
  // Causal: 4-wave workgroups of 128 queries with a 4-tile ring, two per CU, which balanced the triangular work best;
  // up to 512 queries, 2-wave workgroups of 64 queries (four per CU, 2-tile ring), for shorter chains per workgroup.
  // (Measured with the calls replayed from a HIP graph: B=32 h=8 n=128 6.8 -> 5.8 us, B=16 h=8 n_q=200 n_k=256
  // 9.0 -> 6.8 us, causal B=32 h=8 n=256 9.5 -> 9.1 us.)
  // Other head widths: d = 32 as d = 64 (tiles of half the size; unmasked with a 4-tile ring); d = 128 with one
  // query half per wave and a 2-tile ring of 64 KB: unmasked in one 8-wave workgroup per CU, causal and windowed in
  // two 4-wave workgroups per CU (the smaller blocks balance the triangular work).
  switch (d) {
    case 64:
      if (a.windowed) return launch<64, 4, 1, 2, 4, true>(a, stream);
      if (!a.causal && a.n_q >= 512) return launch_attn_fwd_pp_bf16(a, stream);
      if (!a.causal && a.n_q <= 256) return launch<64, 4, 1, 2, 2>(a, stream);
      if (!a.causal) return launch<64, 4, 2, 2, 3>(a, stream);
      if (a.n_q <= 512) return launch<64, 2, 1, 4, 2>(a, stream);
      return launch<64, 4, 1, 2, 4>(a, stream);
    case 32:
      if (a.windowed) return launch<32, 4, 1, 2, 4, true>(a, stream);
      if (!a.causal) return launch<32, 4, 2, 2, 4>(a, stream);
      return launch<32, 4, 1, 2, 4>(a, stream);
    case 128:
      if (a.windowed) return launch<128, 4, 1, 2, 2, true>(a, stream);
      if (!a.causal) return launch<128, 8, 1, 1, 2>(a, stream);
      return launch<128, 4, 1, 2, 2>(a, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace mi355
