// Fused scaled dot-product attention forward, bf16 in/out, d_k = d_v = 64, for gfx950 (MI355X).
//
// Computes, for every (batch, head) and query i:  O_i = sum_j softmax_j(Q_i . K_j / sqrt(64)) V_j, with the optional
// causal mask (keys j > i get score -inf, i.e. weight 0). Definition: "Attention Is All You Need" (lettle.cn
// translation), section 3.2.1, equation Attention(Q,K,V); mask: "Transformer：抛弃循环与卷积的序列建模"
// (jiashun-ye.github.io), section "Transformer 中的三种 Attention".
//
// Design (a workgroup of NW waves owns NW*NSB*32 queries of one head; each wave owns NSB sub-blocks of 32 queries;
// keys are streamed in tiles of 64):
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: queries sit in the lane index
//    (lanes l and l+32 both own query l%32 of a sub-block), keys in the accumulator registers. The row softmax then
//    reduces over registers plus one v_permlane32_swap, and the fp32 accumulator packed to bf16 is directly the B
//    operand of the second product O^T = V^T P^T: the n x n score matrix never leaves registers.
//  * K and V tiles are staged in LDS row-major (16-byte coalesced global loads, 16-byte LDS stores). The K operand is
//    a 16-byte row read; the V^T operand comes from two ds_read_b64_tr_b16 transpose reads, which hand each lane the 4
//    consecutive keys of one d column that the P operand's register layout pairs it with. Every K/V operand read
//    feeds all NSB sub-blocks. Row paddings (144 B for K, 160 B for V) keep the reads free of bank conflicts. Tiles
//    are prefetched into registers two ahead; LDS is double-buffered with one barrier per tile.
//  * The softmax costs about as many VALU-pipe cycles per tile as the MFMAs take on the matrix core (v_exp_f32
//    alone ~9 cycles per wave instruction), and one wave can issue a VALU op only every ~6 cycles. So the kernel
//    is built for several waves per SIMD (the default configuration keeps each wave under 128 VGPRs for 4 waves per
//    SIMD): while some waves run MFMAs, the others run their softmax.
//  * Online softmax in the exp2 domain: p = exp2(s*c - m) with c = log2(e)/sqrt(64). m is a per-row offset raised
//    only when the tile's row max exceeds it by more than 2^8 (the rescale branch is skipped when no row of the wave
//    needs it); p <= 256 is exact enough in bf16 and the fp32 sums. l sums the bf16-rounded p (the values that
//    multiply V) with v_dot2_f32_bf16.
//  * Unmasked tiles run mask-free code; only tiles on the causal diagonal or past n_k take the masked path. Key tiles
//    entirely after a wave's last query are skipped, and query blocks run heaviest first.
#include "device_common.h"
#include "launch.h"

#include <math.h>

namespace mi355 {
namespace {

constexpr int kD = 64;                     // head width
constexpr int kBN = 64;                    // keys per tile
constexpr int kKS = 72;                    // K row stride in LDS (bf16 elements): 144 B
constexpr int kVS = 80;                    // V row stride in LDS (bf16 elements): 160 B
constexpr int kKElems = kBN * kKS;
constexpr int kVElems = kBN * kVS;
constexpr int kBufElems = kKElems + kVElems;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr float kScaleLog2 = (float)(1.4426950408889634 / 8.0);  // log2(e) / sqrt(64)

template <int NSB>
struct WaveState {
  f32x16 o[NSB][2];  // O^T accumulators [sub-block][d rows 0..31 | 32..63], query column li of the sub-block
  float m[NSB];      // exp2 offset in use for this lane's query of each sub-block (scaled-score units)
  float l[NSB];      // sum of rounded p over this lane's keys (the partner lane 32 away holds the rest)
};

// Softmax update of one 32-query sub-block over one 64-key tile; writes the P operand (bf16) for the 4 PV k-steps.
// s[kb] register r holds key k0 + 32kb + 8(r/4) + 4g + r%4 for query q.
template <bool kMasked>
__device__ __forceinline__ void softmax_rows(f32x16 (&s)[2], f32x16& o0, f32x16& o1, float& m, float& l,
                                             bf16x8 (&pf)[4], float c, int k0, int q, int g, int n_k, bool causal) {
  if (kMasked) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
        if (key >= n_k || (causal && key > q)) s[kb][r] = -INFINITY;
      }
  }
  // four independent max3 chains, then combine
  float mx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) mx[j] = fmaxf(fmaxf(s[0][4 * j], s[0][4 * j + 1]), s[0][4 * j + 2]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    mx[j] = fmaxf(fmaxf(mx[j], s[0][4 * j + 3]), s[1][4 * j]);
    mx[j] = fmaxf(fmaxf(mx[j], s[1][4 * j + 1]), s[1][4 * j + 2]);
    mx[j] = fmaxf(mx[j], s[1][4 * j + 3]);
  }
  float rmax = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
  rmax = max_with_partner32(rmax) * c;
  // Raise a row's offset only when its p would otherwise exceed 2^threshold. The decision is per row (the ballot
  // only skips the branch when no row needs it), so a row's arithmetic never depends on other rows' keys.
  const bool need = rmax > m + kRescaleThreshold;  // implies rmax finite
  if (__builtin_amdgcn_ballot_w64(need)) {
    const float alpha = need ? fast_exp2(m - rmax) : 1.f;  // 0 on a row's first tile (m = -inf)
    m = need ? rmax : m;
    l *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      o0[r] *= alpha;
      o1[r] *= alpha;
    }
  }
  const float m_use = (kMasked && m == -INFINITY) ? 0.f : m;
  float lsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const f32x16& sk = s[ks >> 1];
    const int base = 8 * (ks & 1);
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p0 = fast_exp2(fmaf(sk[base + 2 * j], c, -m_use));
      const float p1 = fast_exp2(fmaf(sk[base + 2 * j + 1], c, -m_use));
      w[j] = pack_bf16x2_nonneg(p0, p1);
      lsum[j] += p0 + p1;
    }
    pf[ks] = __builtin_bit_cast(bf16x8, (uint4){w[0], w[1], w[2], w[3]});
  }
  l += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
}

// S^T = K Q^T for every sub-block: s[sb][kb] covers keys 32kb .. 32kb+31 of the tile, query column li of sub-block sb.
// kbase points at K row li, column 32g of the tile. Each K operand read feeds all sub-blocks.
template <int NSB>
__device__ __forceinline__ void s_mfma(f32x16 (&s)[NSB][2], const bf16x8 (&qf)[NSB][4], const uint16_t* kbase) {
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) s[sb][0] = s[sb][1] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kbase + kb * 32 * kKS + 8 * ks);
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) s[sb][kb] = mfma32x32x16(ka, qf[sb][ks], s[sb][kb]);
    }
  }
}

// O^T += V^T P^T for every sub-block. k-step ks pairs P registers 8(ks%2) .. +7 of key block ks/2 with keys
// 16ks + 4g + (0..3) and 16ks + 8 + 4g + (0..3); vbase0/vbase1 are this lane's transpose-read sources for those two
// groups of rows (row 4g + (lane%16)/4, +8).
template <int NSB>
__device__ __forceinline__ void pv_mfma(f32x16 (&o)[NSB][2], const bf16x8 (&pf)[NSB][4], const uint16_t* vbase0,
                                        const uint16_t* vbase1) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const bf16x4 lo = lds_read_tr16x4(vbase0 + ks * 16 * kVS + 32 * mb);
      const bf16x4 hi = lds_read_tr16x4(vbase1 + ks * 16 * kVS + 32 * mb);
      const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) o[sb][mb] = mfma32x32x16(va, pf[sb][ks], o[sb][mb]);
    }
  }
}

// Make this wave's LDS stores visible to the workgroup and wait for every wave. Unlike __syncthreads() it does not
// wait for outstanding global loads, so register prefetches stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Store the O^T accumulators of one sub-block, divided by the row sum, as bf16 row q of the output.
__device__ __forceinline__ void store_rows(uint16_t* Op, int64_t o_stride_row, const f32x16 (&o)[2], float l, int q,
                                           int n_q, int g) {
  const float inv = 1.0f / sum_with_partner32(l);
  if (q >= n_q) return;
  uint16_t* orow = Op + (int64_t)q * o_stride_row;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const uint2 w = {pack_bf16x2(o[mb][4 * rg] * inv, o[mb][4 * rg + 1] * inv),
                       pack_bf16x2(o[mb][4 * rg + 2] * inv, o[mb][4 * rg + 3] * inv)};
      *reinterpret_cast<uint2*>(orow + 32 * mb + 8 * rg + 4 * g) = w;
    }
  }
}

// NSB: 32-query sub-blocks per wave; NW: waves per workgroup; MINB: workgroups per CU the register budget targets.
template <int NSB, int NW, int MINB>
__global__ __launch_bounds__(64 * NW, MINB) void attn_fwd_bf16_d64(AttnArgs a, int n_qblocks) {
  constexpr int kT = 64 * NW;          // threads
  constexpr int kBM = 32 * NSB * NW;   // queries per workgroup
  constexpr int kCH = 1024 / kT;       // 16-byte chunks of the K+V tile each thread stages
  static_assert(1024 % kT == 0, "tile staging assumes 1024 chunks divide evenly");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kBufElems];  // [buffer][K tile | V tile]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, li = lane & 31;
  const int n_q = a.n_q, n_k = a.n_k;
  const bool causal = a.causal != 0;
  const float c = kScaleLog2;

  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  int qb = blk % n_qblocks;
  const int bh = blk / n_qblocks;
  if (causal) qb = n_qblocks - 1 - qb;  // heaviest query blocks first
  const int b = bh / a.H, hh = bh % a.H;
  const uint16_t* Qp = static_cast<const uint16_t*>(a.Q) + (int64_t)bh * a.q_stride_bh;
  const uint16_t* Kp = static_cast<const uint16_t*>(a.K) + (int64_t)bh * a.k_stride_bh;
  const uint16_t* Vp = static_cast<const uint16_t*>(a.V) + (int64_t)bh * a.k_stride_bh;
  uint16_t* Op = static_cast<uint16_t*>(a.O) + b * a.o_stride_b + hh * a.o_stride_h;

  const int q_blk0 = qb * kBM;
  const int qw0 = q_blk0 + wave * 32 * NSB;  // first query of this wave

  // Q as the B operand of S^T = K Q^T: lane supplies Q[q][32g + 8ks + j], ks = 0..3 (the same d permutation as the
  // K operand). Rows at or past n_q are zero.
  bf16x8 qf[NSB][4];
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) {
    const int q = qw0 + 32 * sb + li;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[sb][ks] = q < n_q ? *reinterpret_cast<const bf16x8*>(Qp + (int64_t)q * kD + 32 * g + 8 * ks) : bf16x8{};
  }

  int nt = (n_k + kBN - 1) / kBN;
  if (causal) nt = min(nt, (q_blk0 + kBM - 1) / kBN + 1);
  // tiles before t_mask need no mask for this wave; tiles from t_skip on lie entirely in this wave's future
  const int t_mask = min(causal ? qw0 / kBN : nt, n_k / kBN);
  const int t_skip = causal ? (qw0 + 32 * NSB - 1) / kBN + 1 : nt;

  // Cooperative tile staging: 16-byte chunk id = tid + kT*i of the K (ids 0..511) and V (512..1023) tiles, row
  // (id%512)/8, columns 8*(id%8). Rows at or past n_k load as zeros.
  uint4 rr[kCH];
  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < kCH; ++i) {
      const int id = tid + kT * i, row = t * kBN + ((id & 511) >> 3), col = (id & 7) * 8;
      const uint16_t* src = (id >> 9) ? Vp : Kp;
      rr[i] = row < n_k ? *reinterpret_cast<const uint4*>(src + (int64_t)row * kD + col) : (uint4){0u, 0u, 0u, 0u};
    }
  };
  auto lds_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kCH; ++i) {
      const int id = tid + kT * i, row = (id & 511) >> 3, col = (id & 7) * 8;
      uint16_t* dst = smem + buf * kBufElems + ((id >> 9) ? kKElems + row * kVS : row * kKS) + col;
      *reinterpret_cast<uint4*>(dst) = rr[i];
    }
  };

  WaveState<NSB> st;
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) {
    st.o[sb][0] = st.o[sb][1] = f32x16{};
    st.m[sb] = -INFINITY;
    st.l[sb] = 0.f;
  }

  // per-lane LDS offsets: K operand row li, columns 32g + 8ks; V transpose-read source row 4g + (lane%16)/4 (+8),
  // column 16*((lane/16)%2) + 4*(lane%4)
  const int koff = li * kKS + 32 * g;
  const int vrow = 4 * g + ((lane & 15) >> 2);
  const int voff0 = kKElems + vrow * kVS + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int voff1 = voff0 + 8 * kVS;

  gload(0);
  lds_store(0);
  if (nt > 1) gload(1);
  lds_barrier();
  for (int t = 0; t < nt; ++t) {
    const uint16_t* base = smem + (t & 1) * kBufElems;
    if (t < t_skip) {
      f32x16 s[NSB][2];
      bf16x8 pf[NSB][4];
      s_mfma<NSB>(s, qf, base + koff);
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const int q = qw0 + 32 * sb + li;
        if (t < t_mask)
          softmax_rows<false>(s[sb], st.o[sb][0], st.o[sb][1], st.m[sb], st.l[sb], pf[sb], c, t * kBN, q, g, n_k,
                              causal);
        else
          softmax_rows<true>(s[sb], st.o[sb][0], st.o[sb][1], st.m[sb], st.l[sb], pf[sb], c, t * kBN, q, g, n_k,
                             causal);
      }
      pv_mfma<NSB>(st.o, pf, base + voff0, base + voff1);
    }
    // tile t+1 goes into the other buffer: every wave finished reading it (tile t-1) before the last barrier
    if (t + 1 < nt) {
      lds_store((t + 1) & 1);
      if (t + 2 < nt) gload(t + 2);
    }
    lds_barrier();
  }

  // O = O^T / l; lane holds d = 32mb + 8(r/4) + 4g + r%4 of its query in each sub-block.
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) store_rows(Op, a.o_stride_row, st.o[sb], st.l[sb], qw0 + 32 * sb + li, n_q, g);
}

template <int NSB, int NW, int MINB>
hipError_t launch_cfg(const AttnArgs& a, hipStream_t stream) {
  constexpr int kBM = 32 * NSB * NW;
  const int n_qblocks = (a.n_q + kBM - 1) / kBM;
  const int64_t nblocks = (int64_t)n_qblocks * a.B * a.H;
  if (nblocks <= 0 || nblocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_fwd_bf16_d64<NSB, NW, MINB>), dim3((unsigned)nblocks), dim3(64 * NW), 0, stream, a,
                     n_qblocks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------------------------
// Software-pipelined variant (one 32-query sub-block per wave): while a wave runs the exponentials of tile t it also
// issues the MFMAs of S^T for tile t+1 and of O^T += V^T P^T for tile t, interleaved instruction by instruction, so
// its own matrix-core work overlaps its own VALU work (and other waves on the SIMD fill what remains). K tiles are
// staged one tile ahead of V tiles, so two buffers of each suffice with one barrier per tile.

// First half of the softmax for one tile: masking, the row max and the (rare) offset raise. Returns the offset.
template <bool kMasked>
__device__ __forceinline__ float softmax_max(f32x16 (&s)[2], f32x16& o0, f32x16& o1, float& m, float& l, float c,
                                             int k0, int q, int g, int n_k, bool causal) {
  if (kMasked) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
        if (key >= n_k || (causal && key > q)) s[kb][r] = -INFINITY;
      }
  }
  float mx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) mx[j] = fmaxf(fmaxf(s[0][4 * j], s[0][4 * j + 1]), s[0][4 * j + 2]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    mx[j] = fmaxf(fmaxf(mx[j], s[0][4 * j + 3]), s[1][4 * j]);
    mx[j] = fmaxf(fmaxf(mx[j], s[1][4 * j + 1]), s[1][4 * j + 2]);
    mx[j] = fmaxf(mx[j], s[1][4 * j + 3]);
  }
  float rmax = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
  rmax = max_with_partner32(rmax) * c;
  const bool need = rmax > m + kRescaleThreshold;  // per row; implies rmax finite
  if (__builtin_amdgcn_ballot_w64(need)) {
    const float alpha = need ? fast_exp2(m - rmax) : 1.f;
    m = need ? rmax : m;
    l *= alpha;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      o0[r] *= alpha;
      o1[r] *= alpha;
    }
  }
  return (kMasked && m == -INFINITY) ? 0.f : m;
}

// Operands of one pipelined tile step, read from LDS at the start of the step so that their ~150-cycle latency is
// hidden behind the row-max reduction: K(t+1) for S^T(t+1) and V(t)^T for the PV product of tile t.
struct StepOperands {
  bf16x8 k[4][2];  // [ks][kb]
  bf16x8 v[4][2];  // [ks][mb]
};

__device__ __forceinline__ void read_operands(StepOperands& op, const uint16_t* kbase, const uint16_t* vbase0,
                                              const uint16_t* vbase1) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) op.k[ks][kb] = *reinterpret_cast<const bf16x8*>(kbase + kb * 32 * kKS + 8 * ks);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const bf16x4 lo = lds_read_tr16x4(vbase0 + ks * 16 * kVS + 32 * mb);
      const bf16x4 hi = lds_read_tr16x4(vbase1 + ks * 16 * kVS + 32 * mb);
      op.v[ks][mb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

// Exponentials of tile t interleaved with S^T(t+1) = K(t+1) Q^T and O^T += V(t)^T P(t)^T (operands in registers).
__device__ __forceinline__ void pipe_exp_mfma(const f32x16 (&s_cur)[2], f32x16 (&s_next)[2], f32x16 (&o)[2],
                                              float& l, const bf16x8 (&qf)[4], const StepOperands& op, float c,
                                              float m_use) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float lsum[4] = {0.f, 0.f, 0.f, 0.f};
  bf16x8 pf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const f32x16& sk = s_cur[ks >> 1];
    const int base = 8 * (ks & 1);
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p0 = fast_exp2(fmaf(sk[base + 2 * j], c, -m_use));
      const float p1 = fast_exp2(fmaf(sk[base + 2 * j + 1], c, -m_use));
      w[j] = pack_bf16x2(p0, p1);
      lsum[j] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[j]), ones, lsum[j], false);
    }
    pf[ks] = __builtin_bit_cast(bf16x8, (uint4){w[0], w[1], w[2], w[3]});
  }
  s_next[0] = s_next[1] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s_next[kb] = mfma32x32x16(op.k[ks][kb], qf[ks], s_next[kb]);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) o[mb] = mfma32x32x16(op.v[ks][mb], pf[ks], o[mb]);
  l += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
  // one MFMA, then a share of the VALU work, sixteen times
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);  // VALU
  }
}

template <int NW, int MINB>
__global__ __launch_bounds__(64 * NW, MINB) void attn_fwd_bf16_d64_pipe(AttnArgs a, int n_qblocks) {
  constexpr int kT = 64 * NW;         // threads
  constexpr int kBM = 32 * NW;        // queries per workgroup
  constexpr int kCH = 512 / kT;       // 16-byte chunks of a K (or V) tile each thread stages
  static_assert(512 % kT == 0, "tile staging assumes 512 chunks divide evenly");
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * kKElems + 2 * kVElems];  // K[2] | V[2]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, li = lane & 31;
  const int n_q = a.n_q, n_k = a.n_k;
  const bool causal = a.causal != 0;
  const float c = kScaleLog2;

  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  int qb = blk % n_qblocks;
  const int bh = blk / n_qblocks;
  if (causal) qb = n_qblocks - 1 - qb;
  const int b = bh / a.H, hh = bh % a.H;
  const uint16_t* Qp = static_cast<const uint16_t*>(a.Q) + (int64_t)bh * a.q_stride_bh;
  const uint16_t* Kp = static_cast<const uint16_t*>(a.K) + (int64_t)bh * a.k_stride_bh;
  const uint16_t* Vp = static_cast<const uint16_t*>(a.V) + (int64_t)bh * a.k_stride_bh;
  uint16_t* Op = static_cast<uint16_t*>(a.O) + b * a.o_stride_b + hh * a.o_stride_h;

  const int q_blk0 = qb * kBM;
  const int qw0 = q_blk0 + wave * 32;
  const int q = qw0 + li;
  bf16x8 qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qf[ks] = q < n_q ? *reinterpret_cast<const bf16x8*>(Qp + (int64_t)q * kD + 32 * g + 8 * ks) : bf16x8{};

  int nt = (n_k + kBN - 1) / kBN;
  if (causal) nt = min(nt, (q_blk0 + kBM - 1) / kBN + 1);
  const int t_mask = min(causal ? qw0 / kBN : nt, n_k / kBN);
  const int t_skip = causal ? (qw0 + 31) / kBN + 1 : nt;

  // staging: chunk id = tid + kT*i of a tile, row id/8, columns 8*(id%8); rows at or past n_k load as zeros
  uint4 kr[kCH], vr[kCH];
  auto gload = [&](uint4 (&r)[kCH], const uint16_t* src, int t) {
#pragma unroll
    for (int i = 0; i < kCH; ++i) {
      const int id = tid + kT * i, row = t * kBN + (id >> 3), col = (id & 7) * 8;
      r[i] = row < n_k ? *reinterpret_cast<const uint4*>(src + (int64_t)row * kD + col) : (uint4){0u, 0u, 0u, 0u};
    }
  };
  auto kstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kCH; ++i) {
      const int id = tid + kT * i;
      *reinterpret_cast<uint4*>(smem + buf * kKElems + (id >> 3) * kKS + (id & 7) * 8) = kr[i];
    }
  };
  auto vstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kCH; ++i) {
      const int id = tid + kT * i;
      *reinterpret_cast<uint4*>(smem + 2 * kKElems + buf * kVElems + (id >> 3) * kVS + (id & 7) * 8) = vr[i];
    }
  };

  WaveState<1> st;
  st.o[0][0] = st.o[0][1] = f32x16{};
  st.m[0] = -INFINITY;
  st.l[0] = 0.f;

  const int koff = li * kKS + 32 * g;
  const int vrow = 4 * g + ((lane & 15) >> 2);
  const int voff0 = 2 * kKElems + vrow * kVS + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int voff1 = voff0 + 8 * kVS;

  // prologue: K(0), K(1), V(0) in LDS; K(2), V(1) prefetched; S(0) computed
  gload(kr, Kp, 0);
  kstore(0);
  gload(kr, Kp, 1);
  kstore(1);
  gload(vr, Vp, 0);
  vstore(0);
  gload(kr, Kp, 2);
  gload(vr, Vp, 1);
  lds_barrier();
  f32x16 sA[2], sB[2];
  sA[0] = sA[1] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      sA[kb] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(smem + koff + kb * 32 * kKS + 8 * ks), qf[ks], sA[kb]);
  lds_barrier();

  auto tile = [&](f32x16 (&s_cur)[2], f32x16 (&s_next)[2], int t) {
    if (t < t_skip) {
      const uint16_t* vb = smem + 2 * kKElems + (t & 1) * kVElems - 2 * kKElems;
      StepOperands op;
      read_operands(op, smem + ((t + 1) & 1) * kKElems + koff, vb + voff0, vb + voff1);
      const float m_use = (t < t_mask)
          ? softmax_max<false>(s_cur, st.o[0][0], st.o[0][1], st.m[0], st.l[0], c, t * kBN, q, g, n_k, causal)
          : softmax_max<true>(s_cur, st.o[0][0], st.o[0][1], st.m[0], st.l[0], c, t * kBN, q, g, n_k, causal);
      pipe_exp_mfma(s_cur, s_next, st.o[0], st.l[0], qf, op, c, m_use);
    }
    // stage K(t+2) into the K buffer tile t used, V(t+1) into the V buffer tile t-1 used; prefetch the next ones
    if (t + 2 < nt) kstore(t & 1);
    if (t + 1 < nt) vstore((t + 1) & 1);
    if (t + 3 < nt) gload(kr, Kp, t + 3);
    if (t + 2 < nt) gload(vr, Vp, t + 2);
    lds_barrier();
  };
  for (int t = 0; t < nt; t += 2) {
    tile(sA, sB, t);
    if (t + 1 < nt) tile(sB, sA, t + 1);
  }

  store_rows(Op, a.o_stride_row, st.o[0], st.l[0], q, n_q, g);
}

template <int NW, int MINB>
hipError_t launch_pipe(const AttnArgs& a, hipStream_t stream) {
  constexpr int kBM = 32 * NW;
  const int n_qblocks = (a.n_q + kBM - 1) / kBM;
  const int64_t nblocks = (int64_t)n_qblocks * a.B * a.H;
  if (nblocks <= 0 || nblocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_fwd_bf16_d64_pipe<NW, MINB>), dim3((unsigned)nblocks), dim3(64 * NW), 0, stream, a,
                     n_qblocks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------------------------
// Complementary-schedule variant: 8 waves; waves w and w+4 share a SIMD. Between two barriers, waves 0..3 run
// S^T(t) -> softmax(t) -> PV(t) while waves 4..7 run softmax(t) -> PV(t) -> S^T(t+1) (their S^T(t) was computed in the
// previous interval), so while one wave of a SIMD is on the matrix core the other is mostly on the VALU. K tiles are
// staged one tile ahead of V tiles (three K buffers, two V buffers).
template <int NSB, int MINB>
__global__ __launch_bounds__(512, MINB) void attn_fwd_bf16_d64_ab(AttnArgs a, int n_qblocks) {
  constexpr int NW = 8;
  constexpr int kT = 64 * NW;
  constexpr int kBM = 32 * NSB * NW;
  __shared__ __attribute__((aligned(16))) uint16_t smem[3 * kKElems + 2 * kVElems];  // K[3] | V[2]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, li = lane & 31;
  const bool late = wave >= 4;  // schedule B
  const int n_q = a.n_q, n_k = a.n_k;
  const bool causal = a.causal != 0;
  const float c = kScaleLog2;

  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  int qb = blk % n_qblocks;
  const int bh = blk / n_qblocks;
  if (causal) qb = n_qblocks - 1 - qb;
  const int b = bh / a.H, hh = bh % a.H;
  const uint16_t* Qp = static_cast<const uint16_t*>(a.Q) + (int64_t)bh * a.q_stride_bh;
  const uint16_t* Kp = static_cast<const uint16_t*>(a.K) + (int64_t)bh * a.k_stride_bh;
  const uint16_t* Vp = static_cast<const uint16_t*>(a.V) + (int64_t)bh * a.k_stride_bh;
  uint16_t* Op = static_cast<uint16_t*>(a.O) + b * a.o_stride_b + hh * a.o_stride_h;

  const int q_blk0 = qb * kBM;
  // interleave the query chunks of the two schedules so both reach the causal diagonal together
  const int chunk = 2 * (wave & 3) + (late ? 1 : 0);
  const int qw0 = q_blk0 + chunk * 32 * NSB;
  bf16x8 qf[NSB][4];
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) {
    const int q = qw0 + 32 * sb + li;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[sb][ks] = q < n_q ? *reinterpret_cast<const bf16x8*>(Qp + (int64_t)q * kD + 32 * g + 8 * ks) : bf16x8{};
  }

  int nt = (n_k + kBN - 1) / kBN;
  if (causal) nt = min(nt, (q_blk0 + kBM - 1) / kBN + 1);
  const int t_mask = min(causal ? qw0 / kBN : nt, n_k / kBN);
  const int t_skip = causal ? (qw0 + 32 * NSB - 1) / kBN + 1 : nt;

  // staging: one 16-byte chunk of a K tile and one of a V tile per thread (row tid/8, columns 8*(tid%8))
  uint4 kr, vr;
  const int srow = tid >> 3, scol = (tid & 7) * 8;
  auto kload = [&](int t) {
    const int row = t * kBN + srow;
    kr = row < n_k ? *reinterpret_cast<const uint4*>(Kp + (int64_t)row * kD + scol) : (uint4){0u, 0u, 0u, 0u};
  };
  auto vload = [&](int t) {
    const int row = t * kBN + srow;
    vr = row < n_k ? *reinterpret_cast<const uint4*>(Vp + (int64_t)row * kD + scol) : (uint4){0u, 0u, 0u, 0u};
  };
  auto kstore = [&](int t) { *reinterpret_cast<uint4*>(smem + (t % 3) * kKElems + srow * kKS + scol) = kr; };
  auto vstore = [&](int t) {
    *reinterpret_cast<uint4*>(smem + 3 * kKElems + (t & 1) * kVElems + srow * kVS + scol) = vr;
  };

  WaveState<NSB> st;
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) {
    st.o[sb][0] = st.o[sb][1] = f32x16{};
    st.m[sb] = -INFINITY;
    st.l[sb] = 0.f;
  }
  const int koff = li * kKS + 32 * g;
  const int vrow = 4 * g + ((lane & 15) >> 2);
  const int voff0 = 3 * kKElems + vrow * kVS + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int voff1 = voff0 + 8 * kVS;

  // prologue: K(0), K(1), V(0) in LDS; K(2), V(1) prefetched; schedule-B waves compute S^T(0)
  kload(0);
  kstore(0);
  kload(1);
  kstore(1);
  vload(0);
  vstore(0);
  kload(2);
  vload(1);
  lds_barrier();
  f32x16 s[NSB][2];
  if (late) s_mfma<NSB>(s, qf, smem + koff);

  for (int t = 0; t < nt; ++t) {
    if (t < t_skip) {
      if (!late) s_mfma<NSB>(s, qf, smem + (t % 3) * kKElems + koff);
      bf16x8 pf[NSB][4];
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const int q = qw0 + 32 * sb + li;
        if (t < t_mask)
          softmax_rows<false>(s[sb], st.o[sb][0], st.o[sb][1], st.m[sb], st.l[sb], pf[sb], c, t * kBN, q, g, n_k,
                              causal);
        else
          softmax_rows<true>(s[sb], st.o[sb][0], st.o[sb][1], st.m[sb], st.l[sb], pf[sb], c, t * kBN, q, g, n_k,
                             causal);
      }
      const uint16_t* vb = smem + (t & 1) * kVElems;
      pv_mfma<NSB>(st.o, pf, vb + voff0, vb + voff1);
      if (late && t + 1 < t_skip) s_mfma<NSB>(s, qf, smem + ((t + 1) % 3) * kKElems + koff);
    }
    // stage K(t+2) (its buffer last held K(t-1)) and V(t+1) (buffer of V(t-1)); prefetch K(t+3), V(t+2)
    if (t + 2 < nt) kstore(t + 2);
    if (t + 1 < nt) vstore(t + 1);
    if (t + 3 < nt) kload(t + 3);
    if (t + 2 < nt) vload(t + 2);
    lds_barrier();
  }

#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) store_rows(Op, a.o_stride_row, st.o[sb], st.l[sb], qw0 + 32 * sb + li, n_q, g);
}

template <int NSB, int MINB>
hipError_t launch_ab(const AttnArgs& a, hipStream_t stream) {
  constexpr int kBM = 32 * NSB * 8;
  const int n_qblocks = (a.n_q + kBM - 1) / kBM;
  const int64_t nblocks = (int64_t)n_qblocks * a.B * a.H;
  if (nblocks <= 0 || nblocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_fwd_bf16_d64_ab<NSB, MINB>), dim3((unsigned)nblocks), dim3(512), 0, stream, a, n_qblocks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------------------------
// Asynchronous-staging variant: K/V tiles go global -> LDS directly with global_load_lds_dwordx4 (no staging
// registers, no LDS store instructions) into a STAGES-deep ring, so a tile's loads have STAGES-1 tiles of compute to
// land. Those loads write each wave's 64 x 16 bytes contiguously, so rows are unpadded (128 B) and the 16-byte chunk c
// of row r is stored at chunk c ^ swz(r): with swz below, the K operand row reads and the V transpose reads hit
// distinct LDS banks (checked for 32 and for 64 banks).

// Chunk swizzle of row r (depends on r mod 16).
__device__ __forceinline__ int swz(int r) { return (2 * (r & 3) + ((r >> 2) & 1)) ^ ((r >> 2) & 2); }

constexpr int kTileElemsU = kBN * kD;  // unpadded 64 x 64 tile

template <int NSB>
__device__ __forceinline__ void s_mfma_swz(f32x16 (&s)[NSB][2], const bf16x8 (&qf)[NSB][4], const uint16_t* ktile,
                                           const int (&koff)[4]) {
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) s[sb][0] = s[sb][1] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(ktile + kb * 32 * kD + koff[ks]);
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) s[sb][kb] = mfma32x32x16(ka, qf[sb][ks], s[sb][kb]);
    }
  }
}

template <int NSB>
__device__ __forceinline__ void pv_mfma_swz(f32x16 (&o)[NSB][2], const bf16x8 (&pf)[NSB][4], const uint16_t* vtile,
                                            const int (&voff)[2][2]) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const bf16x4 lo = lds_read_tr16x4(vtile + ks * 16 * kD + voff[mb][0]);
      const bf16x4 hi = lds_read_tr16x4(vtile + ks * 16 * kD + voff[mb][1]);
      const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) o[sb][mb] = mfma32x32x16(va, pf[sb][ks], o[sb][mb]);
    }
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int NSB, int NW, int MINB, int STAGES>
__global__ __launch_bounds__(64 * NW, MINB) void attn_fwd_bf16_d64_async(AttnArgs a, int n_qblocks) {
  constexpr int kBM = 32 * NSB * NW;
  constexpr int kLPW = 16 / NW;  // 1 KB load instructions per wave per tile (16 per K+V tile)
  static_assert(16 % NW == 0, "tile loads split evenly over the waves");
  __shared__ __attribute__((aligned(16))) uint16_t smem[STAGES * 2 * kTileElemsU];  // [stage][K | V]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, li = lane & 31;
  const int n_q = a.n_q, n_k = a.n_k;
  const bool causal = a.causal != 0;
  const float c = kScaleLog2;

  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  int qb = blk % n_qblocks;
  const int bh = blk / n_qblocks;
  if (causal) qb = n_qblocks - 1 - qb;
  const int b = bh / a.H, hh = bh % a.H;
  const uint16_t* Qp = static_cast<const uint16_t*>(a.Q) + (int64_t)bh * a.q_stride_bh;
  const uint16_t* Kp = static_cast<const uint16_t*>(a.K) + (int64_t)bh * a.k_stride_bh;
  const uint16_t* Vp = static_cast<const uint16_t*>(a.V) + (int64_t)bh * a.k_stride_bh;
  uint16_t* Op = static_cast<uint16_t*>(a.O) + b * a.o_stride_b + hh * a.o_stride_h;

  const int q_blk0 = qb * kBM;
  const int qw0 = q_blk0 + wave * 32 * NSB;
  bf16x8 qf[NSB][4];
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) {
    const int q = qw0 + 32 * sb + li;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qf[sb][ks] = q < n_q ? *reinterpret_cast<const bf16x8*>(Qp + (int64_t)q * kD + 32 * g + 8 * ks) : bf16x8{};
  }

  int nt = (n_k + kBN - 1) / kBN;
  if (causal) nt = min(nt, (q_blk0 + kBM - 1) / kBN + 1);
  const int t_mask = min(causal ? qw0 / kBN : nt, n_k / kBN);
  const int t_skip = causal ? (qw0 + 32 * NSB - 1) / kBN + 1 : nt;

  // Tile loads: wave instruction gi (0..15) of a tile moves rows 8*(gi%8) .. +7 of K (gi < 8) or V; lane l brings the
  // logical chunk that belongs at physical chunk l%8 of row 8*(gi%8) + l/8. Rows past n_k read row n_k-1 (their
  // scores are masked and their weights are zero).
  const int lrow = lane >> 3;
  auto issue_tile = [&](int t) {
    uint16_t* stage = smem + (t % STAGES) * 2 * kTileElemsU;
#pragma unroll
    for (int i = 0; i < kLPW; ++i) {
      const int gi = wave * kLPW + i;
      const int row = 8 * (gi & 7) + lrow;
      const int lc = (lane & 7) ^ swz(row);
      const int grow = min(t * kBN + row, n_k - 1);
      const uint16_t* src = (gi < 8 ? Kp : Vp) + (int64_t)grow * kD + lc * 8;
      uint16_t* dst = stage + (gi < 8 ? 0 : kTileElemsU) + 8 * (gi & 7) * kD;
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                       (void __attribute__((address_space(3)))*)dst, 16, 0, 0);
    }
  };

  WaveState<NSB> st;
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) {
    st.o[sb][0] = st.o[sb][1] = f32x16{};
    st.m[sb] = -INFINITY;
    st.l[sb] = 0.f;
  }

  // per-lane swizzled offsets: K operand row li, logical chunk 4g+ks; V transpose-read row 4g + (lane%16)/4 (+8 for
  // the second half), logical chunk 4mb + 2*((lane/16)%2) + (lane%4)/2, element 4*(lane%2) of the chunk
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
      voff[mb][hi] = kTileElemsU + row * kD + ((lchunk ^ swz(row)) << 3) + 4 * (lane & 1);
    }

#pragma unroll
  for (int t = 0; t < STAGES - 1; ++t) issue_tile(t);
  for (int t = 0; t < nt; ++t) {
    wait_vmcnt<(STAGES - 2) * kLPW>();  // this wave's loads of tile t have landed
    lds_barrier();                      // everyone's have; everyone is done with tile t-1's stage
    issue_tile(t + STAGES - 1);         // reuses the stage of tile t-1 (rows clamp past n_k)
    if (t < t_skip) {
      const uint16_t* stage = smem + (t % STAGES) * 2 * kTileElemsU;
      f32x16 s[NSB][2];
      bf16x8 pf[NSB][4];
      s_mfma_swz<NSB>(s, qf, stage, koff);
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const int q = qw0 + 32 * sb + li;
        if (t < t_mask)
          softmax_rows<false>(s[sb], st.o[sb][0], st.o[sb][1], st.m[sb], st.l[sb], pf[sb], c, t * kBN, q, g, n_k,
                              causal);
        else
          softmax_rows<true>(s[sb], st.o[sb][0], st.o[sb][1], st.m[sb], st.l[sb], pf[sb], c, t * kBN, q, g, n_k,
                             causal);
      }
      pv_mfma_swz<NSB>(st.o, pf, stage, voff);
    }
  }
  wait_vmcnt<0>();  // drain the trailing (unused) tile loads before the workgroup's LDS goes away

#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) store_rows(Op, a.o_stride_row, st.o[sb], st.l[sb], qw0 + 32 * sb + li, n_q, g);
}

template <int NSB, int NW, int MINB, int STAGES>
hipError_t launch_async(const AttnArgs& a, hipStream_t stream) {
  constexpr int kBM = 32 * NSB * NW;
  const int n_qblocks = (a.n_q + kBM - 1) / kBM;
  const int64_t nblocks = (int64_t)n_qblocks * a.B * a.H;
  if (nblocks <= 0 || nblocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_fwd_bf16_d64_async<NSB, NW, MINB, STAGES>), dim3((unsigned)nblocks), dim3(64 * NW), 0,
                     stream, a, n_qblocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, hipStream_t stream) {
  // Block shape by query length: long unmasked ranges use 8 waves x 64 queries (each K/V operand read feeds two
  // sub-blocks); otherwise 32 queries per wave, with 4-wave blocks when that gives better balance (short or causal).
  if (!a.causal && a.n_q >= 2048) return launch_async<2, 8, 1, 4>(a, stream);
  if (!a.causal && a.n_q >= 512) return launch_async<1, 8, 1, 4>(a, stream);
  return launch_async<1, 4, 2, 4>(a, stream);
}

}  // namespace mi355
