// Fused scaled dot-product attention forward, bf16 in/out, d_k = d_v = 64, for gfx950 (MI355X).
//
// Computes, for every (batch, head) and query i:  O_i = sum_j softmax_j(Q_i . K_j / sqrt(64)) V_j, with the optional
// causal mask (keys j > i get score -inf, i.e. weight 0). Definition: "Attention Is All You Need" (lettle.cn
// translation), section 3.2.1, equation Attention(Q,K,V); mask: "Transformer：抛弃循环与卷积的序列建模"
// (jiashun-ye.github.io), section "Transformer 中的三种 Attention".
//
// Design (one workgroup = 4 waves = 128 queries of one head; keys streamed in tiles of 64):
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: queries sit in the lane index
//    (lane l and l+32 both own query l%32), keys in the accumulator registers. The row softmax then reduces over
//    registers plus one v_permlane32_swap, and the fp32 accumulator packed to bf16 is directly the B operand of the
//    second product O^T = V^T P^T: the n x n score matrix never leaves registers.
//  * K rows are fed to the first MFMA in a permuted order (bits 2 and 3 of the row index swapped) so that the 8 keys
//    a lane contributes per PV k-step are contiguous; the V^T operand is then one 16-byte LDS read.
//  * K is staged in LDS row-major, V transposed (V^T[d][key]) so both operands are 16-byte LDS reads. Global loads are
//    16-byte, coalesced, prefetched into registers one tile ahead.
//  * Online softmax in the exp2 domain: p = exp2(s*c - m) with c = log2(e)/sqrt(64); m is the running row max of s*c,
//    l the running sum of the bf16-rounded p (the same values that multiply V), O rescaled by exp2(m_old - m_new).
//  * Causal: key tiles entirely after a wave's last query are skipped; only diagonal tiles pay for the compare.
//    Query blocks run heaviest first.
#include "device_common.h"
#include "launch.h"

#include <math.h>

namespace mi355 {
namespace {

constexpr int kD = 64;          // head width
constexpr int kBM = 128;        // queries per workgroup (4 waves x 32)
constexpr int kBN = 64;         // keys per tile
constexpr int kLds = 72;        // LDS row stride in bf16 elements (64 + 8 padding: 144 B, 16-B aligned rows)
constexpr int kThreads = 256;

// Row of the K tile that feeds MFMA row i: swap bits 2 and 3 (an involution on 0..31).
__device__ __forceinline__ int key_perm(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

__global__ __launch_bounds__(kThreads) void attn_fwd_bf16_d64(AttnArgs a, int n_qblocks, float c) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBN * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kD * kLds];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, li = lane & 31;

  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  int qb = blk % n_qblocks;
  const int bh = blk / n_qblocks;
  if (a.causal) qb = n_qblocks - 1 - qb;  // heaviest query blocks first
  const int b = bh / a.H, hh = bh % a.H;
  const int n_q = a.n_q, n_k = a.n_k;

  const uint16_t* Qp = static_cast<const uint16_t*>(a.Q) + (int64_t)bh * a.q_stride_bh;
  const uint16_t* Kp = static_cast<const uint16_t*>(a.K) + (int64_t)bh * a.k_stride_bh;
  const uint16_t* Vp = static_cast<const uint16_t*>(a.V) + (int64_t)bh * a.k_stride_bh;
  uint16_t* Op = static_cast<uint16_t*>(a.O) + b * a.o_stride_b + hh * a.o_stride_h;

  const int q_blk0 = qb * kBM;
  const int qw0 = q_blk0 + wave * 32;  // first query of this wave
  const int qi = qw0 + li;             // this lane's query

  // Q as the B operand of S^T = K Q^T: lane supplies Q[qi][32g + 8ks + j], ks = 0..3 (a fixed d permutation that the
  // K operand below uses as well).
  bf16x8 qf[4];
  if (qi < n_q) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(Qp + (int64_t)qi * kD + 32 * g + 8 * ks);
  } else {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = bf16x8{};
  }

  int nt = (n_k + kBN - 1) / kBN;
  if (a.causal) nt = min(nt, (q_blk0 + kBM - 1) / kBN + 1);

  // Cooperative tile loader: K chunks (row tid/8 and 32 + tid/8, 8 columns at 8*(tid%8)); V rows 2*(tid/8) and
  // 2*(tid/8)+1, same 8 columns. Rows at or past n_k load as zeros.
  const int lr = tid >> 3, lc = (tid & 7) * 8;
  uint4 kr0, kr1, vr0, vr1;
  auto gload = [&](int t) {
    const int k0 = t * kBN;
    const uint4 z = {0u, 0u, 0u, 0u};
    const int r0 = k0 + lr, r1 = k0 + 32 + lr, v0 = k0 + 2 * lr, v1 = v0 + 1;
    kr0 = r0 < n_k ? *reinterpret_cast<const uint4*>(Kp + (int64_t)r0 * kD + lc) : z;
    kr1 = r1 < n_k ? *reinterpret_cast<const uint4*>(Kp + (int64_t)r1 * kD + lc) : z;
    vr0 = v0 < n_k ? *reinterpret_cast<const uint4*>(Vp + (int64_t)v0 * kD + lc) : z;
    vr1 = v1 < n_k ? *reinterpret_cast<const uint4*>(Vp + (int64_t)v1 * kD + lc) : z;
  };
  auto lds_store = [&]() {
    *reinterpret_cast<uint4*>(&Ks[lr * kLds + lc]) = kr0;
    *reinterpret_cast<uint4*>(&Ks[(32 + lr) * kLds + lc]) = kr1;
    // V^T: dword (V[2lr][lc+e], V[2lr+1][lc+e]) -> Vt[lc+e][2lr .. 2lr+1]
    const uint32_t va[4] = {vr0.x, vr0.y, vr0.z, vr0.w};
    const uint32_t vb[4] = {vr1.x, vr1.y, vr1.z, vr1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t lo = (e & 1) ? (va[e >> 1] >> 16) : (va[e >> 1] & 0xffffu);
      const uint32_t hi = (e & 1) ? (vb[e >> 1] & 0xffff0000u) : (vb[e >> 1] << 16);
      *reinterpret_cast<uint32_t*>(&Vt[(lc + e) * kLds + 2 * lr]) = lo | hi;
    }
  };

  f32x16 o0 = {}, o1 = {};     // O^T accumulators: d rows 0..31 and 32..63, query column li
  float m = -INFINITY;         // running max of s*c for query qi
  float l = 0.f;               // running sum of rounded p over this lane's keys (partner lane holds the rest)

  const uint16_t* krow = &Ks[key_perm(li) * kLds + 32 * g];
  const uint16_t* vrow = &Vt[li * kLds + 8 * g];

  gload(0);
  for (int t = 0; t < nt; ++t) {
    __syncthreads();
    lds_store();
    __syncthreads();
    if (t + 1 < nt) gload(t + 1);

    const int k0 = t * kBN;
    if (a.causal && k0 > qw0 + 31) continue;  // every key of the tile is after every query of this wave

    // S^T (2 blocks of 32 keys) = K Q^T over d = 64 (4 MFMA k-steps)
    f32x16 s0 = {}, s1 = {};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + 8 * ks);
      const bf16x8 kb = *reinterpret_cast<const bf16x8*>(krow + 32 * kLds + 8 * ks);
      s0 = mfma32x32x16(ka, qf[ks], s0);
      s1 = mfma32x32x16(kb, qf[ks], s1);
    }
    // register r of block kb holds key k0 + 32kb + 16(r/8) + 8g + r%8 for query qi
    const bool need_mask = (k0 + kBN > n_k) || (a.causal && k0 + kBN - 1 > qw0);
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 16 * (r >> 3) + 8 * g + (r & 7);
        if (key >= n_k || (a.causal && key > qi)) s0[r] = -INFINITY;
        if (key + 32 >= n_k || (a.causal && key + 32 > qi)) s1[r] = -INFINITY;
      }
    }
    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    mx = max_with_partner32(mx);
    const float m_new = fmaxf(m, mx * c);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    m = m_new;

    // p = exp2(s*c - m), packed to bf16 as the B operand of O^T = V^T P^T; l sums the rounded values.
    bf16x8 pf[4];
    float lsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const f32x16& s = (ks < 2) ? s0 : s1;
      const int base = 8 * (ks & 1);
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = fast_exp2(fmaf(s[base + 2 * j], c, -m_use));
        const float p1 = fast_exp2(fmaf(s[base + 2 * j + 1], c, -m_use));
        w[j] = pack_bf16x2(p0, p1);
        lsum += bf16_bits_to_f32(w[j] & 0xffffu) + bf16_bits_to_f32(w[j] >> 16);
      }
      pf[ks] = __builtin_bit_cast(bf16x8, (uint4){w[0], w[1], w[2], w[3]});
    }
    l = l * alpha + lsum;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      o0[r] *= alpha;
      o1[r] *= alpha;
    }
    // O^T += V^T P^T: k-step ks covers keys 16ks .. 16ks+15; lane supplies V^T[d][16ks + 8g + j]
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 va = *reinterpret_cast<const bf16x8*>(vrow + 16 * ks);
      const bf16x8 vb = *reinterpret_cast<const bf16x8*>(vrow + 32 * kLds + 16 * ks);
      o0 = mfma32x32x16(va, pf[ks], o0);
      o1 = mfma32x32x16(vb, pf[ks], o1);
    }
  }

  // O = O^T / l; lane holds d = 32mb + 8(r/4) + 4g + r%4 of query qi.
  const float inv = 1.0f / sum_with_partner32(l);
  if (qi < n_q) {
    uint16_t* orow = Op + (int64_t)qi * a.o_stride_row;
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d = 8 * rg + 4 * g;
      uint2 w0 = {pack_bf16x2(o0[4 * rg] * inv, o0[4 * rg + 1] * inv),
                  pack_bf16x2(o0[4 * rg + 2] * inv, o0[4 * rg + 3] * inv)};
      uint2 w1 = {pack_bf16x2(o1[4 * rg] * inv, o1[4 * rg + 1] * inv),
                  pack_bf16x2(o1[4 * rg + 2] * inv, o1[4 * rg + 3] * inv)};
      *reinterpret_cast<uint2*>(orow + d) = w0;
      *reinterpret_cast<uint2*>(orow + 32 + d) = w1;
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, hipStream_t stream) {
  const int n_qblocks = (a.n_q + kBM - 1) / kBM;
  const int64_t nblocks = (int64_t)n_qblocks * a.B * a.H;
  if (nblocks <= 0 || nblocks > 0x7fffffff) return hipErrorInvalidValue;
  const float c = (float)(1.4426950408889634 / 8.0);  // log2(e) / sqrt(64)
  hipLaunchKernelGGL(attn_fwd_bf16_d64, dim3((unsigned)nblocks), dim3(kThreads), 0, stream, a, n_qblocks, c);
  return hipGetLastError();
}

}  // namespace mi355
