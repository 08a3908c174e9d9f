// Building blocks shared by the gfx950 bf16 attention kernels: tile geometry, the HBM -> LDS tile copy with its
// swizzle, wait/barrier primitives, the row-sum selector of the matrix-core row sum, and small cross-lane helpers.
#pragma once

#include <stdint.h>

#include <type_traits>
#include <utility>

#include "device_common.h"

namespace mi355 {

constexpr int kD = 64;                      // head width
constexpr int kBN = 64;                     // keys per tile
constexpr int kTileElems = kBN * kD;        // one 64 x 64 bf16 tile (K or V), 8 KB
constexpr float kScaleLog2 = (float)(1.4426950408889634 / 8.0);  // log2(e) / sqrt(64)
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTileSumLimit = 1048576.0f;  // 2^20: largest accepted per-tile row sum of P

// 16-byte chunk swizzle of tile row r (depends on r mod 16): logical chunk c of row r is stored at chunk c ^ swz(r).
__device__ __forceinline__ int swz(int r) { return (2 * (r & 3) + ((r >> 2) & 1)) ^ ((r >> 2) & 2); }

// The same for a tile of rows of D bf16 (D / 8 chunks of 16 bytes; swz_d<64> is swz). LDS serves 16 lanes of a
// 16-byte read (or 32 lanes of an 8-byte read) from 64 four-byte banks, i.e. sixteen 16-byte bank groups; a row of D
// elements starts at group (r * D / 8) mod 16. The swizzle makes both read patterns of the attention kernels hit
// sixteen different groups: the operand reads (sixteen consecutive rows, one logical chunk) and the transpose reads
// (four consecutive rows from a multiple of 4, four consecutive chunks from a multiple of 4). D = 128 (rows of 256
// bytes, all starting at group 0) needs a bijection of r mod 16 whose low two bits follow r mod 4 in the upper two
// bits of the chunk; D = 32 (four rows per 256 bytes) needs only a bijection of r / 4 mod 4.
template <int D>
__device__ __forceinline__ int swz_d(int r) {
  static_assert(D == 32 || D == 64 || D == 128, "head width");
  if constexpr (D == 64) return swz(r);
  else if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
  else return (r >> 2) & 3;
}

// log2(e) / sqrt(D): the exponent scale of a score of two D-wide rows (the division by sqrt(d_k) of the scaled
// dot product, moved into the exponent of base 2)
template <int D>
constexpr float scale_log2() {
  static_assert(D == 32 || D == 64 || D == 128, "head width");
  return D == 64 ? kScaleLog2 : D == 32 ? (float)(1.4426950408889634 / 5.656854249492381)
                                        : (float)(1.4426950408889634 / 11.313708498984761);
}

// Global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4, scalar-base form): lane l reads
// base + voff(l) and its 16 bytes land at LDS byte address lds + 16*l. Issued as inline assembly with m0 (the LDS
// destination) set in the same statement, so that the compiler does not treat later LDS reads as possibly reading
// these bytes (it would then wait for every outstanding global load before the first LDS read of each tile). The
// kernel orders these copies with explicit vmcnt waits and barriers. Nothing else in this kernel uses m0. An LDS-DMA
// load needs one wait state after an SALU write of m0 (the s_nop 0, as the compiler emits for its own copies).
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// This wave's LDS reads are complete, then every wave of the workgroup has arrived. Unlike __syncthreads() it does
// not wait for outstanding global -> LDS copies (their completion is tracked with explicit vmcnt waits).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The Q operands are loaded once, before the tile loop. Passing them through an empty asm statement makes the
// compiler wait for those loads here, once, instead of at their first use inside the loop, where (not knowing about
// the asm-issued tile copies) it would wait for every outstanding global load on every iteration.
__device__ __forceinline__ void settle(bf16x8& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Row sum on the matrix core: with v_mfma_f32_16x16x32_bf16, lane l supplies B[8(l/16) + j][l%16] from its 8 P
// values and A[m][8(l/16) + j] from this selector; register i of lane l receives D[4(l/16) + i][l%16]. The selector
// is 1 where (m/4 + k/8) is even, so D[4(l/16) + i][l%16] sums the P values of the two lanes that hold the keys of
// query l%32 in the 32x32 layout: every register of every lane gets the sum over this k-step's 16 keys for the lane's
// own query.
__device__ __forceinline__ bf16x8 lsum_selector(int lane) {
  const __bf16 v = ((((lane & 15) >> 2) + (lane >> 4)) & 1) ? (__bf16)0.0f : (__bf16)1.0f;
  return bf16x8{v, v, v, v, v, v, v, v};
}

// s * c - m, one fused multiply-add. Written as a builtin, not inline assembly: s comes straight from an MFMA, and
// only instructions the compiler emits itself get the wait states a VALU read of an MFMA result needs.
template <int D = 64>
__device__ __forceinline__ float scaled_minus(float s, float neg_m) { return __builtin_fmaf(s, scale_log2<D>(), neg_m); }

// The other lane of this lane's query (lane +- 32) has the flag set.
__device__ __forceinline__ bool partner32_any(bool x) {
  const uint32_t v = x ? 1u : 0u;
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (r[0] | r[1]) != 0u;
}

template <class F, int... I>
__device__ __forceinline__ void unroll_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), in order.
template <int N, class F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace mi355
