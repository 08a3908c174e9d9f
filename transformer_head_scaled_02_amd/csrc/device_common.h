// Device helpers shared by the gfx950 kernels: vector types, MFMA wrappers, bf16 packing, cross-lane ops and the
// XCD-aware workgroup remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi355 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16), one wave.
// Lane l supplies A[l%32][8*(l/32) + j] and B[8*(l/32) + j][l%32] for j = 0..7; it receives
// D[8*(r/4) + 4*(l/32) + r%4][l%32] in accumulator register r = 0..15. (Checked against a host matmul on gfx950.)
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two fp32 values -> two bf16 (round to nearest even), packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// v_permlane32_swap with the same value in both operands: r[0] and r[1] together hold this lane's value and the
// value of the lane 32 away (lanes < 32: r[0] own, r[1] partner; lanes >= 32: r[0] partner, r[1] own).
__device__ __forceinline__ float max_with_partner32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ds_read_b64_tr_b16: every lane passes the LDS address of 4 consecutive 16-bit elements. Within each group of 16
// lanes, output lane i receives component j from source lane 4j + i/4, element i%4. (Checked on gfx950.) So if
// source lane 4j + t of a group points at row (r0 + j), column (c0 + 4t) of a row-major tile, output lane i gets
// the 4 elements of column c0 + i in rows r0 .. r0+3: a transposed read.
__device__ __forceinline__ bf16x4 lds_read_tr16x4(const uint16_t* p) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2). Map the hardware block id so that
// every XCD receives one contiguous range of logical block ids: neighbouring logical blocks (same head, same K/V)
// then share an L2. A bijection on [0, nblocks).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcds = 8;
  const int per = nblocks / kXcds, rem = nblocks % kXcds;
  const int xcd = bid % kXcds, slot = bid / kXcds;
  return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

// Causal workloads, whose blocks differ in cost: map the hardware block id to (head slot, block index within the head)
// so that each XCD still owns whole heads (its blocks share K/V in its L2) but dispatches them block-index-major:
// index 0 of all its heads first, then index 1, and so on. The caller makes index 0 the heaviest block, so the
// longest blocks start first and the light ones fill in behind them. Falls back to xcd_remap's head-major order when
// the heads do not divide evenly over the XCDs.
__device__ __forceinline__ void causal_order(int bid, int nblocks, int n_per_head, int& head_slot, int& idx) {
  constexpr int kXcds = 8;
  const int per = nblocks / kXcds;
  if (nblocks % kXcds == 0 && per % n_per_head == 0) {
    const int hx = per / n_per_head, xcd = bid % kXcds, slot = bid / kXcds;
    head_slot = xcd * hx + slot % hx;
    idx = slot / hx;
  } else {
    const int l = xcd_remap(bid, nblocks);
    head_slot = l / n_per_head;
    idx = l % n_per_head;
  }
}

// Head of a workgroup's slot: slots are decoded batch-minor (slot % B is the batch entry), so that the contiguous
// slot range xcd_remap gives each XCD spans every batch entry. Heads are independent, so this costs nothing when
// every entry does the same work, and it keeps the XCDs evenly loaded when entries differ (key padding). Returns the
// batch entry; `bh` receives the head's index b*H + h into the [B, H, ...] tensors.
__device__ __forceinline__ int head_of_slot(int slot, int B, int H, int& bh) {
  const int b = slot % B;
  bh = b * H + slot / B;
  return b;
}

}  // namespace mi355
