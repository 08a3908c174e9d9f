// Measurement kernels (microbenchmarks): matrix-core, v_exp_f32 and LDS read throughput with every CU busy, and HBM
// copy bandwidth. They give the ceilings the attention kernel is compared with on the chip it runs on (the published
// peak assumes the 2.4 GHz clock, which the chip does not hold under dense matrix-core load).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <vector>

#include "../../include/mi355_attn.h"
#include "../../include/mi355_probe.h"
#include "device_common.h"
#include "launch.h"

#define ATTN_EXPORT extern "C" __attribute__((visibility("default")))

namespace mi355 {
namespace {

constexpr int kProbeThreads = 256;  // four waves per workgroup
constexpr int kProbeBlocksPerCU = 2;  // two waves per SIMD
constexpr int kMaxCUs = 1024;
constexpr size_t kCycleBytes = (size_t)kMaxCUs * kProbeBlocksPerCU * 4 * sizeof(unsigned long long);
constexpr size_t kSinkBytes = (size_t)kMaxCUs * kProbeBlocksPerCU * kProbeThreads * sizeof(float);
constexpr size_t kScratchBytes = kCycleBytes + kSinkBytes;

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}
// eight bf16 values uniform in [-2, 2) from a hash of (seed, i)
__device__ bf16x8 hashed_bf16x8(uint32_t seed) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (__bf16)(((float)(mix32(seed * 8u + i) & 0xffffu) * (1.0f / 65536.0f) - 0.5f) * 4.0f);
  return v;
}

__global__ __launch_bounds__(kProbeThreads, kProbeBlocksPerCU) void probe_mfma_kernel(float* sink,
                                                                                    unsigned long long* cycles,
                                                                                    int iters) {
  const uint32_t gid = blockIdx.x * kProbeThreads + threadIdx.x;
  const bf16x8 a0 = hashed_bf16x8(4 * gid + 1), a1 = hashed_bf16x8(4 * gid + 2);
  const bf16x8 b0 = hashed_bf16x8(4 * gid + 3), b1 = hashed_bf16x8(4 * gid + 4);
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    // four accumulation chains; consecutive products share their A operand
    c0 = mfma32x32x16(a0, b0, c0);
    c1 = mfma32x32x16(a0, b1, c1);
    c2 = mfma32x32x16(a0, b0, c2);
    c3 = mfma32x32x16(a0, b1, c3);
    c0 = mfma32x32x16(a1, b0, c0);
    c1 = mfma32x32x16(a1, b1, c1);
    c2 = mfma32x32x16(a1, b0, c2);
    c3 = mfma32x32x16(a1, b1, c3);
  }
  // the MFMA results are read only after the loop; the clock is read after the last product has issued
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[gid] = s;
  if ((threadIdx.x & 63) == 0) cycles[gid >> 6] = t1 - t0;
}

__global__ __launch_bounds__(kProbeThreads, kProbeBlocksPerCU) void probe_exp_kernel(float* sink,
                                                                                   unsigned long long* cycles,
                                                                                   int iters) {
  const uint32_t gid = blockIdx.x * kProbeThreads + threadIdx.x;
  float r[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) r[i] = (float)(mix32(gid * 32u + i) & 0xffu) * (1.0f / 256.0f);
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 32; ++i) r[i] = __builtin_amdgcn_exp2f(-r[i]);  // stays in (0.5, 1]
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) s += r[i];
  sink[gid] = s;
  if ((threadIdx.x & 63) == 0) cycles[gid >> 6] = t1 - t0;
}

// LDS reads as the attention kernels issue them: row reads of 16 bytes a lane (ds_read_b128, the score operands) or
// transposed reads of four 16-bit values from four rows (ds_read_b64_tr_b16, the V operands), 32 in flight per
// wave, over a 32 KB buffer. Every address stays inside the buffer; the values only feed the sink.
template <bool kTr>
__global__ __launch_bounds__(kProbeThreads, kProbeBlocksPerCU) void probe_lds_kernel(float* sink,
                                                                                   unsigned long long* cycles,
                                                                                   int iters) {
  constexpr int kElems = 16384;  // 32 KB of 16-bit values
  __shared__ __attribute__((aligned(16))) uint16_t buf[kElems];
  for (int i = threadIdx.x; i < kElems; i += kProbeThreads) buf[i] = (uint16_t)(mix32((uint32_t)i) & 0x3fffu);
  __syncthreads();
  const uint32_t gid = blockIdx.x * kProbeThreads + threadIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t base = (uint32_t)(uintptr_t)buf;
  // per-lane element offset inside a 1 KB (row reads) or 512-byte (transposed reads) piece: a row read takes 8
  // consecutive elements per lane; a transposed read takes row 4g + (lane%16)/4 (+8 for lanes 16..31 of each half)
  // and 4 elements at column 8(2((lane/16)%2) + (lane%4)/2) + 4(lane%2) of a 64-column block, as the kernels do
  const int g = lane >> 5, jj = (lane & 15) >> 2;
  const uint32_t loff = kTr ? (uint32_t)((4 * g + jj) * 64 + 8 * (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) +
                                         4 * (lane & 1)) * 2u
                            : (uint32_t)lane * 16u;
  uint32_t acc = 0;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    // 32 reads, then one wait: piece (wave * 4 + j + it) mod 16 of the buffer (2 KB apart), all in bounds
    uint32_t r[32][4];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t addr = base + (uint32_t)(((wave * 4 + j + it) & 15) * 2048) + loff;
      if constexpr (kTr) {
        asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(*reinterpret_cast<uint64_t*>(&r[j][0])) : "v"(addr));
        r[j][2] = r[j][3] = 0u;
      } else {
        asm volatile("ds_read_b128 %0, %1" : "=v"(*reinterpret_cast<uint4*>(&r[j][0])) : "v"(addr));
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // (one word of each read passes through an empty volatile statement after the wait, so it is read only once it
    // has landed; one XOR per read keeps the VALU out of the way of the LDS)
#pragma unroll
    for (int j = 0; j < 32; ++j) asm volatile("" : "+v"(r[j][0]));
#pragma unroll
    for (int j = 0; j < 32; ++j) acc ^= r[j][0];
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  sink[gid] = (float)(acc & 0xffffu);
  if ((threadIdx.x & 63) == 0) cycles[gid >> 6] = t1 - t0;
}

__global__ __launch_bounds__(256) void probe_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                         size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

int cu_count(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail_status(ATTN_ERR_HIP, "probe: hipGetDevice failed");
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return fail_status(ATTN_ERR_HIP, "probe: cannot read the compute-unit count");
  if (n > kMaxCUs) return fail_status(ATTN_ERR_UNSUPPORTED, "probe: more compute units than the scratch layout holds");
  *out = n;
  return ATTN_OK;
}

// Launch `launch` twice (the first run warms up), time the second with events on `stream`, and return the time in
// milliseconds and the median per-wave cycle count read back from the scratch.
template <class F>
int timed_probe(F&& launch, hipStream_t stream, const unsigned long long* cycles_dev, int waves, float* ms,
                double* median_cycles) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return fail_status(ATTN_ERR_HIP, "probe: hipEventCreate failed");
  }
  int rc = ATTN_OK;
  launch();
  if (hipGetLastError() != hipSuccess || hipEventRecord(e0, stream) != hipSuccess) rc = ATTN_ERR_HIP;
  if (rc == ATTN_OK) {
    launch();
    if (hipGetLastError() != hipSuccess || hipEventRecord(e1, stream) != hipSuccess ||
        hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(ms, e0, e1) != hipSuccess)
      rc = ATTN_ERR_HIP;
  }
  if (rc == ATTN_OK && cycles_dev != nullptr) {
    std::vector<unsigned long long> c((size_t)waves);
    if (hipMemcpy(c.data(), cycles_dev, c.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost) != hipSuccess) {
      rc = ATTN_ERR_HIP;
    } else {
      std::nth_element(c.begin(), c.begin() + c.size() / 2, c.end());
      *median_cycles = (double)c[c.size() / 2];
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (rc != ATTN_OK) return fail_status(rc, "probe: a launch or event call failed");
  return ATTN_OK;
}

int check_scratch(void* scratch, size_t bytes, int64_t iters, const char* who) {
  if (!scratch) return fail_status(ATTN_ERR_INVALID, "%s: null scratch pointer", who);
  if ((reinterpret_cast<uintptr_t>(scratch) & 15u) != 0)
    return fail_status(ATTN_ERR_INVALID, "%s: scratch must be 16-byte aligned", who);
  if (bytes < kScratchBytes)
    return fail_status(ATTN_ERR_INVALID, "%s: scratch of %zu bytes, %zu needed", who, bytes, kScratchBytes);
  if (iters < 1 || iters > 1000000) return fail_status(ATTN_ERR_INVALID, "%s: iters %lld outside [1, 1e6]", who,
                                                       (long long)iters);
  return ATTN_OK;
}

}  // namespace
}  // namespace mi355

using namespace mi355;

ATTN_EXPORT size_t probe_scratch_size(void) { return kScratchBytes; }

ATTN_EXPORT int probe_mfma_bf16(void* scratch, size_t scratch_bytes, int64_t iters, void* stream, double* tflops,
                                double* clock_ghz) {
  if (!tflops || !clock_ghz) return fail_status(ATTN_ERR_INVALID, "probe_mfma_bf16: null result pointer");
  int rc = check_scratch(scratch, scratch_bytes, iters, "probe_mfma_bf16");
  if (rc != ATTN_OK) return rc;
  int cus = 0;
  if ((rc = cu_count(&cus)) != ATTN_OK) return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  auto* cycles = static_cast<unsigned long long*>(scratch);
  auto* sink = reinterpret_cast<float*>(static_cast<char*>(scratch) + kCycleBytes);
  const int blocks = cus * kProbeBlocksPerCU, waves = blocks * (kProbeThreads / 64);
  float ms = 0.f;
  double cyc = 0.0;
  rc = timed_probe([&] { hipLaunchKernelGGL(probe_mfma_kernel, dim3(blocks), dim3(kProbeThreads), 0, s, sink, cycles,
                                            (int)iters); }, s, cycles, waves, &ms, &cyc);
  if (rc != ATTN_OK) return rc;
  const double flops = (double)waves * (double)iters * 8.0 * (2.0 * 32 * 32 * 16);
  *tflops = flops / (ms * 1e-3) / 1e12;
  *clock_ghz = cyc / (ms * 1e-3) / 1e9;
  return ATTN_OK;
}

ATTN_EXPORT int probe_exp_f32(void* scratch, size_t scratch_bytes, int64_t iters, void* stream,
                              double* exp_per_clock_per_cu, double* clock_ghz) {
  if (!exp_per_clock_per_cu || !clock_ghz) return fail_status(ATTN_ERR_INVALID, "probe_exp_f32: null result pointer");
  int rc = check_scratch(scratch, scratch_bytes, iters, "probe_exp_f32");
  if (rc != ATTN_OK) return rc;
  int cus = 0;
  if ((rc = cu_count(&cus)) != ATTN_OK) return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  auto* cycles = static_cast<unsigned long long*>(scratch);
  auto* sink = reinterpret_cast<float*>(static_cast<char*>(scratch) + kCycleBytes);
  const int blocks = cus * kProbeBlocksPerCU, waves = blocks * (kProbeThreads / 64);
  float ms = 0.f;
  double cyc = 0.0;
  rc = timed_probe([&] { hipLaunchKernelGGL(probe_exp_kernel, dim3(blocks), dim3(kProbeThreads), 0, s, sink, cycles,
                                            (int)iters); }, s, cycles, waves, &ms, &cyc);
  if (rc != ATTN_OK) return rc;
  const double lanes = (double)waves * 64.0 * (double)iters * 32.0;
  *exp_per_clock_per_cu = lanes / cyc / cus;
  *clock_ghz = cyc / (ms * 1e-3) / 1e9;
  return ATTN_OK;
}

ATTN_EXPORT int probe_lds_read(void* scratch, size_t scratch_bytes, int64_t iters, int transposed, void* stream,
                               double* bytes_per_clock_per_cu, double* clock_ghz) {
  if (!bytes_per_clock_per_cu || !clock_ghz) return fail_status(ATTN_ERR_INVALID, "probe_lds_read: null result pointer");
  if (transposed != 0 && transposed != 1) return fail_status(ATTN_ERR_INVALID, "probe_lds_read: transposed must be 0 or 1");
  int rc = check_scratch(scratch, scratch_bytes, iters, "probe_lds_read");
  if (rc != ATTN_OK) return rc;
  int cus = 0;
  if ((rc = cu_count(&cus)) != ATTN_OK) return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  auto* cycles = static_cast<unsigned long long*>(scratch);
  auto* sink = reinterpret_cast<float*>(static_cast<char*>(scratch) + kCycleBytes);
  const int blocks = cus * kProbeBlocksPerCU, waves = blocks * (kProbeThreads / 64);
  float ms = 0.f;
  double cyc = 0.0;
  rc = timed_probe([&] {
    if (transposed)
      hipLaunchKernelGGL(probe_lds_kernel<true>, dim3(blocks), dim3(kProbeThreads), 0, s, sink, cycles, (int)iters);
    else
      hipLaunchKernelGGL(probe_lds_kernel<false>, dim3(blocks), dim3(kProbeThreads), 0, s, sink, cycles, (int)iters);
  }, s, cycles, waves, &ms, &cyc);
  if (rc != ATTN_OK) return rc;
  const double bytes = (double)waves * (double)iters * 32.0 * 64.0 * (transposed ? 8.0 : 16.0);
  *bytes_per_clock_per_cu = bytes / cyc / cus;
  *clock_ghz = cyc / (ms * 1e-3) / 1e9;
  return ATTN_OK;
}

ATTN_EXPORT int probe_hbm_copy(const void* src, void* dst, size_t bytes, int reps, void* stream, double* gbps) {
  if (!src || !dst || !gbps) return fail_status(ATTN_ERR_INVALID, "probe_hbm_copy: null pointer");
  if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) != 0)
    return fail_status(ATTN_ERR_INVALID, "probe_hbm_copy: pointers must be 16-byte aligned");
  if (bytes == 0 || bytes % 16 != 0 || bytes > (size_t(1) << 34))
    return fail_status(ATTN_ERR_INVALID, "probe_hbm_copy: bytes %zu must be a positive multiple of 16, at most 2^34",
                       bytes);
  if (reps < 1 || reps > 1000) return fail_status(ATTN_ERR_INVALID, "probe_hbm_copy: reps %d outside [1, 1000]", reps);
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + bytes && b < a + bytes) return fail_status(ATTN_ERR_INVALID, "probe_hbm_copy: src and dst overlap");
  int cus = 0;
  int rc = cu_count(&cus);
  if (rc != ATTN_OK) return rc;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t n = bytes / 16;
  const int blocks = cus * 8;
  float ms = 0.f;
  rc = timed_probe([&] {
    for (int r = 0; r < reps; ++r)
      hipLaunchKernelGGL(probe_copy_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const uint4*>(src),
                         static_cast<uint4*>(dst), n);
  }, s, nullptr, 0, &ms, nullptr);
  if (rc != ATTN_OK) return rc;
  *gbps = 2.0 * (double)bytes * reps / (ms * 1e-3) / 1e9;
  return ATTN_OK;
}
