/* mi355_probe.h - C ABI of the measurement kernels (microbenchmarks) shipped with the attention library.
 *
 * They measure what this chip actually delivers to the attention kernel, so its throughput can be stated against a
 * measured ceiling as well as against the published one:
 *   - probe_mfma_bf16: dense bf16 matrix-core throughput (v_mfma_f32_32x32x16_bf16, fp32 accumulate) with every CU
 *     busy, two waves per SIMD, operands drawn from a hash of the lane (so they toggle like real data; the chip's
 *     clock under matrix-core load depends on how many operand bits change), and consecutive products sharing one
 *     operand, the order the attention kernel uses;
 *   - probe_exp_f32: the rate of v_exp_f32 (the softmax's transcendental) with every CU busy;
 *   - probe_lds_read: LDS read throughput with every CU busy, for the two read forms the attention kernels use;
 *   - probe_hbm_copy: device-to-device copy bandwidth (bytes read + bytes written per second).
 *
 * Conventions: pointers are caller-owned DEVICE pointers (16-byte aligned); `stream` is a hipStream_t (NULL: the
 * default stream). Unlike the attention entry points, every probe SYNCHRONISES `stream` (it times itself with HIP
 * events) and writes its results to the caller's host doubles. Return values are attn_status codes (mi355_attn.h);
 * attn_last_error() has the detail. The probes allocate nothing; `scratch` must hold probe_scratch_size() bytes.
 */
#ifndef MI355_PROBE_H
#define MI355_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of device scratch the MFMA and exp probes need (per-wave cycle counts and sink outputs). */
size_t probe_scratch_size(void);

/* Matrix-core throughput: `iters` loop trips of 8 dependent-chain MFMAs per wave (iters in [1, 1e6]).
 *   tflops:    achieved dense bf16 TFLOP/s (2*32*32*16 flops per MFMA) over the whole launch
 *   clock_ghz: shader cycles per wave (s_memtime) divided by the launch time: the clock the chip held */
int probe_mfma_bf16(void* scratch, size_t scratch_bytes, int64_t iters, void* stream, double* tflops,
                    double* clock_ghz);

/* v_exp_f32 throughput: `iters` loop trips of 32 independent exp2 per wave (iters in [1, 1e6]).
 *   exp_per_clock_per_cu: lane results per shader cycle per CU; clock_ghz as above */
int probe_exp_f32(void* scratch, size_t scratch_bytes, int64_t iters, void* stream, double* exp_per_clock_per_cu,
                  double* clock_ghz);

/* LDS read throughput: `iters` loop trips of 32 reads per wave (iters in [1, 1e6]), two 4-wave workgroups per CU, each
 * reading its own 32 KB; transposed = 0: ds_read_b128 (16 bytes a lane), 1: ds_read_b64_tr_b16 (8 bytes a lane).
 *   bytes_per_clock_per_cu: bytes delivered to lanes per shader cycle per CU; clock_ghz as above */
int probe_lds_read(void* scratch, size_t scratch_bytes, int64_t iters, int transposed, void* stream,
                   double* bytes_per_clock_per_cu, double* clock_ghz);

/* Copy `bytes` (a multiple of 16, at most 2^34) from src to dst `reps` times (reps in [1, 1000]); src and dst must
 * not overlap. gbps: (bytes read + bytes written) per second, in GB/s (1e9 B/s). */
int probe_hbm_copy(const void* src, void* dst, size_t bytes, int reps, void* stream, double* gbps);

#ifdef __cplusplus
}
#endif

#endif /* MI355_PROBE_H */
