/*
 * vsa_probe.h - hardware probes beside the attention library (C ABI of
 * libvsa_probe.so).
 *
 * Not part of the attention boundary (vsa.h): these calls measure facts of
 * this part that the measurement and the parity tests rely on, so that none
 * of those facts rests on code outside the repository.  They compute
 * nothing of the method.
 *   - two same-run ceilings: what the matrix cores deliver on data-dependent
 *     operands at the attention kernel's occupancy, and what a plain HBM read
 *     stream reaches (a kernel's achieved rate is then set against ceilings
 *     measured beside it, not only against the datasheet's 2.5 PFLOP/s
 *     dense bf16 and 8 TB/s);
 *   - one bare E4M3 matrix product, whose summation error bounds the E4M3
 *     attention's parity tolerance.
 *
 * Conventions as in vsa.h: device pointers are caller-owned HIP device
 * memory, `stream` is a hipStream_t passed as void* (NULL = default
 * stream), calls are asynchronous and return a status code (0 = OK,
 * 1 = invalid argument, 4 = a HIP call failed).  No call allocates.
 */
#ifndef VSA_PROBE_H
#define VSA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Waves per workgroup of the MFMA rate probe (three per SIMD, as in the
 * attention kernel's 384-token tiles). */
#define VSA_PROBE_WAVES 12

/* Matrix-core rate with data-dependent operands.
 *
 * `workgroups` workgroups of VSA_PROBE_WAVES waves each run `iters`
 * iterations of 64 v_mfma_f32_32x32x16_bf16 products (32x32 outputs,
 * k = 16: 32768 FLOP each) over eight A and eight B fragments that every
 * wave loads once from `src` (bf16 bits; wave w takes the 16 KB slice
 * w mod (src_bytes / 16384)), cycling through them so that both operands
 * change from one product to the next; four independent accumulator
 * chains.  No memory traffic inside the loop.
 * FLOPs per call = workgroups * 12 * iters * 64 * 32768.
 *
 * out: workgroups * 12 * 64 floats; lane l of wave w writes the sum of its
 *      accumulator registers to out[w * 64 + l] (over the 64 lanes of a
 *      wave this is the sum of every output element of its products, which
 *      a host check can recompute from the column and row sums of the
 *      fragments).
 * src_bytes must be a positive multiple of 16384; src and out 16-byte
 * aligned; workgroups and iters positive.
 */
int vsa_probe_mfma_rate(const void* src, size_t src_bytes, float* out, int workgroups, int iters,
                        void* stream);

/* HBM read rate: `workgroups` workgroups of 256 threads read the `bytes` of
 * `src` once, grid-stride in 16-byte units (eight loads in flight per
 * thread; non-temporal loads when `nontemporal` is nonzero), and XOR-fold
 * what they read: thread t writes the XOR of its units' four 32-bit words
 * to out[t] (workgroups * 256 uint32).
 * bytes must be a positive multiple of 16; src 16-byte aligned.
 */
int vsa_probe_read_rate(const void* src, size_t bytes, uint32_t* out, int workgroups, int nontemporal,
                        void* stream);

/* One E4M3 matrix product per problem, as the E4M3 attention computes its
 * scores: D_p = A_p B_p with a single v_mfma_f32_32x32x64_f8f6f4 (both
 * operands OCP E4M3, unscaled, zero accumulator input), one wave per
 * problem p < n.
 *   a: n x [32 rows m][64 k] E4M3 bytes (row-major);
 *   b: n x [32 columns][64 k] E4M3 bytes (B transposed: column j's 64 k
 *      values are contiguous);
 *   d: n x [32 rows][32 columns] float, row-major.
 * a and b 16-byte aligned; n positive.
 */
int vsa_probe_mfma_f8(const uint8_t* a, const uint8_t* b, float* d, int n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VSA_PROBE_H */
