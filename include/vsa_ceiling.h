/*
 * vsa_ceiling.h - same-run ceilings of this part for the bounds the
 * attention path meets (C ABI of libvsa_ceiling.so).
 *
 * Not part of the attention boundary (vsa.h): these two calls measure what
 * the matrix cores and HBM deliver on this part and in this process, so a
 * kernel's achieved rate can be set against a practical ceiling measured
 * beside it rather than only against the datasheet figures (2.5 PFLOP/s
 * dense bf16, 8 TB/s HBM).  They compute nothing of the method.
 *
 * Conventions as in vsa.h: device pointers are caller-owned HIP device
 * memory, `stream` is a hipStream_t passed as void* (NULL = default
 * stream), calls are asynchronous and return a status code
 * (0 = OK, 1 = invalid argument, 4 = a HIP call failed).  Neither call
 * allocates.
 */
#ifndef VSA_CEILING_H
#define VSA_CEILING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Waves per workgroup of the MFMA probe (three per SIMD, as in the
 * attention kernel's 384-token tiles). */
#define VSA_CEILING_WAVES 12

/* Matrix-core ceiling with data-dependent operands.
 *
 * `workgroups` workgroups of VSA_CEILING_WAVES waves each run `iters`
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
int vsa_ceiling_mfma_bf16(const void* src, size_t src_bytes, float* out, int workgroups,
                          int iters, void* stream);

/* HBM read ceiling: `workgroups` workgroups of 256 threads read the
 * `bytes` of `src` once, grid-stride in 16-byte units (eight loads in
 * flight per thread; non-temporal loads when `nontemporal` is nonzero), and
 * XOR-fold what they read: thread t writes the XOR of its units' four
 * 32-bit words to out[t] (workgroups * 256 uint32).
 * bytes must be a positive multiple of 16; src 16-byte aligned.
 */
int vsa_ceiling_read(const void* src, size_t bytes, uint32_t* out, int workgroups, int nontemporal,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VSA_CEILING_H */
