// Hardware probes of this part (gfx950): the matrix cores' rate with
// data-dependent operands, the HBM read rate, and one bare E4M3 product.
// Measurement only; nothing of the attention method is computed here.
//
// The MFMA probe issues the attention kernel's product shape
// (v_mfma_f32_32x32x16_bf16) back to back at the attention kernel's
// occupancy (12 waves per CU, 3 per SIMD), with operands that change from
// one product to the next, so the matrix pipes' switching activity, and
// with it the power-limited clock, is that of real data rather than of
// constant registers.  The read probe streams a buffer once with 16-byte
// loads.  The E4M3 probe issues the E4M3 attention's score product
// (v_mfma_f32_32x32x64_f8f6f4) once on caller data, so a test can measure
// its summation error against exact sums.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vsa_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = VSA_PROBE_WAVES;
constexpr int kSliceUnits = 16 * 64;  // 16-byte units of one wave's 16 fragments

__global__ __launch_bounds__(kWaves * 64, 3) void mfma_chain_kernel(const uint4* __restrict__ src,
                                                                    long n_slices,
                                                                    float* __restrict__ out,
                                                                    int iters) {
  const int lane = threadIdx.x & 63;
  const long gw = (long)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const uint4* p = src + (gw % n_slices) * kSliceUnits + lane;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = __builtin_bit_cast(bf16x8, p[i * 64]);
    b[i] = __builtin_bit_cast(bf16x8, p[(8 + i) * 64]);
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
    // product (ia, ib) multiplies A fragment ia by B fragment (ia + ib) mod 8
    // into chain ia mod 4: both operands change at every product
#pragma unroll
    for (int ib = 0; ib < 8; ++ib)
#pragma unroll
      for (int ia = 0; ia < 8; ++ia)
        acc[ia & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ia], b[(ia + ib) & 7], acc[ia & 3], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[gw * 64 + lane] = s;
}

// Eight 16-byte loads in flight per thread; NT: non-temporal loads (no
// allocation in the caches on the way).
template <bool NT>
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, long n,
                                                   uint32_t* __restrict__ out) {
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const long stride = (long)gridDim.x * 256;
  uint32_t x = 0;
  long i = t;
  for (; i + 7 * stride < n; i += 8 * stride) {
    u32x4 u[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      u[k] = NT ? __builtin_nontemporal_load(src + i + k * stride) : src[i + k * stride];
#pragma unroll
    for (int k = 0; k < 8; ++k) x ^= u[k].x ^ u[k].y ^ u[k].z ^ u[k].w;
  }
  for (; i < n; i += stride) {
    const u32x4 u = src[i];
    x ^= u.x ^ u.y ^ u.z ^ u.w;
  }
  out[t] = x;
}

// Lane layout of the 32x32x64 E4M3 product: row m of A (column n of B)
// sits in lane m (n) % 32, whose 32 bytes cover k = 32 * (lane / 32) ..
// +31; output register r of lane (n, h) holds row 8 * (r / 4) + 4h + r % 4
// of column n.
__global__ __launch_bounds__(64) void mfma_f8_kernel(const uint8_t* __restrict__ a,
                                                     const uint8_t* __restrict__ b,
                                                     float* __restrict__ d) {
  const int lane = threadIdx.x;
  const int m = lane & 31, h = lane >> 5;
  const long p = blockIdx.x;
  const i32x8 fa = *reinterpret_cast<const i32x8*>(a + p * 2048 + m * 64 + h * 32);
  const i32x8 fb = *reinterpret_cast<const i32x8*>(b + p * 2048 + m * 64 + h * 32);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  // format 0 (E4M3) for both operands; zero scale operands: unscaled
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, acc, 0, 0, 0, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) d[p * 1024 + (8 * (r >> 2) + 4 * h + (r & 3)) * 32 + m] = acc[r];
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

extern "C" int vsa_probe_mfma_rate(const void* src, size_t src_bytes, float* out, int workgroups,
                                   int iters, void* stream) {
  if (!src || !out || !aligned16(src) || !aligned16(out) || src_bytes == 0 ||
      src_bytes % (kSliceUnits * 16) != 0 || workgroups <= 0 || iters <= 0)
    return 1;
  hipLaunchKernelGGL(mfma_chain_kernel, dim3(workgroups), dim3(kWaves * 64), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint4*>(src), (long)(src_bytes / (kSliceUnits * 16)), out,
                     iters);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int vsa_probe_read_rate(const void* src, size_t bytes, uint32_t* out, int workgroups,
                                   int nontemporal, void* stream) {
  if (!src || !out || !aligned16(src) || bytes == 0 || bytes % 16 != 0 || workgroups <= 0) return 1;
  if (nontemporal)
    hipLaunchKernelGGL(read_kernel<true>, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const u32x4*>(src), (long)(bytes / 16), out);
  else
    hipLaunchKernelGGL(read_kernel<false>, dim3(workgroups), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const u32x4*>(src), (long)(bytes / 16), out);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int vsa_probe_mfma_f8(const uint8_t* a, const uint8_t* b, float* d, int n, void* stream) {
  if (!a || !b || !d || !aligned16(a) || !aligned16(b) || n <= 0) return 1;
  hipLaunchKernelGGL(mfma_f8_kernel, dim3(n), dim3(64), 0, (hipStream_t)stream, a, b, d);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
