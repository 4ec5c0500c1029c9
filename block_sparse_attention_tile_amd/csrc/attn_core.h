// Per-wave flash-attention core shared by the tile and the fine-grained
// attention kernels (CDNA4 / gfx950, v_mfma_f32_32x32x16_bf16).
//
// A wave owns 32 query rows.  For each chunk of up to 64 keys staged in LDS
// (K by key rows, V transposed [d][key], both swizzled) it computes S^T = K Q^T, masks keys
// past the chunk's valid count, updates the online softmax (running max and
// sum; the result equals masked softmax attention, SPADE review page,
// ledger axiom on FlashAttention-style online softmax) and accumulates
// O^T += V^T P^T.
//
// Lane layout (32x32x16 MFMA): output column = lane % 32, so each lane owns
// one query; its 16 accumulator registers hold rows 8*(r/4) + 4*(lane/32) +
// r%4.  K rows are fed in the order key_perm(row) (bits 2 and 3 swapped), so
// register r of key block mt holds key mt*32 + 16*(r/8) + 8*(lane/32) + r%8:
// eight consecutive keys per lane half, exactly the B-operand layout of the
// P^T V^T product.
#pragma once

#include <hip/hip_runtime.h>

namespace vsa {
namespace core {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

constexpr int kKC = 64;  // keys per chunk

__device__ __forceinline__ int key_perm(int m) {
  return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}


// LDS stage: K chunk [64 keys][D] and V^T chunk [D][64 keys], bf16, rows
// unpadded so that a wave's 64 x 16-byte direct global->LDS load fills 1 KB
// contiguously.  Bank conflicts of the 16-byte fragment reads are avoided by
// XOR-swizzling the 16-byte column index with a function of the row chosen
// so that any 8 (and any 16) consecutive lanes of a fragment read touch
// distinct bank groups.
template <int D>
struct Lds {
  static constexpr int KE = kKC * D;       // K elements per stage
  static constexpr int VE = D * kKC;       // V^T elements per stage
  static constexpr int STAGE = KE + VE;
  static constexpr int KC16 = D / 8;       // 16-byte columns per K row
  static constexpr int VC16 = kKC / 8;     // 16-byte columns per V^T row (8)
  // K row r (key), 16-byte column c -> element offset
  __device__ __forceinline__ static int k_off(int r, int c) {
    return r * D + ((c ^ (key_perm(r & 31) & (KC16 - 1))) << 3);
  }
  // V^T row d (channel), 16-byte column c (8 keys) -> element offset
  __device__ __forceinline__ static int v_off(int d, int c) {
    return d * kKC + ((c ^ ((d & 7) ^ ((d >> 3) & 1))) << 3);
  }
};

template <int D>
struct WaveState {
  static constexpr int DK = D / 16;  // MFMA k-steps over the head dimension
  static constexpr int DT = D / 32;  // 32-row blocks of O^T
  bf16x8 qf[DK];                     // Q fragment (B operand: k = head dim, n = query)
  f32x16 acc[DT];                    // O^T accumulators
  float m_run;                       // running max (raw score units)
  float l_part;                      // this lane half's partial row sum

  __device__ __forceinline__ void init(const uint16_t* qrow_ptr, int hi) {
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
      qf[kk] = *reinterpret_cast<const bf16x8*>(qrow_ptr + kk * 16 + hi * 8);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
    m_run = -INFINITY;
    l_part = 0.f;
  }

  // One 32-key block (keys kb*32 .. kb*32+31 of the staged chunk), of which
  // the first nk are valid.  c2 = softmax scale * log2(e).
  __device__ __forceinline__ void block32(const uint16_t* lk, const uint16_t* lvt, int kb, int nk,
                                          float c2, int col, int hi) {
    // S^T = K Q^T for 32 keys x 32 queries
    const int row = kb * 32 + key_perm(col);
    f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        *reinterpret_cast<const bf16x8*>(lk + Lds<D>::k_off(row, hi)), qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
    for (int kk = 1; kk < DK; ++kk)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *reinterpret_cast<const bf16x8*>(lk + Lds<D>::k_off(row, 2 * kk + hi)), qf[kk], s, 0, 0, 0);
    // keys past the valid count (only in a tile's last block)
    if (nk < 32) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (16 * (r >> 3) + 8 * hi + (r & 7) >= nk) s[r] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Lazy rescaling: raise the running max only when a score exceeds it by
    // more than 2^8 in exp2 units; probabilities stay <= 256 and the final
    // normalisation by the same running sum is exact.
    const float m_new = fmaxf(m_run, mx);
    if (__any((m_new - m_run) * c2 > 8.0f)) {
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
      m_run = m_new;
    }
    const float mc = m_run * c2;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      bf16x8 pb;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        pb[t] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[half * 8 + t], c2, -mc));
      // row sum of the rounded probabilities actually multiplied with V
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        bf16x2 pr = {pb[t], pb[t + 1]};
        l_part = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes2, l_part, false);
      }
      const int ks = kb * 2 + half;  // 16-key step inside the chunk
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(lvt + Lds<D>::v_off(dt * 32 + col, 2 * ks + hi)), pb,
            acc[dt], 0, 0, 0);
    }
  }

  // One staged chunk with ck valid keys (1..64).
  __device__ __forceinline__ void chunk(const uint16_t* lk, const uint16_t* lvt, int ck, float c2,
                                        int col, int hi) {
    block32(lk, lvt, 0, min(ck, 32), c2, col, hi);
    if (ck > 32) block32(lk, lvt, 1, ck - 32, c2, col, hi);
  }

  // Normalise and write this lane's query row (d channels, bf16) to op.
  // Must be called by both lane halves (they exchange their partial sums).
  __device__ __forceinline__ void store(uint16_t* op, int hi, bool write) {
    const float l_tot = l_part + __shfl_xor(l_part, 32);
    if (!write) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = dt * 32 + 8 * r4 + 4 * hi;
        __bf16 h[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) h[x] = (__bf16)(acc[dt][4 * r4 + x] * inv);
        uint2 pk;
        pk.x = (uint32_t)__builtin_bit_cast(uint16_t, h[0]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, h[1]) << 16);
        pk.y = (uint32_t)__builtin_bit_cast(uint16_t, h[2]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, h[3]) << 16);
        *reinterpret_cast<uint2*>(op + d0) = pk;
      }
    }
  }
};

}  // namespace core
}  // namespace vsa
