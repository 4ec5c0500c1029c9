// Per-wave flash-attention core shared by the tile and the fine-grained
// attention kernels (CDNA4 / gfx950, v_mfma_f32_32x32x16_bf16).
//
// A wave owns QT x 32 query rows.  For each chunk of up to 64 keys staged in LDS
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

// QT 32-query column tiles per wave: every K / V^T fragment read from LDS
// feeds QT MFMAs, which divides the LDS read traffic per FLOP by QT.
template <int D, int QT = 1>
struct WaveState {
  static constexpr int DK = D / 16;  // MFMA k-steps over the head dimension
  static constexpr int DT = D / 32;  // 32-row blocks of O^T
  bf16x8 qf[QT][DK];                 // Q fragments (B operand: k = head dim, n = query)
  f32x16 acc[QT][DT];                // O^T accumulators
  float m_run[QT];                   // running max (raw score units)
  float l_part[QT];                  // this lane half's partial row sum

  // q_ptr(qt) points at the query row of column tile qt owned by this lane.
  template <class QPtr>
  __device__ __forceinline__ void init(QPtr q_ptr, int hi) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const uint16_t* p = q_ptr(qt);
#pragma unroll
      for (int kk = 0; kk < DK; ++kk) qf[qt][kk] = *reinterpret_cast<const bf16x8*>(p + kk * 16 + hi * 8);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[qt][dt][r] = 0.f;
      m_run[qt] = -INFINITY;
      l_part[qt] = 0.f;
    }
  }
  __device__ __forceinline__ void init(const uint16_t* qrow_ptr, int hi) {
    init([&](int qt) { return qrow_ptr + (long)qt * 32 * D; }, hi);
  }

  // One 32-key block (keys kb*32 .. kb*32+31 of the staged chunk), of which
  // the first nk are valid.  c2 = softmax scale * log2(e).
  __device__ __forceinline__ void block32(const uint16_t* lk, const uint16_t* lvt, int kb, int nk,
                                          float c2, int col, int hi) {
    // S^T = K Q^T for 32 keys x 32 queries, one query column tile at a time
    // (K fragments read from LDS once and reused by every tile), followed
    // directly by that tile's softmax so only one S tile is live.
    const int row = kb * 32 + key_perm(col);
    bf16x8 ka[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
      ka[kk] = *reinterpret_cast<const bf16x8*>(lk + Lds<D>::k_off(row, 2 * kk + hi));
    bf16x8 pb[QT][2];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qf[qt][0], f32x16{}, 0, 0, 0);
#pragma unroll
      for (int kk = 1; kk < DK; ++kk)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qf[qt][kk], s, 0, 0, 0);
      // keys past the valid count (only in a tile's last block)
      if (nk < 32) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (16 * (r >> 3) + 8 * hi + (r & 7) >= nk) s[r] = -INFINITY;
      }
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      // Lazy rescaling: the running max (the same value in both lane halves
      // of a query) is raised only when some score exceeds it by more than
      // 2^8 in exp2 units, so every probability stays <= 256 and the final
      // normalisation by the same running sum is exact.  The decision needs
      // only each lane's own 16 keys and a wave vote; the exchange between
      // the two halves happens only on the (rare) raise.
      if (__any((mx - m_run[qt]) * c2 > 8.0f)) {
        const float m_new = fmaxf(m_run[qt], fmaxf(mx, __shfl_xor(mx, 32)));
        const float alpha = __builtin_amdgcn_exp2f((m_run[qt] - m_new) * c2);
        l_part[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[qt][dt][r] *= alpha;
        m_run[qt] = m_new;
      }
      const float mc = m_run[qt] * c2;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
          pb[qt][half][t] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[half * 8 + t], c2, -mc));
        // row sum of the rounded probabilities actually multiplied with V
#pragma unroll
        for (int t = 0; t < 8; t += 2) {
          bf16x2 pr = {pb[qt][half][t], pb[qt][half][t + 1]};
          l_part[qt] = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes2, l_part[qt], false);
        }
      }
      // keep the scheduler from overlapping several tiles' S (register bound)
      if (QT > 1) __builtin_amdgcn_sched_barrier(0);
    }
    // O^T += V^T P^T
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int ks = kb * 2 + half;  // 16-key step inside the chunk
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(lvt + Lds<D>::v_off(dt * 32 + col, 2 * ks + hi));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          acc[qt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qt][half], acc[qt][dt], 0, 0, 0);
      }
    }
  }

  // One staged chunk with ck valid keys (1..64).
  __device__ __forceinline__ void chunk(const uint16_t* lk, const uint16_t* lvt, int ck, float c2,
                                        int col, int hi) {
    block32(lk, lvt, 0, min(ck, 32), c2, col, hi);
    if (ck > 32) block32(lk, lvt, 1, ck - 32, c2, col, hi);
  }

  // Normalise and write the query row of column tile qt (d channels, bf16)
  // to op.  Both lane halves must call it (they exchange partial sums).
  __device__ __forceinline__ void store(int qt, uint16_t* op, int hi, bool write) {
    const float l_tot = l_part[qt] + __shfl_xor(l_part[qt], 32);
    if (!write) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = dt * 32 + 8 * r4 + 4 * hi;
        __bf16 h[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) h[x] = (__bf16)(acc[qt][dt][4 * r4 + x] * inv);
        uint2 pk;
        pk.x = (uint32_t)__builtin_bit_cast(uint16_t, h[0]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, h[1]) << 16);
        pk.y = (uint32_t)__builtin_bit_cast(uint16_t, h[2]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, h[3]) << 16);
        *reinterpret_cast<uint2*>(op + d0) = pk;
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* op, int hi, bool write) { store(0, op, hi, write); }
};

}  // namespace core
}  // namespace vsa
