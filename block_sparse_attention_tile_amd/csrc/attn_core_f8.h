// Per-wave flash-attention core of the E4M3 (FP8) tile path (CDNA4 /
// gfx950, v_mfma_f32_32x32x64_f8f6f4 with both operands E4M3).
//
// A wave owns 32 query rows.  For each chunk of up to 64 keys staged in LDS
// (K by key rows, V transposed [d][key]) it computes S^T = K Q^T per 32-key
// block, updates the online softmax over the whole chunk, rounds the
// probabilities to E4M3 and accumulates O^T += V^T P^T and the row sums
// l += 1^T P^T (one more MFMA with an all-ones operand), once per 64 keys.  The row sum is then exactly
// the sum of the rounded probabilities that multiply V.
//
// Lane layout (32x32x64): row m of A and column n of B sit in lane m (n) %
// 32; the 32 bytes of a lane cover one half of the 64-long k range, the
// half chosen by lane / 32; A and B are fed alike, so any assignment of k to
// (half, byte) that both share gives the same product.  Output register r of
// lane (n, h) holds row 8*(r/4) + 4h + r%4.
//  * S^T: lane m reads K row kb*32 + m (natural key order) and lane n the
//    query row n, bytes kk*64 + 32h .. +31 of the head dimension for MFMA kk.
//  * P^T (the B operand of the PV product): byte i < 16 of lane (n, h) is
//    register i of block 0, byte 16 + i register i of block 1, i.e. key
//    32b + 8(i/4) + 4h + i%4.
//  * V^T: the E4M3 layout stores, inside every 32-slot group, slot bits
//    (b4 b3 b2 b1 b0) at position (b2 b4 b3 b1 b0), so those 16 keys of
//    block b and half h are the consecutive bytes 32b + 16h .. +15 of a V^T
//    row: two 16-byte reads per operand.
#pragma once

#include <hip/hip_runtime.h>

namespace vsa {
namespace core8 {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kKC = 64;  // keys per chunk

// LDS stage (bytes): K chunk [64 keys][D] and V^T chunk [D][64 keys].  Every
// row is padded by one 16-byte unit, so the 16-byte reads of 16 consecutive
// lanes (16 consecutive rows, one column) fall in distinct bank groups.  A
// stage is a whole number of 1 KB blocks (the unit of a direct load).
template <int D>
struct Lds {
  static constexpr int KROW = D + 16;    // bytes per K row (padded)
  static constexpr int VROW = kKC + 16;  // bytes per V^T row (padded)
  static constexpr int KE = kKC * KROW;  // K bytes per stage
  static constexpr int VE = D * VROW;    // V^T bytes per stage
  static constexpr int STAGE = KE + VE;
  static constexpr int KC16 = D / 16;    // 16-byte data units per K row
  static constexpr int VC16 = kKC / 16;  // 16-byte data units per V^T row
  static_assert(KE % 1024 == 0 && VE % 1024 == 0, "stage parts are whole 1 KB blocks");
  // key held by physical K row p of a stage
  __device__ __forceinline__ static int key_of_row(int p) { return p; }
};

__device__ __forceinline__ i32x8 read32(const uint8_t* p0, const uint8_t* p1) {
  const i32x4 a = *reinterpret_cast<const i32x4*>(p0);
  const i32x4 b = *reinterpret_cast<const i32x4*>(p1);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // format 0 (E4M3) for both operands; zero scale operands select the
  // unscaled instruction
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// A wave's state for 32 query rows.
//
// Online softmax against an integer reference: p = 2^(c2 s - mo) with c2 =
// scale * log2(e) * 2^-(e_q + e_k) and mo + 8 an integer at or above every
// score seen so far (in exp2 units), so every p <= 256 fits E4M3.  mo + 8 is
// raised to the ceiling of the running max whenever a score exceeds it; the
// rescale factor 2^(mo_old - mo_new) is a power of two, so rounded
// probabilities already accumulated stay exactly what rounding against the
// final reference would have given (outside E4M3's subnormal range).
template <int D>
struct WaveState {
  static constexpr int DK = D / 64;  // MFMA k-steps over the head dimension
  static constexpr int DT = D / 32;  // 32-row blocks of O^T
  i32x8 qf[DK];                      // Q bytes (B operand)
  f32x16 acc[DT];                    // O^T accumulators
  f32x16 lacc;                       // row sums (every register: this lane's query)
  float mo;                          // reference - 8 in exp2 units; -inf before any key

  // qrow_ptr points at the E4M3 query row owned by this lane.
  __device__ __forceinline__ void init(const uint8_t* qrow_ptr, int hi) {
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) qf[kk] = *reinterpret_cast<const i32x8*>(qrow_ptr + kk * 64 + hi * 32);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) lacc[r] = 0.f;
    mo = -INFINITY;
  }

  // S^T for the 32 keys kb*32 .. kb*32+31 of the staged chunk.
  __device__ __forceinline__ f32x16 scores(const uint8_t* lk, int kb, int col, int hi) const {
    const uint8_t* kp = lk + (kb * 32 + col) * Lds<D>::KROW + hi * 32;
    i32x8 ka[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) ka[kk] = read32(kp + kk * 64, kp + kk * 64 + 16);
    f32x16 s = mfma8(ka[0], qf[0], f32x16{});
#pragma unroll
    for (int kk = 1; kk < DK; ++kk) s = mfma8(ka[kk], qf[kk], s);
    return s;
  }

  // Keys at or past nk of a block get -inf (none for nk >= 32, all for
  // nk <= 0).  Register r holds key
  // 8*(r/4) + 4*hi + r%4 of the block; the threshold is laundered through an
  // empty asm so that the compares stay against immediates.
  __device__ __forceinline__ static void mask(f32x16& s, int nk, int hi) {
    int thr = nk - 4 * hi;
    asm volatile("" : "+v"(thr));
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (8 * (r >> 2) + (r & 3) >= thr) s[r] = -INFINITY;
  }

  // E4M3 probabilities of a block against the current reference, packed
  // four to a dword in register order.
  __device__ __forceinline__ void probs(const f32x16& s, float c2, int pk[4]) const {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = __builtin_amdgcn_exp2f(fmaf(s[4 * w], c2, -mo));
      const float b = __builtin_amdgcn_exp2f(fmaf(s[4 * w + 1], c2, -mo));
      const float c = __builtin_amdgcn_exp2f(fmaf(s[4 * w + 2], c2, -mo));
      const float d = __builtin_amdgcn_exp2f(fmaf(s[4 * w + 3], c2, -mo));
      int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
      pk[w] = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    }
  }

  // Largest score of a block (a three-level tree).
  __device__ __forceinline__ static float block_max(const f32x16& s) {
    float m3[6];
#pragma unroll
    for (int k = 0; k < 5; ++k) m3[k] = fmaxf(fmaxf(s[3 * k], s[3 * k + 1]), s[3 * k + 2]);
    m3[5] = s[15];
    return fmaxf(fmaxf(fmaxf(m3[0], m3[1]), m3[2]), fmaxf(fmaxf(m3[3], m3[4]), m3[5]));
  }

  // Softmax of a whole chunk: the probabilities of both blocks go into one
  // PV product, so they must share one reference and the max is taken over
  // the chunk first.  If some score exceeds the reference (a wave vote;
  // both lane halves of a query take the same new reference) it is raised
  // to the ceiling of the max and the accumulators are rescaled by the
  // power of two; then the probabilities are rounded against it.
  __device__ __forceinline__ void softmax(const f32x16& s0, const f32x16& s1, float c2, int pk[8]) {
    const float mxc = fmaxf(block_max(s0), block_max(s1)) * c2;
    if (__any(mxc - mo > 8.0f)) {
      const float mn = fmaxf(mo, ceilf(fmaxf(mxc, __shfl_xor(mxc, 32))) - 8.0f);
      // 2^(mo - mn) exactly; 0 before the first key (nothing accumulated yet)
      const float alpha = mo == -INFINITY ? 0.f : __builtin_amdgcn_ldexpf(1.0f, (int)(mo - mn));
#pragma unroll
      for (int r = 0; r < 16; ++r) lacc[r] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
      mo = mn;
    }
    probs(s0, c2, pk);
    probs(s1, c2, pk + 4);
  }

  // O^T += V^T P^T and l += 1^T P^T for the 64 keys of a chunk.  Lane col
  // reads channel row dt*32 + col, bytes 16*hi .. +15 (block 0) and
  // 32 + 16*hi .. +15 (block 1).
  __device__ __forceinline__ void pv(const uint8_t* lvt, int col, int hi, const i32x8& p) {
    const uint8_t* vp = lvt + col * Lds<D>::VROW + hi * 16;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint8_t* r = vp + dt * 32 * Lds<D>::VROW;
      acc[dt] = mfma8(read32(r, r + 32), p, acc[dt]);
    }
    constexpr int kOne = 0x38;  // 1.0 in E4M3
    constexpr int kOnes = kOne | (kOne << 8) | (kOne << 16) | (kOne << 24);
    const i32x8 ones = {kOnes, kOnes, kOnes, kOnes, kOnes, kOnes, kOnes, kOnes};
    lacc = mfma8(ones, p, lacc);
  }

  // One staged chunk with ck valid keys (1..64).  A 32-key chunk masks all
  // of block 1 (its LDS rows hold tile data, never stale memory), so both
  // chunk sizes run one code path.
  __device__ __forceinline__ void chunk(const uint8_t* lk, const uint8_t* lvt, int ck, float c2,
                                        int col, int hi) {
    f32x16 s0 = scores(lk, 0, col, hi);
    f32x16 s1 = scores(lk, 1, col, hi);
    if (ck < 64) {
      mask(s0, ck, hi);
      mask(s1, ck - 32, hi);
    }
    int pk[8];
    softmax(s0, s1, c2, pk);
    const i32x8 p = {pk[0], pk[1], pk[2], pk[3], pk[4], pk[5], pk[6], pk[7]};
    pv(lvt, col, hi, p);
  }

  // One staged chunk of two 32-key units (block b holds unit b) with n0, n1
  // (0..32, wave-uniform, not both 0) valid keys.
  __device__ __forceinline__ void chunk_units(const uint8_t* lk, const uint8_t* lvt, int n0, int n1,
                                              float c2, int col, int hi) {
    f32x16 s0 = scores(lk, 0, col, hi);
    f32x16 s1 = scores(lk, 1, col, hi);
    if (n0 < 32 || n1 < 32) {
      mask(s0, n0, hi);
      mask(s1, n1, hi);
    }
    int pk[8];
    softmax(s0, s1, c2, pk);
    const i32x8 p = {pk[0], pk[1], pk[2], pk[3], pk[4], pk[5], pk[6], pk[7]};
    pv(lvt, col, hi, p);
  }

  // Normalise (times oscale = 2^-e_v) and write this lane's query row (d
  // channels, bf16) to op.
  __device__ __forceinline__ void store(uint16_t* op, int hi, bool write, float oscale) const {
    if (!write) return;
    const float l = lacc[0];
    const float inv = l > 0.f ? oscale / l : 0.f;
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

}  // namespace core8
}  // namespace vsa
