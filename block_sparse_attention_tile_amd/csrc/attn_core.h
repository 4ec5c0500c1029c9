// Per-wave flash-attention core shared by the tile and the fine-grained
// attention kernels (CDNA4 / gfx950, v_mfma_f32_32x32x16_bf16).
//
// A wave owns 32 query rows.  For each chunk of up to 64 keys staged in LDS
// (K by key rows, V transposed [d][key]) it computes S^T = K Q^T, masks keys
// past the chunk's valid count, updates the online softmax (running offset
// and sum; the result equals masked softmax attention, SPADE review page,
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


// LDS stage: K chunk [64 keys][D] and V^T chunk [D][64 keys], bf16.  Every
// row is padded by one 16-byte unit, so that consecutive rows start in
// consecutive 16-byte bank groups: the 16-byte fragment reads of 8 (and of
// 16) consecutive lanes, which read consecutive rows at one column, touch
// distinct banks, and every fragment a lane reads sits at a compile-time
// offset from one per-lane base address.  K rows are stored in MFMA lane order:
// physical row p holds key (p & ~31) | key_perm(p & 31).  A stage is a whole
// number of 1 KB blocks, the unit of a wave's direct global->LDS load.
template <int D>
struct Lds {
  static constexpr int KROW = D + 8;          // elements per K row (padded)
  static constexpr int VROW = kKC + 8;        // elements per V^T row (padded)
  static constexpr int KE = kKC * KROW;       // K elements per stage
  static constexpr int VE = D * VROW;         // V^T elements per stage
  static constexpr int STAGE = KE + VE;
  static constexpr int KC16 = D / 8;          // 16-byte data units per K row
  static constexpr int VC16 = kKC / 8;        // 16-byte data units per V^T row
  static_assert(KE % 512 == 0 && VE % 512 == 0, "stage parts are whole 1 KB blocks");
  // key r of the chunk, 16-byte column c -> element offset
  __device__ __forceinline__ static int k_off(int r, int c) {
    return ((r & ~31) | key_perm(r & 31)) * KROW + c * 8;
  }
  // V^T row d (channel), 16-byte column c (keys 8c .. 8c+7) -> element offset
  __device__ __forceinline__ static int v_off(int d, int c) { return d * VROW + c * 8; }
  // key held by physical K row p of a stage
  __device__ __forceinline__ static int key_of_row(int p) { return (p & ~31) | key_perm(p & 31); }
};

// A wave's flash-attention state for 32 query rows.
//
// Online softmax with a lazily raised, integer offset: probabilities are
// p = 2^(c2 s - mo) with c2 = scale * log2(e) and mo an integer held per
// query.  mo is raised (to the ceiling of the running max of c2 s) only when
// some score exceeds it by more than 8, so every p stays <= 256, and every
// rescale factor 2^(mo_old - mo_new) is a power of two: rescaling the
// accumulators, the row sum and already rounded bf16 probabilities is exact.
// The final normalisation divides by the sum of the rounded probabilities
// that were actually multiplied with V.
template <int D>
struct WaveState {
  static constexpr int DK = D / 16;  // MFMA k-steps over the head dimension
  static constexpr int DT = D / 32;  // 32-row blocks of O^T
  bf16x8 qf[DK];                     // Q fragments (B operand: k = head dim, n = query)
  f32x16 acc[DT];                    // O^T accumulators
  float mo;                          // offset in exp2 units (integer valued; -inf before any key)
  float l_part;                      // this lane half's partial row sum

  // qrow_ptr points at the query row owned by this lane.
  __device__ __forceinline__ void init(const uint16_t* qrow_ptr, int hi) {
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qrow_ptr + kk * 16 + hi * 8);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
    mo = -INFINITY;
    l_part = 0.f;
  }

  // S^T = K Q^T for the 32 keys kb*32 .. kb*32+31 of the staged chunk
  // (lane col reads physical row kb*32 + col): all K fragments, then the
  // MFMA chain.
  __device__ __forceinline__ f32x16 scores(const uint16_t* lk, int kb, int col, int hi) const {
    const uint16_t* kp = lk + (kb * 32 + col) * Lds<D>::KROW + hi * 8;
    bf16x8 ka[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) ka[kk] = *reinterpret_cast<const bf16x8*>(kp + kk * 16);
    f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
    for (int kk = 1; kk < DK; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qf[kk], s, 0, 0, 0);
    // at most four fragment reads ahead of the MFMA chain (register budget)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int kk = 0; kk < DK - 4; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    return s;
  }

  // K fragments of the next block read during a PV step (the first PRE of its DK).
  static constexpr int PRE = DK < 4 ? DK : 4;

  // scores() for a block whose first PRE K fragments were prefetched: the
  // chain starts on them and the rest are read right after its first MFMA
  // (the same products in the same order).
  __device__ __forceinline__ f32x16 scores_pre(const uint16_t* lk, int kb, int col, int hi,
                                               const bf16x8 pre[PRE]) const {
    const uint16_t* kp = lk + (kb * 32 + col) * Lds<D>::KROW + hi * 8;
    bf16x8 ka[DK];
#pragma unroll
    for (int kk = 0; kk < PRE; ++kk) ka[kk] = pre[kk];
#pragma unroll
    for (int kk = PRE; kk < DK; ++kk) ka[kk] = *reinterpret_cast<const bf16x8*>(kp + kk * 16);
    f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[0], qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
    for (int kk = 1; kk < DK; ++kk) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qf[kk], s, 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (DK > PRE) __builtin_amdgcn_sched_group_barrier(0x100, DK - PRE, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, DK - 1, 0);
    return s;
  }

  // Keys at or past nk (< 32) of a block get -inf.  Register r holds key
  // 16*(r/8) + 8*hi + r%8, invalid when 16*(r/8) + r%8 >= nk - 8*hi; the
  // threshold is laundered through an empty asm so that the compares stay
  // against immediates (no per-register key constants kept live).
  __device__ __forceinline__ static void mask(f32x16& s, int nk, int hi) {
    int thr = nk - 8 * hi;
    asm volatile("" : "+v"(thr));
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (16 * (r >> 3) + (r & 7) >= thr) s[r] = -INFINITY;
  }

  // Per 16-key half h of a block (registers 8h .. 8h+7): keys at or past
  // n_h (0..16) of the half get -inf.
  __device__ __forceinline__ static void mask_halves(f32x16& s, int n0, int n1, int hi) {
    int t0 = n0 - 8 * hi, t1 = n1 - 8 * hi;
    asm volatile("" : "+v"(t0), "+v"(t1));
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (r >= t0) s[r] = -INFINITY;
      if (r >= t1) s[8 + r] = -INFINITY;
    }
  }

  // Probabilities of a block against the current offset, as the bf16 B
  // operands of the two 16-key steps.
  __device__ __forceinline__ void probs(const f32x16& s, float c2, bf16x8 pb[2]) const {
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int t = 0; t < 8; ++t) pb[half][t] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[half * 8 + t], c2, -mo));
  }

  // Softmax of one block.  The probabilities are computed against the
  // current offset while this lane's block max is reduced (a three-level
  // tree); the offset is raised, and the probabilities recomputed, only
  // when some score exceeds it by more than 8 in exp2 units (a wave vote;
  // both lane halves of a query take the same new offset), so every
  // probability stays <= 256.  The rounded probabilities are then summed
  // into the row sum.
  __device__ __forceinline__ void softmax(const f32x16& s, float c2, bf16x8 pb[2]) {
    probs(s, c2, pb);
    float m3[6];
#pragma unroll
    for (int k = 0; k < 5; ++k) m3[k] = fmaxf(fmaxf(s[3 * k], s[3 * k + 1]), s[3 * k + 2]);
    m3[5] = s[15];
    const float mx = fmaxf(fmaxf(fmaxf(m3[0], m3[1]), m3[2]), fmaxf(fmaxf(m3[3], m3[4]), m3[5]));
    const float mxc = mx * c2;
    if (__any(mxc - mo > 8.0f)) {
      const float mn = fmaxf(mo, ceilf(fmaxf(mxc, __shfl_xor(mxc, 32))));
      // 2^(mo - mn) exactly; 0 before the first key (nothing accumulated yet)
      const float alpha = mo == -INFINITY ? 0.f : __builtin_amdgcn_ldexpf(1.0f, (int)(mo - mn));
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
      mo = mn;
      probs(s, c2, pb);
    }
    // row sum of the rounded probabilities actually multiplied with V
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        bf16x2 pr = {pb[half][t], pb[half][t + 1]};
        l_part = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes2, l_part, false);
      }
  }

  // O^T += V^T P^T for block kb.  Lane col reads channel row dt*32 + col,
  // keys 16*ks + 8*hi .. +7 of the 16-key step ks = 2*kb + half.
  // The fragment reads run PV_AHEAD ahead of the MFMAs (each accumulator
  // still takes half 0, then half 1).
  static constexpr int PV_AHEAD = 2 * DT < 4 ? 2 * DT : 4;
  __device__ __forceinline__ void pv(const uint16_t* lvt, int kb, int col, int hi, const bf16x8 pb[2]) {
    const uint16_t* vp = lvt + col * Lds<D>::VROW + kb * 32 + hi * 8;
    bf16x8 va[2 * DT];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        va[half * DT + dt] = *reinterpret_cast<const bf16x8*>(vp + dt * 32 * Lds<D>::VROW + half * 16);
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[half * DT + dt], pb[half], acc[dt], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, PV_AHEAD, 0);
#pragma unroll
    for (int x = 0; x < 2 * DT - PV_AHEAD; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, PV_AHEAD, 0);
  }

  // pv() that also reads the first PRE K fragments of block kn for the next
  // scores_pre(): the V^T reads run PV_AHEAD ahead of the MFMAs as in pv(),
  // then the K reads go out one per MFMA over the last PRE MFMAs.
  __device__ __forceinline__ void pv_pf(const uint16_t* lvt, int kb, int col, int hi, const bf16x8 pb[2],
                                        const uint16_t* lk, int kn, bf16x8 pre[PRE]) {
    static_assert(PV_AHEAD >= PRE, "the K reads follow the V^T reads");
    const uint16_t* vp = lvt + col * Lds<D>::VROW + kb * 32 + hi * 8;
    bf16x8 va[2 * DT];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        va[half * DT + dt] = *reinterpret_cast<const bf16x8*>(vp + dt * 32 * Lds<D>::VROW + half * 16);
    const uint16_t* kp = lk + (kn * 32 + col) * Lds<D>::KROW + hi * 8;
#pragma unroll
    for (int kk = 0; kk < PRE; ++kk) pre[kk] = *reinterpret_cast<const bf16x8*>(kp + kk * 16);
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[half * DT + dt], pb[half], acc[dt], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, PV_AHEAD, 0);
#pragma unroll
    for (int x = 0; x < 2 * DT - PV_AHEAD + PRE; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (PV_AHEAD > PRE) __builtin_amdgcn_sched_group_barrier(0x008, PV_AHEAD - PRE, 0);
  }

  // One staged chunk with ck valid keys (1..64), block by block.  PF: block
  // 1's first K fragments are read during block 0's PV step (the stage always
  // holds 64 rows, so the reads stay in it for a 32-key chunk); off where the
  // register budget has no room for them.
  template <bool PF = true>
  __device__ __forceinline__ void chunk(const uint16_t* lk, const uint16_t* lvt, int ck, float c2,
                                        int col, int hi) {
    f32x16 s0 = scores(lk, 0, col, hi);
    if (ck < 32) mask(s0, ck, hi);
    bf16x8 p0[2];
    softmax(s0, c2, p0);
    bf16x8 pre[PRE];
    if constexpr (PF)
      pv_pf(lvt, 0, col, hi, p0, lk, 1, pre);
    else
      pv(lvt, 0, col, hi, p0);
    if (ck > 32) {
      f32x16 s1 = PF ? scores_pre(lk, 1, col, hi, pre) : scores(lk, 1, col, hi);
      if (ck < 64) mask(s1, ck - 32, hi);
      bf16x8 p1[2];
      softmax(s1, c2, p1);
      pv(lvt, 1, col, hi, p1);
    }
  }

  // One staged chunk of four 16-key units with n[u] (0..16) valid keys each
  // (wave-uniform).  A block whose two units hold no valid key is skipped;
  // any other has a valid key in every query row, so its softmax is finite.
  __device__ __forceinline__ void chunk_units(const uint16_t* lk, const uint16_t* lvt, const int n[4],
                                              float c2, int col, int hi) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int na = n[2 * kb], nb = n[2 * kb + 1];
      if (na + nb == 0) continue;
      f32x16 s = scores(lk, kb, col, hi);
      if (na < 16 || nb < 16) mask_halves(s, na, nb, hi);
      bf16x8 p[2];
      softmax(s, c2, p);
      pv(lvt, kb, col, hi, p);
    }
  }

  // Normalise and write this lane's query row (d channels, bf16) to op.
  // Both lane halves must call it (they exchange partial sums).
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
