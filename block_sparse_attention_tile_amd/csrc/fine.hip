// Fine-grained M x 1 sparse attention (FG-Attn verdict page, arXiv
// 2509.16518: pith_extraction.key_machinery, referee_report.summary and
// major_comments[1]).
//
// The unit of skipping is an M x 1 slice: M consecutive queries against one
// key.  The pooling mask averages the queries of a group into q_avg and keeps
// the keys whose score k . q_avg passes a threshold.  The page's threshold
// formula is garbled and its constant undefined; it is monotone in the score,
// so the threshold is read as a per-head quantile: keep the K = ceil(keep * G
// * N) highest (group, key) scores of the head (ties at the threshold kept).
//
// The mask, exactly (every input):
//   q_avg   exact fp64 sum of the group's bf16 rows, one fp64 division, one
//           rounding to fp32;
//   score   s_gj = sum_c q_avg_g[c] * k_j[c], fp64, added in channel order
//           c = 0..d-1 (every product is exact in fp64);
//   tau     the K-th largest score of the head;
//   lists   per group, the ascending key indices with s >= tau.
//
// How it is evaluated without scoring every pair in fp64:
//   1. Every pair is scored on the matrix cores: q_avg is split into two bf16
//      parts (hi + lo, |q - hi - lo| <= 2^-16 |q|) and
//      v_mfma_f32_32x32x16_bf16 accumulates k . hi + k . lo in fp32, giving
//      a.  The exact score lies in [a - e, a + e] with
//      e = 2^-12 |q_avg| |k| + 2^-22 |a| + 2^-119 |k| + 2^-100 (Euclidean
//      norms rounded up; by Cauchy-Schwarz |q_avg||k| >= sum_c |q_c k_c|,
//      and this MFMA chain stays within 2^-17 of that sum of the exact value,
//      so the first term alone has a 32x margin; the others cover the fp32
//      rounding of a +- e and flushed subnormals).
//   2. Radix histograms over the fp32 order keys of the upper ends u = a + e
//      and of the lower ends l = a - e (two 12-bit levels: sign, exponent and
//      15 mantissa bits) find 24-bit bins holding the K-th largest u and the
//      K-th largest l; tau lies between them.  A pair whose l lies above the
//      u bin is kept for sure (s >= l > tau), one whose u lies below the l
//      bin is dropped for sure (s <= u < tau).
//   3. The pairs in between, a thin band around tau, are rescored exactly and
//      tau is their (K - #kept-for-sure)-th largest score (MSB-first radix
//      select over order-preserving 64-bit keys).
//   4. Kept pairs are set in a bitmask of ceil(N/32) words per group, then
//      compacted per group into ascending key lists of capacity N (ties at
//      tau may keep every pair, and the lists can always hold them).
//   A head whose band overflows the rescoring buffer, whose approximations
//   are not finite, or whose band cannot hold that rank takes the exact
//   path: a radix select over the exact scores of every pair (six passes of
//   12/12/12/12/12/4-bit digits), then the bitmask from exact scores.
// Attention: per group, the kept K and V rows are gathered into LDS (V
// transposed on the way in, address generation spread over all threads) and
// fed to the same MFMA / online-softmax core as the tile path.
#include <hip/hip_runtime.h>

#include <float.h>

#include "attn_core.h"
#include "vsa_internal.h"

namespace vsa {
namespace {

using core::bf16x8;
using core::f32x16;
using core::kKC;
using core::Lds;
using core::u32x4;

constexpr int kBins = 4096;            // 12-bit digits
constexpr long kCandCap = 1L << 18;    // band pairs rescored exactly, per head

struct FineHead {
  int full;                   // 1: the exact path over every pair
  int b1u, b1l;               // level-1 bins of the K-th largest u and l
  int r1u, r1l;               // their ranks inside those bins (1 = largest)
  float vu;                   // largest fp32 value of the u bin: l > vu is kept for sure
  float vl;                   // smallest fp32 value of the l bin: u < vl is dropped for sure
  int ndef;                   // pairs kept for sure
  int ncand;                  // band pairs (may exceed kCandCap)
  int pad0;
  unsigned long long ckmin;   // smallest and largest exact order key of the band
  unsigned long long ckmax;
  int pad[2];
};

struct FineScratch {
  FineHead* head;             // [BH]
  int* hist;                  // [BH][6][kBins]: level-1 u, level-1 l, level-2 u, level-2 l;
                              // the exact path's six digits reuse all six
  uint16_t* qhi;              // [BH][G][D] bf16 high part of q_avg
  uint16_t* qlo;              // [BH][G][D] bf16 low part
  float* nq;                  // [BH][G] |q_avg|, rounded up
  float* nk;                  // [BH][NW * 32] |k_j|, rounded up (0 past N)
  unsigned long long* ckey;   // [BH][kCandCap] exact order keys of band pairs
  int* cpos;                  // [BH][kCandCap] their positions g * N + j
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
__host__ __device__ inline int n_words(int N) { return (N + 31) / 32; }

FineScratch carve(const Geo& g, unsigned char* base) {
  const long BH = (long)g.B * g.H;
  FineScratch f;
  size_t off = 0;
  f.head = reinterpret_cast<FineHead*>(base + off);
  off = align256(off + BH * sizeof(FineHead));
  f.hist = reinterpret_cast<int*>(base + off);
  off = align256(off + (size_t)BH * 6 * kBins * sizeof(int));
  f.qhi = reinterpret_cast<uint16_t*>(base + off);
  off = align256(off + (size_t)BH * g.fine_G * g.d * sizeof(uint16_t));
  f.qlo = reinterpret_cast<uint16_t*>(base + off);
  off = align256(off + (size_t)BH * g.fine_G * g.d * sizeof(uint16_t));
  f.nq = reinterpret_cast<float*>(base + off);
  off = align256(off + (size_t)BH * g.fine_G * sizeof(float));
  f.nk = reinterpret_cast<float*>(base + off);
  off = align256(off + (size_t)BH * n_words(g.N) * 32 * sizeof(float));
  f.ckey = reinterpret_cast<unsigned long long*>(base + off);
  off = align256(off + (size_t)BH * kCandCap * sizeof(unsigned long long));
  f.cpos = reinterpret_cast<int*>(base + off);
  return f;
}

// Order-preserving keys (larger value -> larger key).  fkey is applied to
// l = a - e and u = a + e with e > 0 only: a zero result of a sum of nonzero
// finite values is +0 under round to nearest, so no -0 reaches it.  okey maps
// a zero of either sign to the key of +0, so that key order and value order
// agree on ties.
__device__ __forceinline__ unsigned fkey(float x) {
  const unsigned u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_value(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
__device__ __forceinline__ unsigned long long okey(double v) {
  const unsigned long long u = v == 0.0 ? 0ull : (unsigned long long)__double_as_longlong(v);
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}
__device__ __forceinline__ double okey_value(unsigned long long k) {
  const unsigned long long u = (k & 0x8000000000000000ull) ? (k & 0x7fffffffffffffffull) : ~k;
  return __longlong_as_double((long long)u);
}

// Upward-rounded fp32 of a non-negative fp64 value (a few ulps above).
__device__ __forceinline__ float round_up_f32(double x) {
  return (float)x * (1.0f + 0x1p-20f);
}

__global__ __launch_bounds__(256) void fine_init_kernel(FineScratch f) {
  const long bh = blockIdx.x;
  if (threadIdx.x == 0) {
    FineHead h = {};
    h.ckmin = ~0ull;
    f.head[bh] = h;
  }
  for (int b = threadIdx.x; b < 4 * kBins; b += 256) f.hist[bh * 6 * kBins + b] = 0;
}

// Group means of Q: exact fp64 sums of at most M bf16 values per channel;
// also the bf16 split of each mean for the MFMA scores and its norm.
template <int D>
__global__ __launch_bounds__(D) void fine_qbar_kernel(Geo g, const uint16_t* __restrict__ q,
                                                      float* __restrict__ qbar, FineScratch f) {
  __shared__ double red[D];
  const int gi = blockIdx.x;
  const long bh = blockIdx.y;
  const int c = threadIdx.x;
  const int r0 = gi * g.fine_M;
  const int r1 = min(r0 + g.fine_M, g.N);
  const uint16_t* x = q + bh * (long)g.N * D;
  // eight rows per batch of loads; the fp64 sum of bf16 values is exact (the
  // oracle asserts it), so the grouping of the additions does not matter
  double s = 0.0;
  int r = r0;
  for (; r + 8 <= r1; r += 8) {
    uint16_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = x[(long)(r + i) * D + c];
#pragma unroll
    for (int i = 0; i < 8; ++i) s += (double)__uint_as_float((uint32_t)v[i] << 16);
  }
  for (; r < r1; ++r) s += (double)__uint_as_float((uint32_t)x[(long)r * D + c] << 16);
  const float m = (float)(s / (double)(r1 - r0));
  const long at = (bh * g.fine_G + gi) * D + c;
  qbar[at] = m;
  const __bf16 h = (__bf16)m;                  // round to nearest even
  const __bf16 l = (__bf16)(m - (float)h);     // m - h is exact (Sterbenz)
  f.qhi[at] = __builtin_bit_cast(uint16_t, h);
  f.qlo[at] = __builtin_bit_cast(uint16_t, l);
  red[c] = (double)m * (double)m;
  __syncthreads();
  for (int w = D / 2; w > 0; w >>= 1) {
    if (c < w) red[c] += red[c + w];
    __syncthreads();
  }
  if (c == 0) f.nq[bh * g.fine_G + gi] = round_up_f32(sqrt(red[0]));
}

// Key norms |k_j| (fp64 sums of squares, rounded up); 0 on the pad keys of
// the last 32-key block.
template <int D>
__global__ __launch_bounds__(256) void fine_knorm_kernel(Geo g, const uint16_t* __restrict__ k, FineScratch f) {
  const long bh = blockIdx.y;
  const int NW = n_words(g.N);
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= NW * 32) return;
  float out = 0.f;
  if (j < g.N) {
    const uint16_t* kr = k + (bh * (long)g.N + j) * D;
    double s = 0.0;
#pragma unroll 4
    for (int c8 = 0; c8 < D; c8 += 8) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(kr + c8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double lo = (double)__uint_as_float(w[e] << 16);
        const double hi = (double)__uint_as_float(w[e] & 0xffff0000u);
        s += lo * lo + hi * hi;
      }
    }
    out = round_up_f32(sqrt(s));
  }
  f.nk[bh * (long)NW * 32 + j] = out;
}

// MFMA passes over every (group, key) pair: one workgroup = kAW waves, each
// owning 32 groups (their split means held as B operands), over a segment of
// kSeg 32-key blocks.  Each block's K rows (and key norms) are loaded once
// per workgroup into LDS (double-buffered, rows padded by 16 bytes so that the
// A-fragment reads of 16 consecutive lanes hit distinct banks) and shared by
// the waves.  Lane (col, hi) owns group g0 + col and keys 8 (r / 4) + 4 hi +
// r % 4 of the block in its accumulator registers r.
//   MODE 1: level-1 histograms of u and l (12 leading key bits); a head with
//           a non-finite approximation goes to the exact path.
//   MODE 2: level-2 histograms (next 12 bits) inside the level-1 bins.
//   MODE 3: kept-for-sure bits into the bitmask, kept-for-sure count, band
//           pairs' positions into the rescoring buffer (staged per wave in
//           LDS, one global atomic per 256 or so).
constexpr int kAW = 8;
constexpr int kSeg = 16;
constexpr int kStage = 1280;  // band positions staged per wave (a block adds at most 1024)

template <int D, int MODE>
__global__ __launch_bounds__(kAW * 64, 2) void fine_approx_kernel(
    Geo g, const uint16_t* __restrict__ k, FineScratch f, uint32_t* __restrict__ mask) {
  constexpr int ST = D / 16;
  constexpr int KR = D + 8;            // padded K row (elements)
  constexpr int PIECES = 32 * D / 8;   // 16-byte pieces of a 32-key block
  static_assert(PIECES <= kAW * 64, "one piece per thread");
  constexpr int HB = MODE == 3 ? 1 : kBins;
  __shared__ int hu[HB];
  __shared__ int hl[HB];
  __shared__ int stage[MODE == 3 ? kAW * kStage : 1];
  __shared__ __align__(16) uint16_t kbuf[2][32 * KR];
  __shared__ __align__(16) float nkbuf[2][32];
  __shared__ int sdef;
  const long bh = blockIdx.z;
  const FineHead hd = f.head[bh];
  if (hd.full) return;  // uniform over the workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hi = lane >> 5;
  if constexpr (MODE != 3) {
    for (int b = tid; b < kBins; b += kAW * 64) hu[b] = hl[b] = 0;
  } else {
    if (tid == 0) sdef = 0;
  }
  const int G = g.fine_G, N = g.N, NW = n_words(N);
  const int g0 = (blockIdx.y * kAW + wave) * 32;
  const int gq = min(g0 + col, G - 1);
  const bool gvalid = g0 + col < G;
  const uint16_t* kh = k + bh * (long)N * D;
  const float* nkh = f.nk + bh * (long)NW * 32;
  // this thread's piece of each block: K row pr, 16-byte column pc; threads
  // 0..7 also carry four key norms
  const int pr = tid / (D / 8), pc = tid % (D / 8);
  u32x4 pre = {};
  float4 pre_nk = {};
  auto gload = [&](int kb) {
    if (tid < PIECES) pre = *reinterpret_cast<const u32x4*>(kh + (long)min(kb * 32 + pr, N - 1) * D + pc * 8);
    if (tid < 8) pre_nk = *reinterpret_cast<const float4*>(nkh + kb * 32 + 4 * tid);
  };
  auto lstore = [&](int buf) {
    if (tid < PIECES) *reinterpret_cast<u32x4*>(&kbuf[buf][pr * KR + pc * 8]) = pre;
    if (tid < 8) *reinterpret_cast<float4*>(&nkbuf[buf][4 * tid]) = pre_nk;
  };
  int nonfinite = 0, def = 0;
  int* const wst = stage + (MODE == 3 ? wave * kStage : 0);
  int nst = 0;  // staged band positions (wave-uniform)
  auto flush = [&]() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's staging writes have landed
    int base = 0;
    if (lane == 0) base = atomicAdd(&f.head[bh].ncand, nst);
    base = __shfl(base, 0);
    for (int i = lane; i < nst; i += 64)
      if (base + i < kCandCap) f.cpos[bh * kCandCap + base + i] = wst[i];
    nst = 0;
  };
  bf16x8 qh[ST], ql[ST];
  const long qrow = (bh * G + gq) * (long)D + hi * 8;
#pragma unroll
  for (int st = 0; st < ST; ++st) {
    qh[st] = *reinterpret_cast<const bf16x8*>(f.qhi + qrow + st * 16);
    ql[st] = *reinterpret_cast<const bf16x8*>(f.qlo + qrow + st * 16);
  }
  // e = |k| (2^-12 |q| + 2^-119) + 2^-100 + 2^-22 |a|
  const float cq = 0x1p-12f * f.nq[bh * G + gq] + 0x1p-119f;
  const int kb0 = blockIdx.x * kSeg;
  const int kb_end = min(kb0 + kSeg, NW);
  if (kb0 < kb_end) {
    gload(kb0);
    lstore(0);
  }
  __syncthreads();
  for (int kb = kb0, it = 0; kb < kb_end; ++kb, ++it) {
    const bool nxt = kb + 1 < kb_end;
    if (nxt) gload(kb + 1);
    if (g0 < G) {  // wave-uniform: waves past the last group only join the barriers
      const uint16_t* kr = &kbuf[it & 1][col * KR + hi * 8];
      bf16x8 a[ST];
#pragma unroll
      for (int st = 0; st < ST; ++st) a[st] = *reinterpret_cast<const bf16x8*>(kr + st * 16);
      float4 nk4[4];
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) nk4[qd] = *reinterpret_cast<const float4*>(&nkbuf[it & 1][8 * qd + 4 * hi]);
      f32x16 acc = {};
#pragma unroll
      for (int st = 0; st < ST; ++st) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[st], qh[st], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[st], ql[st], acc, 0, 0, 0);
      }
      unsigned bits = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kin = 8 * (r >> 2) + 4 * hi + (r & 3);  // key inside the block
        const bool valid = gvalid && kb * 32 + kin < N;
        const float av = acc[r];
        const float e = fmaf(0x1p-22f, fabsf(av), fmaf(nk4[r >> 2][r & 3], cq, 0x1p-100f));
        const float lv = av - e, uv = av + e;
        if constexpr (MODE == 1) {
          if (valid) {
            if (!(fabsf(lv) <= FLT_MAX && fabsf(uv) <= FLT_MAX)) nonfinite = 1;
            atomicAdd(&hu[fkey(uv) >> 20], 1);
            atomicAdd(&hl[fkey(lv) >> 20], 1);
          }
        } else if constexpr (MODE == 2) {
          const unsigned ku = fkey(uv), kl = fkey(lv);
          if (valid && (int)(ku >> 20) == hd.b1u) atomicAdd(&hu[(ku >> 8) & (kBins - 1)], 1);
          if (valid && (int)(kl >> 20) == hd.b1l) atomicAdd(&hl[(kl >> 8) & (kBins - 1)], 1);
        } else {
          const bool sure = valid && lv > hd.vu;
          const bool band = valid && !sure && uv >= hd.vl;
          bits |= (unsigned)sure << kin;
          const unsigned long long m = __ballot(band);
          if (band) wst[nst + __popcll(m & ((1ull << lane) - 1ull))] = (g0 + col) * N + kb * 32 + kin;
          nst += __popcll(m);
        }
      }
      if constexpr (MODE == 3) {
        def += __popc(bits);
        const unsigned word = bits | __shfl_xor(bits, 32);
        if (hi == 0 && gvalid) mask[(bh * G + g0 + col) * (long)NW + kb] = word;
        if (nst > kStage - 1024) flush();
      }
    }
    if (nxt) lstore((it + 1) & 1);
    __syncthreads();
  }
  if constexpr (MODE == 3) {
    if (nst) flush();
  }
  if constexpr (MODE == 1) {
    if (__any(nonfinite) && lane == 0) atomicOr(&f.head[bh].full, 1);
  }
  if constexpr (MODE == 3) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) def += __shfl_xor(def, m);
    if (lane == 0 && def) atomicAdd(&sdef, def);
  }
  __syncthreads();
  if constexpr (MODE == 3) {
    if (tid == 0 && sdef) atomicAdd(&f.head[bh].ndef, sdef);
  } else {
    int* gh = f.hist + (bh * 6 + (MODE == 1 ? 0 : 2)) * kBins;
    for (int b = tid; b < kBins; b += kAW * 64) {
      if (hu[b]) atomicAdd(&gh[b], hu[b]);
      if (hl[b]) atomicAdd(&gh[kBins + b], hl[b]);
    }
  }
}

// The bin of an NB-bin histogram (ascending keys) holding the rank-th
// largest element (rank >= 1), and the rank inside that bin; bin = -1 when
// the histogram holds fewer than rank elements.  All NT threads call it.
template <int NT, int NB>
__device__ void rank_bin(const int* h, long rank, int* bin_out, long* rank_out) {
  static_assert(NB % NT == 0, "whole bins per thread");
  constexpr int PER = NB / NT;
  __shared__ long part[NT];
  __shared__ int bin_s;
  __shared__ long rank_s;
  const int t = threadIdx.x;
  long s = 0;
  for (int i = 0; i < PER; ++i) s += h[t * PER + i];
  part[t] = s;
  if (t == 0) bin_s = -1;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {  // inclusive suffix sums
    const long v = t + off < NT ? part[t + off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  const long above = part[t] - s;  // elements in the bins above this thread's range
  if (above < rank && above + s >= rank) {
    long a = above;
    for (int i = PER - 1; i >= 0; --i) {
      const int b = t * PER + i;
      if (a + h[b] >= rank) {
        bin_s = b;
        rank_s = rank - a;
        break;
      }
      a += h[b];
    }
  }
  __syncthreads();
  *bin_out = bin_s;
  *rank_out = bin_s >= 0 ? rank_s : 0;
  __syncthreads();
}

__device__ __forceinline__ void top_rank_bin(const int* h, long rank, int* bin_out, long* rank_out) {
  rank_bin<256, kBins>(h, rank, bin_out, rank_out);
}

__global__ __launch_bounds__(256) void fine_find1_kernel(Geo g, FineScratch f) {
  const long bh = blockIdx.x;
  if (f.head[bh].full) return;
  const int* h = f.hist + bh * 6 * kBins;
  int bu, bl;
  long ru, rl;
  top_rank_bin(h, g.fine_keep, &bu, &ru);
  top_rank_bin(h + kBins, g.fine_keep, &bl, &rl);
  if (threadIdx.x == 0) {
    FineHead& hd = f.head[bh];
    if (bu < 0 || bl < 0) {
      hd.full = 1;
    } else {
      hd.b1u = bu;
      hd.r1u = (int)ru;
      hd.b1l = bl;
      hd.r1l = (int)rl;
    }
  }
}

__global__ __launch_bounds__(256) void fine_find2_kernel(Geo g, FineScratch f) {
  const long bh = blockIdx.x;
  if (f.head[bh].full) return;
  const int* h = f.hist + bh * 6 * kBins;
  const FineHead hd = f.head[bh];
  int bu, bl;
  long ru, rl;
  top_rank_bin(h + 2 * kBins, hd.r1u, &bu, &ru);
  top_rank_bin(h + 3 * kBins, hd.r1l, &bl, &rl);
  if (threadIdx.x == 0) {
    if (bu < 0 || bl < 0) {
      f.head[bh].full = 1;
    } else {
      // keys below 0x00800000 are not finite values: such bins are never
      // reached here (a non-finite approximation sends the head to the exact path)
      f.head[bh].vu = fkey_value(((unsigned)hd.b1u << 20) | ((unsigned)bu << 8) | 0xffu);
      f.head[bh].vl = fkey_value(((unsigned)hd.b1l << 20) | ((unsigned)bl << 8));
    }
  }
}

// Exact fp64 score of one pair: the fixed channel order of the definition.
template <int D>
__device__ __forceinline__ double exact_score(const float* __restrict__ qr, const uint16_t* __restrict__ kr) {
  double s = 0.0;
#pragma unroll 4
  for (int c8 = 0; c8 < D; c8 += 8) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(kr + c8);
    const float4 q0 = *reinterpret_cast<const float4*>(qr + c8);
    const float4 q1 = *reinterpret_cast<const float4*>(qr + c8 + 4);
    const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t wv = w[e >> 1];
      const float kv = __uint_as_float((e & 1) ? (wv & 0xffff0000u) : (wv << 16));
      s = fma((double)qv[e], (double)kv, s);
    }
  }
  return s;
}

// Exact scores of the band pairs (their order keys).
template <int D>
__global__ __launch_bounds__(256) void fine_cand_exact_kernel(Geo g, const uint16_t* __restrict__ k,
                                                              const float* __restrict__ qbar, FineScratch f) {
  const long bh = blockIdx.y;
  const FineHead hd = f.head[bh];
  if (hd.full || hd.ncand > kCandCap) return;
  unsigned long long kmin = ~0ull, kmax = 0ull;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < hd.ncand; i += gridDim.x * 256) {
    const int pos = f.cpos[bh * kCandCap + i];
    const int gi = pos / g.N, j = pos - gi * g.N;
    const double s = exact_score<D>(qbar + (bh * g.fine_G + gi) * (long)D, k + (bh * (long)g.N + j) * D);
    const unsigned long long key = okey(s);
    f.ckey[bh * kCandCap + i] = key;
    kmin = min(kmin, key);
    kmax = max(kmax, key);
  }
  for (int m = 1; m < 64; m <<= 1) {
    kmin = min(kmin, (unsigned long long)__shfl_xor((long long)kmin, m));
    kmax = max(kmax, (unsigned long long)__shfl_xor((long long)kmax, m));
  }
  if ((threadIdx.x & 63) == 0 && kmax >= kmin) {
    atomicMin(&f.head[bh].ckmin, kmin);
    atomicMax(&f.head[bh].ckmax, kmax);
  }
}

// tau of a head whose band was rescored: its (K - kept-for-sure)-th largest
// exact score, by an MSB-first radix select (11-bit digits) over the bits
// below the band's common key prefix.  A head that cannot be finished this
// way (band beyond the buffer, rank outside the band) is switched to the
// exact path here, whose histograms start at zero.
constexpr int kSelBits = 11;
__global__ __launch_bounds__(1024) void fine_select_kernel(Geo g, FineScratch f, double* __restrict__ tau) {
  __shared__ int h[1 << kSelBits];
  __shared__ unsigned long long prefix_s;
  __shared__ int need_s, ok_s;
  const long bh = blockIdx.x;
  const int tid = threadIdx.x;
  if (tid == 0) {
    FineHead& hd = f.head[bh];
    const long need = g.fine_keep - (long)hd.ndef;
    const int ok = !hd.full && hd.ncand <= kCandCap && need >= 1 && need <= hd.ncand;
    if (!ok) hd.full = 1;
    ok_s = ok;
    need_s = (int)need;
  }
  __syncthreads();
  if (!ok_s) {
    for (int b = tid; b < 6 * kBins; b += 1024) f.hist[bh * 6 * kBins + b] = 0;
    return;
  }
  const FineHead hd = f.head[bh];
  const int n = hd.ncand;
  const unsigned long long* c = f.ckey + bh * kCandCap;
  const unsigned long long diff = hd.ckmin ^ hd.ckmax;
  if (diff == 0) {  // every band score is the same value
    if (tid == 0) tau[bh] = okey_value(hd.ckmin);
    return;
  }
  const int top = 63 - __clzll((long long)diff);  // highest bit that differs inside the band
  if (tid == 0) prefix_s = top == 63 ? 0ull : (hd.ckmin & ~((2ull << top) - 1ull));
  for (int hb = top; hb >= 0; hb -= kSelBits) {
    const int lb = max(hb - kSelBits + 1, 0);
    const unsigned long long pm = hb == 63 ? 0ull : ~((2ull << hb) - 1ull);
    const unsigned dm = (1u << (hb - lb + 1)) - 1u;
    for (int b = tid; b < (1 << kSelBits); b += 1024) h[b] = 0;
    __syncthreads();
    const unsigned long long prefix = prefix_s;
    for (int e0 = tid; e0 < n; e0 += 4 * 1024) {
      unsigned long long key[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) key[u] = e0 + u * 1024 < n ? c[e0 + u * 1024] : 0ull;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (e0 + u * 1024 < n && (key[u] & pm) == prefix) atomicAdd(&h[(key[u] >> lb) & dm], 1);
    }
    __syncthreads();
    int d;
    long r;
    rank_bin<1024, (1 << kSelBits)>(h, need_s, &d, &r);  // bins above dm are empty
    if (tid == 0) {
      prefix_s = prefix | ((unsigned long long)max(d, 0) << lb);
      need_s = (int)r;
    }
    __syncthreads();
  }
  if (tid == 0) tau[bh] = okey_value(prefix_s);
}

// Band pairs at or above tau join the kept-for-sure bits.
__global__ __launch_bounds__(256) void fine_cand_emit_kernel(Geo g, FineScratch f, const double* __restrict__ tau,
                                                             uint32_t* __restrict__ mask) {
  const long bh = blockIdx.y;
  const FineHead hd = f.head[bh];
  if (hd.full) return;
  const double t = tau[bh];
  const int NW = n_words(g.N);
  for (int i = blockIdx.x * 256 + threadIdx.x; i < hd.ncand; i += gridDim.x * 256) {
    if (okey_value(f.ckey[bh * kCandCap + i]) >= t) {
      const int pos = f.cpos[bh * kCandCap + i];
      const int gi = pos / g.N, j = pos - gi * g.N;
      atomicOr(&mask[(bh * g.fine_G + gi) * (long)NW + (j >> 5)], 1u << (j & 31));
    }
  }
}

// ---- the exact path (heads flagged full) -----------------------------------
// Tiles of 16 groups x 1024 keys: 4 keys per thread (256 apart, so 64 lanes
// hold 64 consecutive keys), group means staged channel-major in LDS and read
// as broadcasts, fixed-order fp64 sums.
constexpr int kXG = 16;
constexpr int kXK = 4;
constexpr int kXBlocks = 128;  // workgroups per head (grid-stride over tiles)
__constant__ int kXShift[6] = {52, 40, 28, 16, 4, 0};
__constant__ int kXBits[6] = {12, 12, 12, 12, 12, 4};

template <int D>
__device__ __forceinline__ void exact_tile(const Geo& g, long bh, int tile, const float* __restrict__ qbar,
                                           const uint16_t* __restrict__ k, double (*qs)[kXG],
                                           double acc[kXK][kXG], int& g0, int& jb) {
  const int tiles_k = (g.N + 256 * kXK - 1) / (256 * kXK);
  g0 = (tile / tiles_k) * kXG;
  jb = (tile % tiles_k) * 256 * kXK;
  const int ng = min(kXG, g.fine_G - g0);
  __syncthreads();  // the previous tile's reads of qs are done
  for (int i = threadIdx.x; i < D * kXG; i += 256) {
    const int x = i / D, c = i % D;
    qs[c][x] = x < ng ? (double)qbar[(bh * g.fine_G + g0 + x) * (long)D + c] : 0.0;
  }
  __syncthreads();
  const uint16_t* kr[kXK];
#pragma unroll
  for (int t = 0; t < kXK; ++t) kr[t] = k + (bh * (long)g.N + min(jb + 256 * t + (int)threadIdx.x, g.N - 1)) * D;
#pragma unroll
  for (int t = 0; t < kXK; ++t)
#pragma unroll
    for (int x = 0; x < kXG; ++x) acc[t][x] = 0.0;
  for (int p8 = 0; p8 < D / 8; ++p8) {
    u32x4 w4[kXK];
#pragma unroll
    for (int t = 0; t < kXK; ++t) w4[t] = *reinterpret_cast<const u32x4*>(kr[t] + p8 * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = p8 * 8 + e;
      double kv[kXK];
#pragma unroll
      for (int t = 0; t < kXK; ++t) {
        const uint32_t w = w4[t][e >> 1];
        kv[t] = (double)__uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
      }
#pragma unroll
      for (int x = 0; x < kXG; x += 2) {
        const double2 qq = *reinterpret_cast<const double2*>(&qs[c][x]);
#pragma unroll
        for (int t = 0; t < kXK; ++t) {
          acc[t][x] = fma(qq.x, kv[t], acc[t][x]);
          acc[t][x + 1] = fma(qq.y, kv[t], acc[t][x + 1]);
        }
      }
    }
  }
}

// The exact path's key prefix after npass digits and the rank inside it,
// from the histograms of those digits (every workgroup works it out itself,
// so no launch of its own is needed between two passes).  All 256 threads.
__device__ void exact_prefix(const Geo& g, const FineScratch& f, long bh, int npass, unsigned long long* prefix,
                             long* need) {
  unsigned long long p = 0ull;
  long r = g.fine_keep;
  for (int q = 0; q < npass; ++q) {
    int d;
    long rr;
    top_rank_bin(f.hist + (bh * 6 + q) * kBins, r, &d, &rr);  // d >= 0: every pair is counted
    p |= (unsigned long long)max(d, 0) << kXShift[q];
    r = rr;
  }
  *prefix = p;
  *need = r;
}

// Digit `pass` of the radix select over the exact scores of every pair.
template <int D>
__global__ __launch_bounds__(256) void fine_exact_pass_kernel(Geo g, const uint16_t* __restrict__ k,
                                                              const float* __restrict__ qbar, FineScratch f,
                                                              int pass) {
  __shared__ __align__(16) double qs[D][kXG];
  __shared__ int h[kBins];
  const long bh = blockIdx.y;
  if (!f.head[bh].full) return;
  unsigned long long prefix;
  long need;
  exact_prefix(g, f, bh, pass, &prefix, &need);
  const int shift = kXShift[pass], bits = kXBits[pass];
  const unsigned long long pm = pass == 0 ? 0ull : (~0ull << (shift + bits));
  const unsigned long long dm = (1ull << bits) - 1ull;
  for (int b = threadIdx.x; b < kBins; b += 256) h[b] = 0;
  const int tiles = ((g.fine_G + kXG - 1) / kXG) * ((g.N + 256 * kXK - 1) / (256 * kXK));
  for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    double acc[kXK][kXG];
    int g0, jb;
    exact_tile<D>(g, bh, tile, qbar, k, qs, acc, g0, jb);
#pragma unroll
    for (int t = 0; t < kXK; ++t) {
      const int j = jb + 256 * t + threadIdx.x;
#pragma unroll
      for (int x = 0; x < kXG; ++x) {
        if (j < g.N && g0 + x < g.fine_G) {
          const unsigned long long key = okey(acc[t][x]);
          if ((key & pm) == prefix) atomicAdd(&h[(key >> shift) & dm], 1);
        }
      }
    }
  }
  __syncthreads();
  int* gh = f.hist + (bh * 6 + pass) * kBins;
  for (int b = threadIdx.x; b < kBins; b += 256)
    if (h[b]) atomicAdd(&gh[b], h[b]);
}

// tau of an exact-path head (all six digits) and its kept bits from exact
// scores (every word written).
template <int D>
__global__ __launch_bounds__(256) void fine_exact_emit_kernel(Geo g, const uint16_t* __restrict__ k,
                                                              const float* __restrict__ qbar, FineScratch f,
                                                              double* __restrict__ tau,
                                                              uint32_t* __restrict__ mask) {
  __shared__ __align__(16) double qs[D][kXG];
  const long bh = blockIdx.y;
  if (!f.head[bh].full) return;
  unsigned long long prefix;
  long need;
  exact_prefix(g, f, bh, 6, &prefix, &need);
  const double tv = okey_value(prefix);
  if (blockIdx.x == 0 && threadIdx.x == 0) tau[bh] = tv;
  const int NW = n_words(g.N);
  const int lane = threadIdx.x & 63;
  const int tiles = ((g.fine_G + kXG - 1) / kXG) * ((g.N + 256 * kXK - 1) / (256 * kXK));
  for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    double acc[kXK][kXG];
    int g0, jb;
    exact_tile<D>(g, bh, tile, qbar, k, qs, acc, g0, jb);
#pragma unroll
    for (int t = 0; t < kXK; ++t) {
      const int j = jb + 256 * t + threadIdx.x;
      const int w0 = (j - lane) >> 5;  // this wave's 64 keys start on a word boundary
#pragma unroll
      for (int x = 0; x < kXG; ++x) {
        const unsigned long long b = __ballot(j < g.N && acc[t][x] >= tv);
        if (g0 + x < g.fine_G) {
          uint32_t* row = mask + (bh * g.fine_G + g0 + x) * (long)NW;
          if (lane == 0 && w0 < NW) row[w0] = (uint32_t)b;
          if (lane == 32 && w0 + 1 < NW) row[w0 + 1] = (uint32_t)(b >> 32);
        }
      }
    }
  }
}

// Per group: the kept bits as an ascending key list (capacity N) and its
// length.  The words of a chunk of 8192 keys go to LDS; each wave counts a
// quarter of them, then writes its quarter's kept keys in order, 64 keys per
// ballot (coalesced stores).
constexpr int kCompactWords = 256;
__global__ __launch_bounds__(256) void fine_compact_kernel(Geo g, const uint32_t* __restrict__ mask,
                                                           int* __restrict__ count, int* __restrict__ idx) {
  __shared__ uint32_t wl[kCompactWords];
  __shared__ int qcnt[4];
  const int gi = blockIdx.x;
  const long bh = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int NW = n_words(g.N);
  const long row = bh * g.fine_G + gi;
  const uint32_t* m = mask + row * NW;
  int* out = idx + row * (long)g.N;
  int base = 0;
  for (int c0 = 0; c0 < NW; c0 += kCompactWords) {
    const int nw = min(kCompactWords, NW - c0);
    const uint32_t w = t < nw ? m[c0 + t] : 0u;
    wl[t] = w;
    int pc = __popc(w);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) pc += __shfl_xor(pc, o);
    if (lane == 0) qcnt[wave] = pc;
    __syncthreads();
    int o = base;
    for (int x = 0; x < wave; ++x) o += qcnt[x];
    const int total = qcnt[0] + qcnt[1] + qcnt[2] + qcnt[3];
    // this wave's 64 words, two per ballot
    for (int p = 0; p < 32; ++p) {
      const int wi = wave * 64 + 2 * p + (lane >> 5);
      const bool keep = (wl[wi] >> (lane & 31)) & 1u;
      const unsigned long long bal = __ballot(keep);
      if (keep) out[o + __popcll(bal & ((1ull << lane) - 1ull))] = (c0 + wi) * 32 + (lane & 31);
      o += __popcll(bal);
    }
    base += total;
    __syncthreads();
  }
  if (t == 0) count[row] = base;
}

// ---------------------------------------------------------------------------
// Gathered attention: one workgroup per (head, group), M/32 waves.

template <int D, int NW>
struct GatherLoader {
  static constexpr int P = D / 8;                  // 16-byte pieces per row
  static constexpr int T = NW * 64;
  static constexpr int NP = (kKC * P + T - 1) / T; // K pieces per thread
  static constexpr int NQ = (kKC / 4 * P + T - 1) / T;  // V quads (4 keys x 8 channels) per thread
  u32x4 kr[NP];
  u32x4 vr[NQ][4];

  // K pieces: piece-fastest (a key row is read by consecutive lanes).
  // V quads: 4 consecutive keys x 8 channels per thread, key quads fastest,
  // so that 16 lanes write one 128-byte run of a transposed LDS row.  Rows
  // past the chunk re-read its last valid key.  The chunk's key indices come
  // from an LDS copy (keys), so the row loads issue without waiting on a
  // global load.
  int n_tok;  // tokens per head (key indices are clamped below it)
  __device__ __forceinline__ int key_at(const int* keys, int r) const {
    return min(max(keys[r], 0), n_tok - 1);
  }

  __device__ __forceinline__ void load(const uint16_t* __restrict__ kh, const uint16_t* __restrict__ vh,
                                       const int* keys, int nk) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int x = 0; x < NP; ++x) {
      const int pc = min(tid + x * T, kKC * P - 1);
      const int kr_row = min(pc / P, nk - 1), kp = pc % P;
      kr[x] = *reinterpret_cast<const u32x4*>(kh + (long)key_at(keys, kr_row) * D + kp * 8);
    }
#pragma unroll
    for (int x = 0; x < NQ; ++x) {
      const int qd = min(tid + x * T, kKC / 4 * P - 1);
      const int j = qd % (kKC / 4), p = qd / (kKC / 4);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        vr[x][t] = *reinterpret_cast<const u32x4*>(vh + (long)key_at(keys, min(4 * j + t, nk - 1)) * D + p * 8);
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds) {
    const int tid = threadIdx.x;
    uint16_t* lk = lds;
    uint16_t* lvt = lds + Lds<D>::KE;
#pragma unroll
    for (int x = 0; x < NP; ++x) {
      const int pc = min(tid + x * T, kKC * P - 1);
      *reinterpret_cast<u32x4*>(lk + Lds<D>::k_off(pc / P, pc % P)) = kr[x];
    }
#pragma unroll
    for (int x = 0; x < NQ; ++x) {
      const int qd = min(tid + x * T, kKC / 4 * P - 1);
      const int j = qd % (kKC / 4), p = qd / (kKC / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // channels p*8 + 2e (low halves) and p*8 + 2e + 1 (high halves) of keys 4j .. 4j+3
        const uint32_t w0 = vr[x][0][e], w1 = vr[x][1][e], w2 = vr[x][2][e], w3 = vr[x][3][e];
        uint2 lo, hi;
        lo.x = (w0 & 0xffffu) | (w1 << 16);
        lo.y = (w2 & 0xffffu) | (w3 << 16);
        hi.x = (w0 >> 16) | (w1 & 0xffff0000u);
        hi.y = (w2 >> 16) | (w3 & 0xffff0000u);
        const int d0 = p * 8 + 2 * e;
        *reinterpret_cast<uint2*>(lvt + Lds<D>::v_off(d0, 0) + 4 * j) = lo;
        *reinterpret_cast<uint2*>(lvt + Lds<D>::v_off(d0 + 1, 0) + 4 * j) = hi;
      }
    }
  }
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void fine_attend_kernel(Geo g, const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ v,
                                                              const int* __restrict__ count,
                                                              const int* __restrict__ idx,
                                                              uint16_t* __restrict__ o) {
  extern __shared__ __align__(16) uint16_t lds[];
  // XCD-major: the hardware deals consecutive workgroups to the eight XCDs
  // in turn; each XCD takes one contiguous range of (head, group) items, so
  // neighbouring groups, whose kept keys overlap (about half of them for
  // adjacent groups of smooth inputs), gather through the same L2
  const long n_items = (long)g.B * g.H * g.fine_G;
  const long per_xcd = (n_items + kNumXcd - 1) / kNumXcd;
  const long item = (blockIdx.x % kNumXcd) * per_xcd + blockIdx.x / kNumXcd;
  if (item >= n_items) return;
  const int gi = (int)(item % g.fine_G);
  const long bh = item / g.fine_G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hi = lane >> 5;
  const int row0 = gi * g.fine_M + wave * 32;                 // first query row of this wave
  const int rows_end = min(gi * g.fine_M + g.fine_M, g.N);
  const bool active = row0 < rows_end;
  const int qrow = min(row0 + col, g.N - 1);
  const long head = bh * (long)g.N * D;
  core::WaveState<D> ws;
  if (active) ws.init(q + head + (long)qrow * D, hi);
  const float c2 = (float)(g.scale * 1.4426950408889634);
  // (the list length is clamped to its capacity N: a mask that was never
  // written still keeps every access in bounds; key indices are clamped on
  // load)
  const long row = bh * g.fine_G + gi;
  const int n = min(max(count[row], 0), g.N);
  const int* keys = idx + row * (long)g.N;

  // One LDS stage: the next chunk's rows are gathered into registers while
  // the current one is multiplied, then written over it between two
  // barriers (a small stage lets four workgroups share a CU).  Two 64-entry
  // LDS buffers hold the key indices of the next chunks: chunk c's in buffer
  // c % 2.  While chunk c is multiplied, wave 0 fetches the indices of chunk
  // c + 2 into a register and writes them over chunk c's between the
  // barriers.
  int* const ibuf = reinterpret_cast<int*>(lds + Lds<D>::STAGE);
  for (int x = tid; x < 2 * kKC; x += NW * 64) ibuf[x] = n > 0 ? keys[min(x, n - 1)] : 0;
  __syncthreads();
  GatherLoader<D, NW> ld;
  ld.n_tok = g.N;
  if (n > 0) {
    ld.load(k + head, v + head, ibuf, min(kKC, n));
    ld.store(lds);
  }
  __syncthreads();
  for (int e0 = 0, c = 0; e0 < n; e0 += kKC, ++c) {
    const int e1 = e0 + kKC;
    const bool has_next = e1 < n;
    const bool has_next2 = e1 + kKC < n;
    int pf = 0;
    if (has_next2 && tid < kKC) pf = keys[min(e1 + kKC + tid, n - 1)];
    if (has_next) ld.load(k + head, v + head, ibuf + ((c + 1) & 1) * kKC, min(kKC, n - e1));
    if (active) ws.chunk(lds, lds + Lds<D>::KE, min(kKC, n - e0), c2, col, hi);
    if (has_next) {
      __syncthreads();
      ld.store(lds);
      if (has_next2 && tid < kKC) ibuf[(c & 1) * kKC + tid] = pf;
      __syncthreads();
    }
  }
  if (!active) return;
  const bool valid = row0 + col < rows_end;
  ws.store(o + head + (long)qrow * D, hi, valid);
}

template <int D, int NW>
hipError_t launch_fine_attend_t(const Geo& g, const Ws& w, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, uint16_t* o, hipStream_t s) {
  const size_t shmem = Lds<D>::STAGE * sizeof(uint16_t) + 2 * kKC * sizeof(int);  // stage, index buffers
  hipError_t e = ensure_dyn_lds(reinterpret_cast<const void*>(&fine_attend_kernel<D, NW>), shmem);
  if (e != hipSuccess) return e;
  const long items = (long)g.B * g.H * g.fine_G;  // below 2^31 (checked at plan time)
  const long per_xcd = (items + kNumXcd - 1) / kNumXcd;
  hipLaunchKernelGGL((fine_attend_kernel<D, NW>), dim3((unsigned)(per_xcd * kNumXcd)), dim3(NW * 64), shmem, s,
                     g, q, k, v, w.fine_count, w.fine_idx, o);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fine_attend_d(const Geo& g, const Ws& w, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, uint16_t* o, hipStream_t s) {
  int nw = (g.fine_M + 31) / 32;
  // At d = 128 one wave would hold a whole gathered chunk in its registers
  // and spill; a second wave (whose rows belong to the next group, so it
  // only gathers) halves that.
  if (D == 128 && nw < 2) nw = 2;
  switch (nw) {
    case 1: return launch_fine_attend_t<D, 1>(g, w, q, k, v, o, s);
    case 2: return launch_fine_attend_t<D, 2>(g, w, q, k, v, o, s);
    case 3: return launch_fine_attend_t<D, 3>(g, w, q, k, v, o, s);
    case 4: return launch_fine_attend_t<D, 4>(g, w, q, k, v, o, s);
    case 5: return launch_fine_attend_t<D, 5>(g, w, q, k, v, o, s);
    case 6: return launch_fine_attend_t<D, 6>(g, w, q, k, v, o, s);
    case 7: return launch_fine_attend_t<D, 7>(g, w, q, k, v, o, s);
    default: return launch_fine_attend_t<D, 8>(g, w, q, k, v, o, s);
  }
}

}  // namespace

size_t fine_scratch_bytes(const Geo& g) {
  const long BH = (long)g.B * g.H;
  size_t off = align256(BH * sizeof(FineHead));
  off = align256(off + (size_t)BH * 6 * kBins * sizeof(int));
  off = align256(off + (size_t)BH * g.fine_G * g.d * sizeof(uint16_t));
  off = align256(off + (size_t)BH * g.fine_G * g.d * sizeof(uint16_t));
  off = align256(off + (size_t)BH * g.fine_G * sizeof(float));
  off = align256(off + (size_t)BH * n_words(g.N) * 32 * sizeof(float));
  off = align256(off + (size_t)BH * kCandCap * sizeof(unsigned long long));
  off += (size_t)BH * kCandCap * sizeof(int);
  return off;
}

template <int D>
hipError_t launch_fine_select_d(const Geo& g, const Ws& w, const uint16_t* q, const uint16_t* k,
                                hipStream_t s) {
  const FineScratch f = carve(g, w.scratch);
  const unsigned BH = (unsigned)(g.B * g.H);
  const int NW = n_words(g.N);
  uint32_t* mask = w.fine_mask;
  hipLaunchKernelGGL(fine_init_kernel, dim3(BH), dim3(256), 0, s, f);
  hipLaunchKernelGGL(fine_qbar_kernel<D>, dim3(g.fine_G, BH), dim3(D), 0, s, g, q, w.fine_qbar, f);
  hipLaunchKernelGGL(fine_knorm_kernel<D>, dim3((NW * 32 + 255) / 256, BH), dim3(256), 0, s, g, k, f);
  const dim3 ag((NW + kSeg - 1) / kSeg, (g.fine_G + kAW * 32 - 1) / (kAW * 32), BH);
  hipLaunchKernelGGL((fine_approx_kernel<D, 1>), ag, dim3(kAW * 64), 0, s, g, k, f, mask);
  hipLaunchKernelGGL(fine_find1_kernel, dim3(BH), dim3(256), 0, s, g, f);
  hipLaunchKernelGGL((fine_approx_kernel<D, 2>), ag, dim3(kAW * 64), 0, s, g, k, f, mask);
  hipLaunchKernelGGL(fine_find2_kernel, dim3(BH), dim3(256), 0, s, g, f);
  hipLaunchKernelGGL((fine_approx_kernel<D, 3>), ag, dim3(kAW * 64), 0, s, g, k, f, mask);
  hipLaunchKernelGGL(fine_cand_exact_kernel<D>, dim3(64, BH), dim3(256), 0, s, g, k, w.fine_qbar, f);
  hipLaunchKernelGGL(fine_select_kernel, dim3(BH), dim3(1024), 0, s, g, f, w.fine_tau);
  hipLaunchKernelGGL(fine_cand_emit_kernel, dim3(64, BH), dim3(256), 0, s, g, f, w.fine_tau, mask);
  // the exact path: every launch returns at once for heads not on it
  for (int pass = 0; pass < 6; ++pass)
    hipLaunchKernelGGL(fine_exact_pass_kernel<D>, dim3(kXBlocks, BH), dim3(256), 0, s, g, k, w.fine_qbar, f,
                       pass);
  hipLaunchKernelGGL(fine_exact_emit_kernel<D>, dim3(kXBlocks, BH), dim3(256), 0, s, g, k, w.fine_qbar, f,
                     w.fine_tau, mask);
  hipLaunchKernelGGL(fine_compact_kernel, dim3(g.fine_G, BH), dim3(256), 0, s, g, mask, w.fine_count,
                     w.fine_idx);
  return hipGetLastError();
}

hipError_t launch_fine_select(const Geo& g, const Ws& w, const uint16_t* q, const uint16_t* k,
                              hipStream_t s) {
  return g.d == 128 ? launch_fine_select_d<128>(g, w, q, k, s) : launch_fine_select_d<64>(g, w, q, k, s);
}

hipError_t launch_fine_attend(const Geo& g, const Ws& w, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, uint16_t* o, hipStream_t s) {
  return g.d == 128 ? launch_fine_attend_d<128>(g, w, q, k, v, o, s)
                    : launch_fine_attend_d<64>(g, w, q, k, v, o, s);
}

}  // namespace vsa
