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
// Mask (bit-reproducible by construction):
//   q_avg   exact fp64 sum of the group's bf16 rows, one fp64 division, one
//           rounding to fp32;
//   score   s_gj = sum_c q_avg_g[c] * k_j[c], fp64, added in channel order
//           c = 0..d-1 (every product is exact in fp64, so fused and unfused
//           multiply-add agree);
//   tau     the K-th largest score of the head: a 4096-bin value histogram
//           between the head's min and max finds the bin holding it, the
//           scores of that bin are gathered and an MSB-first radix select over
//           their order-preserving 64-bit keys finds the exact value;
//   lists   per group, the ascending key indices with s >= tau (CSR).
// Attention: per group, the kept K and V rows are gathered into LDS (V
// transposed on the way in, address generation spread over all threads) and
// fed to the same MFMA / online-softmax core as the tile path.
#include <hip/hip_runtime.h>

#include "attn_core.h"
#include "vsa_internal.h"

namespace vsa {
namespace {

using core::kKC;
using core::Lds;
using core::u32x4;

constexpr int kBins = 4096;
constexpr long kCandCap = 1L << 20;  // gathered scores of the threshold bin, per head

struct FineHead {
  unsigned long long kmin, kmax;  // order-preserving keys of the min / max score
  int bin;                        // histogram bin holding the K-th largest score
  int above;                      // scores in higher bins
  int need;                       // rank of tau inside `bin` (1 = largest)
  int ncand;                      // gathered candidates
  int overflow;                   // 1: candidates overflowed, 2: list capacity overflowed
  int pad[7];
};

struct FineScratch {
  FineHead* head;                 // [BH]
  int* hist;                      // [BH][kBins]
  double* qbar64;                 // [BH][G][D]
  unsigned long long* cand;       // [BH][kCandCap]
  int* cpos;                      // [BH][kCandCap] position g * N + j of each candidate
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

FineScratch carve(const Geo& g, unsigned char* base) {
  const long BH = (long)g.B * g.H;
  FineScratch f;
  size_t off = 0;
  f.head = reinterpret_cast<FineHead*>(base + off);
  off = align256(off + BH * sizeof(FineHead));
  f.hist = reinterpret_cast<int*>(base + off);
  off = align256(off + BH * kBins * sizeof(int));
  f.qbar64 = reinterpret_cast<double*>(base + off);
  off = align256(off + (size_t)BH * g.fine_G * g.d * sizeof(double));
  f.cand = reinterpret_cast<unsigned long long*>(base + off);
  off = align256(off + (size_t)BH * kCandCap * sizeof(unsigned long long));
  f.cpos = reinterpret_cast<int*>(base + off);
  return f;
}

__device__ __forceinline__ unsigned long long okey(double v) {
  const unsigned long long u = __double_as_longlong(v);
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}
__device__ __forceinline__ double okey_value(unsigned long long k) {
  const unsigned long long u = (k & 0x8000000000000000ull) ? (k & 0x7fffffffffffffffull) : ~k;
  return __longlong_as_double((long long)u);
}

__device__ __forceinline__ int score_bin(double s, double lo, double inv_w) {
  const double t = (s - lo) * inv_w;
  int b = (int)t;
  return b < 0 ? 0 : (b >= kBins ? kBins - 1 : b);
}

__global__ __launch_bounds__(256) void fine_init_kernel(Geo g, FineScratch f, int* __restrict__ count) {
  const long bh = blockIdx.x;
  if (threadIdx.x == 0) {
    FineHead h = {};
    h.kmin = ~0ull;
    h.kmax = 0ull;
    f.head[bh] = h;
  }
  for (int b = threadIdx.x; b < kBins; b += 256) f.hist[bh * kBins + b] = 0;
  for (int gi = threadIdx.x; gi < g.fine_G; gi += 256) count[bh * g.fine_G + gi] = 0;
}

// Group means of Q: exact fp64 sums of at most M bf16 values per channel.
template <int D>
__global__ __launch_bounds__(D) void fine_qbar_kernel(Geo g, const uint16_t* __restrict__ q,
                                                      float* __restrict__ qbar, FineScratch f) {
  const int gi = blockIdx.x;
  const long bh = blockIdx.y;
  const int c = threadIdx.x;
  const int r0 = gi * g.fine_M;
  const int r1 = min(r0 + g.fine_M, g.N);
  const uint16_t* x = q + bh * (long)g.N * D;
  double s = 0.0;
  for (int r = r0; r < r1; ++r) s += (double)__uint_as_float((uint32_t)x[(long)r * D + c] << 16);
  const float m = (float)(s / (double)(r1 - r0));
  qbar[(bh * g.fine_G + gi) * D + c] = m;
  f.qbar64[(bh * g.fine_G + gi) * D + c] = (double)m;
}

constexpr int kScoreGroups = 16;
constexpr int kScoreKeys = 4;

// Scores of 16 groups x 1024 keys per workgroup, four keys per thread (keys
// 256 apart, so every load instruction is coalesced).  The 16 group means
// are staged channel-major in LDS and read as wave-wide broadcasts, each
// feeding 4 keys x 2 groups of fp64 FMAs.  Every score is the sequential
// fp64 sum over channels c = 0 .. D-1 of the exact products qbar[c] * k[c].
template <int D>
__global__ __launch_bounds__(256, 2) void fine_score_kernel(Geo g, const uint16_t* __restrict__ k,
                                                            const double* __restrict__ qbar64,
                                                            double* __restrict__ score, FineScratch f) {
  __shared__ __align__(16) double qs[D][kScoreGroups];
  const int g0 = blockIdx.y * kScoreGroups;
  const long bh = blockIdx.z;
  const int ng = min(kScoreGroups, g.fine_G - g0);
  const double* qb = qbar64 + (bh * g.fine_G + g0) * (long)D;
  for (int i = threadIdx.x; i < D * kScoreGroups; i += 256) {
    const int x = i / D, c = i % D;
    qs[c][x] = x < ng ? qb[(long)x * D + c] : 0.0;
  }
  __syncthreads();
  const int jb = blockIdx.x * 256 * kScoreKeys + threadIdx.x;
  const uint16_t* kr[kScoreKeys];
#pragma unroll
  for (int t = 0; t < kScoreKeys; ++t) kr[t] = k + (bh * (long)g.N + min(jb + 256 * t, g.N - 1)) * D;
  double acc[kScoreKeys][kScoreGroups];
#pragma unroll
  for (int t = 0; t < kScoreKeys; ++t)
#pragma unroll
    for (int x = 0; x < kScoreGroups; ++x) acc[t][x] = 0.0;
  // the next 8 channels of every key are loaded while these 8 are summed
  u32x4 w4[kScoreKeys], nx[kScoreKeys];
#pragma unroll
  for (int t = 0; t < kScoreKeys; ++t) w4[t] = *reinterpret_cast<const u32x4*>(kr[t]);
  for (int p8 = 0; p8 < D / 8; ++p8) {
    if (p8 + 1 < D / 8) {
#pragma unroll
      for (int t = 0; t < kScoreKeys; ++t) nx[t] = *reinterpret_cast<const u32x4*>(kr[t] + (p8 + 1) * 8);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = p8 * 8 + e;
      double kv[kScoreKeys];
#pragma unroll
      for (int t = 0; t < kScoreKeys; ++t) {
        const uint32_t w = w4[t][e >> 1];
        kv[t] = (double)__uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
      }
#pragma unroll
      for (int x = 0; x < kScoreGroups; x += 2) {
        const double2 qq = *reinterpret_cast<const double2*>(&qs[c][x]);
#pragma unroll
        for (int t = 0; t < kScoreKeys; ++t) {
          acc[t][x] = fma(qq.x, kv[t], acc[t][x]);
          acc[t][x + 1] = fma(qq.y, kv[t], acc[t][x + 1]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < kScoreKeys; ++t) w4[t] = nx[t];
  }
  unsigned long long kmin = ~0ull, kmax = 0ull;
#pragma unroll
  for (int t = 0; t < kScoreKeys; ++t) {
    const int j = jb + 256 * t;
    if (j < g.N) {
      double* dst = score + (bh * g.fine_G + g0) * (long)g.N + j;
#pragma unroll
      for (int x = 0; x < kScoreGroups; ++x) {
        if (x < ng) {
          dst[(long)x * g.N] = acc[t][x];
          const unsigned long long kk = okey(acc[t][x]);
          kmin = min(kmin, kk);
          kmax = max(kmax, kk);
        }
      }
    }
  }
  for (int m = 1; m < 64; m <<= 1) {
    kmin = min(kmin, (unsigned long long)__shfl_xor((long long)kmin, m));
    kmax = max(kmax, (unsigned long long)__shfl_xor((long long)kmax, m));
  }
  if ((threadIdx.x & 63) == 0) {
    atomicMin(&f.head[bh].kmin, kmin);
    atomicMax(&f.head[bh].kmax, kmax);
  }
}

constexpr int kSpan = 1 << 16;  // scores per workgroup in the histogram / gather passes

__global__ __launch_bounds__(256) void fine_hist_kernel(Geo g, const double* __restrict__ score,
                                                        FineScratch f) {
  __shared__ int h[kBins];
  const long bh = blockIdx.y;
  const long total = (long)g.fine_G * g.N;
  const long s0 = (long)blockIdx.x * kSpan;
  if (s0 >= total) return;
  for (int b = threadIdx.x; b < kBins; b += 256) h[b] = 0;
  __syncthreads();
  const double lo = okey_value(f.head[bh].kmin), hi = okey_value(f.head[bh].kmax);
  const double inv_w = hi > lo ? (double)kBins / (hi - lo) : 0.0;
  const double* s = score + bh * total;
  const long s1 = min(total, s0 + kSpan);
  for (long e = s0 + threadIdx.x; e < s1; e += 256) atomicAdd(&h[score_bin(s[e], lo, inv_w)], 1);
  __syncthreads();
  for (int b = threadIdx.x; b < kBins; b += 256)
    if (h[b]) atomicAdd(&f.hist[bh * kBins + b], h[b]);
}

__global__ __launch_bounds__(64) void fine_find_kernel(Geo g, FineScratch f) {
  const long bh = blockIdx.x;
  if (threadIdx.x != 0) return;
  const long K = g.fine_keep;
  long above = 0;
  int b = kBins - 1;
  for (; b > 0; --b) {
    const long c = f.hist[bh * kBins + b];
    if (above + c >= K) break;
    above += c;
  }
  f.head[bh].bin = b;
  f.head[bh].above = (int)above;
  f.head[bh].need = (int)(K - above);
  f.head[bh].ncand = 0;
}

// Candidates of the threshold bin (order key and position), and per group
// the scores of higher bins: those are all kept, since the binning is
// monotone and tau lies in the threshold bin.  Each thread counts its run of
// one group in a register and adds it when the group changes, into LDS for
// the span's first kSpanGroups groups (every one, unless N < 64), else into
// the global count.
constexpr int kSpanGroups = 1024;
__global__ __launch_bounds__(256) void fine_gather_kernel(Geo g, const double* __restrict__ score,
                                                          FineScratch f, int* __restrict__ count) {
  __shared__ int cnt[kSpanGroups];
  const long bh = blockIdx.y;
  const long total = (long)g.fine_G * g.N;
  const long s0 = (long)blockIdx.x * kSpan;
  if (s0 >= total) return;
  for (int x = threadIdx.x; x < kSpanGroups; x += 256) cnt[x] = 0;
  __syncthreads();
  const double lo = okey_value(f.head[bh].kmin), hi = okey_value(f.head[bh].kmax);
  const double inv_w = hi > lo ? (double)kBins / (hi - lo) : 0.0;
  const int bin = f.head[bh].bin;
  const double* s = score + bh * total;
  int* const gcount = count + bh * g.fine_G;
  const long s1 = min(total, s0 + kSpan);
  const int g_first = (int)(s0 / g.N);
  long e = s0 + threadIdx.x;
  int gi = (int)(e / g.N);
  long g_end = (long)(gi + 1) * g.N;
  int run = 0;
  auto flush = [&]() {
    if (run == 0) return;
    if (gi - g_first < kSpanGroups) atomicAdd(&cnt[gi - g_first], run);
    else atomicAdd(&gcount[gi], run);
    run = 0;
  };
  for (; e < s1; e += 256) {
    while (e >= g_end) {
      flush();
      ++gi;
      g_end += g.N;
    }
    const double v = s[e];
    const int sb = score_bin(v, lo, inv_w);
    if (sb > bin) {
      ++run;
    } else if (sb == bin) {
      const int slot = atomicAdd(&f.head[bh].ncand, 1);
      if (slot < kCandCap) {
        f.cand[bh * kCandCap + slot] = okey(v);
        f.cpos[bh * kCandCap + slot] = (int)e;
      } else {
        f.head[bh].overflow = 1;
      }
    }
  }
  flush();
  __syncthreads();
  const int n_local = (int)min((long)kSpanGroups, (s1 - 1) / g.N - g_first + 1);
  for (int x = threadIdx.x; x < n_local; x += 256)
    if (cnt[x]) atomicAdd(&gcount[g_first + x], cnt[x]);
}

// Exact K-th largest: MSB-first radix select, 8 bits per pass, over the
// gathered candidates of one head.
__global__ __launch_bounds__(1024) void fine_select_kernel(Geo g, FineScratch f,
                                                           double* __restrict__ tau) {
  __shared__ int h[256];
  __shared__ unsigned long long prefix_s;
  __shared__ int need_s;
  const long bh = blockIdx.x;
  const int n = min((long)f.head[bh].ncand, kCandCap);
  const unsigned long long* c = f.cand + bh * kCandCap;
  if (threadIdx.x == 0) {
    prefix_s = 0ull;
    need_s = f.head[bh].need;
  }
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int b = threadIdx.x; b < 256; b += 1024) h[b] = 0;
    __syncthreads();
    const unsigned long long prefix = prefix_s;
    const unsigned long long mask = (shift == 56) ? 0ull : (~0ull << (shift + 8));
    for (int e = threadIdx.x; e < n; e += 1024) {
      const unsigned long long key = c[e];
      if ((key & mask) == prefix) atomicAdd(&h[(key >> shift) & 255], 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int need = need_s;
      int d = 255;
      for (; d > 0; --d) {
        if (h[d] >= need) break;
        need -= h[d];
      }
      prefix_s = prefix | ((unsigned long long)d << shift);
      need_s = need;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) tau[bh] = okey_value(prefix_s);
}

// Kept scores per group, the threshold bin's share: candidates at or above
// tau (the same fp64 comparison as the emit pass), added to the higher bins'
// counts of the gather pass.
__global__ __launch_bounds__(256) void fine_cand_count_kernel(Geo g, FineScratch f,
                                                              const double* __restrict__ tau,
                                                              int* __restrict__ count) {
  const long bh = blockIdx.y;
  if (f.head[bh].overflow & 1) return;  // the full count below runs instead
  const int n = min((long)f.head[bh].ncand, kCandCap);
  const double t = tau[bh];
  for (int e = blockIdx.x * 256 + threadIdx.x; e < n; e += gridDim.x * 256)
    if (okey_value(f.cand[bh * kCandCap + e]) >= t)
      atomicAdd(&count[bh * g.fine_G + f.cpos[bh * kCandCap + e] / g.N], 1);
}

// Full count of one group's kept scores, only when the candidates
// overflowed (tau then comes from a partial candidate set, and the counts
// must still match the emit pass).
__global__ __launch_bounds__(256) void fine_count_kernel(Geo g, const double* __restrict__ score,
                                                         const double* __restrict__ tau,
                                                         FineScratch f, int* __restrict__ count) {
  __shared__ int part[4];
  const int gi = blockIdx.x;
  const long bh = blockIdx.y;
  if (!(f.head[bh].overflow & 1)) return;
  const double t = tau[bh];
  const double* s = score + (bh * g.fine_G + gi) * (long)g.N;
  int c = 0;
  for (int j = threadIdx.x; j < g.N; j += 256) c += (s[j] >= t) ? 1 : 0;
  for (int m = 1; m < 64; m <<= 1) c += __shfl_xor(c, m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) count[bh * g.fine_G + gi] = part[0] + part[1] + part[2] + part[3];
}

__global__ __launch_bounds__(64) void fine_scan_kernel(Geo g, const int* __restrict__ count,
                                                       int* __restrict__ ptr, FineScratch f) {
  const long bh = blockIdx.x;
  if (threadIdx.x != 0) return;
  long run = 0;
  for (int gi = 0; gi < g.fine_G; ++gi) {
    ptr[bh * (g.fine_G + 1) + gi] = (int)min(run, g.fine_cap);
    run += count[bh * g.fine_G + gi];
  }
  ptr[bh * (g.fine_G + 1) + g.fine_G] = (int)min(run, g.fine_cap);
  if (run > g.fine_cap) f.head[bh].overflow |= 2;
}

// Ascending kept-key list of one group (ordered block compaction).
__global__ __launch_bounds__(256) void fine_emit_kernel(Geo g, const double* __restrict__ score,
                                                        const double* __restrict__ tau,
                                                        const int* __restrict__ ptr,
                                                        int* __restrict__ idx) {
  __shared__ int wsum[4];
  const int gi = blockIdx.x;
  const long bh = blockIdx.y;
  const double t = tau[bh];
  const double* s = score + (bh * g.fine_G + gi) * (long)g.N;
  const int lo = ptr[bh * (g.fine_G + 1) + gi];
  const int hi = ptr[bh * (g.fine_G + 1) + gi + 1];
  int* out = idx + bh * g.fine_cap;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int base = lo;
  for (int j0 = 0; j0 < g.N; j0 += 256) {
    const int j = j0 + threadIdx.x;
    const bool keep = j < g.N && s[j] >= t;
    const unsigned long long ball = __ballot(keep);
    const int before = __popcll(ball & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(ball);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    if (keep && off + before < hi) out[off + before] = j;
    base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
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
                                                              const int* __restrict__ ptr,
                                                              const int* __restrict__ idx,
                                                              uint16_t* __restrict__ o) {
  extern __shared__ __align__(16) uint16_t lds[];
  const int gi = blockIdx.x;
  const long bh = blockIdx.y;
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
  // (list bounds clamped to the capacity: a mask that was never written
  // still keeps every access in bounds; key indices are clamped on load)
  const int lo = min(max(ptr[bh * (g.fine_G + 1) + gi], 0), g.fine_cap);
  const int n = min(max(ptr[bh * (g.fine_G + 1) + gi + 1] - lo, 0), g.fine_cap - lo);
  const int* keys = idx + bh * g.fine_cap + lo;

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
  hipLaunchKernelGGL((fine_attend_kernel<D, NW>), dim3(g.fine_G, g.B * g.H), dim3(NW * 64), shmem, s,
                     g, q, k, v, w.fine_ptr, w.fine_idx, o);
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
  off = align256(off + BH * kBins * sizeof(int));
  off = align256(off + (size_t)BH * g.fine_G * g.d * sizeof(double));
  off = align256(off + (size_t)BH * kCandCap * sizeof(unsigned long long));
  off += (size_t)BH * kCandCap * sizeof(int);
  return off;
}

hipError_t launch_fine_select(const Geo& g, const Ws& w, const uint16_t* q, const uint16_t* k,
                              hipStream_t s) {
  const FineScratch f = carve(g, w.scratch);
  const unsigned BH = (unsigned)(g.B * g.H);
  hipError_t e;
  hipLaunchKernelGGL(fine_init_kernel, dim3(BH), dim3(256), 0, s, g, f, w.fine_count);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (g.d == 128)
    hipLaunchKernelGGL(fine_qbar_kernel<128>, dim3(g.fine_G, BH), dim3(128), 0, s, g, q, w.fine_qbar, f);
  else
    hipLaunchKernelGGL(fine_qbar_kernel<64>, dim3(g.fine_G, BH), dim3(64), 0, s, g, q, w.fine_qbar, f);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dim3 sg((g.N + 256 * kScoreKeys - 1) / (256 * kScoreKeys), (g.fine_G + kScoreGroups - 1) / kScoreGroups, BH);
  double* score = reinterpret_cast<double*>(w.fine_score);
  if (g.d == 128)
    hipLaunchKernelGGL(fine_score_kernel<128>, sg, dim3(256), 0, s, g, k, f.qbar64, score, f);
  else
    hipLaunchKernelGGL(fine_score_kernel<64>, sg, dim3(256), 0, s, g, k, f.qbar64, score, f);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const long total = (long)g.fine_G * g.N;
  dim3 hg((unsigned)((total + kSpan - 1) / kSpan), BH);
  hipLaunchKernelGGL(fine_hist_kernel, hg, dim3(256), 0, s, g, score, f);
  hipLaunchKernelGGL(fine_find_kernel, dim3(BH), dim3(64), 0, s, g, f);
  hipLaunchKernelGGL(fine_gather_kernel, hg, dim3(256), 0, s, g, score, f, w.fine_count);
  hipLaunchKernelGGL(fine_select_kernel, dim3(BH), dim3(1024), 0, s, g, f, w.fine_tau);
  hipLaunchKernelGGL(fine_cand_count_kernel, dim3(64, BH), dim3(256), 0, s, g, f, w.fine_tau, w.fine_count);
  hipLaunchKernelGGL(fine_count_kernel, dim3(g.fine_G, BH), dim3(256), 0, s, g, score, w.fine_tau, f,
                     w.fine_count);
  hipLaunchKernelGGL(fine_scan_kernel, dim3(BH), dim3(64), 0, s, g, w.fine_count, w.fine_ptr, f);
  hipLaunchKernelGGL(fine_emit_kernel, dim3(g.fine_G, BH), dim3(256), 0, s, g, score, w.fine_tau,
                     w.fine_ptr, w.fine_idx);
  return hipGetLastError();
}

hipError_t launch_fine_attend(const Geo& g, const Ws& w, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, uint16_t* o, hipStream_t s) {
  return g.d == 128 ? launch_fine_attend_d<128>(g, w, q, k, v, o, s)
                    : launch_fine_attend_d<64>(g, w, q, k, v, o, s);
}

}  // namespace vsa
