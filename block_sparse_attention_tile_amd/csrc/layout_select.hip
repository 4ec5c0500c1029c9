// Tile layout transform (raster <-> tile-major), pooled tile means, and the
// tile selection (window / Top-K / Top-P) that produces the kept key tiles of
// every query tile.
//
// Tile geometry: the T x H x W token grid is cut into tiles of tt x th x tw
// tokens; a tile is one attention block and its tokens stay consecutive
// (Sliding Tile Attention verdict page, pith_extraction.key_machinery).
// Tiles are numbered in raster order of tile coordinates; inside a tile the
// valid tokens keep raster order and the padded slots (edge tiles, and the
// rounding of the tile size up to 32) come last and are zero.
//
// Selection follows the SPADE review page: mean summaries of Q and K per
// block (Figure 4, MEAN summarizer), block score = product of the summaries,
// and a Top-K / Top-P filter united with a local window ("Core claim").
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>

#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kLayoutThreads = 256;
constexpr int kChunk = 64;  // slots per layout step

struct TileRef {
  int it, ih, iw;  // tile coordinates
  int et, eh, ew;  // extents inside the grid
  int nvalid;
};

__device__ __forceinline__ TileRef tile_ref(const Geo& g, const BlkGeo& b, int i) {
  TileRef t;
  t.it = i / (b.nt[1] * b.nt[2]);
  t.ih = (i / b.nt[2]) % b.nt[1];
  t.iw = i % b.nt[2];
  t.et = min(b.tile[0], g.grid[0] - t.it * b.tile[0]);
  t.eh = min(b.tile[1], g.grid[1] - t.ih * b.tile[1]);
  t.ew = min(b.tile[2], g.grid[2] - t.iw * b.tile[2]);
  t.nvalid = t.et * t.eh * t.ew;
  return t;
}

// Raster token of valid slot s (< nvalid) of tile t.
__device__ __forceinline__ long token_of(const Geo& g, const BlkGeo& b, const TileRef& t, int s) {
  const int ehw = t.eh * t.ew;
  const int st = s / ehw;
  const int r = s - st * ehw;
  const int sh = r / t.ew;
  const int sw = r - sh * t.ew;
  return ((long)(t.it * b.tile[0] + st) * g.grid[1] + (t.ih * b.tile[1] + sh)) * g.grid[2] +
         (t.iw * b.tile[2] + sw);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---- E4M3 quantization (VSA_COMPUTE_FP8) ------------------------------------
// Per (head, tensor) power-of-two factor 2^e: the largest integer e with
// amax * 2^e <= 448 = 0.875 * 2^9, clamped to [-32, 32] (0 for an all-zero
// head).  With amax = m * 2^x, m in [0.5, 1): e = 9 - x if m <= 0.875, else
// 8 - x.  Below 2^-24 the clamp decides (e would exceed 32).
__device__ __forceinline__ int f8_exponent(uint32_t amax_bf16_bits) {
  const float a = __uint_as_float(amax_bf16_bits << 16);
  if (!(a > 0.f)) return 0;
  if (a < 0x1p-24f) return 32;
  int x;
  const float m = frexpf(a, &x);
  const int e = m <= 0.875f ? 9 - x : 8 - x;
  return min(max(e, -32), 32);
}

// Four floats (each |x| <= 448) to E4M3, round to nearest even, packed
// little-endian (a in the low byte).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}

// Eight bf16 values (one 16-byte piece) times 2^e to eight E4M3 bytes; the
// scaling is exact.
__device__ __forceinline__ uint2 quant8(const uint4& w, int e) {
  uint2 o;
  o.x = e4m3x4(ldexpf(bf16_lo(w.x), e), ldexpf(bf16_hi(w.x), e), ldexpf(bf16_lo(w.y), e),
               ldexpf(bf16_hi(w.y), e));
  o.y = e4m3x4(ldexpf(bf16_lo(w.z), e), ldexpf(bf16_hi(w.z), e), ldexpf(bf16_lo(w.w), e),
               ldexpf(bf16_hi(w.w), e));
  return o;
}

// Slot (relative to its 32-slot group) stored at position pp of an E4M3 V^T
// row: slot bits (b4 b3 b2 b1 b0) sit at position (b2 b4 b3 b1 b0), so the
// keys one MFMA lane half multiplies (bit 2 fixed) are 16 consecutive bytes.
__device__ __forceinline__ int f8_vslot(int pp) {
  return (pp & ~31) | (((pp >> 2) & 3) << 3) | (((pp >> 4) & 1) << 2) | (pp & 3);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Partial max |x| (as bf16 bits, sign cleared) of Q, K, V: one workgroup per
// (slice, head, tensor); slice p covers a contiguous 1/kAmaxParts of the
// head's N*d raster values.  Integer maxima of the magnitude bits order
// finite bf16 values exactly; no atomics, so the result is deterministic.
constexpr int kAmaxThreads = 512;
__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(Geo g, const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v,
                                                           uint32_t* __restrict__ part) {
  const int p = blockIdx.x;
  const long bh = blockIdx.y;
  const int which = blockIdx.z;
  const uint16_t* x = (which == 0 ? q : which == 1 ? k : v) + bh * (long)g.N * g.d;
  const long n16 = (long)g.N * g.d / 8;  // 16-byte units of the head
  const long per = (n16 + kAmaxParts - 1) / kAmaxParts;
  const long lo = p * per;
  const long hi = min(n16, lo + per);
  const uint4* x4 = reinterpret_cast<const uint4*>(x);
  u16x2 m = {0, 0};
  constexpr int U = 4;  // loads in flight per thread
  for (long u0 = lo + threadIdx.x; u0 < hi; u0 += (long)kAmaxThreads * U) {
    uint4 w[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const long u = u0 + (long)j * kAmaxThreads;
      w[j] = u < hi ? x4[u] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const uint32_t ww[4] = {w[j].x, w[j].y, w[j].z, w[j].w};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, ww[c] & 0x7fff7fffu));
    }
  }
  uint32_t r = m[0] > m[1] ? m[0] : m[1];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) r = max(r, (uint32_t)__shfl_xor((int)r, o));
  __shared__ uint32_t wmax[kAmaxThreads / 64];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = r;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = wmax[0];
    for (int i = 1; i < kAmaxThreads / 64; ++i) t = max(t, wmax[i]);
    part[(bh * 3 + which) * kAmaxParts + p] = t;
  }
}

// One workgroup per (head, tile): copies Q and K rows to tile-major order,
// writes V transposed per tile ([d][slots]) through LDS, and optionally the
// exact per-tile means of Q and K (fp64 sums of bf16 values, one rounding).
// The Q/K copy runs first with no barrier in it (four rows per thread in
// flight); only the V transpose is staged through LDS.  With F8 the copies
// are E4M3 bytes (per-head power-of-two factors from the partial maxima of
// amax_kernel, recorded in f8_exp by tile 0) and V^T rows are permuted
// inside each 32-slot group (f8_vslot); the summaries still use bf16.
template <int D, bool F8>
__global__ __launch_bounds__(kLayoutThreads) void layout_kernel(
    Geo g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ qt, uint16_t* __restrict__ kt,
    uint16_t* __restrict__ vt, float* __restrict__ pooled_q, float* __restrict__ pooled_k,
    float* __restrict__ pooled_kmin, const int* __restrict__ cand, int pool,
    const uint32_t* __restrict__ f8_amax, int* __restrict__ f8_exp) {
  constexpr int P = D / 8;                       // 16-byte pieces per row
  constexpr int RPP = kLayoutThreads / P;        // rows per pass
  constexpr int LVW = D / 2 + 1;                 // V chunk row stride in words (odd: no bank conflicts)
  constexpr int kWords = kChunk * LVW > kLayoutThreads * 16 ? kChunk * LVW : kLayoutThreads * 16;
  __shared__ uint32_t smem[kWords];              // V chunk; reused for the pooled-sum reduction
  constexpr int U = 4;                           // rows per thread in flight (Q/K copy)

  const int i = blockIdx.x;
  const long bh = blockIdx.y;
  const int c = cand_of(g, cand, bh);
  const BlkGeo b = pick_blk(g, c);
  if (i >= b.n_tiles) return;
  const TileRef t = tile_ref(g, b, i);
  const int tid = threadIdx.x;
  const int p = tid % P;
  const int r0 = tid / P;
  const long in_base = bh * (long)g.N * D;
  const long tm_base = bh * g.tok_cap * D + (long)i * b.slots * D;
  uint8_t* const qt8 = reinterpret_cast<uint8_t*>(qt);
  uint8_t* const kt8 = reinterpret_cast<uint8_t*>(kt);
  uint8_t* const vt8 = reinterpret_cast<uint8_t*>(vt);
  int eq = 0, ek = 0, ev = 0;
  if constexpr (F8) {
    // every wave reduces the head's partial maxima on its own (no barrier)
    const int lane = tid & 63;
    uint32_t m3[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      uint32_t m = 0u;
      for (int y = lane; y < kAmaxParts; y += 64) m = max(m, f8_amax[(bh * 3 + x) * kAmaxParts + y]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
      m3[x] = m;
    }
    eq = f8_exponent(m3[0]);
    ek = f8_exponent(m3[1]);
    ev = f8_exponent(m3[2]);
    if (i == 0 && tid < 3) f8_exp[bh * 3 + tid] = tid == 0 ? eq : (tid == 1 ? ek : ev);
  }

  double sq[8], sk[8];
  float kmx[8], kmn[8];  // per-channel extrema of K over the valid tokens
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    sq[x] = sk[x] = 0.0;
    kmx[x] = -INFINITY;
    kmn[x] = INFINITY;
  }
  const bool extrema = pool && g.summ != VSA_SUMM_MEAN;
  // Q and K: gather raster rows, store contiguous tile-major rows (Q only for
  // E4M3: the bf16 attention reads Q in raster order).
  for (int s0 = r0; s0 < b.slots; s0 += RPP * U) {
    uint4 qv[U], kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * RPP;
      qv[u] = make_uint4(0, 0, 0, 0);
      kv[u] = qv[u];
      if (s < t.nvalid) {
        const long off = in_base + token_of(g, b, t, s) * D + p * 8;
        if (F8 || pool) qv[u] = *reinterpret_cast<const uint4*>(q + off);  // bf16: summaries only
        kv[u] = *reinterpret_cast<const uint4*>(k + off);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * RPP;
      if (s < b.slots) {
        if constexpr (F8) {
          *reinterpret_cast<uint2*>(qt8 + tm_base + (long)s * D + p * 8) = quant8(qv[u], eq);
          *reinterpret_cast<uint2*>(kt8 + tm_base + (long)s * D + p * 8) = quant8(kv[u], ek);
        } else {
          *reinterpret_cast<uint4*>(kt + tm_base + (long)s * D + p * 8) = kv[u];
        }
      }
      if (pool) {
        const uint32_t qw[4] = {qv[u].x, qv[u].y, qv[u].z, qv[u].w};
        const uint32_t kw[4] = {kv[u].x, kv[u].y, kv[u].z, kv[u].w};
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          sq[2 * x] += (double)bf16_lo(qw[x]);
          sq[2 * x + 1] += (double)bf16_hi(qw[x]);
          sk[2 * x] += (double)bf16_lo(kw[x]);
          sk[2 * x + 1] += (double)bf16_hi(kw[x]);
        }
        if (extrema && s < t.nvalid) {  // padded slots are not tokens
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            kmx[2 * x] = fmaxf(kmx[2 * x], bf16_lo(kw[x]));
            kmx[2 * x + 1] = fmaxf(kmx[2 * x + 1], bf16_hi(kw[x]));
            kmn[2 * x] = fminf(kmn[2 * x], bf16_lo(kw[x]));
            kmn[2 * x + 1] = fminf(kmn[2 * x + 1], bf16_hi(kw[x]));
          }
        }
      }
    }
  }

  // V: chunks of 64 slots through LDS, written transposed ([d][slots]).
  const long vt_base = bh * g.tok_cap * D + (long)i * D * b.slots;
  for (int s0 = 0; s0 < b.slots; s0 += kChunk) {
    uint4 vv[kChunk / RPP];
#pragma unroll
    for (int u = 0; u < kChunk / RPP; ++u) {
      const int s = s0 + r0 + u * RPP;
      vv[u] = make_uint4(0, 0, 0, 0);
      if (s < t.nvalid)
        vv[u] = *reinterpret_cast<const uint4*>(v + in_base + token_of(g, b, t, s) * D + p * 8);
    }
#pragma unroll
    for (int u = 0; u < kChunk / RPP; ++u) {
      uint32_t* row = smem + (r0 + u * RPP) * LVW + p * 4;
      row[0] = vv[u].x;
      row[1] = vv[u].y;
      row[2] = vv[u].z;
      row[3] = vv[u].w;
    }
    __syncthreads();
    // V^T pieces: 8 consecutive slots of one channel row; 8 lanes cover a
    // 128-byte run of the row.
    for (int pc = tid; pc < D * (kChunk / 8); pc += kLayoutThreads) {
      const int s8 = pc % (kChunk / 8);
      const int dd = pc / (kChunk / 8);
      const int sl = s0 + s8 * 8;
      if (sl >= b.slots) continue;
      uint32_t h[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = F8 ? f8_vslot(s8 * 8 + j) : s8 * 8 + j;
        const uint32_t wv = smem[row * LVW + (dd >> 1)];
        h[j] = (dd & 1) ? (wv >> 16) : (wv & 0xffffu);
      }
      if constexpr (F8) {
        uint2 o8;
        o8.x = e4m3x4(ldexpf(__uint_as_float(h[0] << 16), ev), ldexpf(__uint_as_float(h[1] << 16), ev),
                      ldexpf(__uint_as_float(h[2] << 16), ev), ldexpf(__uint_as_float(h[3] << 16), ev));
        o8.y = e4m3x4(ldexpf(__uint_as_float(h[4] << 16), ev), ldexpf(__uint_as_float(h[5] << 16), ev),
                      ldexpf(__uint_as_float(h[6] << 16), ev), ldexpf(__uint_as_float(h[7] << 16), ev));
        *reinterpret_cast<uint2*>(vt8 + vt_base + (long)dd * b.slots + sl) = o8;
        continue;
      }
      uint4 out;
      out.x = h[0] | (h[1] << 16);
      out.y = h[2] | (h[3] << 16);
      out.z = h[4] | (h[5] << 16);
      out.w = h[6] | (h[7] << 16);
      *reinterpret_cast<uint4*>(vt + vt_base + (long)dd * b.slots + sl) = out;
    }
    __syncthreads();
  }

  if (!pool) return;
  // Exact sums: every partial sum of bf16 values of moderate range is exact
  // in fp64, so the reduction order does not change the result.  Extrema
  // are exact in any order too.
  double* red = reinterpret_cast<double*>(smem);  // [kLayoutThreads][8]
  float* redf = reinterpret_cast<float*>(smem);   // [kLayoutThreads][8]
  // Q summaries [head][tile][d]; K summaries channel-major [head][d][tile],
  // so that the selection's per-key-tile dot products read them coalesced
  const long q_off = (bh * g.max_tiles + i) * D;
  const long k_off = bh * D * (long)g.max_tiles + i;
  for (int which = 0; which < 2; ++which) {
    if (which == 1 && extrema) break;  // K gets its extrema below instead of its mean
#pragma unroll
    for (int x = 0; x < 8; ++x) red[tid * 8 + x] = which ? sk[x] : sq[x];
    __syncthreads();
    if (tid < D) {
      const int pp = tid / 8, xx = tid % 8;
      double s = 0.0;
      for (int r = 0; r < RPP; ++r) s += red[(r * P + pp) * 8 + xx];
      const float m = (float)(s / (double)t.nvalid);
      if (which)
        pooled_k[k_off + (long)tid * g.max_tiles] = m;
      else
        pooled_q[q_off + tid] = m;
    }
    __syncthreads();
  }
  if (!extrema) return;
  for (int which = 0; which < 2; ++which) {
    if (which == 1 && g.summ != VSA_SUMM_MINMAX) break;
#pragma unroll
    for (int x = 0; x < 8; ++x) redf[tid * 8 + x] = which ? kmn[x] : kmx[x];
    __syncthreads();
    if (tid < D) {
      const int pp = tid / 8, xx = tid % 8;
      float m = redf[pp * 8 + xx];
      for (int r = 1; r < RPP; ++r) {
        const float v = redf[(r * P + pp) * 8 + xx];
        m = which ? fminf(m, v) : fmaxf(m, v);
      }
      (which ? pooled_kmin : pooled_k)[k_off + (long)tid * g.max_tiles] = m;
    }
    __syncthreads();
  }
}

// Tile-major rows back to raster order (valid slots only).
template <int D>
__global__ __launch_bounds__(kLayoutThreads) void untile_kernel(Geo g, const uint16_t* __restrict__ xt,
                                                               const int* __restrict__ cand,
                                                               uint16_t* __restrict__ out) {
  constexpr int P = D / 8;
  const int i = blockIdx.x;
  const long bh = blockIdx.y;
  const int c = cand_of(g, cand, bh);
  const BlkGeo b = pick_blk(g, c);
  if (i >= b.n_tiles) return;
  const TileRef t = tile_ref(g, b, i);
  const long tm_base = bh * g.tok_cap * D + (long)i * b.slots * D;
  for (int e = threadIdx.x; e < t.nvalid * P; e += kLayoutThreads) {
    const int s = e / P, p = e % P;
    const uint4 val = *reinterpret_cast<const uint4*>(xt + tm_base + (long)s * D + p * 8);
    *reinterpret_cast<uint4*>(out + bh * (long)g.N * D + token_of(g, b, t, s) * D + p * 8) = val;
  }
}

// ---------------------------------------------------------------------------
// Selection: one workgroup per (head, query tile).

constexpr int kSelThreads = 256;
constexpr int kMaxTiles = 4096;

__device__ __forceinline__ bool ranks_before(double sa, int ia, double sb, int ib) {
  return sa > sb || (sa == sb && ia < ib);
}

// One compare-exchange of the bitonic network for the element this thread
// holds at sorted position x against its partner (so, io): the lower
// position of an ascending block (x & kk == 0) keeps the element that ranks
// first, every other position the one that ranks second.
__device__ __forceinline__ void bitonic_keep(double& s, int& id, double so, int io, bool lower, bool up) {
  const bool other_first = ranks_before(so, io, s, id);
  if (other_first == (lower == up)) {
    s = so;
    id = io;
  }
}

// In-register stage of stride JJ (< E): positions tid*E + r and tid*E + (r^JJ).
template <int E, int JJ>
__device__ __forceinline__ void bitonic_reg(double (&sv)[E], int (&si)[E], int kk) {
  if constexpr (JJ < E) {
#pragma unroll
    for (int r = 0; r < E; ++r) {
      constexpr int dummy = 0;
      (void)dummy;
      const int pr = r ^ JJ;
      if (pr > r) {
        const bool up = (((int)threadIdx.x * E + r) & kk) == 0;
        // r is the lower position of the pair
        if (ranks_before(sv[pr], si[pr], sv[r], si[r]) == up) {
          const double ts = sv[r];
          sv[r] = sv[pr];
          sv[pr] = ts;
          const int ti = si[r];
          si[r] = si[pr];
          si[pr] = ti;
        }
      }
    }
  }
}

// Sort of m = 256 E (score, tile) pairs held E per thread in blocked order
// (thread t holds positions t*E .. t*E + E - 1): highest score first, ties
// by lower tile index.  Strides below E stay in registers, strides below
// 64 E are lane shuffles inside a wave, the rest go through LDS (xs, xi).
template <int E>
__device__ void bitonic_sort_blocked(double (&sv)[E], int (&si)[E], double* xs, int* xi) {
  const int tid = threadIdx.x;
  constexpr int M = kSelThreads * E;
  for (int kk = 2; kk <= M; kk <<= 1) {
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      if (jj < E) {
        switch (jj) {
          case 1: bitonic_reg<E, 1>(sv, si, kk); break;
          case 2: bitonic_reg<E, 2>(sv, si, kk); break;
          case 4: bitonic_reg<E, 4>(sv, si, kk); break;
          default: bitonic_reg<E, 8>(sv, si, kk); break;
        }
      } else if (jj < 64 * E) {
        const int dl = jj / E;  // lane distance of the partner
#pragma unroll
        for (int r = 0; r < E; ++r) {
          const double so = __shfl_xor(sv[r], dl);
          const int io = __shfl_xor(si[r], dl);
          const int x = tid * E + r;
          bitonic_keep(sv[r], si[r], so, io, (x & jj) == 0, (x & kk) == 0);
        }
      } else {
#pragma unroll
        for (int r = 0; r < E; ++r) {
          xs[tid * E + r] = sv[r];
          xi[tid * E + r] = si[r];
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < E; ++r) {
          const int x = tid * E + r;
          bitonic_keep(sv[r], si[r], xs[x ^ jj], xi[x ^ jj], (x & jj) == 0, (x & kk) == 0);
        }
        __syncthreads();
      }
    }
  }
}

// Order-preserving key of a finite double: a larger value gives a larger
// key, and -0 and +0 give the same key (they compare equal).
__device__ __forceinline__ uint64_t order_key(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x + 0.0);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Exclusive prefix sum of v over the workgroup's threads in thread order;
// *total receives the sum over all threads.  wtot: kSelThreads / 64 ints.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wtot, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) wtot[wave] = inc;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    if (w < wave) before += wtot[w];
    all += wtot[w];
  }
  __syncthreads();  // wtot is reused by the next scan
  *total = all;
  return before + inc - v;
}

// Top-K alone (no Top-P): the K highest scores of each of the nq rows, ties
// to the lower key tile, without sorting.  An MSB-first radix select over
// the scores' 64-bit order keys (8-bit digits, one histogram per row in
// LDS; lanes of a wave with the same digit add their count in one atomic)
// finds the K-th largest key T and how many of the keys equal to T belong
// to the top K; keys above T are kept, and the keys equal to T are kept in
// ascending tile order up to that number.  The keys of row q are held E per
// thread (key tile tid * E + r), as the scores were computed.
// A row is done early when the digits found so far single out one key: that
// key is the K-th largest, and no other key equals it.
static_assert(kSelThreads == 256, "one thread per 8-bit digit");
template <int E, int QB>
__device__ __forceinline__ void topk_radix(const uint64_t (&key)[QB][E], int nq, int n, int K,
                                           int (*hist)[256], int (*wtot)[kSelThreads / 64],
                                           int* rdig, int* rneed, int* rcnt, uint64_t* rkey,
                                           unsigned char* keep, int ks) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j0 = tid * E;
  uint64_t pre[QB];
  int need[QB];
  bool done[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    pre[q] = 0;
    need[q] = K;
    done[q] = q >= nq;
  }
  for (int pass = 0; pass < 8; ++pass) {
    bool all_done = true;
#pragma unroll
    for (int q = 0; q < QB; ++q) all_done = all_done && done[q];
    if (all_done) break;  // uniform
    const int sh = 56 - 8 * pass;
    const uint64_t hm = pass == 0 ? 0ull : (~0ull << (sh + 8));  // the digits found so far
#pragma unroll
    for (int q = 0; q < QB; ++q) hist[q][tid] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      if (done[q]) continue;  // uniform
#pragma unroll
      for (int r = 0; r < E; ++r) {
        const bool m = j0 + r < n && (key[q][r] & hm) == pre[q];
        const int dg = (int)((key[q][r] >> sh) & 255);
        uint64_t act = __ballot(m);
        while (act) {  // one atomic per distinct digit of the wave
          const int leader = __ffsll((unsigned long long)act) - 1;
          const int dl = __shfl(dg, leader);
          const uint64_t same = __ballot(m && dg == dl);
          if (lane == leader) atomicAdd(&hist[q][dl], __popcll(same));
          act &= ~same;
        }
      }
    }
    __syncthreads();
    // counts from the highest digit down: thread t holds digit 255 - t; the
    // digit of the K-th largest is where the running count reaches need
    int c[QB], run[QB];
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      c[q] = hist[q][255 - tid];
      run[q] = c[q];
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        const int t = __shfl_up(run[q], o);
        if (lane >= o) run[q] += t;
      }
    if (lane == 63)
#pragma unroll
      for (int q = 0; q < QB; ++q) wtot[q][wave] = run[q];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      if (done[q]) continue;
#pragma unroll
      for (int w = 0; w < kSelThreads / 64; ++w)
        if (w < wave) run[q] += wtot[q][w];
      if (run[q] >= need[q] && run[q] - c[q] < need[q]) {
        rdig[q] = 255 - tid;
        rneed[q] = need[q] - (run[q] - c[q]);
        rcnt[q] = c[q];
      }
    }
    __syncthreads();
    bool single = false;
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      if (done[q]) continue;
      pre[q] |= (uint64_t)rdig[q] << sh;
      need[q] = rneed[q];
      if (rcnt[q] == 1) {  // one key left with these digits: it is the K-th largest
        const uint64_t m = ~0ull << sh;
#pragma unroll
        for (int r = 0; r < E; ++r)
          if (j0 + r < n && (key[q][r] & m) == pre[q]) rkey[q] = key[q][r];
        single = true;
      }
    }
    __syncthreads();  // rkey written; rdig / rneed / rcnt read by every thread
    if (single) {  // uniform (rcnt is read from LDS by every thread)
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        if (done[q] || rcnt[q] != 1) continue;
        pre[q] = rkey[q];
        done[q] = true;
      }
      __syncthreads();  // rcnt / rkey are rewritten in the next pass
    }
  }
  // pre[q]: the K-th largest key; need[q]: how many keys equal to it are kept
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    if (q >= nq) break;  // uniform
    int ties = 0;
#pragma unroll
    for (int r = 0; r < E; ++r) ties += (j0 + r < n && key[q][r] == pre[q]) ? 1 : 0;
    int total;
    int before = block_exclusive_scan(ties, wtot[0], &total);
#pragma unroll
    for (int r = 0; r < E; ++r) {
      if (j0 + r >= n) continue;
      if (key[q][r] > pre[q]) {
        keep[q * ks + j0 + r] = 1;
      } else if (key[q][r] == pre[q]) {
        if (before < need[q]) keep[q * ks + j0 + r] = 1;
        ++before;
      }
    }
  }
}

// One workgroup per (head, QB consecutive query tiles): window and sink flags,
// then the block scores of every key tile against each query tile (fixed-order
// fp64 dot products of the summaries; one pass over the key summaries serves
// all QB query tiles), held E per thread; for Top-K / Top-P each query tile's
// row is sorted (bitonic, mostly in registers) and its first K positions, or
// the shortest prefix whose softmax mass reaches p, are kept (Top-K alone:
// the K highest by a radix select, no sort); the kept flags are compacted in
// ascending order.
template <int E, int QB>
__global__ __launch_bounds__(kSelThreads) void select_kernel(Geo g, const float* __restrict__ pooled_q,
                                                             const float* __restrict__ pooled_k,
                                                             const float* __restrict__ pooled_kmin,
                                                             const int* __restrict__ cand,
                                                             int* __restrict__ row_len,
                                                             int* __restrict__ col_idx) {

  __shared__ float qbar[QB][128];
  __shared__ int wtot_i[QB][kSelThreads / 64];
  __shared__ double wsum[kSelThreads / 64];
  __shared__ double top_s;
  // dynamic LDS: the kept flags [QB][ks], then (Top-P) the sort's exchange
  // double [256 E], int [256 E]
  extern __shared__ __align__(16) unsigned char sel_dyn[];
  const int ks = (g.max_tiles + 15) & ~15;
  unsigned char* const keep = sel_dyn;
  double* const xs = reinterpret_cast<double*>(sel_dyn + QB * ks);
  int* const xi = reinterpret_cast<int*>(xs + kSelThreads * E);

  const int i0 = blockIdx.x * QB;
  const long bh = blockIdx.y;
  const int c = cand_of(g, cand, bh);
  const BlkGeo b = pick_blk(g, c);
  const int n = b.n_tiles;
  if (i0 >= n) return;
  const int nq = min(QB, n - i0);  // query tiles of this workgroup
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int D = g.d;
  const bool dense = (g.flags & VSA_DENSE) != 0;
  for (int x = tid; x < QB * n; x += kSelThreads) keep[(x / n) * ks + x % n] = (dense || x % n < g.sink) ? 1 : 0;
  __syncthreads();

  if (g.flags & VSA_WINDOW) {
    for (int qt = 0; qt < nq; ++qt) {
      const int i = i0 + qt;
      const int ci[3] = {i / (b.nt[1] * b.nt[2]), (i / b.nt[2]) % b.nt[1], i % b.nt[2]};
      int lo[3], hi[3];
#pragma unroll
      for (int a = 0; a < 3; ++a) {
        const int r = (g.win[a] - 1) / 2;
        const int nn = b.nt[a];
        if (g.win_mode == VSA_WIN_CLAMP && nn >= 2 * r + 1) {
          lo[a] = min(max(ci[a] - r, 0), nn - (2 * r + 1));
          hi[a] = lo[a] + 2 * r;
        } else {
          lo[a] = max(ci[a] - r, 0);
          hi[a] = min(ci[a] + r, nn - 1);
        }
      }
      const int e1 = hi[1] - lo[1] + 1, e2 = hi[2] - lo[2] + 1;
      const int cells = (hi[0] - lo[0] + 1) * e1 * e2;
      for (int x = tid; x < cells; x += kSelThreads) {
        const int a0 = lo[0] + x / (e1 * e2);
        const int a1 = lo[1] + (x / e2) % e1;
        const int a2 = lo[2] + x % e2;
        keep[(qt) * ks + (a0 * b.nt[1] + a1) * b.nt[2] + a2] = 1;
      }
    }
  }

  const bool topp = (g.flags & VSA_TOPP) != 0;
  const int K = b.topk;
  if (topp || K > 0) {
    for (int x = tid; x < QB * D; x += kSelThreads) {
      const int qt = x / D, ch = x % D;
      qbar[qt][ch] = qt < nq ? pooled_q[(bh * g.max_tiles + i0 + qt) * D + ch] : 0.f;
    }
    __syncthreads();
    // scores of key tiles j = tid * E + r (E consecutive tiles per thread:
    // each channel's loads of a thread are contiguous) against the QB query tiles
    const float* kr = pooled_k + bh * D * (long)g.max_tiles;
    const float* kn = pooled_kmin + bh * D * (long)g.max_tiles;
    double acc[QB][E];
#pragma unroll
    for (int qt = 0; qt < QB; ++qt)
#pragma unroll
      for (int r = 0; r < E; ++r) acc[qt][r] = 0.0;
    const int j0 = tid * E;
    if (j0 < n) {
      // channel x of key tile j at [x][j]; loads past the row re-read its last
      // tile.  A batch of BT channels' loads is in flight before the sums,
      // which run in the fixed channel order (each fp32 x fp32 product is
      // exact in fp64).
      constexpr int BT = E >= 8 ? 2 : 32 / E;
      if (g.summ == VSA_SUMM_MINMAX) {
        constexpr int BM = BT / 2;  // two summaries per channel
        for (int x0 = 0; x0 < D; x0 += BM) {
          float a[BM][E], cm[BM][E];
#pragma unroll
          for (int u = 0; u < BM; ++u)
#pragma unroll
            for (int r = 0; r < E; ++r) {
              a[u][r] = kr[(long)(x0 + u) * g.max_tiles + min(j0 + r, n - 1)];
              cm[u][r] = kn[(long)(x0 + u) * g.max_tiles + min(j0 + r, n - 1)];
            }
#pragma unroll
          for (int u = 0; u < BM; ++u)
#pragma unroll
            for (int qt = 0; qt < QB; ++qt) {
              const double qv = (double)qbar[qt][x0 + u];
#pragma unroll
              for (int r = 0; r < E; ++r) acc[qt][r] += fmax(qv * (double)a[u][r], qv * (double)cm[u][r]);
            }
        }
      } else {
        for (int x0 = 0; x0 < D; x0 += BT) {
          float a[BT][E];
#pragma unroll
          for (int u = 0; u < BT; ++u)
#pragma unroll
            for (int r = 0; r < E; ++r) a[u][r] = kr[(long)(x0 + u) * g.max_tiles + min(j0 + r, n - 1)];
#pragma unroll
          for (int u = 0; u < BT; ++u)
#pragma unroll
            for (int qt = 0; qt < QB; ++qt) {
              const double qv = (double)qbar[qt][x0 + u];
#pragma unroll
              for (int r = 0; r < E; ++r) acc[qt][r] = fma(qv, (double)a[u][r], acc[qt][r]);
            }
        }
      }
    }
    if (!topp) {
      if (K >= n) {  // every tile
        for (int x = tid; x < nq * n; x += kSelThreads) keep[(x / n) * ks + x % n] = 1;
      } else {
        __shared__ int rhist[QB][256];
        __shared__ int rdig[QB], rneed[QB], rcnt[QB];
        __shared__ uint64_t rkey[QB];
        uint64_t key[QB][E];
#pragma unroll
        for (int qt = 0; qt < QB; ++qt)
#pragma unroll
          for (int r = 0; r < E; ++r) key[qt][r] = order_key(acc[qt][r] * g.scale);
        topk_radix<E, QB>(key, nq, n, K, rhist, wtot_i, rdig, rneed, rcnt, rkey, keep, ks);
      }
    }
#pragma unroll
    for (int qt = 0; qt < QB; ++qt) {
      if (!topp || qt >= nq) break;  // uniform
      double sv[E];
      int si[E];
#pragma unroll
      for (int r = 0; r < E; ++r) {
        const bool valid = j0 + r < n;
        sv[r] = valid ? acc[qt][r] * g.scale : -DBL_MAX;
        si[r] = valid ? j0 + r : INT_MAX;
      }
      bitonic_sort_blocked<E>(sv, si, xs, xi);
#pragma unroll
      for (int r = 0; r < E; ++r)
        if (tid * E + r < K) keep[(qt) * ks + si[r]] = 1;
      if (topp) {
        // softmax weights in sorted order, their exclusive prefix sums (a
        // fixed-order block scan), and the shortest prefix whose mass reaches
        // p (the crossing tile included; every tile if the mass never does)
        if (tid == 0) top_s = sv[0];
        __syncthreads();
        const double mx = top_s;
        double e[E], loc = 0.0;
#pragma unroll
        for (int r = 0; r < E; ++r) {
          e[r] = si[r] < n ? exp(sv[r] - mx) : 0.0;
          loc += e[r];
        }
        double inc = loc;  // inclusive scan inside the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const double v = __shfl_up(inc, o);
          if (lane >= o) inc += v;
        }
        if (lane == 63) wsum[wave] = inc;
        __syncthreads();
        double before_wave = 0.0, z = 0.0;
#pragma unroll
        for (int w = 0; w < kSelThreads / 64; ++w) {
          if (w < wave) before_wave += wsum[w];
          z += wsum[w];
        }
        double before = before_wave + inc - loc;
#pragma unroll
        for (int r = 0; r < E; ++r) {
          if (si[r] < n && before / z < g.topp) keep[(qt) * ks + si[r]] = 1;
          before += e[r];
        }
        __syncthreads();  // top_s and wsum are reused by the next query tile
      }
    }
  }
  __syncthreads();

  // Ascending compaction of each query tile's kept flags.
  const int per = (n + kSelThreads - 1) / kSelThreads;
  const int c0 = tid * per;
  const int c1 = min(n, c0 + per);
  for (int qt = 0; qt < nq; ++qt) {
    const int i = i0 + qt;
    int local = 0;
    for (int j = c0; j < c1; ++j) local += keep[(qt) * ks + j];
    int total;
    int pos = block_exclusive_scan(local, wtot_i[0], &total);
    if (tid == 0) row_len[bh * g.max_tiles + i] = min(total, g.row_cap);
    int* dst = col_idx + (bh * g.max_tiles + i) * (long)g.row_cap;
    for (int j = c0; j < c1; ++j)
      if (keep[(qt) * ks + j]) {
        if (pos < g.row_cap) dst[pos] = j;
        ++pos;
      }
  }
}

// Explicit instantiations of the layout kernels the launcher picks by value.
#define VSA_LAYOUT_INST(D, F8)                                                                     \
  template __global__ void layout_kernel<D, F8>(Geo, const uint16_t*, const uint16_t*,            \
                                                const uint16_t*, uint16_t*, uint16_t*, uint16_t*, \
                                                float*, float*, float*, const int*, int,          \
                                                const uint32_t*, int*);
VSA_LAYOUT_INST(128, false)
VSA_LAYOUT_INST(128, true)
VSA_LAYOUT_INST(64, false)
VSA_LAYOUT_INST(64, true)
#undef VSA_LAYOUT_INST

}  // namespace


hipError_t launch_layout(const Geo& g, const Ws& w, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, bool pool, hipStream_t s) {
  dim3 grid(g.max_tiles, g.B * g.H);
  const int* cand = per_head_blocking(g) ? w.cand : nullptr;
  auto kern = g.d == 128 ? (g.f8 ? layout_kernel<128, true> : layout_kernel<128, false>)
                         : (g.f8 ? layout_kernel<64, true> : layout_kernel<64, false>);
  hipLaunchKernelGGL(kern, grid, dim3(kLayoutThreads), 0, s, g, q, k, v, w.qt, w.kt, w.vt,
                     w.pooled_q, w.pooled_k, w.pooled_kmin, cand, pool ? 1 : 0, w.f8_amax, w.f8_exp);
  return hipGetLastError();
}

hipError_t launch_amax(const Geo& g, const Ws& w, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, hipStream_t s) {
  hipLaunchKernelGGL(amax_kernel, dim3(kAmaxParts, g.B * g.H, 3), dim3(kAmaxThreads), 0, s, g, q, k,
                     v, w.f8_amax);
  return hipGetLastError();
}

hipError_t launch_untile(const Geo& g, const Ws& w, int which, uint16_t* out, hipStream_t s) {
  dim3 grid(g.max_tiles, g.B * g.H);
  const int* cand = per_head_blocking(g) ? w.cand : nullptr;
  const uint16_t* src = which ? w.kt : w.qt;
  if (g.d == 128)
    hipLaunchKernelGGL(untile_kernel<128>, grid, dim3(kLayoutThreads), 0, s, g, src, cand, out);
  else
    hipLaunchKernelGGL(untile_kernel<64>, grid, dim3(kLayoutThreads), 0, s, g, src, cand, out);
  return hipGetLastError();
}

hipError_t launch_select(const Geo& g, const Ws& w, hipStream_t s) {
  dim3 grid(g.max_tiles, g.B * g.H);
  const int* cand = per_head_blocking(g) ? w.cand : nullptr;
  // elements per thread: the largest row, padded to a power of two >= 256
  int m = kSelThreads;
  while (m < g.max_tiles) m <<= 1;
  const int E = m / kSelThreads;
  const size_t ks = ((size_t)g.max_tiles + 15) & ~(size_t)15;
  // query tiles per workgroup: 4 while the row's scores fit in registers and
  // the launch still has a few workgroups per SIMD (one pass over the key
  // summaries then serves four rows: Wan-14B selection 1.43 -> 0.90 ms), else
  // 1 (Wan-480p's 2,940 rows run faster one per workgroup)
  const bool four = E <= 4 && (long)g.B * g.H * ((g.max_tiles + 3) / 4) >= 4096;
  auto kern = four ? (E <= 1 ? select_kernel<1, 4> : E == 2 ? select_kernel<2, 4> : select_kernel<4, 4>)
                   : (E <= 1 ? select_kernel<1, 1> : E == 2 ? select_kernel<2, 1> : E == 4 ? select_kernel<4, 1>
                      : E == 8 ? select_kernel<8, 1> : select_kernel<16, 1>);
  const int qb = four ? 4 : 1;
  grid.x = (g.max_tiles + qb - 1) / qb;
  // kept flags of the workgroup's rows; the sort's exchange only under Top-P
  const size_t dyn = qb * ks + ((g.flags & VSA_TOPP) ? (size_t)m * (sizeof(double) + sizeof(int)) : 0);
  hipLaunchKernelGGL(kern, grid, dim3(kSelThreads), dyn, s, g, w.pooled_q, w.pooled_k, w.pooled_kmin, cand,
                     w.row_len, w.col_idx);
  return hipGetLastError();
}

}  // namespace vsa
