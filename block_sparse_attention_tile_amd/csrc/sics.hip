// SICS: per-head choice of a blocking by intra-block cosine similarity.
//
// SPADE review page ("Core claim", "What carries the argument", Figure 3):
// every candidate 3D blocking of the Q/K token grid is scored by the sum of
// the pairwise cosine similarities of the tokens inside each block, computed
// in O(BS * d) with running partial sums; per head the best blocking wins.
// With unit vectors u = x / |x| the pair sum of a block is
//     SICS = sum_{a<b} u_a . u_b = (|sum_a u_a|^2 - #{a : x_a != 0}) / 2,
// which is the running-partial-sum form evaluated at the block's end.
//
// Readings (the equations are not printed on the page): blockings with
// different block sizes are compared by the mean pair cosine SICS_i/(n_i
// (n_i-1)/2) averaged over tiles with n_i >= 2; Q and K are both scored and
// averaged; ties go to the lower candidate index.
//
// Three kernels, no floating-point atomics (deterministic):
//   1. atom_kernel: one read of raster Q and K; per "atom" (the per-axis gcd
//      of the candidate tile extents, so every candidate tile is a union of
//      atoms) the sum of unit vectors and the count of non-zero tokens.
//   2. tile_kernel: per (head, candidate, tile) the sum of its atoms and
//      SICS of Q and of K.
//   3. choose_kernel: per head the mean pair cosine of each candidate and
//      the argmax.
#include <hip/hip_runtime.h>

#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kAtomWaves = 4;

// One wave per (head, tensor, atom).  Lanes are split into groups of D/8
// lanes; each group handles one token at a time (8 channels per lane).
template <int D>
__global__ __launch_bounds__(kAtomWaves * 64) void atom_kernel(Geo g, const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              float* __restrict__ atoms,
                                                              int* __restrict__ atom_nz) {
  constexpr int LPT = D / 8;       // lanes per token
  constexpr int TPW = 64 / LPT;    // tokens per wave pass
  const int lane = threadIdx.x & 63;
  const long wid = (long)blockIdx.x * kAtomWaves + (threadIdx.x >> 6);
  const long per_head = 2L * g.n_atoms;
  const long total = (long)g.B * g.H * per_head;
  if (wid >= total) return;
  const long bh = wid / per_head;
  const int which = (int)((wid / g.n_atoms) % 2);
  const int a = (int)(wid % g.n_atoms);
  const int at = a / (g.na[1] * g.na[2]);
  const int ah = (a / g.na[2]) % g.na[1];
  const int aw = a % g.na[2];
  const int t0 = at * g.atom[0], h0 = ah * g.atom[1], w0 = aw * g.atom[2];
  const int et = min(g.atom[0], g.grid[0] - t0);
  const int eh = min(g.atom[1], g.grid[1] - h0);
  const int ew = min(g.atom[2], g.grid[2] - w0);
  const int n = et * eh * ew;
  const uint16_t* x = (which ? k : q) + bh * (long)g.N * D;
  const int grp = lane / LPT, sub = lane % LPT;

  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.f;
  int nz = 0;
  constexpr int UP = 4;  // passes whose loads are in flight together
  for (int s0 = 0; s0 < n; s0 += TPW * UP) {
    uint4 raw[UP];
#pragma unroll
    for (int u = 0; u < UP; ++u) {
      const int s = s0 + u * TPW + grp;
      raw[u] = make_uint4(0, 0, 0, 0);
      if (s < n) {
        const int st = s / (eh * ew), sh = (s / ew) % eh, sw = s % ew;
        const long tok = ((long)(t0 + st) * g.grid[1] + (h0 + sh)) * g.grid[2] + (w0 + sw);
        raw[u] = *reinterpret_cast<const uint4*>(x + tok * D + sub * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < UP; ++u) {
      float v[8];
      const uint32_t w4[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        v[2 * c] = __uint_as_float(w4[c] << 16);
        v[2 * c + 1] = __uint_as_float(w4[c] & 0xffff0000u);
      }
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) ss = fmaf(v[c], v[c], ss);
#pragma unroll
      for (int m = 1; m < LPT; m <<= 1) ss += __shfl_xor(ss, m);
      if (ss > 0.f) {  // a pass beyond the atom reads zeros: no contribution
        const float inv = 1.0f / sqrtf(ss);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = fmaf(v[c], inv, acc[c]);
        nz += (sub == 0) ? 1 : 0;
      }
    }
  }
  // reduce over the token groups of the wave
#pragma unroll
  for (int m = LPT; m < 64; m <<= 1) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] += __shfl_xor(acc[c], m);
    nz += __shfl_xor(nz, m);
  }
  if (lane < LPT) {
    float* dst = atoms + ((bh * 2 + which) * (long)g.n_atoms + a) * D + lane * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) dst[c] = acc[c];
    if (lane == 0) atom_nz[(bh * 2 + which) * (long)g.n_atoms + a] = nz;
  }
}

// One workgroup of D threads per (head, candidate, tile): SICS of Q and K.
template <int D>
__global__ __launch_bounds__(D) void tile_kernel(Geo g, const float* __restrict__ atoms,
                                                 const int* __restrict__ atom_nz,
                                                 float* __restrict__ tile_sics) {
  __shared__ float red[D / 64];
  const int i = blockIdx.x;
  const int c = blockIdx.y;
  const long bh = blockIdx.z;
  const BlkGeo b = pick_blk(g, c);
  if (i >= b.n_tiles) return;
  const int it = i / (b.nt[1] * b.nt[2]), ih = (i / b.nt[2]) % b.nt[1], iw = i % b.nt[2];
  const int lo[3] = {it * b.tile[0], ih * b.tile[1], iw * b.tile[2]};
  int alo[3], ahi[3];
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    const int hi = min(lo[x] + b.tile[x], g.grid[x]);
    alo[x] = lo[x] / g.atom[x];
    ahi[x] = (hi + g.atom[x] - 1) / g.atom[x];
  }
  const int d = threadIdx.x;
  for (int which = 0; which < 2; ++which) {
    const float* base = atoms + (bh * 2 + which) * (long)g.n_atoms * D;
    const int* nzb = atom_nz + (bh * 2 + which) * (long)g.n_atoms;
    float s = 0.f;
    int nz = 0;
    for (int t = alo[0]; t < ahi[0]; ++t)
      for (int h = alo[1]; h < ahi[1]; ++h)
        for (int w = alo[2]; w < ahi[2]; ++w) {
          const int a = (t * g.na[1] + h) * g.na[2] + w;
          s += base[(long)a * D + d];
          nz += nzb[a];
        }
    float sq = s * s;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) sq += __shfl_xor(sq, m);
    if ((d & 63) == 0) red[d >> 6] = sq;
    __syncthreads();
    if (d == 0) {
      float tot = 0.f;
#pragma unroll
      for (int x = 0; x < D / 64; ++x) tot += red[x];
      tile_sics[((bh * g.nb + c) * 2 + which) * g.max_tiles + i] = 0.5f * (tot - (float)nz);
    }
    __syncthreads();
  }
}

// One workgroup per head: mean pair cosine of every candidate, argmax.
__global__ __launch_bounds__(256) void choose_kernel(Geo g, const float* __restrict__ tile_sics,
                                                     float* __restrict__ cand_score,
                                                     int* __restrict__ cand) {
  __shared__ double red[2][256];
  __shared__ int redn[256];
  __shared__ float score[VSA_MAX_CAND];
  const long bh = blockIdx.x;
  const int tid = threadIdx.x;
  for (int c = 0; c < g.nb; ++c) {
    const BlkGeo b = pick_blk(g, c);
    double sq = 0.0, sk = 0.0;
    int cnt = 0;
    for (int i = tid; i < b.n_tiles; i += 256) {
      const int it = i / (b.nt[1] * b.nt[2]), ih = (i / b.nt[2]) % b.nt[1], iw = i % b.nt[2];
      const long n = (long)min(b.tile[0], g.grid[0] - it * b.tile[0]) *
                     min(b.tile[1], g.grid[1] - ih * b.tile[1]) *
                     min(b.tile[2], g.grid[2] - iw * b.tile[2]);
      if (n < 2) continue;
      const double pairs = 0.5 * (double)n * (double)(n - 1);
      sq += (double)tile_sics[((bh * g.nb + c) * 2 + 0) * g.max_tiles + i] / pairs;
      sk += (double)tile_sics[((bh * g.nb + c) * 2 + 1) * g.max_tiles + i] / pairs;
      ++cnt;
    }
    red[0][tid] = sq;
    red[1][tid] = sk;
    redn[tid] = cnt;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (tid < s) {
        red[0][tid] += red[0][tid + s];
        red[1][tid] += red[1][tid + s];
        redn[tid] += redn[tid + s];
      }
      __syncthreads();
    }
    if (tid == 0) {
      const double m = redn[0] > 0 ? 0.5 * (red[0][0] + red[1][0]) / redn[0] : -1e30;
      score[c] = (float)m;
      cand_score[bh * g.nb + c] = (float)m;
    }
    __syncthreads();
  }
  if (tid == 0) {
    int best = 0;
    for (int c = 1; c < g.nb; ++c)
      if (score[c] > score[best]) best = c;
    cand[bh] = best;
  }
}

}  // namespace

hipError_t launch_sics(const Geo& g, const Ws& w, const uint16_t* q, const uint16_t* k,
                       hipStream_t s) {
  const long BH = (long)g.B * g.H;
  const long waves = BH * 2 * g.n_atoms;
  const long blocks = (waves + kAtomWaves - 1) / kAtomWaves;
  int* atom_nz = reinterpret_cast<int*>(w.atoms + BH * 2 * (long)g.n_atoms * g.d);
  if (g.d == 128)
    hipLaunchKernelGGL(atom_kernel<128>, dim3((unsigned)blocks), dim3(kAtomWaves * 64), 0, s, g, q, k,
                       w.atoms, atom_nz);
  else
    hipLaunchKernelGGL(atom_kernel<64>, dim3((unsigned)blocks), dim3(kAtomWaves * 64), 0, s, g, q, k,
                       w.atoms, atom_nz);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 tg(g.max_tiles, g.nb, (unsigned)BH);
  if (g.d == 128)
    hipLaunchKernelGGL(tile_kernel<128>, tg, dim3(128), 0, s, g, w.atoms, atom_nz, w.tile_sics);
  else
    hipLaunchKernelGGL(tile_kernel<64>, tg, dim3(64), 0, s, g, w.atoms, atom_nz, w.tile_sics);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(choose_kernel, dim3((unsigned)BH), dim3(256), 0, s, g, w.tile_sics, w.cand_score,
                     w.cand);
  return hipGetLastError();
}

}  // namespace vsa
