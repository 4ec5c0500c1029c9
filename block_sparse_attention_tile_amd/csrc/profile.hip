// Online profiling selector (VSA_PROFILE_SELECT): per head, the candidate
// blocking whose masked attention on a sample of query rows is closest, in
// mean squared error, to full attention on the same rows (Sparse VideoGen
// verdict page, pith_extraction.key_machinery and core_discovery: spatial vs
// temporal heads decided by a ~1% row sample).
//
// Readings: the candidates are the plan's candidate blockings under the
// policy's static tile mask (window and / or sink, or dense); the sample is
// an evenly spread set of runs of 32 consecutive raster tokens; MSE is the
// mean over the sampled rows and channels; ties go to the lower candidate.
//
// The full pass visits a segment's keys (a range of whole lines of the
// raster grid, a line = the W tokens of one (t, h)) in chunks of 64
// consecutive keys; the masked pass visits them line by line.  A chunk is staged in LDS by
// direct global->LDS loads: K into the padded, lane-ordered rows the MFMA
// core reads, V into padded natural rows, then transposed LDS to LDS into
// the core's V^T rows (16-byte reads of 16 consecutive rows hit distinct
// banks; 4-byte writes of consecutive key pairs are consecutive).
//
// profile_full_kernel: kProfWaves waves (runs of 32 sampled rows of one head)
// share each staged chunk; the keys of a head are split into prof_segs
// ranges of lines, one workgroup each, so the launch fills the chip.  A
// chunk is loaded two iterations ahead and transposed one ahead, with one
// barrier per chunk.  Each wave stores its unnormalised partial (O^T, row
// sum, integer exp2 reference) per segment.
// profile_masked_kernel: one wave per (head, run, candidate) merges the
// segments into the full outputs (exact power-of-two rescales), then visits
// only the lines that some row's kept keys reach (K by direct loads, V
// through VGPRs with every load of a chunk in flight; 35 KB of LDS, so four
// of these latency-bound waves share a CU).  A candidate's kept keys
// on a line are, per query row, one interval of w (its window is a box of
// token coordinates) plus, for every row alike, one interval of sink tiles;
// the wave sums the squared differences of its masked outputs to the full
// ones.
// choose_profile_kernel: per head, the MSE of every candidate (fixed-order
// sums over the runs) and the argmin, into the workspace's CAND /
// CAND_SCORE regions that the layout, selection and attention read.
#include <hip/hip_runtime.h>

#include "attn_core.h"
#include "vsa_internal.h"

namespace vsa {
namespace {

using core::bf16x2;
using core::bf16x8;
using core::f32x16;
using core::kKC;
using core::Lds;

constexpr int kRun = 32;  // query rows per sampled run (one wave)

// Inclusive token range of axis a kept by a blocking's window around the
// query coordinate x (the window is in tiles; clamp mode shifts it inward).
__device__ __forceinline__ void window_axis(const Geo& g, const BlkGeo& b, int a, int x, int* lo,
                                            int* hi) {
  const int tile = a == 0 ? b.tile[0] : (a == 1 ? b.tile[1] : b.tile[2]);
  const int n = a == 0 ? b.nt[0] : (a == 1 ? b.nt[1] : b.nt[2]);
  const int grid = a == 0 ? g.grid[0] : (a == 1 ? g.grid[1] : g.grid[2]);
  const int win = a == 0 ? g.win[0] : (a == 1 ? g.win[1] : g.win[2]);
  if ((g.flags & VSA_DENSE) || !(g.flags & VSA_WINDOW)) {
    *lo = 0;
    *hi = grid - 1;
    return;
  }
  const int c = x / tile;
  const int r = (win - 1) / 2;
  int tl, th;
  if (g.win_mode == VSA_WIN_CLAMP && n >= 2 * r + 1) {
    tl = min(max(c - r, 0), n - (2 * r + 1));
    th = tl + 2 * r;
  } else {
    tl = max(c - r, 0);
    th = min(c + r, n - 1);
  }
  *lo = tl * tile;
  *hi = min((th + 1) * tile, grid) - 1;
}

// Accumulators of one candidate's masked attention.  Unlike the tile path,
// a row may see no kept key in a block (masks differ per row), so a row
// whose reference is still -inf takes zero probabilities instead of
// exp2(-inf + inf).
template <int D>
struct MaskedAcc {
  static constexpr int DT = D / 32;
  f32x16 acc[DT];
  float mo;
  float l_part;

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
    mo = -INFINITY;
    l_part = 0.f;
  }

  __device__ __forceinline__ void softmax(const f32x16& s, float c2, bf16x8 pb[2]) {
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    const float mxc = mx * c2;
    if (__any(mxc - mo > 8.0f)) {
      const float mn = fmaxf(mo, ceilf(fmaxf(mxc, __shfl_xor(mxc, 32))));
      const float alpha = mo == -INFINITY ? 0.f : __builtin_amdgcn_ldexpf(1.0f, (int)(mo - mn));
      l_part *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
      mo = mn;
    }
    const float off = mo == -INFINITY ? 0.f : mo;  // no key yet: every s is -inf
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int t = 0; t < 8; ++t) pb[half][t] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[half * 8 + t], c2, -off));
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        bf16x2 pr = {pb[half][t], pb[half][t + 1]};
        l_part = __builtin_amdgcn_fdot2_f32_bf16(pr, core::kOnes2, l_part, false);
      }
  }

  // VROW: elements per V^T row of the staged chunk
  template <int VROW>
  __device__ __forceinline__ void pv(const uint16_t* lvt, int kb, int col, int hi, const bf16x8 pb[2]) {
    const uint16_t* vp = lvt + col * VROW + kb * 32 + hi * 8;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(vp + dt * 32 * VROW + half * 16);
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[half], acc[dt], 0, 0, 0);
      }
  }
};

// Keys of a 32-key block outside [a1, b1] and [a2, b2] (block-relative key
// indices) get -inf.  Register r of lane half hi holds key 16*(r/8) +
// 8*hi + r%8 of the block (the lane order of attn_core.h); the thresholds
// are shifted by 8*hi and laundered so the compares stay against
// immediates.
__device__ __forceinline__ void mask_intervals(f32x16& s, int a1, int b1, int a2, int b2, int hi) {
  int t0 = a1 - 8 * hi, t1 = b1 - 8 * hi, t2 = a2 - 8 * hi, t3 = b2 - 8 * hi;
  asm volatile("" : "+v"(t0), "+v"(t1), "+v"(t2), "+v"(t3));
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int j = 16 * (r >> 3) + (r & 7);
    const bool keep = (j >= t0 && j <= t1) || (j >= t2 && j <= t3);
    if (!keep) s[r] = -INFINITY;
  }
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kFullWaves = kProfWaves;  // runs sharing one full-pass workgroup

// LDS parts of a chunk (bf16 elements): K rows in MFMA lane order and V rows
// in key order, both padded to D + 8 elements; V^T rows of Lds<D>.
template <int D>
struct Chunk {
  static constexpr int ROW = D + 8;
  static constexpr int KE = kKC * ROW;  // == Lds<D>::KE
  static constexpr int KC16 = D / 8;
  static constexpr int INS = kKC * (KC16 + 1) / 64;  // 1 KB direct loads per part
  static_assert(KE == Lds<D>::KE, "same K stage as the tile kernel");
};

// Issue the direct loads of keys [0, nk) of a chunk (rows past nk re-read row
// nk - 1; masks drop them): K into kbuf (lane order), V into vraw (key
// order).  The 2 * INS instructions are dealt round-robin over NW waves.
template <int D, int NW>
__device__ __forceinline__ void issue_chunk(uint16_t* kbuf, uint16_t* vraw, const uint16_t* __restrict__ k0,
                                            const uint16_t* __restrict__ v0, int nk, int wave, int lane) {
  constexpr int INS = Chunk<D>::INS, KC16 = Chunk<D>::KC16;
#pragma unroll
  for (int x = 0; x < (2 * INS + NW - 1) / NW; ++x) {
    const int ins = wave + x * NW;
    if (ins >= 2 * INS) break;  // wave-uniform
    const bool isv = ins >= INS;
    const int li = isv ? ins - INS : ins;
    const int u = li * 64 + lane;
    const int p = u / (KC16 + 1);
    const int c = min(u % (KC16 + 1), KC16 - 1);
    const int key = min(isv ? p : Lds<D>::key_of_row(p), nk - 1);
    __builtin_amdgcn_global_load_lds((isv ? v0 : k0) + (long)key * D + c * 8,
                                     (lds_ptr_t)((isv ? vraw : kbuf) + li * 512), 16, 0, 0);
  }
}

// V rows (key order, padded) -> V^T rows of Lds<D>, by NT threads: each
// work item packs one key pair of 8 channels into 8 dwords.
template <int D, int NT>
__device__ __forceinline__ void transpose_v(const uint16_t* vraw, uint16_t* lvt, int tid) {
  constexpr int ITEMS = (kKC / 2) * (D / 8);
#pragma unroll
  for (int x = 0; x < (ITEMS + NT - 1) / NT; ++x) {
    const int u = tid + x * NT;
    if (ITEMS % NT != 0 && u >= ITEMS) break;
    const int m = u % (kKC / 2), c8 = u / (kKC / 2);
    const uint4 a = *reinterpret_cast<const uint4*>(vraw + (2 * m) * Chunk<D>::ROW + c8 * 8);
    const uint4 b = *reinterpret_cast<const uint4*>(vraw + (2 * m + 1) * Chunk<D>::ROW + c8 * 8);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<uint32_t*>(lvt + (c8 * 8 + 2 * j) * Lds<D>::VROW + 2 * m) =
          (aw[j] & 0xffffu) | (bw[j] << 16);
      *reinterpret_cast<uint32_t*>(lvt + (c8 * 8 + 2 * j + 1) * Lds<D>::VROW + 2 * m) =
          (aw[j] >> 16) | (bw[j] & 0xffff0000u);
    }
  }
}

// V^T of keys [0, nk) of a chunk (keys past nk zero) through VGPRs: one
// channel pair per lane (with d = 64 the two lane halves split the keys),
// every load of the chunk in flight at once, then 16-byte writes of 8 keys.
template <int D>
__device__ __forceinline__ void stage_v_regs(uint16_t* lvt, const uint16_t* __restrict__ v0, int nk, int lane) {
  constexpr int PAIRS = D / 2;
  static_assert(PAIRS == 64 || PAIRS == 32, "d is 64 or 128");
  constexpr int KEYS = PAIRS == 64 ? 64 : 32;  // keys handled by one lane
  const int pp = lane % PAIRS;
  const int k_first = (lane / PAIRS) * KEYS;
  uint32_t wv[KEYS];
#pragma unroll
  for (int j = 0; j < KEYS; ++j) {
    const int key = k_first + j;
    wv[j] = key < nk ? *reinterpret_cast<const uint32_t*>(v0 + (long)key * D + 2 * pp) : 0u;
  }
#pragma unroll
  for (int g8 = 0; g8 < KEYS / 8; ++g8) {
    const uint32_t* w8 = wv + g8 * 8;
    uint4 lo, hv;
    lo.x = (w8[0] & 0xffffu) | (w8[1] << 16);
    lo.y = (w8[2] & 0xffffu) | (w8[3] << 16);
    lo.z = (w8[4] & 0xffffu) | (w8[5] << 16);
    lo.w = (w8[6] & 0xffffu) | (w8[7] << 16);
    hv.x = (w8[0] >> 16) | (w8[1] & 0xffff0000u);
    hv.y = (w8[2] >> 16) | (w8[3] & 0xffff0000u);
    hv.z = (w8[4] >> 16) | (w8[5] & 0xffff0000u);
    hv.w = (w8[6] >> 16) | (w8[7] & 0xffff0000u);
    const int c = k_first / 8 + g8;
    *reinterpret_cast<uint4*>(lvt + Lds<D>::v_off(2 * pp, c)) = lo;
    *reinterpret_cast<uint4*>(lvt + Lds<D>::v_off(2 * pp + 1, c)) = hv;
  }
}

// K of keys [0, nk) of a chunk by direct loads into lane-ordered rows (rows
// past nk re-read row nk - 1), one wave.
template <int D>
__device__ __forceinline__ void issue_k(uint16_t* kbuf, const uint16_t* __restrict__ k0, int nk, int lane) {
  constexpr int INS = Chunk<D>::INS, KC16 = Chunk<D>::KC16;
#pragma unroll
  for (int ins = 0; ins < INS; ++ins) {
    const int u = ins * 64 + lane;
    const int p = u / (KC16 + 1);
    const int c = min(u % (KC16 + 1), KC16 - 1);
    const int key = min(Lds<D>::key_of_row(p), nk - 1);
    __builtin_amdgcn_global_load_lds(k0 + (long)key * D + c * 8, (lds_ptr_t)(kbuf + ins * 512), 16, 0, 0);
  }
}

// The masked pass stages 32-key chunks: one wave per workgroup, no sharing,
// so a smaller stage lets more waves (and their loads) into a CU.  K rows in
// MFMA lane order, padded like the tile kernel's (the core's score reads);
// the K part is a whole number of 1 KB direct loads, rows past 31 are slack.
// V^T rows hold 32 keys plus one 16-byte pad.
template <int D>
struct MChunk {
  static constexpr int KC = 32;
  static constexpr int KC16 = D / 8;
  static constexpr int INS = (KC * (KC16 + 1) + 63) / 64;  // 1 KB direct loads of the K part
  static constexpr int KE = INS * 512;                     // elements of the K part
  static constexpr int VROW = KC + 8;                      // elements per V^T row
  static constexpr int VE = D * VROW;
};

// K of keys [0, nk <= 32) by direct loads into lane-ordered rows (rows past
// nk re-read row nk - 1), one wave.
template <int D>
__device__ __forceinline__ void issue_k32(uint16_t* kbuf, const uint16_t* __restrict__ k0, int nk, int lane) {
  constexpr int INS = MChunk<D>::INS, KC16 = MChunk<D>::KC16;
#pragma unroll
  for (int ins = 0; ins < INS; ++ins) {
    const int u = ins * 64 + lane;
    const int p = u / (KC16 + 1);
    const int c = min(u % (KC16 + 1), KC16 - 1);
    const int key = min(Lds<D>::key_of_row(p), nk - 1);
    __builtin_amdgcn_global_load_lds(k0 + (long)key * D + c * 8, (lds_ptr_t)(kbuf + ins * 512), 16, 0, 0);
  }
}

// V^T of keys [0, nk <= 32) (keys past nk zero) through VGPRs: one channel
// pair per lane (with d = 64 the two lane halves split the keys), every load
// in flight at once, then 16-byte writes of 8 keys.
template <int D>
__device__ __forceinline__ void stage_v32(uint16_t* lvt, const uint16_t* __restrict__ v0, int nk, int lane) {
  constexpr int PAIRS = D / 2;
  static_assert(PAIRS == 64 || PAIRS == 32, "d is 64 or 128");
  constexpr int KEYS = PAIRS == 64 ? 32 : 16;  // keys handled by one lane
  const int pp = lane % PAIRS;
  const int k_first = (lane / PAIRS) * KEYS;
  uint32_t wv[KEYS];
#pragma unroll
  for (int j = 0; j < KEYS; ++j) {
    const int key = k_first + j;
    wv[j] = key < nk ? *reinterpret_cast<const uint32_t*>(v0 + (long)key * D + 2 * pp) : 0u;
  }
#pragma unroll
  for (int g8 = 0; g8 < KEYS / 8; ++g8) {
    const uint32_t* w8 = wv + g8 * 8;
    uint4 lo, hv;
    lo.x = (w8[0] & 0xffffu) | (w8[1] << 16);
    lo.y = (w8[2] & 0xffffu) | (w8[3] << 16);
    lo.z = (w8[4] & 0xffffu) | (w8[5] << 16);
    lo.w = (w8[6] & 0xffffu) | (w8[7] << 16);
    hv.x = (w8[0] >> 16) | (w8[1] & 0xffff0000u);
    hv.y = (w8[2] >> 16) | (w8[3] & 0xffff0000u);
    hv.z = (w8[4] >> 16) | (w8[5] & 0xffff0000u);
    hv.w = (w8[6] >> 16) | (w8[7] & 0xffff0000u);
    const int c = k_first / 8 + g8;
    *reinterpret_cast<uint4*>(lvt + (2 * pp) * MChunk<D>::VROW + c * 8) = lo;
    *reinterpret_cast<uint4*>(lvt + (2 * pp + 1) * MChunk<D>::VROW + c * 8) = hv;
  }
}

// Full attention of the sampled rows over the keys of one segment of lines:
// kFullWaves waves (runs) share each chunk.  Three-deep pipeline with one
// barrier per chunk: chunk j's direct loads are issued two iterations ahead
// (K into one of three buffers, V rows into one of two), its V is
// transposed one iteration ahead (into one of two V^T buffers), and it is
// multiplied in iteration j.  Output per (run, segment, row): the
// unnormalised O^T registers, the row sum and the reference.
template <int D>
struct FullLds {
  static constexpr int K0 = 0;
  static constexpr int V0 = 3 * Chunk<D>::KE;          // V rows, two buffers
  static constexpr int T0 = V0 + 2 * Chunk<D>::KE;     // V^T, two buffers
  static constexpr int TOTAL = T0 + 2 * Lds<D>::VE;    // elements
};

template <int D>
__global__ __launch_bounds__(kFullWaves * 64, kFullWaves / 4) void profile_full_kernel(
    Geo g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    float* __restrict__ part_acc, float2* __restrict__ part_lm) {
  extern __shared__ __align__(16) uint16_t lds[];
  using F = FullLds<D>;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31, hi = lane >> 5;
  const int run = blockIdx.x * kFullWaves + wave;
  const bool active = run < g.prof_runs;
  const long bh = blockIdx.y;
  const int seg = blockIdx.z;
  const long N = g.N;
  const int W = g.grid[2];
  const long lines = (long)g.grid[0] * g.grid[1];
  const long l0 = lines * seg / g.prof_segs, l1 = lines * (seg + 1) / g.prof_segs;
  // the segment's keys are the contiguous raster range [l0 * W, l1 * W):
  // chunks of 64 run across line ends, so only the segment's last is partial
  const long seg_keys = (l1 - l0) * W;
  const long n = (seg_keys + kKC - 1) / kKC;
  const long row0 = N < kRun ? 0 : (long)min(run, g.prof_runs - 1) * N / g.prof_runs;
  const long qtok = min(row0 + col, N - 1);
  const long head = bh * N * D;

  core::WaveState<D> full;
  full.init(q + head + qtok * D, hi);
  const float c2 = (float)(g.scale * 1.4426950408889634);
  auto keys_of = [&](long i) { return (int)min((long)kKC, seg_keys - i * kKC); };
  auto issue = [&](long j) {
    const long key0 = l0 * W + j * kKC;
    issue_chunk<D, kFullWaves>(lds + F::K0 + (j % 3) * Chunk<D>::KE, lds + F::V0 + (j & 1) * Chunk<D>::KE,
                               k + head + key0 * D, v + head + key0 * D, keys_of(j), wave, lane);
  };
  if (n > 0) issue(0);
  if (n > 1) issue(1);
  if (n > 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    transpose_v<D, kFullWaves * 64>(lds + F::V0, lds + F::T0, tid);
  }
  for (long i = 0; i < n; ++i) {
    // chunk i + 1 has landed (every wave waited for its own loads) and its
    // V buffer is free to transpose; chunk i's V^T is complete; everything
    // chunk i - 1 read is free
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (i + 2 < n) issue(i + 2);
    if (i + 1 < n)
      transpose_v<D, kFullWaves * 64>(lds + F::V0 + ((i + 1) & 1) * Chunk<D>::KE,
                                      lds + F::T0 + ((i + 1) & 1) * Lds<D>::VE, tid);
    if (active) {
      const uint16_t* kcur = lds + F::K0 + (i % 3) * Chunk<D>::KE;
      const uint16_t* vcur = lds + F::T0 + (i & 1) * Lds<D>::VE;
      const int nk = keys_of(i);
      for (int kb = 0; kb < 2; ++kb) {
        const int nkb = nk - 32 * kb;
        if (nkb <= 0) break;
        f32x16 s = full.scores(kcur, kb, col, hi);
        if (nkb < 32) core::WaveState<D>::mask(s, nkb, hi);
        bf16x8 pb[2];
        full.softmax(s, c2, pb);
        full.pv(vcur, kb, col, hi, pb);
      }
    }
  }
  const float lt = full.l_part + __shfl_xor(full.l_part, 32);  // every lane of the wave takes part
  if (!active) return;
  const long slot = ((bh * g.prof_runs + run) * g.prof_segs + seg) * kRun + col;
  if (hi == 0) part_lm[slot] = make_float2(lt, full.mo);
  float* out = part_acc + slot * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float4 x;
      x.x = full.acc[dt][4 * r4 + 0];
      x.y = full.acc[dt][4 * r4 + 1];
      x.z = full.acc[dt][4 * r4 + 2];
      x.w = full.acc[dt][4 * r4 + 3];
      *reinterpret_cast<float4*>(out + dt * 32 + 8 * r4 + 4 * hi) = x;
    }
}

// The chunks a candidate visits for one run (wave-uniform): the lines that
// some row's window box (hull ulo..uhi) or the sink reaches, on each the hull
// of those w ranges, in steps of 64 keys.
struct MaskedChunks {
  int t, h, w0, w_hi, sink_end;
  bool valid;

  __device__ __forceinline__ bool line_at(const Geo& g, const BlkGeo& b, const int ulo[3],
                                          const int uhi[3]) {
    const int W = g.grid[2];
    const bool box_line = t >= ulo[0] && t <= uhi[0] && h >= ulo[1] && h <= uhi[1];
    // sink tiles on this line: tile index base + w / tw < sink
    const int base = ((t / b.tile[0]) * b.nt[1] + h / b.tile[1]) * b.nt[2];
    const int ms = g.sink - base;
    sink_end = ms > 0 ? (int)min((long)ms * b.tile[2], (long)W) : 0;  // w < sink_end
    if (!box_line && sink_end == 0) return false;
    w0 = box_line ? ulo[2] : W;
    w_hi = box_line ? uhi[2] : -1;
    if (sink_end > 0) {
      w0 = 0;
      w_hi = max(w_hi, sink_end - 1);
    }
    return true;
  }
  // from line (t, h) on, the first line that is visited
  __device__ __forceinline__ void seek(const Geo& g, const BlkGeo& b, const int ulo[3], const int uhi[3]) {
    for (; t < g.grid[0]; ++t, h = 0)
      for (; h < g.grid[1]; ++h)
        if (line_at(g, b, ulo, uhi)) {
          valid = true;
          return;
        }
    valid = false;
  }
  __device__ __forceinline__ void start(const Geo& g, const BlkGeo& b, const int ulo[3], const int uhi[3]) {
    t = 0;
    h = 0;
    seek(g, b, ulo, uhi);
  }
  __device__ __forceinline__ void next(const Geo& g, const BlkGeo& b, const int ulo[3], const int uhi[3]) {
    w0 += MChunk<128>::KC;
    if (w0 <= w_hi) return;
    if (++h == g.grid[1]) {
      h = 0;
      ++t;
    }
    seek(g, b, ulo, uhi);
  }
  __device__ __forceinline__ int keys() const { return min(MChunk<128>::KC, w_hi + 1 - w0); }
};

// One candidate (blockIdx.z) on one run: merge the full-pass segments of the
// 32 rows, then the masked attention over the keys the candidate's static
// mask keeps, and the sum over rows and channels of the squared difference.
template <int D>
__global__ __launch_bounds__(64, 2) void profile_masked_kernel(
    Geo g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ part_acc, const float2* __restrict__ part_lm, float* __restrict__ sse) {
  __shared__ __align__(16) uint16_t lds[MChunk<D>::KE + MChunk<D>::VE];
  uint16_t* const lk = lds;
  uint16_t* const lvt = lds + MChunk<D>::KE;
  const int run = blockIdx.x;
  const long bh = blockIdx.y;
  const int cand = blockIdx.z;
  const int lane = threadIdx.x;
  const int col = lane & 31, hi = lane >> 5;
  const int H = g.grid[1], W = g.grid[2];
  const long N = g.N;
  const long row0 = N < kRun ? 0 : (long)run * N / g.prof_runs;
  const bool valid = row0 + col < N;
  const long qtok = min(row0 + col, N - 1);
  const long head = bh * N * D;
  const BlkGeo b = pick_blk(g, cand);

  core::WaveState<D> qs;  // Q fragments and the score product only
  qs.init(q + head + qtok * D, hi);
  MaskedAcc<D> acc;
  acc.reset();
  const int qt = (int)(qtok / ((long)H * W)), qh = (int)((qtok / W) % H), qw = (int)(qtok % W);
  int blo[3], bhi[3];
  window_axis(g, b, 0, qt, &blo[0], &bhi[0]);
  window_axis(g, b, 1, qh, &blo[1], &bhi[1]);
  window_axis(g, b, 2, qw, &blo[2], &bhi[2]);
  // wave-uniform hull of the rows' boxes
  int ulo[3], uhi[3];
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    int lo = blo[a], hv = bhi[a];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      lo = min(lo, __shfl_xor(lo, m));
      hv = max(hv, __shfl_xor(hv, m));
    }
    ulo[a] = __builtin_amdgcn_readfirstlane(lo);
    uhi[a] = __builtin_amdgcn_readfirstlane(hv);
  }
  const float c2 = (float)(g.scale * 1.4426950408889634);

  MaskedChunks cur;
  for (cur.start(g, b, ulo, uhi); cur.valid; cur.next(g, b, ulo, uhi)) {
    const int nk = cur.keys();
    const long key0 = ((long)cur.t * H + cur.h) * W + cur.w0;
    // this row's interval on the line (box) and the line's sink interval;
    // a chunk that no row keeps a key of is not loaded
    const bool in = cur.t >= blo[0] && cur.t <= bhi[0] && cur.h >= blo[1] && cur.h <= bhi[1];
    const int ba = in ? blo[2] : 1, bb = in ? bhi[2] : 0;
    const int lo_k = cur.w0, hi_k = lo_k + nk - 1;  // w of the chunk's keys
    const int a1 = max(ba, lo_k), b1 = min(bb, hi_k);
    const int a2 = lo_k, b2 = min(cur.sink_end - 1, hi_k);
    if (!__any(a1 <= b1 || a2 <= b2)) continue;
    __syncthreads();  // the previous chunk's reads are done
    issue_k32<D>(lk, k + head + key0 * D, nk, lane);
    stage_v32<D>(lvt, v + head + key0 * D, nk, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the direct K loads have landed
    __syncthreads();
    f32x16 s = qs.scores(lk, 0, col, hi);
    mask_intervals(s, a1 - lo_k, b1 - lo_k, a2 - lo_k, b2 - lo_k, hi);
    bf16x8 pb[2];
    acc.softmax(s, c2, pb);
    acc.template pv<MChunk<D>::VROW>(lvt, 0, col, hi, pb);
  }

  // full outputs of this lane's row and channels: merge of the segments
  // (after the masked pass, so that their registers are free during it)
  float of[D / 32][16];
  {
    const long base = (bh * g.prof_runs + run) * g.prof_segs;
    float M = -INFINITY;
    for (int sg = 0; sg < g.prof_segs; ++sg) M = fmaxf(M, part_lm[(base + sg) * kRun + col].y);
    float l = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) of[dt][r] = 0.f;
    for (int sg = 0; sg < g.prof_segs; ++sg) {
      const float2 lm = part_lm[(base + sg) * kRun + col];
      if (lm.y == -INFINITY) continue;  // a segment that saw no key
      const float f = __builtin_amdgcn_ldexpf(1.0f, (int)(lm.y - M));
      l = fmaf(lm.x, f, l);
      const float* src = part_acc + ((base + sg) * kRun + col) * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const float4 x = *reinterpret_cast<const float4*>(src + dt * 32 + 8 * r4 + 4 * hi);
          of[dt][4 * r4 + 0] = fmaf(x.x, f, of[dt][4 * r4 + 0]);
          of[dt][4 * r4 + 1] = fmaf(x.y, f, of[dt][4 * r4 + 1]);
          of[dt][4 * r4 + 2] = fmaf(x.z, f, of[dt][4 * r4 + 2]);
          of[dt][4 * r4 + 3] = fmaf(x.w, f, of[dt][4 * r4 + 3]);
        }
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) of[dt][r] *= inv;
  }

  const float l = acc.l_part + __shfl_xor(acc.l_part, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float e = 0.f;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float d = acc.acc[dt][r] * inv - of[dt][r];
      e = fmaf(d, d, e);
    }
  if (!valid) e = 0.f;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) e += __shfl_xor(e, m);
  if (lane == 0) sse[(bh * g.prof_runs + run) * g.nb + cand] = e;
}

// Per head: MSE of every candidate (runs summed in order, fp64) and the
// argmin (ties to the lower index).
__global__ void choose_profile_kernel(Geo g, const float* __restrict__ sse, float* __restrict__ score,
                                      int* __restrict__ cand) {
  const long bh = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (bh >= (long)g.B * g.H) return;
  const double rows = (double)(g.N < kRun ? g.N : (long)kRun * g.prof_runs);
  int best = 0;
  double best_v = 0.0;
  for (int c = 0; c < g.nb; ++c) {
    double s = 0.0;
    for (int r = 0; r < g.prof_runs; ++r) s += (double)sse[(bh * g.prof_runs + r) * g.nb + c];
    const double mse = s / (rows * g.d);
    score[bh * g.nb + c] = (float)mse;
    if (c == 0 || mse < best_v) {
      best = c;
      best_v = mse;
    }
  }
  cand[bh] = best;
}

// Explicit instantiations of the kernels the launcher picks.
template __global__ void profile_full_kernel<128>(Geo, const uint16_t*, const uint16_t*, const uint16_t*,
                                                  float*, float2*);
template __global__ void profile_full_kernel<64>(Geo, const uint16_t*, const uint16_t*, const uint16_t*,
                                                 float*, float2*);
template __global__ void profile_masked_kernel<128>(Geo, const uint16_t*, const uint16_t*, const uint16_t*,
                                                    const float*, const float2*, float*);
template __global__ void profile_masked_kernel<64>(Geo, const uint16_t*, const uint16_t*, const uint16_t*,
                                                   const float*, const float2*, float*);

template <int D>
hipError_t launch_profile_d(const Geo& g, const Ws& w, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, hipStream_t s) {
  const size_t shmem = (size_t)FullLds<D>::TOTAL * sizeof(uint16_t);
  // more than 64 KB of dynamic LDS must be requested (per device)
  hipError_t e = ensure_dyn_lds(reinterpret_cast<const void*>(&profile_full_kernel<D>), shmem);
  if (e != hipSuccess) return e;
  float2* part_lm = reinterpret_cast<float2*>(w.prof_part);
  float* part_acc = w.prof_part + (size_t)g.B * g.H * g.prof_runs * g.prof_segs * kRun * 2;
  hipLaunchKernelGGL(profile_full_kernel<D>, dim3((g.prof_runs + kFullWaves - 1) / kFullWaves, g.B * g.H, g.prof_segs),
                     dim3(kFullWaves * 64), shmem, s, g, q, k, v, part_acc, part_lm);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(profile_masked_kernel<D>, dim3(g.prof_runs, g.B * g.H, g.nb), dim3(64), 0, s, g, q,
                     k, v, part_acc, part_lm, w.prof_sse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_profile(const Geo& g, const Ws& w, const uint16_t* q, const uint16_t* k,
                          const uint16_t* v, hipStream_t s) {
  hipError_t e = g.d == 128 ? launch_profile_d<128>(g, w, q, k, v, s) : launch_profile_d<64>(g, w, q, k, v, s);
  if (e != hipSuccess) return e;
  const int BH = g.B * g.H;
  hipLaunchKernelGGL(choose_profile_kernel, dim3((BH + 255) / 256), dim3(256), 0, s, g, w.prof_sse,
                     w.cand_score, w.cand);
  return hipGetLastError();
}

}  // namespace vsa
