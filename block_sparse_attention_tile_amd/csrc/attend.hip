// Block-sparse flash attention over tile-major Q, K, V^T (CDNA4 / gfx950).
//
// For every (head, query tile i) the kept key tiles J(i) come from the
// selection stage; the kernel computes O_i = softmax(scale Q_i K_J^T) V_J with
// an online softmax (running max and sum), so skipped tiles cost nothing and
// the result equals masked softmax attention (SPADE review page, ledger
// axiom on FlashAttention-style online softmax; Sliding Tile Attention
// verdict page, pith_extraction.key_machinery: mask logic stays outside the
// dense compute, every computed block is dense).
//
// Design for gfx950:
//  * One workgroup = NW waves = NW*32 query rows of one query tile; a wave
//    owns 32 query rows for the whole KV sweep (its Q fragment stays in
//    VGPRs).
//  * K and V^T are streamed in chunks of 64 (or a final 32) keys through LDS,
//    double-buffered: the global loads of chunk c+1 are in flight while chunk
//    c is multiplied.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the output column is the
//    query, so each lane owns one query and 16 keys and the softmax row
//    reductions are lane-local (plus one swap between the wave halves).
//  * A-operand rows of K are read in a permuted order (bits 2 and 3 of the
//    row swapped) so that the fp32 S^T accumulator, converted to bf16, is
//    already the B operand of the next MFMA: O^T += V^T P^T.
//  * Lazy rescaling: the running max is only raised (and O rescaled) when a
//    new score exceeds it by more than 2^8 in exp2 units, which keeps every
//    probability <= 256 and is exact in the final normalisation.
//  * The epilogue writes O straight to the raster layout (the inverse
//    permutation is fused here), skipping padded query slots.
//  * Workgroups are mapped XCD-major: consecutive work items (same head,
//    neighbouring query tiles, which share most of their key tiles) land on
//    the same XCD and its L2.
#include <hip/hip_runtime.h>

#include "attn_core.h"
#include "vsa_internal.h"

namespace vsa {
namespace {

using core::kKC;
using core::Lds;
using core::u32x4;

constexpr int kMaxWaves = 8;
constexpr int kNumXcd = 8;

struct TileInfo {
  int it, ih, iw, et, eh, ew, nvalid;
};

__device__ __forceinline__ TileInfo tinfo(const Geo& g, const BlkGeo& b, int i) {
  TileInfo t;
  t.it = i / (b.nt[1] * b.nt[2]);
  t.ih = (i / b.nt[2]) % b.nt[1];
  t.iw = i % b.nt[2];
  t.et = min(b.tile[0], g.grid[0] - t.it * b.tile[0]);
  t.eh = min(b.tile[1], g.grid[1] - t.ih * b.tile[1]);
  t.ew = min(b.tile[2], g.grid[2] - t.iw * b.tile[2]);
  t.nvalid = t.et * t.eh * t.ew;
  return t;
}

__device__ __forceinline__ int tile_nvalid(const Geo& g, const BlkGeo& b, int j) {
  const int it = j / (b.nt[1] * b.nt[2]);
  const int ih = (j / b.nt[2]) % b.nt[1];
  const int iw = j % b.nt[2];
  return min(b.tile[0], g.grid[0] - it * b.tile[0]) * min(b.tile[1], g.grid[1] - ih * b.tile[1]) *
         min(b.tile[2], g.grid[2] - iw * b.tile[2]);
}

__device__ __forceinline__ long token_of(const Geo& g, const BlkGeo& b, const TileInfo& t, int s) {
  const int ehw = t.eh * t.ew;
  const int st = s / ehw;
  const int r = s - st * ehw;
  const int sh = r / t.ew;
  const int sw = r - sh * t.ew;
  return ((long)(t.it * b.tile[0] + st) * g.grid[1] + (t.ih * b.tile[1] + sh)) * g.grid[2] +
         (t.iw * b.tile[2] + sw);
}

// Iterator over the key chunks of one query tile's kept list.
struct ChunkIter {
  int e;      // position in the kept list
  int j;      // key tile
  int off;    // first slot of the chunk inside tile j
  int nv;     // valid keys of tile j
};

template <int D, int NW>
struct Loader {
  // per thread: K pieces + V^T pieces of one 64-key chunk
  static constexpr int KP = kKC * (D / 8);        // 16-byte pieces of K
  static constexpr int VP = D * (kKC / 8);        // 16-byte pieces of V^T
  static constexpr int T = NW * 64;
  static constexpr int NK = (KP + T - 1) / T;
  static constexpr int NV = (VP + T - 1) / T;
  u32x4 kr[NK];
  u32x4 vr[NV];

  // Unconditional loads from clamped, always in-bounds addresses keep the
  // staging arrays in VGPRs: pieces past `rows` (a 32-key chunk) re-read the
  // last valid row and are never used, pieces past the chunk duplicate the
  // last piece.
  __device__ __forceinline__ void load(const uint16_t* __restrict__ kt, const uint16_t* __restrict__ vt,
                                       long head_tm, int slots, int j, int off, int rows) {
    const int tid = threadIdx.x;
    const uint16_t* kbase = kt + head_tm + ((long)j * slots + off) * D;
    const uint16_t* vbase = vt + head_tm + (long)j * D * slots + off;
#pragma unroll
    for (int x = 0; x < NK; ++x) {
      const int pc = min(tid + x * T, KP - 1);
      const int r = min(pc / (D / 8), rows - 1), p = pc % (D / 8);
      kr[x] = *reinterpret_cast<const u32x4*>(kbase + (long)r * D + p * 8);
    }
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      const int pc = min(tid + x * T, VP - 1);
      const int dd = pc / (kKC / 8), p = min(pc % (kKC / 8), rows / 8 - 1);
      vr[x] = *reinterpret_cast<const u32x4*>(vbase + (long)dd * slots + p * 8);
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds) {
    const int tid = threadIdx.x;
    uint16_t* lk = lds;
    uint16_t* lvt = lds + Lds<D>::KE;
#pragma unroll
    for (int x = 0; x < NK; ++x) {
      const int pc = min(tid + x * T, KP - 1);
      const int r = pc / (D / 8), p = pc % (D / 8);
      *reinterpret_cast<u32x4*>(lk + r * Lds<D>::KS + p * 8) = kr[x];
    }
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      const int pc = min(tid + x * T, VP - 1);
      const int dd = pc / (kKC / 8), p = pc % (kKC / 8);
      *reinterpret_cast<u32x4*>(lvt + dd * Lds<D>::VS + p * 8) = vr[x];
    }
  }
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attend_kernel(Geo g, int blocking,
                                                         const uint16_t* __restrict__ qt,
                                                         const uint16_t* __restrict__ kt,
                                                         const uint16_t* __restrict__ vt,
                                                         const int* __restrict__ row_len,
                                                         const int* __restrict__ col_idx,
                                                         const int* __restrict__ cand,
                                                         uint16_t* __restrict__ o, int nsb,
                                                         int n_items) {
  extern __shared__ __align__(16) uint16_t lds[];

  // XCD-major mapping of workgroups to work items.
  const int per_xcd = (n_items + kNumXcd - 1) / kNumXcd;
  const int item = (blockIdx.x % kNumXcd) * per_xcd + blockIdx.x / kNumXcd;
  if (item >= n_items) return;
  const int sb = item % nsb;
  const int i = (item / nsb) % g.max_tiles;
  const long bh = item / (nsb * g.max_tiles);
  if (cand && cand[bh] != blocking) return;
  const BlkGeo b = pick_blk(g, blocking);
  if (i >= b.n_tiles) return;
  const int slots = b.slots;
  const int q0 = sb * NW * 32;
  if (q0 >= slots) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;      // query column inside the wave's 32 rows
  const int hi = lane >> 5;       // wave half
  const int qrow = q0 + wave * 32;
  const bool active = qrow < slots;
  const long head_tm = bh * g.tok_cap * D;
  const TileInfo ti = tinfo(g, b, i);

  core::WaveState<D> ws;
  if (active) ws.init(qt + head_tm + ((long)i * slots + qrow + col) * D, hi);
  const float c2 = (float)(g.scale * 1.4426950408889634);  // scale * log2(e)

  const int L = row_len[bh * g.max_tiles + i];
  const int* cols = col_idx + (bh * g.max_tiles + i) * (long)g.row_cap;

  // chunk iterator
  ChunkIter cur;
  cur.e = 0;
  cur.off = 0;
  if (L > 0) {
    cur.j = cols[0];
    cur.nv = tile_nvalid(g, b, cur.j);
  }
  auto rows_of = [&](const ChunkIter& it) {
    const int ck = min(kKC, it.nv - it.off);
    return ck > 32 ? 64 : 32;
  };
  auto advance = [&](ChunkIter it) {
    it.off += kKC;
    if (it.off >= it.nv) {
      it.off = 0;
      ++it.e;
      if (it.e < L) {
        it.j = cols[it.e];
        it.nv = tile_nvalid(g, b, it.j);
      }
    }
    return it;
  };

  Loader<D, NW> ld;
  int stage = 0;
  if (L > 0) {
    ld.load(kt, vt, head_tm, slots, cur.j, cur.off, rows_of(cur));
    ld.store(lds);
  }
  __syncthreads();

  while (cur.e < L) {
    const ChunkIter nxt = advance(cur);
    const bool has_next = nxt.e < L;
    if (has_next) ld.load(kt, vt, head_tm, slots, nxt.j, nxt.off, rows_of(nxt));
    const uint16_t* lk = lds + stage * Lds<D>::STAGE;
    if (active) ws.chunk(lk, lk + Lds<D>::KE, min(kKC, cur.nv - cur.off), c2, col, hi);
    if (has_next) ld.store(lds + (stage ^ 1) * Lds<D>::STAGE);
    __syncthreads();
    stage ^= 1;
    cur = nxt;
  }

  if (!active) return;
  const int qs = qrow + col;  // slot of this lane's query
  const bool valid = qs < ti.nvalid;
  uint16_t* op = o + (bh * (long)g.N + (valid ? token_of(g, b, ti, qs) : 0)) * D;
  ws.store(op, hi, valid);
}

template <int D, int NW>
hipError_t launch_one(const Geo& g, const Ws& w, int blocking, const int* cand, uint16_t* o,
                      hipStream_t s) {
  const BlkGeo& b = g.blk[blocking];
  const int slabs = b.slots / 32;
  const int nsb = (slabs + NW - 1) / NW;
  const long items = (long)g.B * g.H * g.max_tiles * nsb;
  const int per_xcd = (int)((items + kNumXcd - 1) / kNumXcd);
  const size_t shmem = 2 * Lds<D>::STAGE * sizeof(uint16_t);
  static bool attr_set = false;   // more than 64 KB of dynamic LDS must be requested
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attend_kernel<D, NW>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((attend_kernel<D, NW>), dim3(per_xcd * kNumXcd), dim3(NW * 64), shmem, s, g,
                     blocking, w.qt, w.kt, w.vt, w.row_len, w.col_idx, cand, o, nsb, (int)items);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Geo& g, const Ws& w, int blocking, const int* cand, uint16_t* o,
                    hipStream_t s) {
  // Waves per workgroup: split the tile's 32-row slabs into as few groups of
  // at most kMaxWaves as possible, balanced.
  const int slabs = g.blk[blocking].slots / 32;
  const int groups = (slabs + kMaxWaves - 1) / kMaxWaves;
  const int nw = (slabs + groups - 1) / groups;
  switch (nw) {
    case 1: return launch_one<D, 1>(g, w, blocking, cand, o, s);
    case 2: return launch_one<D, 2>(g, w, blocking, cand, o, s);
    case 3: return launch_one<D, 3>(g, w, blocking, cand, o, s);
    case 4: return launch_one<D, 4>(g, w, blocking, cand, o, s);
    case 5: return launch_one<D, 5>(g, w, blocking, cand, o, s);
    case 6: return launch_one<D, 6>(g, w, blocking, cand, o, s);
    case 7: return launch_one<D, 7>(g, w, blocking, cand, o, s);
    default: return launch_one<D, 8>(g, w, blocking, cand, o, s);
  }
}

}  // namespace

hipError_t launch_attend(const Geo& g, const Ws& w, uint16_t* o, hipStream_t s) {
  const int* cand = (g.flags & VSA_SICS_SELECT) ? w.cand : nullptr;
  // One launch per blocking (heads grouped by their chosen blocking); a
  // workgroup whose head chose another blocking exits at once.
  for (int c = 0; c < g.nb; ++c) {
    hipError_t e = (g.d == 128) ? launch_d<128>(g, w, c, cand, o, s) : launch_d<64>(g, w, c, cand, o, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace vsa
