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
//  * K and V^T are streamed in chunks of 64 (or a final 32) keys through LDS
//    with direct global->LDS loads, double-buffered: chunk c+1 is in flight
//    while chunk c is multiplied.
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

constexpr int kMaxWaves = 4;
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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Direct global->LDS loads of one chunk (K: 64 keys x D, V^T: D x 64 keys).
// Each wave instruction moves 64 lanes x 16 B into 1 KB of contiguous LDS;
// the lane's global source is picked so that LDS ends up in the swizzled
// layout of Lds<D>.  The per-lane source offsets depend only on the lane and
// the tile's slot count, so they are computed once per kernel.  A 32-key
// chunk skips the K instructions of rows 32..63 and the V^T lanes of keys
// 32..63, so every access stays inside the tile.  No VGPR staging and no LDS
// stores: the data is in flight while the previous chunk is multiplied.
template <int D, int NW>
struct ChunkLoader {
  static constexpr int KI = Lds<D>::KC16;    // K instructions (1 KB each)
  static constexpr int VI = D / 8;           // V^T instructions
  static constexpr int NI = KI + VI;
  static constexpr int PER = (NI + NW - 1) / NW;
  int off[PER];        // source element offset inside the chunk's tile data
  unsigned vhi;        // bit x: this lane's V^T piece of instruction x holds keys 32..63

  __device__ __forceinline__ void init(int wave, int lane, int slots) {
    vhi = 0;
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int ins = wave + x * NW;
      const int P = ins * 64 + lane;
      if (ins < KI) {
        const int r = P / Lds<D>::KC16, pc = P % Lds<D>::KC16;
        const int c = pc ^ (core::key_perm(r & 31) & (Lds<D>::KC16 - 1));
        off[x] = r * D + c * 8;
      } else {
        const int Pv = P - KI * 64;
        const int d = Pv / 8, pc = Pv % 8;
        const int c = pc ^ ((d & 7) ^ ((d >> 3) & 1));
        off[x] = d * slots + c * 8;
        if (c >= 4) vhi |= 1u << x;
      }
    }
  }

  __device__ __forceinline__ void issue(uint16_t* stage, const uint16_t* __restrict__ kbase,
                                        const uint16_t* __restrict__ vbase, bool half, int wave) const {
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int ins = wave + x * NW;
      if (ins >= NI) break;
      if (ins < KI) {
        if (half && ins * 64 / Lds<D>::KC16 >= 32) continue;
        __builtin_amdgcn_global_load_lds(kbase + off[x], (lds_ptr_t)(stage + ins * 512), 16, 0, 0);
      } else if (!(half && ((vhi >> x) & 1u))) {
        __builtin_amdgcn_global_load_lds(vbase + off[x], (lds_ptr_t)(stage + ins * 512), 16, 0, 0);
      }
    }
  }
};

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 2) void attend_kernel(Geo g, int blocking,
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

  int stage = 0;
  const uint16_t* kt_head = kt + head_tm;
  const uint16_t* vt_head = vt + head_tm;
  auto kaddr = [&](const ChunkIter& it) { return kt_head + ((long)it.j * slots + it.off) * D; };
  auto vaddr = [&](const ChunkIter& it) { return vt_head + (long)it.j * D * slots + it.off; };
  ChunkLoader<D, NW> ldr;
  ldr.init(wave, lane, slots);
  if (L > 0) ldr.issue(lds, kaddr(cur), vaddr(cur), rows_of(cur) == 32, wave);
  wait_loads();
  __syncthreads();

  while (cur.e < L) {
    const ChunkIter nxt = advance(cur);
    const bool has_next = nxt.e < L;
    if (has_next)
      ldr.issue(lds + (stage ^ 1) * Lds<D>::STAGE, kaddr(nxt), vaddr(nxt), rows_of(nxt) == 32, wave);
    const uint16_t* lk = lds + stage * Lds<D>::STAGE;
    if (active) ws.chunk(lk, lk + Lds<D>::KE, min(kKC, cur.nv - cur.off), c2, col, hi);
    wait_loads();
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
