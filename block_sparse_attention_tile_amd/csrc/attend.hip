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
//  * One workgroup covers a whole query tile when it has at most 12 slabs of
//    32 rows (a 384-token tile is 12 waves, 3 per SIMD), so every K/V chunk
//    crosses from L2 into LDS once per query tile.  A wave owns 32 query rows
//    for the whole KV sweep; its Q fragment stays in VGPRs.
//  * K and V^T stream in chunks of 64 (or a final 32) keys through a ring of
//    LDS stages filled by direct global->LDS loads (no VGPR staging); half of
//    the ring is multiplied per barrier while the other half is in flight.
//  * The kept-tile list is copied to LDS first, so the loop issues no other
//    global loads that would drain the queue.
//  * The MFMA / online-softmax math per 32-key block is in attn_core.h
//    (bf16) and attn_core_f8.h (E4M3, VSA_COMPUTE_FP8: Sparse VideoGen
//    verdict page, optional FP8 attention; per-head power-of-two scales
//    from the layout stage).
//  * bf16: each wave reads its 32 query rows straight from the raster input
//    (once per workgroup, so the tile permutation costs nothing there); the
//    layout stage copies only K and V^T.
//  * The epilogue writes O straight to the raster layout (the inverse
//    permutation is fused here), skipping padded query slots.
//  * Workgroups are mapped XCD-major: consecutive work items (same head,
//    neighbouring query tiles, which share most of their key tiles) land on
//    the same XCD and its L2.
#include <hip/hip_runtime.h>

#include "attn_core.h"
#include "attn_core_f8.h"
#include "vsa_internal.h"

namespace vsa {
namespace {

using core::kKC;
static_assert(core::kKC == core8::kKC, "one chunk size");

// The two arithmetic variants of the kernel: element type of the staged
// tiles, LDS stage layout and per-wave core.
template <int D_>
struct Bf16Core {
  static constexpr int D = D_;
  static constexpr bool kF8 = false;
  using T = uint16_t;
  using L = core::Lds<D>;
  using WS = core::WaveState<D>;
};
template <int D_>
struct F8Core {
  static constexpr int D = D_;
  static constexpr bool kF8 = true;
  using T = uint8_t;
  using L = core8::Lds<D>;
  using WS = core8::WaveState<D>;
};

constexpr int kMaxWaves = 12;

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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// The kept-tile list in LDS holds, per entry, the key tile j in the low
// kTileBits bits, its valid key count in the next kTileBits bits (tiles are
// limited to 4096 of at most 4096 tokens, so the chunk iterators never
// divide), and above them which of the workgroup's query tiles keep it
// (bit 0: the first, bit 1: the second of a pair).
constexpr int kTileBits = 13;
constexpr int kFlagShift = 2 * kTileBits;
constexpr int kUnitNvShift = kTileBits + 8;  // unit-table entries: valid keys of the unit, minus 1
__device__ __forceinline__ int entry_nv(int x) { return (x >> kTileBits) & ((1 << kTileBits) - 1); }

// Visiting order of the query tiles of a static window mask (window alone,
// truncated at the grid edge): longest rows first, so that a launch ends on
// short rows and its last wave of workgroups leaves fewer CUs idle.  Along
// each axis the coordinates whose window is not cut by the edge come first,
// in order, then the edge coordinates by decreasing window extent (pairs
// r-1, n-r; r-2, n-r+1; ...).  Any order is correct: each tile is one
// workgroup's and its output rows are its own.
__device__ __forceinline__ int long_rows_first(const Geo& g, const BlkGeo& b, int i) {
  const int rk[3] = {i / (b.nt[1] * b.nt[2]), (i / b.nt[2]) % b.nt[1], i % b.nt[2]};
  int co[3];
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    const int n = b.nt[a], r = (g.win[a] - 1) / 2, inner = n - 2 * r;
    if (inner < 1 || rk[a] < inner) {
      co[a] = inner < 1 ? rk[a] : r + rk[a];
    } else {
      const int k = rk[a] - inner, p = k >> 1;
      co[a] = (k & 1) ? n - r + p : r - 1 - p;
    }
  }
  return (co[0] * b.nt[1] + co[1]) * b.nt[2] + co[2];
}

// How many heads chose `blocking` (every head without a per-head choice).
// Wave-uniform.
__device__ __forceinline__ int heads_with(const Geo& g, const int* cand, int blocking) {
  const long BH = (long)g.B * g.H;
  if (!cand) return (int)BH;
  const int lane = threadIdx.x & 63;
  int n = 0;
  for (long base = 0; base < BH; base += 64) {
    const long h = base + lane;
    n += __popcll(__ballot(h < BH && cand_of(g, cand, h) == blocking));
  }
  return n;
}

// The r-th head, in head order, whose chosen blocking is `blocking` (every
// head without a per-head choice); -1 past the last.  Wave-uniform: each
// lane tests one head of a 64-head window, a ballot counts the hits.
__device__ __forceinline__ long nth_head(const Geo& g, const int* cand, int blocking, int r) {
  const long BH = (long)g.B * g.H;
  if (!cand) return r < BH ? r : -1;
  const int lane = threadIdx.x & 63;
  for (long base = 0; base < BH; base += 64) {
    const long h = base + lane;
    const uint64_t hits = __ballot(h < BH && cand_of(g, cand, h) == blocking);
    const int n = __popcll(hits);
    if (r < n) {
      const bool mine = ((hits >> lane) & 1) && __popcll(hits & ((1ull << lane) - 1)) == r;
      return base + __ffsll((unsigned long long)__ballot(mine)) - 1;
    }
    r -= n;
  }
  return -1;
}

// Iterator over the 64-key chunks of a query tile's kept key tiles.
struct ChunkIter {
  int e;    // position in the kept list
  int j;    // key tile
  int off;  // first slot of the chunk inside tile j
  int nv;   // valid keys of tile j
  int fl;   // query tiles of the workgroup that keep tile j
  __device__ __forceinline__ void load(const int* cols) {
    const int x = __builtin_amdgcn_readfirstlane(cols[e]);  // uniform: keep the iterator scalar
    j = x & ((1 << kTileBits) - 1);
    nv = entry_nv(x);
    fl = x >> kFlagShift;
  }
  __device__ __forceinline__ void start(const int* cols, int L) {
    e = 0;
    off = 0;
    j = 0;
    nv = 0;
    fl = 0;
    if (L > 0) load(cols);
  }
  __device__ __forceinline__ void next(const int* cols, int L) {
    off += kKC;
    if (off >= nv) {
      off = 0;
      if (++e < L) load(cols);
    }
  }
  __device__ __forceinline__ int keys() const { return min(kKC, nv - off); }
};

// Interleaved pair schedule (interleaved_pairs): one entry per chunk, with
// the key tile in the low kTileBits bits, the chunk's index inside the tile
// in the next 4, its valid keys minus one from bit kCkKeysShift (6 bits)
// and the query-tile flags from kFlagShift.  Tiles are paired only when
// they hold at most 6 slabs (192 keys, three chunks), so the chunk index
// fits its 4 bits.
constexpr int kCkKeysShift = kTileBits + 4;
static_assert(kCkKeysShift + 6 <= kFlagShift, "schedule fields do not overlap");

struct ListIter {
  int c;    // position in the schedule
  int j;    // key tile
  int off;  // first slot of the chunk inside tile j
  int kv;   // valid keys of the chunk
  int fl;   // query tiles of the workgroup that keep tile j
  __device__ __forceinline__ void load(const int* ck) {
    const int x = __builtin_amdgcn_readfirstlane(ck[c]);  // uniform: keep the iterator scalar
    j = x & ((1 << kTileBits) - 1);
    off = ((x >> kTileBits) & 15) * kKC;
    kv = ((x >> kCkKeysShift) & 63) + 1;
    fl = x >> kFlagShift;
  }
  __device__ __forceinline__ void start(const int* ck, int n) {
    c = 0;
    j = off = kv = fl = 0;
    if (n > 0) load(ck);
  }
  __device__ __forceinline__ void next(const int* ck, int n) {
    if (++c < n) load(ck);
  }
  __device__ __forceinline__ int keys() const { return kv; }
};

// Unit mode: element offsets of the first key of a chunk's four 16-key
// units in the head's K (k0..k3) and V^T (v0..v3).
struct UnitBases {
  int k0, k1, k2, k3, v0, v1, v2, v3;
};

// Direct global->LDS loads of one chunk (K: 64 keys x D, V^T: D x 64 keys).
// Each wave instruction moves 64 lanes x 16 B into 1 KB of contiguous LDS;
// the lane's global source is picked so that LDS ends up in the padded,
// lane-ordered layout of the stage (a padding unit re-reads its row's last
// data unit).  The NI instructions of a chunk are dealt round-robin over the
// waves.  A 32-key chunk clamps the source rows / key columns past 32 to the
// last valid ones: every access stays inside the tile, and every LDS byte
// of the stage holds tile data (slots the math does not use are multiplied
// by zero probabilities, never by stale memory).
template <class C, int NW>
struct ChunkLoader {
  static constexpr int D = C::D;
  using L = typename C::L;
  using T = typename C::T;
  static constexpr int E = 16 / (int)sizeof(T);        // elements per 16-byte unit
  static constexpr int KU = kKC * (L::KC16 + 1);       // 16-byte units of the K part
  static constexpr int VU = D * (L::VC16 + 1);         // and of the V^T part
  static constexpr int KI = KU / 64;                   // K instructions (1 KB each)
  static constexpr int VI = VU / 64;                   // V^T instructions
  static constexpr int NI = KI + VI;
  static constexpr int PER = (NI + NW - 1) / NW;
  static_assert(KU % 64 == 0 && VU % 64 == 0, "whole instructions per part");
  static constexpr int SZ = (int)sizeof(T);
  int wave;                // wave-uniform
  int lane;
  uint32_t off_full[PER];  // source byte offsets of this lane's pieces from the chunk's K or
                           // V^T base, 64-key chunk (a scalar base plus a 32-bit lane offset
                           // is the load's own addressing form: no per-load address math)

  __device__ __forceinline__ static int ins_of(int wave, int x) {
    return min(wave + x * NW, NI - 1);  // past the last: clamped, never issued
  }

  __device__ __forceinline__ void init(int w, int ln, int slots) {
    wave = __builtin_amdgcn_readfirstlane(w);
    __builtin_assume(wave >= 0 && wave < NW);  // settles most per-piece branches at compile time
    lane = ln;
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int ins = ins_of(wave, x);
      const int u = ins * 64 + lane;
      if (ins < KI) {
        const int p = u / (L::KC16 + 1);                   // physical row
        const int c = min(u % (L::KC16 + 1), L::KC16 - 1);
        off_full[x] = (uint32_t)((L::key_of_row(p) * D + c * E) * SZ);
      } else {
        const int v = u - KU;
        const int d = v / (L::VC16 + 1);
        const int c = min(v % (L::VC16 + 1), L::VC16 - 1);
        off_full[x] = (uint32_t)((d * slots + c * E) * SZ);
      }
    }
  }

  // The source byte offset of piece x for a 32-key chunk: K rows past 31 and
  // V^T key columns past 31 are clamped to the last valid ones (derived from
  // the 64-key offset: K rows are D elements apart, the V^T column unit is
  // recomputed).
  // With six or more pieces per lane, holding these offsets across the
  // loop beside the 64-key ones spills; they are recomputed per 32-key chunk
  // instead (the empty asm keeps the compiler from hoisting them).
  __device__ __forceinline__ uint32_t off_half(int x) const {
    constexpr int HU = L::VC16 / 2;  // data units of 32 keys
    uint32_t o = off_full[x];
    int ln = lane;
    if constexpr (PER >= 6) asm volatile("" : "+v"(o), "+v"(ln));
    const int ins = ins_of(wave, x);
    if (ins < KI) return min(o, (uint32_t)(31 * D * SZ) + (o & (uint32_t)(D * SZ - 1)));
    const int c = min((ins * 64 + ln - KU) % (L::VC16 + 1), L::VC16 - 1);
    return o - (uint32_t)(max(c - (HU - 1), 0) * 16);  // 16 bytes per data unit
  }

  template <bool HALF>
  __device__ __forceinline__ void issue_t(T* stage, const T* __restrict__ kbase,
                                          const T* __restrict__ vbase) const {
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      if (wave + x * NW >= NI) break;  // wave-uniform
      const int ins = ins_of(wave, x);
      const char* base = reinterpret_cast<const char*>(ins < KI ? kbase : vbase);
      uint32_t o = HALF ? off_half(x) : off_full[x];
      // (the empty asm keeps the offset 32-bit up to the load, which then
      // takes the scalar-base form instead of a 64-bit VGPR address)
      asm volatile("" : "+v"(o));
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const T*>(base + o),
                                       (lds_ptr_t)(stage + ins * (1024 / (int)sizeof(T))), 16, 0, 0);
    }
  }
  // one branch per chunk on its size, not one per piece
  __device__ __forceinline__ void issue(T* stage, const T* __restrict__ kbase,
                                        const T* __restrict__ vbase, bool half) const {
    if (half)
      issue_t<true>(stage, kbase, vbase);
    else
      issue_t<false>(stage, kbase, vbase);
  }

  // Unit mode: a chunk is 64 / KU units of KU keys (16 for bf16, 32 for
  // E4M3, whose V^T slot permutation stays inside 32-slot groups), each from
  // its own key tile.  Piece x of this lane belongs to unit unit_of[x] (K:
  // key row / KU; V^T: the 16-byte key column's first key / KU) and sits at
  // off_full[x] inside it.
  static constexpr int KU_ = C::kF8 ? 32 : 16;
  int unit_of[PER];

  __device__ __forceinline__ void init_units(int w, int ln, int slots) {
    static_assert(KU_ % E == 0, "a 16-byte V^T column lies inside one unit");
    wave = __builtin_amdgcn_readfirstlane(w);
    __builtin_assume(wave >= 0 && wave < NW);
    lane = ln;
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int ins = ins_of(wave, x);
      const int u = ins * 64 + lane;
      if (ins < KI) {
        const int key = L::key_of_row(u / (L::KC16 + 1));
        const int c = min(u % (L::KC16 + 1), L::KC16 - 1);
        unit_of[x] = key / KU_;
        off_full[x] = (uint32_t)(((key % KU_) * D + c * E) * SZ);
      } else {
        const int v = u - KU;
        const int d = v / (L::VC16 + 1);
        const int c = min(v % (L::VC16 + 1), L::VC16 - 1);
        unit_of[x] = c * E / KU_;
        off_full[x] = (uint32_t)((d * slots + (c * E) % KU_) * SZ);
      }
    }
  }

  // u.k[t] / u.v[t]: element offsets of unit t's first key in the head's K
  // and V^T (wave-uniform; named scalars, so the per-lane pick stays two
  // levels of selects instead of an indexed private array).
  __device__ __forceinline__ static int pick(int u, int b0, int b1, int b2, int b3) {
    const int lo = (u & 1) ? b1 : b0;
    const int hi = (u & 1) ? b3 : b2;
    return (u & 2) ? hi : lo;
  }
  __device__ __forceinline__ void issue_units(T* stage, const T* __restrict__ kt_head,
                                              const T* __restrict__ vt_head, const UnitBases& ub) const {
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      if (wave + x * NW >= NI) break;  // wave-uniform
      const int ins = ins_of(wave, x);
      // element offsets of a head's K or V^T fit 31 bits (checked before a
      // unit-mode launch), so the byte offset fits the 32-bit lane offset
      const int ue = ins < KI ? pick(unit_of[x], ub.k0, ub.k1, ub.k2, ub.k3)
                              : pick(unit_of[x], ub.v0, ub.v1, ub.v2, ub.v3);
      const char* head = reinterpret_cast<const char*>(ins < KI ? kt_head : vt_head);
      uint32_t o = (uint32_t)ue * (uint32_t)SZ + off_full[x];
      asm volatile("" : "+v"(o));
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const T*>(head + o),
                                       (lds_ptr_t)(stage + ins * (1024 / (int)sizeof(T))),
                                       16, 0, 0);
    }
  }
};

// K and V^T element offsets of the first key of a unit-table entry.
template <int D, int KU>
__device__ __forceinline__ void unit_bases(int entry, int slots, int& kb, int& vb) {
  const int x = __builtin_amdgcn_readfirstlane(entry);
  const int j = x & ((1 << kTileBits) - 1);
  const int uo = KU * ((x >> kTileBits) & 255);
  kb = (j * slots + uo) * D;
  vb = j * D * slots + uo;
}

// All of this wave's outstanding loads have landed, then barrier: after it
// every wave's pieces of the chunks issued so far are visible in LDS, and
// every wave is done with the stages the next loads will overwrite.
__device__ __forceinline__ void wait_loads_and_barrier() {
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

// Waves per SIMD the register budget is sized for: one- and two-wave groups
// (whose loaders keep many per-lane offsets) get 2; all others 3 (168 VGPRs),
// so two small workgroups can share a CU.
constexpr int waves_per_simd(int nw) { return nw > 2 ? 3 : 2; }

// TPW query tiles per workgroup (1, or 2 for a pair of adjacent tiles whose
// waves share the staged chunks of the union of their kept lists); NW / TPW
// waves per query tile.  UN (pairs whose tile sizes leave short tails): the
// kept keys are cut into 16-key (E4M3: 32-key)
// units (a tile of nv keys gives ceil(nv / 16), or ceil(nv / 32)), taken
// four (two) per chunk in list order, so a tile's short tail shares its chunk
// with the next tile's keys instead of occupying a chunk of its own.
template <class C, int NW, int STAGES, int TPW, bool UN>
__global__ __launch_bounds__(NW * 64, waves_per_simd(NW)) void attend_kernel(
    Geo g, int blocking, const typename C::T* __restrict__ qt, const typename C::T* __restrict__ kt,
    const typename C::T* __restrict__ vt, const int* __restrict__ row_len,
    const int* __restrict__ col_idx, const int* __restrict__ cand, const int* __restrict__ f8_exp,
    uint16_t* __restrict__ o, int nsb, int n_items, const uint16_t* __restrict__ qr) {
  constexpr int D = C::D;
  using T = typename C::T;
  using Stage = typename C::L;
  extern __shared__ __align__(16) unsigned char lds_bytes[];
  T* const lds = reinterpret_cast<T*>(lds_bytes);
  using Loader = ChunkLoader<C, NW>;
  constexpr int WPT = NW / TPW;  // waves per query tile
  static_assert(TPW == 1 || TPW == 2, "one tile or a pair per workgroup");
  static_assert(!UN || TPW == 2, "units: pairs");
  constexpr int KU = C::kF8 ? 32 : 16;  // keys per unit (unit mode)
  constexpr int UPC = kKC / KU;         // units per chunk

  // Workgroups to work items (head, query tile or pair, slab group).  The
  // hardware deals consecutive workgroups to the eight XCDs in turn.
  const BlkGeo b = pick_blk(g, blocking);
  int sb, i0;
  long bh;
  if (g.head_sync) {
    // Head-synchronous: every XCD takes one contiguous eighth of each head's
    // items, and all XCDs walk the heads that chose this blocking in order.
    const int per_head = (b.n_tiles + TPW - 1) / TPW * nsb;
    const int per_hx = (per_head + kNumXcd - 1) / kNumXcd;
    const int j = blockIdx.x / kNumXcd;
    const int in_head = (blockIdx.x % kNumXcd) * per_hx + j % per_hx;
    if (in_head >= per_head) return;
    bh = nth_head(g, cand, blocking, j / per_hx);
    if (bh < 0) return;
    sb = in_head % nsb;
    i0 = in_head / nsb * TPW;
  } else if (cand) {
    // XCD-major over the heads that chose this blocking (their count comes
    // from the choices; the grid covers every head): each XCD takes one
    // contiguous range of those heads' items, so the XCDs get equal shares
    // however the choices fall.
    const int per_head = (b.n_tiles + TPW - 1) / TPW * nsb;
    const long n_act = (long)heads_with(g, cand, blocking) * per_head;
    const long per_x = (n_act + kNumXcd - 1) / kNumXcd;
    const long j = blockIdx.x / kNumXcd;
    const long item = (blockIdx.x % kNumXcd) * per_x + j;
    if (j >= per_x || item >= n_act) return;
    bh = nth_head(g, cand, blocking, (int)(item / per_head));
    if (bh < 0) return;
    const int in_head = (int)(item % per_head);
    sb = in_head % nsb;
    i0 = in_head / nsb * TPW;
  } else {
    // XCD-major: each XCD takes one contiguous range of all items, so
    // neighbouring query tiles of a head (sharing window tiles) run on the
    // same XCD and its L2.
    const int units = (g.max_tiles + TPW - 1) / TPW;  // tiles (or pairs) per head
    const int per_xcd = (n_items + kNumXcd - 1) / kNumXcd;
    const int item = (blockIdx.x % kNumXcd) * per_xcd + blockIdx.x / kNumXcd;
    if (item >= n_items) return;
    sb = item % nsb;
    i0 = ((item / nsb) % units) * TPW;  // first query tile of the workgroup
    bh = item / (nsb * units);
    if (cand_of(g, cand, bh) != blocking) return;
  }
  if (i0 >= b.n_tiles) return;
  // a static window truncated at the edge: longest rows first
  // (HunyuanVideo: attention 15.42 -> 15.29 ms)
  if (TPW == 1 && (g.flags & VSA_WINDOW) && g.win_mode == VSA_WIN_TRUNCATE &&
      !(g.flags & (VSA_DENSE | VSA_TOPK | VSA_TOPK_FRAC | VSA_TOPP)))
    i0 = long_rows_first(g, b, i0);
  const int slots = b.slots;
  const int q0 = sb * WPT * 32;
  if (q0 >= slots) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;  // query column inside the wave's 32 rows
  const int hi = lane >> 5;   // wave half
  const int sub = wave / WPT;          // which query tile of the workgroup this wave serves
  const int i = i0 + sub;              // that query tile
  const int qrow = q0 + (wave - sub * WPT) * 32;  // first query row of this wave
  const bool active = i < b.n_tiles && qrow < slots;
  const long head_tm = bh * g.tok_cap * D;

  // kept-tile list -> LDS (after the K/V stages)
  int* cols = reinterpret_cast<int*>(lds + STAGES * Stage::STAGE);
  // (row lengths and tile indices clamped: a selection that was never
  // written still keeps every access in bounds)
  int L;
  if constexpr (TPW == 1) {
    L = min(max(row_len[bh * g.max_tiles + i0], 0), g.row_cap);
    const int* gcols = col_idx + (bh * g.max_tiles + i0) * (long)g.row_cap;
    for (int e = tid; e < L; e += NW * 64) {
      const int j = min(max(gcols[e], 0), b.n_tiles - 1);
      cols[e] = (1 << kFlagShift) | (tile_nvalid(g, b, j) << kTileBits) | j;
    }
  } else {
    // both tiles' lists, then their ascending union with per-tile flags
    // (each tile then meets its own kept tiles in its own list's order)
    int* la = cols + 2 * g.row_cap;
    int* lb = la + g.row_cap;
    int* nu = lb + g.row_cap;
    const bool has_b = i0 + 1 < b.n_tiles;
    const int na = min(max(row_len[bh * g.max_tiles + i0], 0), g.row_cap);
    const int nb = has_b ? min(max(row_len[bh * g.max_tiles + i0 + 1], 0), g.row_cap) : 0;
    const int* ga = col_idx + (bh * g.max_tiles + i0) * (long)g.row_cap;
    const int* gb = ga + g.row_cap;
    for (int e = tid; e < na; e += NW * 64) la[e] = min(max(ga[e], 0), b.n_tiles - 1);
    for (int e = tid; e < nb; e += NW * 64) lb[e] = min(max(gb[e], 0), b.n_tiles - 1);
    __syncthreads();
    if (tid == 0) {
      int ia = 0, ib = 0, n = 0;
      while (ia < na || ib < nb) {  // every pass consumes at least one entry
        const int ja = ia < na ? la[ia] : 0x7fffffff;
        const int jb = ib < nb ? lb[ib] : 0x7fffffff;
        const int j = min(ja, jb);
        const int fl = (ja == j ? 1 : 0) | (jb == j ? 2 : 0);
        ia += ja == j;
        ib += jb == j;
        cols[n++] = (fl << kFlagShift) | (tile_nvalid(g, b, j) << kTileBits) | j;
      }
      *nu = n;
      if constexpr (!UN) {
        if (interleaved_pairs(g)) {
          // the chunks both tiles keep (ascending), then the chunks only one
          // keeps, taken from the two tiles' ascending lists in turn
          int* ck = cols + ((4 * g.row_cap + 2 + 3) & ~3);
          int m = 0;
          auto emit = [&](int x, int off) {
            ck[m++] = (x & ((1 << kTileBits) - 1)) | ((off / kKC) << kTileBits) |
                      ((min(kKC, entry_nv(x) - off) - 1) << kCkKeysShift) | ((x >> kFlagShift) << kFlagShift);
          };
          for (int e = 0; e < n; ++e)
            if ((cols[e] >> kFlagShift) == 3)
              for (int off = 0; off < entry_nv(cols[e]); off += kKC) emit(cols[e], off);
          auto next_of = [&](int e, int f) {
            do ++e; while (e < n && ((cols[e] >> kFlagShift) != f || entry_nv(cols[e]) == 0));
            return e;
          };
          int ea = next_of(-1, 1), eb = next_of(-1, 2), oa = 0, ob = 0;
          while (ea < n || eb < n) {
            if (ea < n) {
              emit(cols[ea], oa);
              if ((oa += kKC) >= entry_nv(cols[ea])) { oa = 0; ea = next_of(ea, 1); }
            }
            if (eb < n) {
              emit(cols[eb], ob);
              if ((ob += kKC) >= entry_nv(cols[eb])) { ob = 0; eb = next_of(eb, 2); }
            }
          }
        }
      }
      if constexpr (UN) {
        // first unit of each union entry (la, lb are free now), total units
        // (ascending tile order: a 32-key block that mixes tiles kept by one
        // query tile each keeps both halves of the workgroup busy)
        int U = 0;
        for (int e = 0; e < n; ++e) {
          la[e] = U;
          U += (entry_nv(cols[e]) + KU - 1) / KU;
        }
        nu[1] = U;
      }
    }
    __syncthreads();
    L = *nu;
  }
  // Unit table: entry t holds tile (bits 0..12), unit within the tile
  // (13..20), valid keys of the unit minus one (21..25) and the pair flags
  // (26, 27); padded to whole chunks with units of a kept tile that no query
  // tile keeps (no flags).
  int* const utab = cols + ((4 * g.row_cap + 2 + 3) & ~3);
  int n_units = 0;
  if constexpr (UN) {
    const int* ust = cols + 2 * g.row_cap;
    for (int e = tid; e < L; e += NW * 64) {
      const int x = cols[e];
      const int j = x & ((1 << kTileBits) - 1);
      const int nv = entry_nv(x);
      const int hd = j | ((x >> kFlagShift) << kFlagShift);
      int* dst = utab + ust[e];
      for (int t = 0; KU * t < nv; ++t) dst[t] = hd | (t << kTileBits) | ((min(KU, nv - KU * t) - 1) << kUnitNvShift);
    }
    n_units = cols[4 * g.row_cap + 1];  // nu[1]
    if (tid < (UPC - n_units % UPC) % UPC) utab[n_units + tid] = cols[0] & ((1 << kTileBits) - 1);
  }

  typename C::WS ws;
  if constexpr (C::kF8) {
    if (active) ws.init(qt + head_tm + ((long)i * slots + qrow + col) * D, hi);
  } else if (active) {
    // bf16: the lane's query row straight from the raster input (a padded
    // slot re-reads the tile's last token; its output is never stored)
    const TileInfo tq = tinfo(g, b, i);
    ws.init(qr + (bh * (long)g.N + token_of(g, b, tq, min(qrow + col, tq.nvalid - 1))) * D, hi);
  }
  float c2 = (float)(g.scale * 1.4426950408889634);  // scale * log2(e)
  float oscale = 1.f;
  if constexpr (C::kF8) {
    // scores carry 2^(e_q + e_k), values 2^e_v (clamped like the layout's
    // exponents, so an unwritten workspace still gives finite factors)
    const int eq = min(max(f8_exp[bh * 3 + 0], -32), 32);
    const int ek = min(max(f8_exp[bh * 3 + 1], -32), 32);
    const int ev = min(max(f8_exp[bh * 3 + 2], -32), 32);
    c2 = __builtin_amdgcn_ldexpf(c2, -(eq + ek));
    oscale = __builtin_amdgcn_ldexpf(1.f, -ev);
  }
  Loader ldr;
  if constexpr (UN)
    ldr.init_units(wave, lane, slots);
  else
    ldr.init(wave, lane, slots);
  __syncthreads();  // cols (and the unit table) visible

  // total chunks of the row (each wave sums the list on its own)
  int total = 0;
  if constexpr (UN) {
    total = (n_units + UPC - 1) / UPC;
  } else {
    for (int e = lane; e < L; e += 64) total += (entry_nv(cols[e]) + kKC - 1) / kKC;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) total += __shfl_xor(total, m);
  }
  total = __builtin_amdgcn_readfirstlane(total);

  const T* kt_head = kt + head_tm;
  const T* vt_head = vt + head_tm;
  // The ring holds STAGES chunks in two halves of CPB = STAGES/2 chunks.  The
  // prologue loads the first half; each iteration waits for the half it is
  // about to multiply (everything issued so far), refills the other half
  // (freed by the previous iteration) and multiplies CPB chunks: one barrier
  // per CPB chunks, CPB chunks always in flight.
  constexpr int CPB = STAGES / 2;
  static_assert(STAGES >= 2 && STAGES % 2 == 0, "stages come in pairs");
  if constexpr (UN) {
    const int wsub = __builtin_amdgcn_readfirstlane(sub);
    auto issue_chunk = [&](int st, int nc) {
      UnitBases ub;
      unit_bases<D, KU>(utab[UPC * nc + 0], slots, ub.k0, ub.v0);
      unit_bases<D, KU>(utab[UPC * nc + 1], slots, ub.k1, ub.v1);
      if constexpr (UPC == 4) {
        unit_bases<D, KU>(utab[UPC * nc + 2], slots, ub.k2, ub.v2);
        unit_bases<D, KU>(utab[UPC * nc + 3], slots, ub.k3, ub.v3);
      } else {
        ub.k2 = ub.k3 = ub.k0;  // never picked: units 0 and 1 only
        ub.v2 = ub.v3 = ub.v0;
      }
      ldr.issue_units(lds + st * Stage::STAGE, kt_head, vt_head, ub);
    };
#pragma unroll
    for (int s = 0; s < CPB; ++s)
      if (s < total) issue_chunk(s, s);
    for (int c = 0; c < total; c += CPB) {
      wait_loads_and_barrier();
#pragma unroll
      for (int u = 0; u < CPB; ++u) {
        const int nc = c + CPB + u;
        if (nc < total) issue_chunk(nc % STAGES, nc);
      }
#pragma unroll
      for (int u = 0; u < CPB; ++u) {
        if (c + u < total) {
          // valid keys of each unit for this wave's query tile
          int n[UPC];
          int any = 0;
#pragma unroll
          for (int t = 0; t < UPC; ++t) {
            const int x = __builtin_amdgcn_readfirstlane(utab[UPC * (c + u) + t]);
            n[t] = ((x >> (kFlagShift + wsub)) & 1) ? ((x >> kUnitNvShift) & 31) + 1 : 0;
            any += n[t];
          }
          const T* lk = lds + ((c + u) % STAGES) * Stage::STAGE;
          if (active && any > 0) {
            if constexpr (C::kF8)
              ws.chunk_units(lk, lk + Stage::KE, n[0], n[UPC - 1], c2, col, hi);
            else
              ws.chunk_units(lk, lk + Stage::KE, n, c2, col, hi);
          }
        }
      }
    }
  } else {
    // one chunk sequence: the kept list (or the pair's union) chunk by
    // chunk, or the interleaved pair schedule (same chunks, other order)
    auto stream = [&](auto ld_it, const int* lst, int nl) {
      auto cur = ld_it;
#pragma unroll
      for (int s = 0; s < CPB; ++s) {
        if (s < total) {
          ldr.issue(lds + s * Stage::STAGE, kt_head + ((long)ld_it.j * slots + ld_it.off) * D,
                    vt_head + (long)ld_it.j * D * slots + ld_it.off, ld_it.keys() <= 32);
          ld_it.next(lst, nl);
        }
      }
      for (int c = 0; c < total; c += CPB) {
        wait_loads_and_barrier();
#pragma unroll
        for (int u = 0; u < CPB; ++u) {
          const int nc = c + CPB + u;
          if (nc < total) {
            ldr.issue(lds + (nc % STAGES) * Stage::STAGE,
                      kt_head + ((long)ld_it.j * slots + ld_it.off) * D,
                      vt_head + (long)ld_it.j * D * slots + ld_it.off, ld_it.keys() <= 32);
            ld_it.next(lst, nl);
          }
        }
#pragma unroll
        for (int u = 0; u < CPB; ++u) {
          if (c + u < total) {
            const T* lk = lds + ((c + u) % STAGES) * Stage::STAGE;
            if (active && (TPW == 1 || ((cur.fl >> sub) & 1))) {
              if constexpr (C::kF8)
                ws.chunk(lk, lk + Stage::KE, cur.keys(), c2, col, hi);
              else  // one-tile workgroups read the next block's K fragments during PV
                ws.template chunk<TPW == 1>(lk, lk + Stage::KE, cur.keys(), c2, col, hi);
            }
            cur.next(lst, nl);
          }
        }
      }
    };
    bool ilv = false;
    if constexpr (TPW == 2) ilv = interleaved_pairs(g);
    if (ilv) {
      const int* ck = cols + ((4 * g.row_cap + 2 + 3) & ~3);
      ListIter it;
      it.start(ck, total);
      stream(it, ck, total);
    } else {
      ChunkIter it;
      it.start(cols, L);
      stream(it, cols, L);
    }
  }

  if (!active) return;
  const TileInfo ti = tinfo(g, b, i);
  const int qs = qrow + col;  // slot of this lane's query
  const bool valid = qs < ti.nvalid;
  uint16_t* const orow = o + (bh * (long)g.N + (valid ? token_of(g, b, ti, qs) : 0)) * D;
  if constexpr (C::kF8)
    ws.store(orow, hi, valid, oscale);
  else
    ws.store(orow, hi, valid);
}

// Explicit instantiations of every kernel the launchers can pick.  (With
// several implicit instantiations sharing a wave count, taking a kernel's
// host-side address for hipFuncSetAttribute has left some host stubs
// undefined in the shared library.)
#define VSA_ATTEND_INST(C, NW, ST) VSA_ATTEND_INST_U(C, NW, ST, 1, false)
#define VSA_ATTEND_INST_T(C, NW, ST, TPW) VSA_ATTEND_INST_U(C, NW, ST, TPW, false)
#define VSA_ATTEND_INST_U(C, NW, ST, TPW, UN)                                                  \
  template __global__ void attend_kernel<C, NW, ST, TPW, UN>(Geo, int, const typename C::T*,  \
                                                    const typename C::T*, const typename C::T*, \
                                                    const int*, const int*, const int*,        \
                                                    const int*, uint16_t*, int, int, const uint16_t*);
#define VSA_ATTEND_INST_C(C)                                                               \
  VSA_ATTEND_INST(C, 1, 2) VSA_ATTEND_INST(C, 2, 2) VSA_ATTEND_INST(C, 3, 2)    \
  VSA_ATTEND_INST(C, 4, 2) VSA_ATTEND_INST(C, 5, 2) VSA_ATTEND_INST(C, 6, 2)    \
  VSA_ATTEND_INST(C, 7, 2) VSA_ATTEND_INST(C, 8, 2) VSA_ATTEND_INST(C, 7, 4) VSA_ATTEND_INST(C, 8, 4) VSA_ATTEND_INST(C, 9, 4)    \
  VSA_ATTEND_INST(C, 10, 4) VSA_ATTEND_INST(C, 11, 4) VSA_ATTEND_INST(C, 12, 4)        \
  VSA_ATTEND_INST_T(C, 8, 4, 2) VSA_ATTEND_INST_T(C, 10, 4, 2) VSA_ATTEND_INST_T(C, 12, 4, 2)
#define VSA_ATTEND_INST_UN(C) \
  VSA_ATTEND_INST_U(C, 8, 4, 2, true) VSA_ATTEND_INST_U(C, 10, 4, 2, true) VSA_ATTEND_INST_U(C, 12, 4, 2, true)
VSA_ATTEND_INST_C(Bf16Core<128>)
VSA_ATTEND_INST_C(Bf16Core<64>)
VSA_ATTEND_INST_C(F8Core<128>)
VSA_ATTEND_INST_C(F8Core<64>)
VSA_ATTEND_INST_UN(Bf16Core<128>)
VSA_ATTEND_INST_UN(Bf16Core<64>)
VSA_ATTEND_INST_UN(F8Core<128>)
VSA_ATTEND_INST_UN(F8Core<64>)
#undef VSA_ATTEND_INST_UN
#undef VSA_ATTEND_INST_C
#undef VSA_ATTEND_INST_U
#undef VSA_ATTEND_INST_T
#undef VSA_ATTEND_INST

// Dynamic LDS of a launch: the K/V ring, then the kept list (TPW = 1) or the
// union (up to twice a row), both tiles' lists and the union's length; in
// unit mode also the total units and the unit table (the union's entries
// times the units of a full tile, padded to whole chunks); for interleaved
// pairs the schedule (the union's entries times the chunks of a full tile).
template <class C, int STAGES, int TPW, bool UN = false>
size_t attend_shmem(const Geo& g, int blocking) {
  size_t list_ints = TPW == 1 ? (size_t)g.row_cap : 4 * (size_t)g.row_cap + 1;
  if (TPW == 2 && !UN && interleaved_pairs(g)) {  // + the interleaved schedule: the union's chunks
    const size_t entries = std::min<size_t>(2 * (size_t)g.row_cap, (size_t)g.blk[blocking].n_tiles);
    list_ints = ((4 * (size_t)g.row_cap + 2 + 3) & ~(size_t)3) +
                entries * (size_t)((g.blk[blocking].slots + kKC - 1) / kKC);
  }
  if (UN) {
    const size_t entries = std::min<size_t>(2 * (size_t)g.row_cap, (size_t)g.blk[blocking].n_tiles);
    list_ints = ((4 * (size_t)g.row_cap + 2 + 3) & ~(size_t)3) +
                ((entries * (g.blk[blocking].slots / 16) + 3) & ~(size_t)3);
  }
  return (size_t)STAGES * C::L::STAGE * sizeof(typename C::T) + list_ints * 4;
}

template <class C, int NW, int STAGES, int TPW = 1, bool UN = false>
hipError_t launch_one(const Geo& g, const Ws& w, int blocking, const int* cand, const uint16_t* q,
                      uint16_t* o, hipStream_t s) {
  using T = typename C::T;
  const BlkGeo& b = g.blk[blocking];
  const int slabs = b.slots / 32;
  const int nsb = (slabs + NW / TPW - 1) / (NW / TPW);
  const long BH = (long)g.B * g.H;
  long items, per_xcd;
  if (g.head_sync) {  // every head's items in eight contiguous ranges (see the kernel)
    const long per_head = (b.n_tiles + TPW - 1) / TPW * (long)nsb;
    items = BH * per_head;
    per_xcd = (per_head + kNumXcd - 1) / kNumXcd * BH;
  } else if (cand) {  // the chosen heads' items in eight ranges: room for every head
    const long per_head = (b.n_tiles + TPW - 1) / TPW * (long)nsb;
    items = BH * per_head;
    per_xcd = (items + kNumXcd - 1) / kNumXcd;
  } else {
    items = BH * ((g.max_tiles + TPW - 1) / TPW) * nsb;
    per_xcd = (items + kNumXcd - 1) / kNumXcd;
  }
  const size_t shmem = attend_shmem<C, STAGES, TPW, UN>(g, blocking);
  // more than 64 KB of dynamic LDS must be requested (per device)
  hipError_t e = ensure_dyn_lds(reinterpret_cast<const void*>(&attend_kernel<C, NW, STAGES, TPW, UN>), shmem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attend_kernel<C, NW, STAGES, TPW, UN>), dim3(per_xcd * kNumXcd), dim3(NW * 64), shmem, s,
                     g, blocking, reinterpret_cast<const T*>(w.qt), reinterpret_cast<const T*>(w.kt),
                     reinterpret_cast<const T*>(w.vt), w.row_len, w.col_idx, cand, w.f8_exp, o, nsb,
                     (int)items, q);
  return hipGetLastError();
}

template <class C>
hipError_t launch_d(const Geo& g, const Ws& w, int blocking, const int* cand, const uint16_t* q,
                    uint16_t* o, hipStream_t s) {
  // Waves per workgroup: the tile's 32-row slabs split into as few balanced
  // groups of at most kMaxWaves as possible.  At 3 waves per SIMD a CU holds
  // 12 waves, so groups of 7 to 12 waves run one workgroup per CU; groups of
  // 9 to 12 get a 4-stage ring, smaller groups 2 stages (two workgroups per
  // CU up to 6 waves).  Seven- and eight-wave E4M3 groups also get 4 stages
  // (measured: 3% faster at Wan-14B; for bf16 the deeper ring was no faster
  // there and 3% slower on short rows).
  const int slabs = g.blk[blocking].slots / 32;
  const int groups = (slabs + kMaxWaves - 1) / kMaxWaves;
  const int nw = (slabs + groups - 1) / groups;
  // a pair of adjacent query tiles per workgroup (the plan decides; 4 to 6
  // waves per tile), when the ring and the lists fit in the CU's LDS
  {
    // pairs cut the kept keys into 16-key (E4M3: 32-key) units where the plan
    // chose them, the table fits and the head's element offsets fit in 32 bits
    if (g.blk[blocking].pair && g.blk[blocking].units && nw >= 4 && nw <= 6 &&
        attend_shmem<C, 4, 2, true>(g, blocking) <= 160 * 1024 && g.tok_cap * C::D <= 0x7fffffffL) {
      switch (nw) {
        case 4: return launch_one<C, 8, 4, 2, true>(g, w, blocking, cand, q, o, s);
        case 5: return launch_one<C, 10, 4, 2, true>(g, w, blocking, cand, q, o, s);
        default: return launch_one<C, 12, 4, 2, true>(g, w, blocking, cand, q, o, s);
      }
    }
  }
  if (g.blk[blocking].pair && nw >= 4 && nw <= 6 && attend_shmem<C, 4, 2>(g, blocking) <= 160 * 1024) {
    switch (nw) {
      case 4: return launch_one<C, 8, 4, 2>(g, w, blocking, cand, q, o, s);
      case 5: return launch_one<C, 10, 4, 2>(g, w, blocking, cand, q, o, s);
      default: return launch_one<C, 12, 4, 2>(g, w, blocking, cand, q, o, s);
    }
  }
  switch (nw) {
    case 1: return launch_one<C, 1, 2>(g, w, blocking, cand, q, o, s);
    case 2: return launch_one<C, 2, 2>(g, w, blocking, cand, q, o, s);
    case 3: return launch_one<C, 3, 2>(g, w, blocking, cand, q, o, s);
    case 4: return launch_one<C, 4, 2>(g, w, blocking, cand, q, o, s);
    case 5: return launch_one<C, 5, 2>(g, w, blocking, cand, q, o, s);
    case 6: return launch_one<C, 6, 2>(g, w, blocking, cand, q, o, s);
    case 7: return C::kF8 ? launch_one<C, 7, 4>(g, w, blocking, cand, q, o, s) : launch_one<C, 7, 2>(g, w, blocking, cand, q, o, s);
    case 8: return C::kF8 ? launch_one<C, 8, 4>(g, w, blocking, cand, q, o, s) : launch_one<C, 8, 2>(g, w, blocking, cand, q, o, s);
    case 9: return launch_one<C, 9, 4>(g, w, blocking, cand, q, o, s);
    case 10: return launch_one<C, 10, 4>(g, w, blocking, cand, q, o, s);
    case 11: return launch_one<C, 11, 4>(g, w, blocking, cand, q, o, s);
    default: return launch_one<C, 12, 4>(g, w, blocking, cand, q, o, s);
  }
}

}  // namespace

hipError_t launch_attend(const Geo& g, const Ws& w, const uint16_t* q, uint16_t* o, hipStream_t s,
                         bool make_streams) {
  const int* cand = per_head_blocking(g) ? w.cand : nullptr;
  auto one = [&](int c, hipStream_t st) -> hipError_t {
    if (g.f8)
      return (g.d == 128) ? launch_d<F8Core<128>>(g, w, c, cand, q, o, st)
                          : launch_d<F8Core<64>>(g, w, c, cand, q, o, st);
    return (g.d == 128) ? launch_d<Bf16Core<128>>(g, w, c, cand, q, o, st)
                        : launch_d<Bf16Core<64>>(g, w, c, cand, q, o, st);
  };
  // One launch per blocking (heads grouped by their chosen blocking); a
  // workgroup whose head chose another blocking exits at once.  The launches
  // write disjoint heads, so blockings after the first go to side streams
  // forked from and joined back into the caller's: the workgroups of a
  // small-tile blocking (4 waves) then fill the CUs beside those of a
  // large-tile one instead of waiting for them.
  SideStreams* ss = g.nb > 1 ? side_streams(s, make_streams) : nullptr;
  if (!ss) {
    for (int c = 0; c < g.nb; ++c) {
      const hipError_t e = one(c, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  std::lock_guard<std::mutex> lock(ss->mu);
  hipError_t e = hipEventRecord(ss->fork, s);
  int forked = 0;
  for (; e == hipSuccess && forked < g.nb - 1; ++forked) e = hipStreamWaitEvent(ss->s[forked], ss->fork, 0);
  for (int c = 0; e == hipSuccess && c < g.nb; ++c) e = one(c, c == 0 ? s : ss->s[c - 1]);
  // Join every stream that was forked, also after an error, so that the
  // caller's stream (or its capture) is never left with work outside it.
  for (int i = 0; i < forked; ++i) {
    hipError_t ej = hipEventRecord(ss->join[i], ss->s[i]);
    if (ej == hipSuccess) ej = hipStreamWaitEvent(s, ss->join[i], 0);
    if (e == hipSuccess) e = ej;
  }
  return e;
}

}  // namespace vsa
