// Internal definitions shared by the host API and the HIP kernels of libvsa.
#pragma once

#include <hip/hip_runtime.h>

#include <mutex>
#include <stddef.h>
#include <stdint.h>

#include "../../include/vsa.h"

namespace vsa {

// One blocking of the token grid (tile extents and derived counts).
struct BlkGeo {
  int tile[3];   // tokens per tile along t, h, w
  int nt[3];     // tiles along t, h, w
  int n_tiles;   // nt[0]*nt[1]*nt[2]
  int slots;     // tokens per tile rounded up to a multiple of 32
  int topk;      // resolved K for this blocking (0 = off)
  int pair;      // attention: two adjacent query tiles per workgroup (their kept lists overlap)
  int units;     // attention (bf16 pairs): keys staged in 16-key units, four per 64-key chunk
};

// Everything a kernel needs to know about the problem; passed by value.
struct Geo {
  int B, H, d, N;
  int grid[3];
  int nb;           // number of blockings (1, or the SICS candidates)
  BlkGeo blk[VSA_MAX_CAND];
  int max_tiles;
  long tok_cap;     // max over blockings of n_tiles*slots (tile-major rows per head)
  int row_cap;      // capacity of one kept-tile row
  uint32_t flags;
  int win[3];
  int win_mode;
  double topp;
  double scale;     // softmax scale
  int summ;         // VSA_SUMM_* (dynamic masks)
  int sink;         // leading key tiles kept for every query tile
  int head_sync;    // attention: head-synchronous workgroup order (masks without a window)
  int f8;           // 1 under VSA_COMPUTE_FP8: E4M3 tile-major Q, K, V and attention
  int prof_runs;    // VSA_PROFILE_SELECT: sampled runs of 32 query rows per head
  int prof_segs;    // key segments (ranges of raster lines) of the full pass
  // fine-grained mask
  int fine_M, fine_G;
  long fine_keep;   // kept (group, key) pairs per head (target count)
  long fine_cap;    // kept-key list capacity per head: G*N (N per group)
  // SICS atoms: common refinement of the candidate blockings
  int atom[3];
  int na[3];
  int n_atoms;
};

// Blocking c of g, field by field with selects: indexing the by-value kernel
// argument with a runtime c would place the whole array in scratch memory.
__host__ __device__ __forceinline__ int sel4(int c, int a0, int a1, int a2, int a3) {
  return c == 0 ? a0 : (c == 1 ? a1 : (c == 2 ? a2 : a3));
}
// Whether the blocking is chosen per head (by SICS or by the profiling
// selector; both write the workspace's CAND region).
__host__ __device__ __forceinline__ bool per_head_blocking(const Geo& g) {
  return (g.flags & (VSA_SICS_SELECT | VSA_PROFILE_SELECT)) != 0;
}

// The blocking chosen for head bh (0 without a per-head choice), clamped to a
// valid index, so that a workspace whose selection was never written (a
// cached call on a fresh workspace) still addresses memory in bounds.
// Whether paired query tiles (whole-chunk mode) stream an interleaved chunk
// schedule instead of their ascending union: the chunks both tiles keep,
// then the chunks only one keeps, the two tiles' alternating, so that in
// each step of two chunks both halves of the workgroup have work.  Used for
// Top-K masks, whose neighbouring rows share only about half their tiles.
__host__ __device__ __forceinline__ bool interleaved_pairs(const Geo& g) {
  return (g.flags & (VSA_TOPK | VSA_TOPK_FRAC)) != 0 && (g.flags & VSA_TOPP) == 0;
}

__device__ __forceinline__ int cand_of(const Geo& g, const int* cand, long bh) {
  return cand ? min(max(cand[bh], 0), g.nb - 1) : 0;
}

__host__ __device__ __forceinline__ BlkGeo pick_blk(const Geo& g, int c) {
  BlkGeo b;
#define VSA_PICK(f) b.f = sel4(c, g.blk[0].f, g.blk[1].f, g.blk[2].f, g.blk[3].f)
  VSA_PICK(tile[0]); VSA_PICK(tile[1]); VSA_PICK(tile[2]);
  VSA_PICK(nt[0]); VSA_PICK(nt[1]); VSA_PICK(nt[2]);
  VSA_PICK(n_tiles); VSA_PICK(slots); VSA_PICK(topk);
#undef VSA_PICK
  return b;
}

// Workspace pointers resolved from the plan's layout.
struct Ws {
  uint16_t* qt;
  uint16_t* kt;
  uint16_t* vt;
  float* pooled_q;
  float* pooled_k;
  float* pooled_kmin;
  int* row_len;
  int* col_idx;
  int* cand;
  float* cand_score;
  float* tile_sics;
  float* atoms;
  float* fine_qbar;
  double* fine_tau;
  int* fine_count;
  int* fine_idx;
  uint32_t* fine_mask;  // [B*H][G][ceil(N/32)] kept-pair bits
  unsigned char* scratch;
  int* f8_exp;          // [B*H][3] E4M3 scale exponents of Q, K, V
  uint32_t* f8_amax;    // [B*H][3][kAmaxParts] partial max |x| (bf16 bits)
  float* prof_sse;      // [B*H][prof_runs][nb] squared-error sums of the profiling selector
  float* prof_part;     // full-pass partials: float2 (row sum, reference) [B*H][runs][segs][32],
                        // then fp32 O^T [B*H][runs][segs][32][d]
};

// Runs of sampled query rows (waves) sharing one workgroup of the profiling
// selector's full pass.
constexpr int kProfWaves = 12;

// Slices per (head, tensor) of the max |x| reduction of the FP8 path.
constexpr int kAmaxParts = 128;

// Bytes of the device array that vsa_forward_noalloc uses as its workspace
// (api.cpp): plans needing more are refused by that entry point.
constexpr size_t kNoAllocBytes = VSA_NOALLOC_BYTES;
// XCDs of the part: the hardware deals consecutive workgroups of a launch to
// them in turn, and each has its own L2.
constexpr int kNumXcd = 8;

// Raises a kernel's dynamic-LDS limit to at least `bytes` on the current
// device, once per (device, kernel); thread-safe (api.cpp).
hipError_t ensure_dyn_lds(const void* kernel, size_t bytes);

// Streams beside the caller's, one per blocking after the first, so that the
// attention launches of different blockings (disjoint heads) can share the
// CUs.  One set per device, made on first use; `mu` is held from the fork
// event to the last join so that calls from several host threads do not mix
// their events.  nullptr: none (not made yet and `create` false, the caller's
// stream is being captured before the set exists, or creation failed); the
// launches then run in order on the caller's stream.
struct SideStreams {
  static constexpr int kN = VSA_MAX_CAND - 1;
  hipStream_t s[kN] = {};
  hipEvent_t fork = nullptr;
  hipEvent_t join[kN] = {};
  std::mutex mu;
};
SideStreams* side_streams(hipStream_t caller, bool create);

// Bytes of internal scratch the fine-grained mask needs (fine.hip).
size_t fine_scratch_bytes(const Geo& g);

// Kernel launchers (layout_select.hip / attend.hip / sics.hip / fine.hip);
// return hipError_t.  launch_layout's pool writes the block summaries of
// dynamic masks (mean of Q, and mean / max / max+min of K per g.summ).
hipError_t launch_layout(const Geo& g, const Ws& w, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, bool pool, hipStream_t s);
// FP8 path: partial max |x| of Q, K, V per head (before launch_layout).
hipError_t launch_amax(const Geo& g, const Ws& w, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, hipStream_t s);
hipError_t launch_untile(const Geo& g, const Ws& w, int which, uint16_t* out, hipStream_t s);
hipError_t launch_select(const Geo& g, const Ws& w, hipStream_t s);
// (bf16 attention reads its query rows from the raster q)
hipError_t launch_attend(const Geo& g, const Ws& w, const uint16_t* q, uint16_t* o, hipStream_t s,
                         bool make_streams);
hipError_t launch_sics(const Geo& g, const Ws& w, const uint16_t* q, const uint16_t* k,
                       hipStream_t s);
// Profiling selector: per-head MSE of every candidate on the sampled rows,
// and the chosen blocking (CAND, CAND_SCORE).
hipError_t launch_profile(const Geo& g, const Ws& w, const uint16_t* q, const uint16_t* k,
                          const uint16_t* v, hipStream_t s);
hipError_t launch_fine_select(const Geo& g, const Ws& w, const uint16_t* q, const uint16_t* k,
                              hipStream_t s);
hipError_t launch_fine_attend(const Geo& g, const Ws& w, const uint16_t* q, const uint16_t* k,
                              const uint16_t* v, uint16_t* o, hipStream_t s);

}  // namespace vsa
