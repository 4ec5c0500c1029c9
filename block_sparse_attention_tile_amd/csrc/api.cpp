// Host side of libvsa: plan validation, tile geometry, workspace layout and
// the extern "C" entry points declared in include/vsa.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <numeric>
#include <string>
#include <utility>
#include <vector>

#include "vsa_internal.h"

using vsa::BlkGeo;
using vsa::Geo;
using vsa::Ws;

struct vsa_plan_s {
  vsa_problem prob;
  vsa_mask_policy pol;
  Geo geo;
  bool dynamic;        // mask depends on the input (scores or SICS)
  int64_t static_pairs;
  double static_flops;
  size_t off[VSA_WS_NREGIONS];
  size_t size[VSA_WS_NREGIONS];
  size_t ws_total;
};

namespace vsa {

hipError_t ensure_dyn_lds(const void* kernel, size_t bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, size_t> raised;
  std::lock_guard<std::mutex> lock(mu);
  size_t& have = raised[{dev, kernel}];
  if (have >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) have = bytes;
  return e;
}

SideStreams* side_streams(hipStream_t caller, bool create) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  // the set belongs to the current device: a caller's stream on another
  // device gets the launches in order on that stream
  hipDevice_t sdev = -1;
  if (hipStreamGetDevice(caller, &sdev) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (sdev != dev) return nullptr;
  static std::mutex mu;
  static SideStreams* made[64] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (made[dev] || !create) return made[dev];
  // Streams are made outside stream capture only: a caller that captures
  // before any uncaptured call on this device gets one stream.
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(caller, &cs) != hipSuccess) {
    (void)hipGetLastError();  // leave no error behind for the launches' checks
    return nullptr;
  }
  if (cs != hipStreamCaptureStatusNone) return nullptr;
  SideStreams* ss = new (std::nothrow) SideStreams();
  if (!ss) return nullptr;
  bool ok = hipEventCreateWithFlags(&ss->fork, hipEventDisableTiming) == hipSuccess;
  for (int i = 0; ok && i < SideStreams::kN; ++i)
    ok = hipStreamCreateWithFlags(&ss->s[i], hipStreamNonBlocking) == hipSuccess &&
         hipEventCreateWithFlags(&ss->join[i], hipEventDisableTiming) == hipSuccess;
  if (!ok) {  // undo a partial set-up; the next call tries again
    for (int i = 0; i < SideStreams::kN; ++i) {
      if (ss->join[i]) (void)hipEventDestroy(ss->join[i]);
      if (ss->s[i]) (void)hipStreamDestroy(ss->s[i]);
    }
    if (ss->fork) (void)hipEventDestroy(ss->fork);
    delete ss;
    (void)hipGetLastError();
    return nullptr;
  }
  made[dev] = ss;
  return ss;
}

}  // namespace vsa

// Device scratch of vsa_forward_noalloc.  One copy of this array exists on
// every device the library's code object is loaded on, at that device's own
// address, and stays until the process ends.  On the host its name is only a
// stand-in: host code passes the address that hipGetSymbolAddress returns
// for the current device (scratch_on_device below), never the name itself.
static __device__ __align__(256) unsigned char scratch[vsa::kNoAllocBytes];

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return VSA_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(VSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

long ceil_div(long a, long b) { return (a + b - 1) / b; }

// K = ceil(frac * n) with slack so an exact product is not bumped up by the
// fp64 representation of frac (0.2 * 315 -> 63).
long frac_count(double frac, long n) {
  long k = (long)std::ceil(frac * (double)n - 1e-9);
  return std::max(1L, k);
}

// Tiles kept by the window along one axis for tile coordinate c.
void axis_range(int c, int r, int n, int mode, int* lo, int* hi) {
  if (mode == VSA_WIN_CLAMP && n >= 2 * r + 1) {
    *lo = std::min(std::max(c - r, 0), n - (2 * r + 1));
    *hi = *lo + 2 * r;
  } else {
    *lo = std::max(c - r, 0);
    *hi = std::min(c + r, n - 1);
  }
}

// Kept key tiles of query tile i under the static part of the policy
// (window box, or every tile under VSA_DENSE / no window, plus the sink),
// marked in `keep` (n_tiles flags).
void static_row(const Geo& g, const BlkGeo& b, int i, std::vector<char>& keep) {
  std::fill(keep.begin(), keep.end(), 0);
  int lo[3] = {0, 0, 0}, hi[3] = {b.nt[0] - 1, b.nt[1] - 1, b.nt[2] - 1};
  if (!(g.flags & VSA_DENSE) && (g.flags & VSA_WINDOW)) {
    const int c3[3] = {i / (b.nt[1] * b.nt[2]), (i / b.nt[2]) % b.nt[1], i % b.nt[2]};
    for (int a = 0; a < 3; ++a) axis_range(c3[a], (g.win[a] - 1) / 2, b.nt[a], g.win_mode, &lo[a], &hi[a]);
  }
  if ((g.flags & (VSA_DENSE | VSA_WINDOW)) != 0)
    for (int t = lo[0]; t <= hi[0]; ++t)
      for (int h = lo[1]; h <= hi[1]; ++h)
        for (int w = lo[2]; w <= hi[2]; ++w) keep[(t * b.nt[1] + h) * b.nt[2] + w] = 1;
  for (int j = 0; j < std::min(g.sink, b.n_tiles); ++j) keep[j] = 1;
}

// Whether the attention launch pairs adjacent query tiles (2p, 2p+1) of a
// blocking in one workgroup that streams the union of their kept lists.
// Only groups of 4 to 6 waves (tiles of 97..192 slots) are paired, giving
// 8- to 12-wave workgroups with a 4-stage ring.  Top-P rows keep most tiles
// and neighbours' rows nearly coincide.  Top-K rows of neighbours share only
// about half their tiles: tiles of 6 slabs are paired with the interleaved
// schedule (interleaved_pairs), which stages each shared tile once and keeps
// both halves busy on the rest (Wan-14B shape, 3x8x8 tiles: 29.5 -> 27.4 ms);
// tiles of 4 slabs are not (7x4x4 tiles: 37.2 -> 41.2 ms, though the
// traffic from beyond L2 fell by 15%: two independent four-wave workgroups
// per CU hide load latency better than one eight-wave workgroup).  Static
// masks are paired when the pairs' lists overlap enough that at least 70% of
// the staged chunks serve both tiles' waves.
int pair_tiles(const Geo& g, const BlkGeo& b) {
  const int slabs = b.slots / 32;
  if (slabs < 4 || slabs > 6) return 0;
  if (g.flags & VSA_TOPP) return 1;
  if (g.flags & (VSA_TOPK | VSA_TOPK_FRAC)) return slabs == 6 ? 1 : 0;
  std::vector<char> ka(b.n_tiles), kb(b.n_tiles);
  double used = 0.0, staged = 0.0;
  for (int i = 0; i < b.n_tiles; i += 2) {
    static_row(g, b, i, ka);
    if (i + 1 < b.n_tiles) static_row(g, b, i + 1, kb); else std::fill(kb.begin(), kb.end(), 0);
    long na = 0, nb = 0, nu = 0;
    for (int j = 0; j < b.n_tiles; ++j) {
      na += ka[j];
      nb += kb[j];
      nu += (ka[j] | kb[j]);
    }
    used += (double)(na + nb);
    staged += 2.0 * (double)nu;
  }
  return staged > 0.0 && used >= 0.7 * staged ? 1 : 0;
}

// Valid tokens of tile (it, ih, iw) of a blocking.
long tile_valid(const Geo& g, const BlkGeo& b, int it, int ih, int iw) {
  long et = std::min(b.tile[0], g.grid[0] - it * b.tile[0]);
  long eh = std::min(b.tile[1], g.grid[1] - ih * b.tile[1]);
  long ew = std::min(b.tile[2], g.grid[2] - iw * b.tile[2]);
  return et * eh * ew;
}

long tile_valid_id(const Geo& g, const BlkGeo& b, int i) {
  int it = i / (b.nt[1] * b.nt[2]);
  int ih = (i / b.nt[2]) % b.nt[1];
  int iw = i % b.nt[2];
  return tile_valid(g, b, it, ih, iw);
}

// Whether the attention of a paired blocking stages the kept keys in units
// (16 keys for bf16, 32 for E4M3; 64 / unit size per 64-key chunk, across
// tile boundaries) instead of per-tile 64-key chunks with a 32-key tail
// chunk: when units cut the chunk iterations over all tiles by at least 5%
// (tile sizes that are not multiples of 64, or ragged edge tiles).
// (One-tile workgroups stay with whole chunks: bf16 units measured no faster
// there, on 112-, 208- and 480-key tiles.)
int unit_tiles(const Geo& g, const BlkGeo& b) {
  if (!b.pair || vsa::interleaved_pairs(g)) return 0;  // the interleaved schedule works on whole chunks
  const long ku = g.f8 ? 32 : 16;
  long units = 0, chunks = 0;
  for (int i = 0; i < b.n_tiles; ++i) {
    const long nv = tile_valid_id(g, b, i);
    units += (nv + ku - 1) / ku;
    chunks += (nv + 63) / 64;
  }
  return 20 * units < 19 * (64 / ku) * chunks ? 1 : 0;
}

int gcd(int a, int b) { return b == 0 ? a : gcd(b, a % b); }

Ws resolve(const vsa_plan_t* p, void* ws) {
  auto at = [&](int r) -> void* {
    return p->size[r] ? (void*)((char*)ws + p->off[r]) : nullptr;
  };
  Ws w;
  w.qt = (uint16_t*)at(VSA_WS_QT);
  w.kt = (uint16_t*)at(VSA_WS_KT);
  w.vt = (uint16_t*)at(VSA_WS_VT);
  w.pooled_q = (float*)at(VSA_WS_POOLED_Q);
  w.pooled_k = (float*)at(VSA_WS_POOLED_K);
  w.pooled_kmin = (float*)at(VSA_WS_POOLED_KMIN);
  w.row_len = (int*)at(VSA_WS_ROW_LEN);
  w.col_idx = (int*)at(VSA_WS_COL_IDX);
  w.cand = (int*)at(VSA_WS_CAND);
  w.cand_score = (float*)at(VSA_WS_CAND_SCORE);
  w.tile_sics = (float*)at(VSA_WS_TILE_SICS);
  w.atoms = (float*)at(VSA_WS_ATOMS);
  w.fine_qbar = (float*)at(VSA_WS_FINE_QBAR);
  w.fine_tau = (double*)at(VSA_WS_FINE_TAU);
  w.fine_count = (int*)at(VSA_WS_FINE_COUNT);
  w.fine_idx = (int*)at(VSA_WS_FINE_IDX);
  w.fine_mask = (uint32_t*)at(VSA_WS_FINE_MASK);
  w.scratch = (unsigned char*)at(VSA_WS_SCRATCH);
  w.f8_exp = (int*)at(VSA_WS_F8_EXP);
  w.f8_amax = (uint32_t*)at(VSA_WS_F8_AMAX);
  w.prof_sse = (float*)at(VSA_WS_PROF_SSE);
  w.prof_part = (float*)at(VSA_WS_PROF_PART);
  return w;
}

int check_exec(const vsa_plan_t* p, const void* ws, size_t ws_bytes) {
  if (!p) return fail(VSA_ERR_INVALID_ARG, "plan is NULL");
  if (!ws) return fail(VSA_ERR_INVALID_ARG, "workspace is NULL");
  if (((uintptr_t)ws & 255) != 0)
    return fail(VSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (ws_bytes < p->ws_total)
    return fail(VSA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, plan needs %zu",
                ws_bytes, p->ws_total);
  return VSA_OK;
}

int check_tensor(const void* t, const char* name) {
  if (!t) return fail(VSA_ERR_INVALID_ARG, "%s is NULL", name);
  if (((uintptr_t)t & 15) != 0) return fail(VSA_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
  return VSA_OK;
}

int build_plan(const vsa_problem* pr, const vsa_mask_policy* po, vsa_plan_s* p) {
  memset(p, 0, sizeof *p);
  p->prob = *pr;
  p->pol = *po;
  Geo& g = p->geo;
  if (pr->B <= 0 || pr->H <= 0 || pr->d <= 0)
    return fail(VSA_ERR_INVALID_ARG, "B, H, d must be positive (got %d, %d, %d)", pr->B, pr->H, pr->d);
  for (int a = 0; a < 3; ++a)
    if (pr->grid[a] <= 0) return fail(VSA_ERR_INVALID_ARG, "grid[%d] must be positive", a);
  if (pr->dtype != VSA_BF16) return fail(VSA_ERR_UNSUPPORTED, "only VSA_BF16 is supported");
  if (pr->d != 64 && pr->d != 128) return fail(VSA_ERR_UNSUPPORTED, "d must be 64 or 128 (got %d)", pr->d);
  long N = (long)pr->grid[0] * pr->grid[1] * pr->grid[2];
  if (N > (1L << 30)) return fail(VSA_ERR_UNSUPPORTED, "too many tokens");
  // several launches put B*H in the second grid dimension
  const long BH = (long)pr->B * pr->H;
  if (BH > 65535) return fail(VSA_ERR_UNSUPPORTED, "B*H = %ld exceeds 65535", BH);
  uint32_t f = po->flags;
  const uint32_t known = VSA_DENSE | VSA_WINDOW | VSA_TOPK | VSA_TOPK_FRAC | VSA_TOPP |
                         VSA_SICS_SELECT | VSA_FINE | VSA_PROFILE_SELECT;
  if (f & ~known) return fail(VSA_ERR_INVALID_ARG, "unknown policy flags 0x%x", f & ~known);
  if (f == 0) return fail(VSA_ERR_INVALID_ARG, "policy selects nothing (flags = 0)");
  if ((f & VSA_FINE) && (f != VSA_FINE))
    return fail(VSA_ERR_INVALID_ARG, "VSA_FINE cannot be combined with other flags");
  if ((f & VSA_TOPK) && (f & VSA_TOPK_FRAC))
    return fail(VSA_ERR_INVALID_ARG, "VSA_TOPK and VSA_TOPK_FRAC are exclusive");
  if ((f & VSA_SICS_SELECT) && !(f & (VSA_DENSE | VSA_WINDOW | VSA_TOPK | VSA_TOPK_FRAC | VSA_TOPP)))
    return fail(VSA_ERR_INVALID_ARG, "VSA_SICS_SELECT needs a tile mask to go with it");
  if ((f & VSA_SICS_SELECT) && (f & VSA_PROFILE_SELECT))
    return fail(VSA_ERR_INVALID_ARG, "VSA_SICS_SELECT and VSA_PROFILE_SELECT are exclusive");
  if ((f & VSA_PROFILE_SELECT) && !(f & (VSA_DENSE | VSA_WINDOW)))
    return fail(VSA_ERR_INVALID_ARG, "VSA_PROFILE_SELECT needs a static tile mask (VSA_DENSE or VSA_WINDOW)");
  if ((f & VSA_PROFILE_SELECT) && (f & (VSA_TOPK | VSA_TOPK_FRAC | VSA_TOPP)))
    return fail(VSA_ERR_UNSUPPORTED, "VSA_PROFILE_SELECT is built for static masks only (no Top-K / Top-P)");
  if (!(po->profile_frac >= 0.0 && po->profile_frac <= 1.0))
    return fail(VSA_ERR_INVALID_ARG, "profile_frac must be in (0, 1] (0 selects 0.01)");
  if (!(f & VSA_FINE) && !(f & (VSA_DENSE | VSA_WINDOW | VSA_TOPK | VSA_TOPK_FRAC | VSA_TOPP)))
    return fail(VSA_ERR_INVALID_ARG, "policy keeps no tiles");
  if (po->scale < 0 || !std::isfinite(po->scale))
    return fail(VSA_ERR_INVALID_ARG, "scale must be finite and >= 0");

  g.B = pr->B; g.H = pr->H; g.d = pr->d; g.N = (int)N;
  for (int a = 0; a < 3; ++a) g.grid[a] = pr->grid[a];
  g.flags = f;
  g.scale = po->scale > 0 ? po->scale : 1.0 / std::sqrt((double)pr->d);
  g.win_mode = po->win_mode;
  g.topp = po->topp;
  if (po->summarizer < VSA_SUMM_MEAN || po->summarizer > VSA_SUMM_MINMAX)
    return fail(VSA_ERR_INVALID_ARG, "summarizer must be VSA_SUMM_MEAN, _MAX or _MINMAX (got %d)",
                po->summarizer);
  if (po->sink < 0) return fail(VSA_ERR_INVALID_ARG, "sink must be >= 0 (got %d)", po->sink);
  if ((f & VSA_FINE) && po->sink > 0)
    return fail(VSA_ERR_INVALID_ARG, "the tile sink does not apply to VSA_FINE");
  g.summ = po->summarizer;
  g.sink = po->sink;
  // Kept tiles chosen by score alone (no window) are scattered over the
  // head: an XCD's L2 finds little to reuse between neighbouring query
  // tiles, and what matters is that the Infinity Cache holds the K and V of
  // the heads in flight.  Their attention then walks the heads in order
  // across the whole GPU.  A window keeps each XCD on its own run of
  // neighbouring query tiles instead.
  g.head_sync = !(f & VSA_WINDOW) && (f & (VSA_TOPK | VSA_TOPK_FRAC | VSA_TOPP)) ? 1 : 0;
  if (po->compute != VSA_COMPUTE_BF16 && po->compute != VSA_COMPUTE_FP8)
    return fail(VSA_ERR_INVALID_ARG, "compute must be VSA_COMPUTE_BF16 or VSA_COMPUTE_FP8 (got %d)",
                po->compute);
  if (po->compute == VSA_COMPUTE_FP8 && (f & VSA_FINE))
    return fail(VSA_ERR_UNSUPPORTED, "VSA_COMPUTE_FP8 is built for tile masks only, not VSA_FINE");
  g.f8 = po->compute == VSA_COMPUTE_FP8 ? 1 : 0;

  if (f & VSA_FINE) {
    int M = po->fine_group;
    if (M < 16 || M % 16 != 0 || M > 256)
      return fail(VSA_ERR_INVALID_ARG, "fine_group must be a multiple of 16 in [16, 256] (got %d)", M);
    if (!(po->fine_keep > 0.0 && po->fine_keep <= 1.0))
      return fail(VSA_ERR_INVALID_ARG, "fine_keep must be in (0, 1]");
    g.fine_M = M;
    g.fine_G = (int)ceil_div(N, M);
    if (BH * g.fine_G > 0x7fffffffL)  // the fine-mask passes index (head, group) pairs in 32 bits
      return fail(VSA_ERR_UNSUPPORTED, "B*H*groups = %ld exceeds 2^31 - 1", BH * g.fine_G);
    if ((long)g.fine_G * N > 0x7fffffffL)  // candidate scores keep their (group, key) position in 32 bits
      return fail(VSA_ERR_UNSUPPORTED, "groups*N = %ld exceeds 2^31 - 1", (long)g.fine_G * N);
    double total = (double)g.fine_G * (double)N;
    g.fine_keep = frac_count(po->fine_keep, (long)total);
    g.fine_cap = (long)g.fine_G * N;  // N keys per group: ties at the threshold may keep every pair
    g.nb = 0;
    g.max_tiles = 0;
    g.tok_cap = 0;
    p->dynamic = true;
    p->static_pairs = -1;
  } else {
    if (f & (VSA_SICS_SELECT | VSA_PROFILE_SELECT)) {
      if (pr->n_cand < 1 || pr->n_cand > VSA_MAX_CAND)
        return fail(VSA_ERR_INVALID_ARG, "n_cand must be in [1, %d]", VSA_MAX_CAND);
      g.nb = pr->n_cand;
    } else {
      g.nb = 1;
    }
    for (int c = 0; c < g.nb; ++c) {
      const int32_t* t = (f & (VSA_SICS_SELECT | VSA_PROFILE_SELECT)) ? pr->cand_tile[c] : pr->tile;
      BlkGeo& b = g.blk[c];
      long bs = 1;
      for (int a = 0; a < 3; ++a) {
        if (t[a] <= 0) return fail(VSA_ERR_INVALID_ARG, "tile extents must be positive");
        if (t[a] > pr->grid[a])
          return fail(VSA_ERR_UNSUPPORTED, "tile extent %d exceeds grid extent %d on axis %d",
                      t[a], pr->grid[a], a);
        b.tile[a] = t[a];
        b.nt[a] = (int)ceil_div(pr->grid[a], t[a]);
        bs *= t[a];
      }
      if (bs > 4096) return fail(VSA_ERR_UNSUPPORTED, "tile of %ld tokens exceeds 4096", bs);
      b.n_tiles = b.nt[0] * b.nt[1] * b.nt[2];
      if (b.n_tiles > 4096) return fail(VSA_ERR_UNSUPPORTED, "%d tiles exceed 4096", b.n_tiles);
      b.slots = (int)ceil_div(bs, 32) * 32;
      if (f & VSA_TOPK) {
        if (po->topk <= 0) return fail(VSA_ERR_INVALID_ARG, "topk must be positive");
        b.topk = std::min(po->topk, b.n_tiles);
      } else if (f & VSA_TOPK_FRAC) {
        if (!(po->topk_frac > 0.0 && po->topk_frac <= 1.0))
          return fail(VSA_ERR_INVALID_ARG, "topk_frac must be in (0, 1]");
        b.topk = (int)std::min<long>(frac_count(po->topk_frac, b.n_tiles), b.n_tiles);
      }
      g.max_tiles = std::max(g.max_tiles, b.n_tiles);
      g.tok_cap = std::max(g.tok_cap, (long)b.n_tiles * b.slots);
    }
    // the attention launch has one workgroup per (head, tile, group of at
    // most 12 slabs of 32 query rows): at most 11 groups per tile, each
    // head's items padded to a multiple of the 8 XCDs in the head-synchronous
    // order
    if (BH * ((long)g.max_tiles * 11 + 7) > 0x7fffffffL)
      return fail(VSA_ERR_UNSUPPORTED, "B*H*tiles = %ld is too large for one launch", BH * g.max_tiles);
    if (f & VSA_TOPP) {
      if (!(po->topp > 0.0 && po->topp <= 1.0))
        return fail(VSA_ERR_INVALID_ARG, "topp must be in (0, 1]");
    }
    long win_cells = 0;
    if (f & VSA_WINDOW) {
      if (po->win_mode != VSA_WIN_TRUNCATE && po->win_mode != VSA_WIN_CLAMP)
        return fail(VSA_ERR_INVALID_ARG, "win_mode must be 0 (truncate) or 1 (clamp)");
      win_cells = 1;
      for (int a = 0; a < 3; ++a) {
        if (po->win[a] < 1 || po->win[a] % 2 == 0)
          return fail(VSA_ERR_INVALID_ARG, "window extents must be odd and >= 1 (axis %d: %d)", a, po->win[a]);
        g.win[a] = po->win[a];
        win_cells *= po->win[a];
      }
    }
    for (int c = 0; c < g.nb; ++c) {
      g.blk[c].pair = pair_tiles(g, g.blk[c]);
      g.blk[c].units = unit_tiles(g, g.blk[c]);
    }
    p->dynamic = (f & (VSA_TOPK | VSA_TOPK_FRAC | VSA_TOPP | VSA_SICS_SELECT | VSA_PROFILE_SELECT)) != 0;
    if ((f & (VSA_DENSE | VSA_TOPP)) || (f & (VSA_SICS_SELECT | VSA_PROFILE_SELECT))) {
      g.row_cap = g.max_tiles;
    } else {
      long cap = win_cells + g.sink;
      int maxk = 0;
      for (int c = 0; c < g.nb; ++c) maxk = std::max(maxk, g.blk[c].topk);
      cap += maxk;
      g.row_cap = (int)std::min<long>(cap, g.max_tiles);
    }
    // Profiling sample: runs of 32 consecutive query rows per head.
    if (f & VSA_PROFILE_SELECT) {
      const double frac = po->profile_frac > 0.0 ? po->profile_frac : 0.01;
      if (N < 32) {
        g.prof_runs = 1;
      } else {
        long r = (long)std::floor(frac * (double)N / 32.0 + 0.5);
        g.prof_runs = (int)std::min(std::max(r, 1L), N / 32);
      }
      // split the keys into ranges of lines until the full pass has about
      // 1024 workgroups (a few rounds over the CUs)
      const long groups = (long)g.B * g.H * ((g.prof_runs + vsa::kProfWaves - 1) / vsa::kProfWaves);
      const long lines = (long)pr->grid[0] * pr->grid[1];
      g.prof_segs = (int)std::max(1L, std::min({(1024 + groups - 1) / groups, lines, 16L}));
    }
    // SICS atoms: per-axis gcd of the candidate tile extents.
    if (f & VSA_SICS_SELECT) {
      g.n_atoms = 1;
      for (int a = 0; a < 3; ++a) {
        int v = g.blk[0].tile[a];
        for (int c = 1; c < g.nb; ++c) v = gcd(v, g.blk[c].tile[a]);
        g.atom[a] = v;
        g.na[a] = (int)ceil_div(pr->grid[a], v);
        g.n_atoms *= g.na[a];
      }
    }
    // Static statistics (input-independent masks).
    if (!p->dynamic) {
      const BlkGeo& b = g.blk[0];
      std::vector<long> nv(b.n_tiles);
      for (int i = 0; i < b.n_tiles; ++i) nv[i] = tile_valid_id(g, b, i);
      int64_t pairs = 0;
      double fl = 0.0;
      for (int i = 0; i < b.n_tiles; ++i) {
        int it = i / (b.nt[1] * b.nt[2]), ih = (i / b.nt[2]) % b.nt[1], iw = i % b.nt[2];
        int lo[3] = {0, 0, 0}, hi[3] = {b.nt[0] - 1, b.nt[1] - 1, b.nt[2] - 1};
        if (!(f & VSA_DENSE)) {
          int c3[3] = {it, ih, iw};
          for (int a = 0; a < 3; ++a)
            axis_range(c3[a], (g.win[a] - 1) / 2, b.nt[a], g.win_mode, &lo[a], &hi[a]);
        }
        auto in_window = [&](int j) {
          const int t = j / (b.nt[1] * b.nt[2]), h = (j / b.nt[2]) % b.nt[1], w = j % b.nt[2];
          return t >= lo[0] && t <= hi[0] && h >= lo[1] && h <= hi[1] && w >= lo[2] && w <= hi[2];
        };
        for (int t = lo[0]; t <= hi[0]; ++t)
          for (int h = lo[1]; h <= hi[1]; ++h)
            for (int w = lo[2]; w <= hi[2]; ++w) {
              int j = (t * b.nt[1] + h) * b.nt[2] + w;
              ++pairs;
              fl += (double)nv[i] * (double)nv[j];
            }
        for (int j = 0; j < std::min(g.sink, b.n_tiles); ++j)  // sink tiles outside the window
          if (!in_window(j)) {
            ++pairs;
            fl += (double)nv[i] * (double)nv[j];
          }
      }
      p->static_pairs = pairs;
      p->static_flops = fl * 4.0 * g.d * g.B * g.H;
    } else {
      p->static_pairs = -1;
    }
  }

  // Workspace layout.
  size_t sz[VSA_WS_NREGIONS] = {0};
  if (!(f & VSA_FINE)) {
    size_t tm = (size_t)BH * g.tok_cap * g.d * 2;
    sz[VSA_WS_KT] = sz[VSA_WS_VT] = tm;
    // bf16 attention reads Q in raster order: tile-major Q only for E4M3
    sz[VSA_WS_QT] = g.f8 ? tm : 0;
    if (f & (VSA_TOPK | VSA_TOPK_FRAC | VSA_TOPP)) {
      sz[VSA_WS_POOLED_Q] = sz[VSA_WS_POOLED_K] = (size_t)BH * g.max_tiles * g.d * 4;
      if (g.summ == VSA_SUMM_MINMAX) sz[VSA_WS_POOLED_KMIN] = sz[VSA_WS_POOLED_K];
    }
    sz[VSA_WS_ROW_LEN] = (size_t)BH * g.max_tiles * 4;
    sz[VSA_WS_COL_IDX] = (size_t)BH * g.max_tiles * g.row_cap * 4;
    sz[VSA_WS_CAND] = (size_t)BH * 4;
    if (g.f8) {
      sz[VSA_WS_F8_EXP] = (size_t)BH * 3 * 4;
      sz[VSA_WS_F8_AMAX] = (size_t)BH * 3 * vsa::kAmaxParts * 4;
    }
    if (f & VSA_PROFILE_SELECT) {
      sz[VSA_WS_CAND_SCORE] = (size_t)BH * g.nb * 4;
      sz[VSA_WS_PROF_SSE] = (size_t)BH * g.prof_runs * g.nb * 4;
      sz[VSA_WS_PROF_PART] = (size_t)BH * g.prof_runs * g.prof_segs * 32 * (g.d + 2) * 4;
    }
    if (f & VSA_SICS_SELECT) {
      sz[VSA_WS_CAND_SCORE] = (size_t)BH * g.nb * 4;
      sz[VSA_WS_TILE_SICS] = (size_t)BH * g.nb * 2 * g.max_tiles * 4;
      sz[VSA_WS_ATOMS] = (size_t)BH * 2 * g.n_atoms * (g.d + 1) * 4;  // sums + non-zero counts
    }
  } else {
    sz[VSA_WS_FINE_QBAR] = (size_t)BH * g.fine_G * g.d * 4;
    sz[VSA_WS_FINE_TAU] = (size_t)BH * 8;
    sz[VSA_WS_FINE_COUNT] = (size_t)BH * g.fine_G * 4;
    sz[VSA_WS_FINE_IDX] = (size_t)BH * g.fine_cap * 4;
    sz[VSA_WS_FINE_MASK] = (size_t)BH * g.fine_G * (size_t)((N + 31) / 32) * 4;
  }
  sz[VSA_WS_SCRATCH] = (f & VSA_FINE) ? vsa::fine_scratch_bytes(g) : 256;
  size_t offv = 0;
  for (int r = 0; r < VSA_WS_NREGIONS; ++r) {
    p->off[r] = sz[r] ? offv : 0;
    p->size[r] = sz[r];
    offv += (sz[r] + 255) & ~(size_t)255;
  }
  p->ws_total = offv;
  return VSA_OK;
}

// Tile layout of q, k, v.  With mask inputs (the default) it also runs the
// SICS blocking choice and the pooled means the selection needs; a cached
// call (mask = false) keeps the blocking and the selection in the workspace.
int enqueue_layout(const vsa_plan_t* p, const void* q, const void* k, const void* v, void* ws,
                   hipStream_t s, bool mask = true) {
  const Geo& g = p->geo;
  if (g.flags & VSA_FINE) return VSA_OK;
  Ws w = resolve(p, ws);
  hipError_t e;
  if (mask && (g.flags & VSA_SICS_SELECT)) {
    e = vsa::launch_sics(g, w, (const uint16_t*)q, (const uint16_t*)k, s);
    if (e != hipSuccess) return hip_fail(e, "SICS kernels");
  }
  if (mask && (g.flags & VSA_PROFILE_SELECT)) {
    e = vsa::launch_profile(g, w, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, s);
    if (e != hipSuccess) return hip_fail(e, "profiling selector kernels");
  }
  bool pool = mask && (g.flags & (VSA_TOPK | VSA_TOPK_FRAC | VSA_TOPP)) != 0;
  if (g.f8) {  // the E4M3 scales need every head's max |x| before the layout
    e = vsa::launch_amax(g, w, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, s);
    if (e != hipSuccess) return hip_fail(e, "max-abs kernel");
  }
  e = vsa::launch_layout(g, w, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, pool, s);
  if (e != hipSuccess) return hip_fail(e, "layout kernel");
  return VSA_OK;
}

int enqueue_select(const vsa_plan_t* p, const void* q, const void* k, void* ws, hipStream_t s) {
  const Geo& g = p->geo;
  Ws w = resolve(p, ws);
  hipError_t e;
  if (g.flags & VSA_FINE) {
    e = vsa::launch_fine_select(g, w, (const uint16_t*)q, (const uint16_t*)k, s);
    if (e != hipSuccess) return hip_fail(e, "fine mask kernels");
    return VSA_OK;
  }
  e = vsa::launch_select(g, w, s);
  if (e != hipSuccess) return hip_fail(e, "select kernel");
  return VSA_OK;
}

int enqueue_attend(const vsa_plan_t* p, const void* q, const void* k, const void* v, void* o,
                   void* ws, hipStream_t s, bool make_streams = true) {
  const Geo& g = p->geo;
  Ws w = resolve(p, ws);
  hipError_t e;
  if (g.flags & VSA_FINE)
    e = vsa::launch_fine_attend(g, w, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                                (uint16_t*)o, s);
  else
    e = vsa::launch_attend(g, w, (const uint16_t*)q, (uint16_t*)o, s, make_streams);
  if (e != hipSuccess) return hip_fail(e, "attention kernel");
  return VSA_OK;
}

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  return VSA_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch`, looked up once
// per device (with that device current) and kept.
int scratch_on_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(VSA_ERR_UNSUPPORTED, "device %d is beyond the %d devices the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || ((uintptr_t)p & 255) != 0)
      return fail(VSA_ERR_HIP, "scratch symbol address %p is not 256-byte aligned", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return VSA_OK;
}

}  // namespace

extern "C" {

int vsa_plan(const vsa_problem* prob, const vsa_mask_policy* pol, vsa_plan_t** out) {
  if (!prob || !pol || !out) return fail(VSA_ERR_INVALID_ARG, "vsa_plan: NULL argument");
  *out = nullptr;
  vsa_plan_s* p = new (std::nothrow) vsa_plan_s;
  if (!p) return fail(VSA_ERR_INVALID_ARG, "out of host memory");
  int st = build_plan(prob, pol, p);
  if (st != VSA_OK) {
    delete p;
    return st;
  }
  *out = p;
  return ok();
}

void vsa_plan_destroy(vsa_plan_t* plan) { delete plan; }

int vsa_plan_get_info(const vsa_plan_t* p, vsa_plan_info* info) {
  if (!p || !info) return fail(VSA_ERR_INVALID_ARG, "vsa_plan_get_info: NULL argument");
  memset(info, 0, sizeof *info);
  const Geo& g = p->geo;
  info->n_blockings = g.nb;
  for (int c = 0; c < g.nb; ++c) {
    for (int a = 0; a < 3; ++a) info->ntiles[c][a] = g.blk[c].nt[a];
    info->n_tiles[c] = g.blk[c].n_tiles;
    info->slots[c] = g.blk[c].slots;
    info->topk[c] = g.blk[c].topk;
    info->pair[c] = g.blk[c].pair;
    info->units[c] = g.blk[c].units;
    info->interleave[c] = g.blk[c].pair && !g.blk[c].units && vsa::interleaved_pairs(g) ? 1 : 0;
  }
  info->max_tiles = g.max_tiles;
  info->row_cap = g.row_cap;
  info->head_sync = g.head_sync;
  info->static_pairs = p->static_pairs;
  info->static_flops = p->static_flops;
  info->fine_groups = g.fine_G;
  info->fine_keep_count = g.fine_keep;
  info->fine_cap = g.fine_cap;
  info->scale = g.scale;
  return ok();
}

int vsa_workspace_bytes(const vsa_plan_t* p, size_t* bytes) {
  if (!p || !bytes) return fail(VSA_ERR_INVALID_ARG, "vsa_workspace_bytes: NULL argument");
  *bytes = p->ws_total;
  return ok();
}

int vsa_workspace_region(const vsa_plan_t* p, int region, size_t* offset, size_t* bytes) {
  if (!p || !offset || !bytes) return fail(VSA_ERR_INVALID_ARG, "vsa_workspace_region: NULL argument");
  if (region < 0 || region >= VSA_WS_NREGIONS)
    return fail(VSA_ERR_INVALID_ARG, "unknown workspace region %d", region);
  *offset = p->off[region];
  *bytes = p->size[region];
  return ok();
}

int vsa_layout(const vsa_plan_t* p, const void* q, const void* k, const void* v, void* ws,
               size_t ws_bytes, void* stream) {
  int st = check_exec(p, ws, ws_bytes);
  if (st) return st;
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(v, "v"))) return st;
  if ((st = check_device())) return st;
  st = enqueue_layout(p, q, k, v, ws, (hipStream_t)stream);
  return st ? st : ok();
}

int vsa_select(const vsa_plan_t* p, const void* q, const void* k, const void* v, void* ws,
               size_t ws_bytes, void* stream) {
  (void)v;
  int st = check_exec(p, ws, ws_bytes);
  if (st) return st;
  if (p->geo.flags & VSA_FINE) {
    if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k"))) return st;
  }
  if ((st = check_device())) return st;
  st = enqueue_select(p, q, k, ws, (hipStream_t)stream);
  return st ? st : ok();
}

int vsa_attend(const vsa_plan_t* p, const void* q, const void* k, const void* v, void* o, void* ws,
               size_t ws_bytes, void* stream) {
  int st = check_exec(p, ws, ws_bytes);
  if (st) return st;
  if ((st = check_tensor(o, "o"))) return st;
  if (p->geo.flags & VSA_FINE) {
    if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(v, "v")))
      return st;
  } else if (!p->geo.f8) {
    if ((st = check_tensor(q, "q"))) return st;  // bf16 attention reads q in raster order
  }
  if ((st = check_device())) return st;
  st = enqueue_attend(p, q, k, v, o, ws, (hipStream_t)stream);
  return st ? st : ok();
}

int vsa_forward(const vsa_plan_t* p, const void* q, const void* k, const void* v, void* o, void* ws,
                size_t ws_bytes, void* stream) {
  int st = check_exec(p, ws, ws_bytes);
  if (st) return st;
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(v, "v")) ||
      (st = check_tensor(o, "o")))
    return st;
  if ((st = check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  if ((st = enqueue_layout(p, q, k, v, ws, s))) return st;
  if ((st = enqueue_select(p, q, k, ws, s))) return st;
  if ((st = enqueue_attend(p, q, k, v, o, ws, s))) return st;
  return ok();
}

int vsa_forward_noalloc(const vsa_plan_t* p, const void* q, const void* k, const void* v, void* o,
                        void* stream) {
  if (!p) return fail(VSA_ERR_INVALID_ARG, "plan is NULL");
  if (p->ws_total > vsa::kNoAllocBytes)
    return fail(VSA_ERR_UNSUPPORTED,
                "vsa_forward_noalloc: the plan needs %zu bytes of scratch, beyond the library's "
                "fixed %zu bytes; use vsa_forward with a caller-provided workspace",
                p->ws_total, vsa::kNoAllocBytes);
  int st;
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(v, "v")) ||
      (st = check_tensor(o, "o")))
    return st;
  if ((st = check_device())) return st;
  void* ws = nullptr;
  if ((st = scratch_on_device(&ws))) return st;
  hipStream_t s = (hipStream_t)stream;
  if ((st = enqueue_layout(p, q, k, v, ws, s))) return st;
  if ((st = enqueue_select(p, q, k, ws, s))) return st;
  // Side streams are used if an earlier call on this device made them; this
  // call makes none.
  if ((st = enqueue_attend(p, q, k, v, o, ws, s, /*make_streams=*/false))) return st;
  return ok();
}

int vsa_forward_cached(const vsa_plan_t* p, const void* q, const void* k, const void* v, void* o,
                       void* ws, size_t ws_bytes, void* stream) {
  int st = check_exec(p, ws, ws_bytes);
  if (st) return st;
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(v, "v")) ||
      (st = check_tensor(o, "o")))
    return st;
  if ((st = check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  if ((st = enqueue_layout(p, q, k, v, ws, s, /*mask=*/false))) return st;
  if ((st = enqueue_attend(p, q, k, v, o, ws, s))) return st;
  return ok();
}

int vsa_untile(const vsa_plan_t* p, int which, const void* ws, size_t ws_bytes, void* out,
               void* stream) {
  int st = check_exec(p, ws, ws_bytes);
  if (st) return st;
  if (p->geo.flags & VSA_FINE) return fail(VSA_ERR_UNSUPPORTED, "no tiled layout under VSA_FINE");
  if (p->geo.f8) return fail(VSA_ERR_UNSUPPORTED, "the tiled layout holds E4M3 under VSA_COMPUTE_FP8");
  if (which != 0 && which != 1) return fail(VSA_ERR_INVALID_ARG, "which must be 0 (Q) or 1 (K)");
  if (which == 0)
    return fail(VSA_ERR_UNSUPPORTED, "no tile-major Q: the bf16 attention reads Q in raster order");
  if ((st = check_tensor(out, "out"))) return st;
  if ((st = check_device())) return st;
  Ws w = resolve(p, (void*)ws);
  hipError_t e = vsa::launch_untile(p->geo, w, which, (uint16_t*)out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "untile kernel");
  return ok();
}

int vsa_read_selection(const vsa_plan_t* p, const void* ws, size_t ws_bytes, int32_t* row_ptr,
                       int32_t* col_idx, size_t col_cap, int64_t* n_kept, int32_t* cand,
                       void* stream) {
  int st = check_exec(p, ws, ws_bytes);
  if (st) return st;
  if (!row_ptr || !n_kept) return fail(VSA_ERR_INVALID_ARG, "row_ptr and n_kept must not be NULL");
  const Geo& g = p->geo;
  if (g.flags & VSA_FINE) return fail(VSA_ERR_UNSUPPORTED, "tile selection does not exist under VSA_FINE");
  if ((st = check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  Ws w = resolve(p, (void*)ws);
  const long BH = (long)g.B * g.H;
  const long rows = BH * g.max_tiles;
  std::vector<int32_t> len(rows), idx((size_t)rows * g.row_cap);
  std::vector<int32_t> cnd(BH, 0);
  hipError_t e = hipMemcpyAsync(len.data(), w.row_len, rows * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(idx.data(), w.col_idx, idx.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && w.cand && vsa::per_head_blocking(g))
    e = hipMemcpyAsync(cnd.data(), w.cand, BH * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading the selection");
  for (long bh = 0; bh < BH; ++bh)
    if (cnd[bh] < 0 || cnd[bh] >= g.nb)
      return fail(VSA_ERR_HIP, "corrupt blocking index %d for head %ld", cnd[bh], bh);
  int64_t n = 0;
  row_ptr[0] = 0;
  for (long r = 0; r < rows; ++r) {
    long bh = r / g.max_tiles;
    int i = (int)(r % g.max_tiles);
    int nt = g.blk[cnd[bh]].n_tiles;
    int L = (i < nt) ? len[r] : 0;
    if (L < 0 || L > g.row_cap) return fail(VSA_ERR_HIP, "corrupt row length %d at row %ld", L, r);
    if (col_idx) {
      if ((size_t)(n + L) > col_cap) return fail(VSA_ERR_WORKSPACE_TOO_SMALL, "col_cap too small");
      memcpy(col_idx + n, idx.data() + (size_t)r * g.row_cap, (size_t)L * 4);
    }
    n += L;
    row_ptr[r + 1] = (int32_t)n;
  }
  *n_kept = n;
  if (cand) memcpy(cand, cnd.data(), BH * 4);
  return ok();
}

int vsa_retained_work(const vsa_plan_t* p, const void* ws, size_t ws_bytes, int64_t* pairs,
                      double* flops, void* stream) {
  int st = check_exec(p, ws, ws_bytes);
  if (st) return st;
  if (!pairs || !flops) return fail(VSA_ERR_INVALID_ARG, "pairs and flops must not be NULL");
  const Geo& g = p->geo;
  if ((st = check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  Ws w = resolve(p, (void*)ws);
  const long BH = (long)g.B * g.H;
  if (g.flags & VSA_FINE) {
    std::vector<int32_t> cnt((size_t)BH * g.fine_G);
    hipError_t e = hipMemcpyAsync(cnt.data(), w.fine_count, cnt.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "reading fine counts");
    int64_t pr = 0;
    double fl = 0;
    for (long bh = 0; bh < BH; ++bh)
      for (int gi = 0; gi < g.fine_G; ++gi) {
        long rowsg = std::min<long>(g.fine_M, (long)g.N - (long)gi * g.fine_M);
        long c = cnt[bh * g.fine_G + gi];
        if (c < 0 || c > g.N) return fail(VSA_ERR_HIP, "corrupt fine count %ld for head %ld", c, bh);
        pr += c;
        fl += 4.0 * g.d * (double)rowsg * (double)c;
      }
    *pairs = pr;
    *flops = fl;
    return ok();
  }
  const long rows = BH * g.max_tiles;
  std::vector<int32_t> len(rows), idx((size_t)rows * g.row_cap), cnd(BH, 0);
  hipError_t e = hipMemcpyAsync(len.data(), w.row_len, rows * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(idx.data(), w.col_idx, idx.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && vsa::per_head_blocking(g))
    e = hipMemcpyAsync(cnd.data(), w.cand, BH * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading the selection");
  int64_t pr = 0;
  double fl = 0;
  for (long bh = 0; bh < BH; ++bh) {
    if (cnd[bh] < 0 || cnd[bh] >= g.nb)
      return fail(VSA_ERR_HIP, "corrupt blocking index %d for head %ld", cnd[bh], bh);
    const BlkGeo& b = g.blk[cnd[bh]];
    std::vector<long> nv(b.n_tiles);
    for (int i = 0; i < b.n_tiles; ++i) nv[i] = tile_valid_id(g, b, i);
    for (int i = 0; i < b.n_tiles; ++i) {
      long r = bh * g.max_tiles + i;
      int L = len[r];
      if (L < 0 || L > g.row_cap) return fail(VSA_ERR_HIP, "corrupt row length");
      for (int e2 = 0; e2 < L; ++e2) {
        int j = idx[(size_t)r * g.row_cap + e2];
        if (j < 0 || j >= b.n_tiles) return fail(VSA_ERR_HIP, "corrupt tile index");
        ++pr;
        fl += (double)nv[i] * (double)nv[j];
      }
    }
  }
  *pairs = pr;
  *flops = fl * 4.0 * g.d;
  return ok();
}

const char* vsa_status_string(int status) {
  switch (status) {
    case VSA_OK: return "VSA_OK";
    case VSA_ERR_INVALID_ARG: return "VSA_ERR_INVALID_ARG";
    case VSA_ERR_UNSUPPORTED: return "VSA_ERR_UNSUPPORTED";
    case VSA_ERR_WORKSPACE_TOO_SMALL: return "VSA_ERR_WORKSPACE_TOO_SMALL";
    case VSA_ERR_HIP: return "VSA_ERR_HIP";
    default: return "VSA_ERR_UNKNOWN";
  }
}

const char* vsa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
