/*
 * vsa.h - block-sparse self-attention over a 3D video token grid (MI355X).
 *
 * C ABI of libvsa.so.  Plain pointers and sizes only.  Device pointers are
 * HIP device memory owned by the caller; `stream` is a hipStream_t passed
 * as void* (NULL = the default stream).  Every call returns a status code
 * (VSA_OK = 0); no C++ exception crosses this boundary.  A failing call
 * leaves a message readable with vsa_last_error() on the calling thread.
 *
 * What is computed (sources are public web pages, cited by page/section):
 *   - the token grid T x H x W is cut into 3D tiles; one tile is one
 *     attention block and tokens inside a tile stay consecutive
 *     (Sliding Tile Attention verdict page, arXiv 2502.04507,
 *     pith_extraction.key_machinery);
 *   - each head may pick, among candidate blockings, the one whose tiles
 *     are most self-similar by SICS, the sum of intra-block cosine
 *     similarities (SPADE review page, arXiv 2608.03335, "Core claim",
 *     "What carries the argument", Figure 3);
 *   - each query tile keeps a set of key tiles: a sliding tile window
 *     (STA page, pith_extraction.pith_summary) and/or a Top-K / Top-P filter
 *     on pooled-mean block scores (SPADE page, "Core claim"; Figure 4);
 *   - alternatively a fine-grained mask keeps individual keys for groups of
 *     M consecutive queries, by thresholding k . mean(q_group)
 *     (FG-Attn verdict page, arXiv 2509.16518, pith_extraction.key_machinery,
 *     referee_report.major_comments[1]);
 *   - attention is then softmax(scale * q k^T) v restricted to the kept
 *     keys, computed with an online softmax (SPADE page, ledger axiom on
 *     FlashAttention-style online softmax).
 *
 * Tensor layout.  q, k, v, o are contiguous bf16 [B, H, N, d] with
 * N = T*H*W tokens in raster order (t, h, w), w fastest; 16-byte aligned.
 * d must be 64 or 128.
 */
#ifndef VSA_H
#define VSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define VSA_OK                      0
#define VSA_ERR_INVALID_ARG         1  /* null pointer, bad size/shape/policy */
#define VSA_ERR_UNSUPPORTED         2  /* valid but outside what is built */
#define VSA_ERR_WORKSPACE_TOO_SMALL 3
#define VSA_ERR_HIP                 4  /* a HIP runtime call failed (text in vsa_last_error) */

/* ---- dtypes ------------------------------------------------------------ */
#define VSA_BF16 1

/* ---- mask policy flags (combine with |) --------------------------------
 * VSA_DENSE       every key tile (all-ones block mask).
 * VSA_WINDOW      sliding tile window of win[] tiles (odd full extents).
 * VSA_TOPK        the `topk` highest-scoring key tiles per query tile.
 * VSA_TOPK_FRAC   Top-K with K = ceil(topk_frac * n_tiles) (per blocking).
 * VSA_TOPP        smallest set of highest-scoring key tiles whose softmax
 *                 mass over the row reaches `topp`.
 * VSA_SICS_SELECT per head, pick among problem.cand_tile[] by SICS.
 * VSA_PROFILE_SELECT per head, pick among problem.cand_tile[] the blocking
 *                 whose masked attention on a sample of query rows is
 *                 closest (MSE) to full attention on them (Sparse VideoGen
 *                 verdict page, pith_extraction.key_machinery: spatial vs
 *                 temporal heads from a ~1% row sample).  Readings: the
 *                 candidates use the policy's static mask (VSA_DENSE or
 *                 VSA_WINDOW, plus the sink); the sample is
 *                 clamp(round(profile_frac * N / 32), 1, N / 32) runs of 32
 *                 consecutive raster tokens, run r starting at
 *                 floor(r * N / runs) (all N tokens when N < 32); MSE is the
 *                 mean over sampled rows and channels; ties go to the lower
 *                 candidate.  Exclusive with VSA_SICS_SELECT; dynamic masks
 *                 (Top-K / Top-P) with it are VSA_ERR_UNSUPPORTED.
 * VSA_FINE        fine-grained M x 1 mask (M = fine_group), keep fraction
 *                 fine_keep of all (group, key) pairs per head.  Exclusive
 *                 with every other flag.
 * Window, Top-K, Top-P and the sink (policy.sink) combine as a union.
 * Top-K over all key tiles, then union with the window.                   */
#define VSA_DENSE        0x01u
#define VSA_WINDOW       0x02u
#define VSA_TOPK         0x04u
#define VSA_TOPK_FRAC    0x08u
#define VSA_TOPP         0x10u
#define VSA_SICS_SELECT  0x20u
#define VSA_FINE         0x40u
#define VSA_PROFILE_SELECT 0x80u

/* Block summarizer and score estimator of dynamic (Top-K / Top-P) masks.
 * The SPADE review page (referee report, minor comment 3; its ledger of
 * axioms) names max, min and mean block summaries (the MEAN-, DSA- and
 * DSA2-SPADE variants) but gives no expressions; the readings taken here,
 * with q_i the mean of query tile i and every reduction per channel over
 * the tile's valid tokens:
 *   VSA_SUMM_MEAN    S_ij = scale * <q_i, mean_j(K)>
 *   VSA_SUMM_MAX     S_ij = scale * <q_i, max_j(K)>
 *   VSA_SUMM_MINMAX  S_ij = scale * sum_c max(q_ic max_j(K)_c, q_ic min_j(K)_c),
 *                    an upper bound of scale * <q_i, k> over the keys k of
 *                    tile j.                                               */
#define VSA_SUMM_MEAN   0
#define VSA_SUMM_MAX    1
#define VSA_SUMM_MINMAX 2

/* Arithmetic of the tile attention (Sparse VideoGen verdict page,
 * pith_extraction.core_discovery / forward_implications and
 * skeptic_critique.rationale: optional FP8 quantization of attention, about
 * 1.3x on HunyuanVideo, scheme not given).  Readings taken:
 *   VSA_COMPUTE_BF16  bf16 Q, K, V and probabilities, fp32 accumulation.
 *   VSA_COMPUTE_FP8   OCP E4M3 (bias 7, largest finite 448, round to nearest
 *                     even) for Q, K, V and the probabilities.  Per (batch,
 *                     head) and tensor, x8 = E4M3(x * 2^e) with e the largest
 *                     integer such that max|x| * 2^e <= 448 (e = 0 when the
 *                     head is all zeros), clamped to [-32, 32]; inputs need
 *                     max|x| <= 448 * 2^32.  Scores are the dequantized
 *                     products s = scale * (q8 . k8) * 2^-(e_q + e_k); with
 *                     t = s * log2(e) and r = ceil(max t) over the row's kept
 *                     keys, p8 = E4M3(2^(t - r + 8)); O = 2^-e_v * sum p8 v8 /
 *                     sum p8, fp32 accumulation.  The selection (SICS, pooled
 *                     summaries, Top-K / Top-P) still reads the bf16 inputs.
 *                     Tile masks only (not with VSA_FINE).                  */
#define VSA_COMPUTE_BF16 0
#define VSA_COMPUTE_FP8  1

#define VSA_WIN_TRUNCATE 0  /* window cut at the grid edge */
#define VSA_WIN_CLAMP    1  /* window shifted inward, keeps its full size */

#define VSA_MAX_CAND 4

typedef struct vsa_problem {
  int32_t B, H, d;
  int32_t grid[3];                    /* T, H, W in tokens */
  int32_t tile[3];                    /* tile extents (t, h, w) when SICS is off */
  int32_t n_cand;                     /* candidate blockings for SICS / profiling (<= 4) */
  int32_t cand_tile[VSA_MAX_CAND][3];
  int32_t dtype;                      /* VSA_BF16 */
} vsa_problem;

typedef struct vsa_mask_policy {
  uint32_t flags;
  int32_t win[3];         /* window extent in tiles per axis, odd, >= 1 */
  int32_t win_mode;       /* VSA_WIN_TRUNCATE or VSA_WIN_CLAMP */
  int32_t topk;           /* for VSA_TOPK */
  double topk_frac;       /* for VSA_TOPK_FRAC, in (0, 1] */
  double topp;            /* for VSA_TOPP, in (0, 1] */
  int32_t fine_group;     /* M for VSA_FINE, multiple of 16, >= 16 */
  double fine_keep;       /* kept fraction for VSA_FINE, in (0, 1] */
  double scale;           /* softmax scale; 0 selects 1/sqrt(d) */
  int32_t summarizer;     /* VSA_SUMM_*; used by Top-K / Top-P only */
  int32_t sink;           /* key tiles 0 .. sink-1 (raster tile order, the
                             first frames) are kept for every query tile, an
                             always-kept attention sink (SPADE review page,
                             ledger free parameters: sink length, no value
                             given); 0 = none.  Not with VSA_FINE. */
  int32_t compute;        /* VSA_COMPUTE_BF16 (0) or VSA_COMPUTE_FP8 */
  double profile_frac;    /* VSA_PROFILE_SELECT: sampled fraction of query
                             rows, in (0, 1]; 0 selects 0.01 */
} vsa_mask_policy;

/* Opaque, immutable plan; safe to share between threads. */
typedef struct vsa_plan_s vsa_plan_t;

/* Facts about a plan (host data). */
typedef struct vsa_plan_info {
  int32_t n_blockings;            /* 1, or n_cand under VSA_SICS_SELECT / VSA_PROFILE_SELECT */
  int32_t ntiles[VSA_MAX_CAND][3];/* tiles per axis of each blocking */
  int32_t n_tiles[VSA_MAX_CAND];  /* tiles of each blocking */
  int32_t slots[VSA_MAX_CAND];    /* tokens per tile rounded up to 32 */
  int32_t topk[VSA_MAX_CAND];     /* resolved K per blocking (0 = off) */
  int32_t max_tiles;              /* max n_tiles over blockings */
  int32_t row_cap;                /* capacity of one kept-tile row */
  int64_t static_pairs;           /* kept tile pairs per head if the mask is
                                     input-independent, else -1 */
  double static_flops;            /* 4 d sum n_i n_j over static pairs, all
                                     heads and batches; 0 if dynamic */
  int32_t fine_groups;            /* G for VSA_FINE, else 0 */
  int64_t fine_keep_count;        /* kept (group, key) pairs per head target */
  int64_t fine_cap;               /* capacity of the kept-key lists per head: G * N
                                     (N per group, so ties at the threshold never
                                     overflow) */
  double scale;                   /* resolved softmax scale */
  int32_t pair[VSA_MAX_CAND];     /* 1: the attention of this blocking runs two adjacent
                                     query tiles per workgroup over the union of their
                                     kept lists (tiles of 4 to 6 slabs; Top-P masks, or
                                     static masks whose neighbours' lists mostly
                                     coincide) */
  int32_t units[VSA_MAX_CAND];    /* 1: the attention of this paired blocking stages
                                     the union's kept keys in units of 16 keys (bf16)
                                     or 32 keys (VSA_COMPUTE_FP8), packed into 64-key
                                     chunks across tile boundaries (when that cuts the
                                     chunk count by 5% or more: tile sizes not
                                     multiples of 64, ragged edge tiles), unless the
                                     unit table does not fit in LDS at launch; 0
                                     without pairing */
  int32_t interleave[VSA_MAX_CAND];/* 1: this paired blocking (Top-K masks) streams an
                                     interleaved schedule instead of the ascending union:
                                     the chunks both tiles keep, then the chunks only one
                                     keeps, alternating between the two tiles, so both
                                     halves of the workgroup compute in every step */
  int32_t head_sync;              /* 1: attention workgroups are ordered head by head
                                     across the whole GPU (each XCD takes one contiguous
                                     range of every head's query tiles): masks without a
                                     window, whose kept tiles have no spatial locality for
                                     an XCD's L2 to use, then keep only a head or two of
                                     K and V in the Infinity Cache at a time. 0: each XCD
                                     takes one contiguous range of all (head, tile)
                                     items, which keeps neighbouring windows together */
} vsa_plan_info;

/* Workspace regions, for inspection by tests (see vsa_workspace_region). */
#define VSA_WS_QT          0  /* tile-major Q, VSA_COMPUTE_FP8 only (0 bytes under bf16: the bf16
                                 attention reads Q in raster order) */
#define VSA_WS_KT          1  /* bf16 [B*H][tiles*slots][d] tile-major K */
#define VSA_WS_VT          2  /* bf16 [B*H][tiles][d][slots] tile-major V, transposed per tile */
#define VSA_WS_POOLED_Q    3  /* fp32 [B*H][max_tiles][d] mean of Q */
#define VSA_WS_POOLED_K    4  /* fp32 [B*H][d][max_tiles] (channel-major) mean (or, VSA_SUMM_MAX / MINMAX, maximum) of K */
#define VSA_WS_ROW_LEN     5  /* int32 [B*H][max_tiles] kept tiles per row */
#define VSA_WS_COL_IDX     6  /* int32 [B*H][max_tiles][row_cap] ascending */
#define VSA_WS_CAND        7  /* int32 [B*H] chosen blocking */
#define VSA_WS_CAND_SCORE  8  /* fp32 [B*H][n_blockings] mean pair cosine (SICS) or MSE (profiling) */
#define VSA_WS_TILE_SICS   9  /* fp32 [B*H][n_blockings][2][max_tiles] SICS of Q, K */
#define VSA_WS_ATOMS      10  /* fp32 [B*H][2][atoms][d] unit-vector sums, then int32 [B*H][2][atoms] non-zero counts */
#define VSA_WS_FINE_QBAR  11  /* fp32 [B*H][G][d] group means of Q */
#define VSA_WS_FINE_TAU   12  /* fp64 [B*H] per-head score threshold */
#define VSA_WS_FINE_COUNT 13  /* int32 [B*H][G] kept keys per group */
#define VSA_WS_FINE_IDX   14  /* int32 [B*H][G][N] kept keys of each group, ascending, in the
                                 first FINE_COUNT entries of the group's row */
#define VSA_WS_FINE_PTR   15  /* unused (0 bytes) */
#define VSA_WS_FINE_MASK  16  /* uint32 [B*H][G][ceil(N/32)] kept (group, key) pairs, key j in bit
                                 j % 32 of word j / 32 */
#define VSA_WS_SCRATCH    17  /* internal */
#define VSA_WS_POOLED_KMIN 18 /* fp32 [B*H][d][max_tiles] (channel-major) per-channel K minimum (VSA_SUMM_MINMAX) */
#define VSA_WS_F8_EXP     19  /* int32 [B*H][3] exponents e_q, e_k, e_v (VSA_COMPUTE_FP8) */
#define VSA_WS_F8_AMAX    20  /* uint32 [B*H][3][parts] partial max |x| as bf16 bits (VSA_COMPUTE_FP8) */
#define VSA_WS_PROF_SSE   21  /* fp32 [B*H][runs][n_blockings] squared-error sums (VSA_PROFILE_SELECT) */
#define VSA_WS_PROF_PART  22  /* profiling full-pass partials per key segment: float2 [B*H][runs][segs][32]
                                 (row sum, exp2 reference), then fp32 [B*H][runs][segs][32][d] */
#define VSA_WS_NREGIONS   23
/* Under VSA_COMPUTE_FP8 the QT, KT and VT regions hold E4M3 bytes in the
 * same layouts with 1-byte elements, except that inside every aligned group
 * of 32 slots of a VT row the key with slot bits (b4 b3 b2 b1 b0) sits at
 * position (b2 b4 b3 b1 b0): the keys that one half of the 64 MFMA lanes
 * multiplies are then contiguous. */

/* ---- plan ---------------------------------------------------------------
 * The policy (candidate blockings, mask expressions and budgets) is fixed
 * here, ahead of and apart from the execution calls (SPADE review page, "What
 * carries the argument": the specification of 3D blocking candidates and
 * summarizer / estimator masks, scheme generation, and a separate sparse
 * executor; "If this is right": policy separated from mechanism).  A tile is
 * a 3D box of tokens kept consecutive (STA verdict page,
 * pith_extraction.key_machinery).
 * Validates `prob` and `pol`, computes the tile geometry of every blocking,
 * the static window statistics and the workspace layout.  Host only: makes
 * no HIP call and needs no GPU.  On success *out owns a plan that the caller
 * releases with vsa_plan_destroy.  Errors: VSA_ERR_INVALID_ARG for null
 * pointers, non-positive sizes, even/zero window extents, fractions outside
 * (0,1], conflicting flags, an unknown compute mode; VSA_ERR_UNSUPPORTED
 * for d not in {64,128}, dtype other than bf16, VSA_COMPUTE_FP8 with
 * VSA_FINE, more than 4096 tiles, a tile larger than the grid, B*H above
 * 65535, more workgroups than one launch holds (B*H*tiles*11 or
 * B*H*groups above 2^31 - 1), or, for VSA_FINE, groups*N above 2^31 - 1
 * (the mask passes index a head's scores in 32 bits). */
int vsa_plan(const vsa_problem* prob, const vsa_mask_policy* pol, vsa_plan_t** out);
void vsa_plan_destroy(vsa_plan_t* plan);
int vsa_plan_get_info(const vsa_plan_t* plan, vsa_plan_info* info);

/* Workspace bytes the caller must provide to the calls below (host only). */
int vsa_workspace_bytes(const vsa_plan_t* plan, size_t* bytes);
/* Byte offset and size of one VSA_WS_* region inside the workspace. */
int vsa_workspace_region(const vsa_plan_t* plan, int region, size_t* offset, size_t* bytes);

/* ---- execution ----------------------------------------------------------
 * All of these enqueue kernels on `stream` and return without waiting; they
 * allocate no device memory and never synchronize.  Argument errors are
 * reported before anything is enqueued; a HIP launch error returns
 * VSA_ERR_HIP.  Kernel faults surface at the caller's next synchronization.
 * The workspace (>= vsa_workspace_bytes, 256-byte aligned) is owned by the
 * caller and must not be shared by calls that overlap in time.
 *
 * Side streams: under a per-head blocking choice (VSA_SICS_SELECT,
 * VSA_PROFILE_SELECT) the attention makes one launch per blocking, and the
 * launches after the first run on library-owned streams (default priority,
 * one set per device, made by the first uncaptured call that needs them and
 * kept until the process ends), forked from `stream` by an event recorded on
 * it and joined back into it before the call returns: work enqueued on
 * `stream` afterwards waits for all of them, as for any single-stream call.
 *
 * Stream capture: the calls enqueue kernel launches and event records /
 * waits only (no memset, copy or allocation), so a captured graph replays
 * them.  The first call of a kernel variant in a process also raises that
 * kernel's dynamic-LDS limit (a host-side function attribute) and makes the
 * side streams: make one uncaptured call with the plan before capturing (a
 * capture that comes first gets the blockings' launches in order on
 * `stream`).  A replay reads the buffers captured, so new inputs go into
 * those buffers.
 *
 * vsa_forward = vsa_layout + vsa_select + vsa_attend.  o receives the
 * attention output in the same raster layout as q. */
int vsa_forward(const vsa_plan_t* plan, const void* q, const void* k, const void* v,
                void* o, void* workspace, size_t ws_bytes, void* stream);

/* Forward with a cached mask (the semi-static class of the SPADE review
 * page, *What carries the argument*: a mask computed once and reused by later
 * calls; the FG-Attn verdict page, pith_summary: a cached mask reused across
 * denoising steps).  Lays out q, k, v and runs the attention against the
 * selection already in `workspace`, written by the last vsa_forward or
 * vsa_select on this workspace with this plan: no SICS choice (the blocking
 * per head is kept), no pooled means, no selection.  Under VSA_FINE only the
 * gathered attention runs.  Arguments, ownership and errors as vsa_forward.
 * A workspace whose selection was never written gives unspecified output
 * but no out-of-bounds access (lengths and indices are clamped in-kernel). */
int vsa_forward_cached(const vsa_plan_t* plan, const void* q, const void* k, const void* v,
                       void* o, void* workspace, size_t ws_bytes, void* stream);

/* Forward for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same computation, arguments, ownership and errors
 * as vsa_forward, except that the workspace is the library's own device
 * array of VSA_NOALLOC_BYTES (256 MiB) per device, held until the process
 * ends; nothing is allocated or freed by this call, and it makes no side
 * streams (it uses a device's side streams only once another call has made
 * them; otherwise the blockings' launches run in order on `stream`).  A plan whose
 * vsa_workspace_bytes exceeds VSA_NOALLOC_BYTES is refused with
 * VSA_ERR_UNSUPPORTED before anything is enqueued.  Every call on one device
 * shares that device's array, which keeps the previous call's contents
 * (each forward rewrites everything it reads): calls that overlap in time on
 * one device (other streams, other threads) race and must be serialized by
 * the caller. */
#define VSA_NOALLOC_BYTES ((size_t)256 << 20)
int vsa_forward_noalloc(const vsa_plan_t* plan, const void* q, const void* k, const void* v,
                        void* o, void* stream);

/* Stage 1, layout (the token-to-tile layout transform, fused with the block
 * summaries as on the SPADE review page, "What carries the argument"; tiles
 * kept consecutive in memory, STA verdict page, pith_extraction.key_machinery;
 * per-head blocking choice by SICS, SPADE "Core claim", or by the sampled-row
 * profiler, Sparse VideoGen verdict page, pith_extraction.key_machinery).
 * Under VSA_SICS_SELECT scores every candidate blocking by
 * SICS (under VSA_PROFILE_SELECT by the sampled-row MSE) and records the
 * chosen one per head; then copies Q, K (tile-major)
 * and V (tile-major, transposed per tile) into the workspace, padding each
 * tile with zeros up to its slot count, and, for dynamic masks, writes the
 * per-tile mean of Q and K.  Nothing to do under VSA_FINE. */
int vsa_layout(const vsa_plan_t* plan, const void* q, const void* k, const void* v,
               void* workspace, size_t ws_bytes, void* stream);

/* Stage 2, selection (block scores from the summaries, then Top-K / Top-P
 * united with the sliding tile window and the sink: SPADE review page, "Core
 * claim" and Figure 4; STA verdict page, pith_extraction.pith_summary; or the
 * per-head quantile of the M x 1 group mask: FG-Attn verdict page,
 * referee_report.major_comments[1]): the kept key tiles of every query tile (ascending,
 * in the workspace's ROW_LEN / COL_IDX regions), or under VSA_FINE the kept
 * keys of every query group.  Reads q, k only under VSA_FINE. */
int vsa_select(const vsa_plan_t* plan, const void* q, const void* k, const void* v,
               void* workspace, size_t ws_bytes, void* stream);

/* Stage 3, attention (dense MFMA work on every kept block, the mask kept out
 * of the inner loop: STA verdict page, pith_extraction.key_machinery; online
 * softmax: SPADE review page, ledger axiom; gathered M x 1 slices: FG-Attn
 * verdict page, pith_extraction.key_machinery): block-sparse (or
 * fine-grained) attention with online softmax, fp32 accumulation, bf16
 * output written straight to raster `o`.
 * Requires stages 1 and 2 on the same workspace. */
int vsa_attend(const vsa_plan_t* plan, const void* q, const void* k, const void* v,
               void* o, void* workspace, size_t ws_bytes, void* stream);
/* (vsa_attend reads q, k, v under VSA_FINE, and q under bf16 tile masks, whose
 * attention reads the query rows in raster order; otherwise they may be NULL.) */

/* Inverse layout: copy the workspace's tile-major K (which = 1) back to
 * raster bf16 [B, H, N, d] in `out`, dropping pads.  which = 0 (Q) is
 * VSA_ERR_UNSUPPORTED: the bf16 attention reads Q in raster order, so no
 * tile-major Q exists; so is any call under VSA_COMPUTE_FP8 (the workspace
 * holds E4M3). */
int vsa_untile(const vsa_plan_t* plan, int which, const void* workspace, size_t ws_bytes,
               void* out, void* stream);

/* ---- debug getters (synchronize `stream`) -------------------------------
 * vsa_read_selection returns the block mask that vsa_select built (the kept
 * key tiles of each query tile: SPADE review page, "Core claim"; STA verdict
 * page, pith_extraction.pith_summary).  The pooled summaries and SICS values
 * are not copied by it: they are read through vsa_workspace_region
 * (VSA_WS_POOLED_Q / _K / _KMIN, VSA_WS_TILE_SICS, VSA_WS_CAND_SCORE).
 * Copies the tile selection to host memory as CSR over rows r = (b*H + h) *
 * max_tiles + i: row_ptr has B*H*max_tiles + 1 entries, col_idx capacity
 * col_cap entries (B*H*max_tiles*row_cap always suffices); *n_kept receives
 * the number of entries written.  cand (may be NULL) receives B*H chosen
 * blockings.  Returns VSA_ERR_WORKSPACE_TOO_SMALL when col_cap is short. */
int vsa_read_selection(const vsa_plan_t* plan, const void* workspace, size_t ws_bytes,
                       int32_t* row_ptr, int32_t* col_idx, size_t col_cap,
                       int64_t* n_kept, int32_t* cand, void* stream);

/* Retained work of the current selection: kept tile pairs (or fine
 * (group, key) pairs) summed over heads, and 4*d*sum(n_query*n_key) FLOPs
 * over valid tokens.  Synchronizes `stream`. */
int vsa_retained_work(const vsa_plan_t* plan, const void* workspace, size_t ws_bytes,
                      int64_t* pairs, double* flops, void* stream);

const char* vsa_status_string(int status);
const char* vsa_last_error(void);   /* thread-local, "" if none */

#ifdef __cplusplus
}
#endif
#endif /* VSA_H */
