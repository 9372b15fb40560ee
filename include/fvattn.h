/*
 * fvattn.h - C ABI of the FVAttn block-sparse attention hot path for AMD
 * Instinct MI355X (gfx950).
 *
 * The library implements the single-GPU data-parallel path of FVAttn
 * ("FVAttn: Adaptive Sparse Attention with Runtime Load Balancing for Video
 * Generation", arXiv 2607.16190):
 *
 *   fva_route        the sparse-routing front end: video-aware 3D-tile blocks,
 *                    mean-pooled Q/K block scores, per-query-block Top-p cut
 *                    with a Top-k floor, slack-aware augmentation up to a
 *                    per-head budget, and the per-head CSR block lists
 *                    (abstract; paperlayer.ai summary, section 3 "FVAttn
 *                    Design": Sparse-routing frontend, Slack-Aware Sparse
 *                    Augmentation);
 *   fva_attn_prepare the list-independent part of fva_sparse_attn (K/V
 *                    copies), for overlap with fva_route on another stream
 *   fva_sparse_attn  exact softmax attention over only the kept key blocks
 *                    (section 2 "Background and Related Work": dynamic
 *                    block-sparse attention), with a work-list balancer that
 *                    spreads long rows over the GPU's compute units - the
 *                    one-GPU counterpart of the pages' Runtime Load Balancing
 *                    (section 3, "Runtime Load Balancing").
 *
 * Conventions shared by every entry point:
 *  - Ownership: the caller owns every buffer (inputs, outputs, workspace,
 *    stats).  The library allocates no device memory and keeps no per-call
 *    state; its only global state is a per-device cache of the CU count.
 *  - Asynchrony: device work is enqueued on `stream` (a hipStream_t; NULL is
 *    the null stream) and the host is never synchronised.  Every
 *    data-dependent size stays on the device; outputs are sized for the
 *    worst case.  Concurrent calls on one stream are ordered; calls that
 *    share a workspace on different streams race.
 *  - Validation: arguments are checked on the host before anything is
 *    launched; on error nothing is enqueued and outputs are untouched.  A
 *    launch failure returns FVA_ERR_HIP (outputs then undefined).  No
 *    exception crosses the ABI.  Calls are thread-safe.
 *  - Pointers marked "device" must be device (or managed) memory, 16-byte
 *    aligned.
 */
#ifndef FVATTN_H
#define FVATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FVA_OK = 0,
    FVA_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, bad size or parameter */
    FVA_ERR_UNSUPPORTED = -2,   /* valid but not implemented (head_dim, dtype, tile volume) */
    FVA_ERR_WORKSPACE = -3,     /* workspace smaller than the matching *_workspace_bytes */
    FVA_ERR_HIP = -4,           /* a HIP runtime call or launch failed */
    FVA_ERR_SCRATCH = -5        /* fva_route_static: the problem needs more than FVA_STATIC_SCRATCH_BYTES */
} fva_status;

typedef enum { FVA_BF16 = 0, FVA_F32 = 1 } fva_dtype;

/*
 * Problem geometry.  Q, K, V and O are [batch, heads, N, head_dim] with
 * N = grid_t*grid_y*grid_x latent tokens, token n = (t*grid_y + y)*grid_x + x,
 * head_dim contiguous, and the given element strides (identical for q, k, v
 * and o; stride_n >= head_dim, all multiples of 8).
 *
 * Blocks (the video-aware block organisation of the routing front end,
 * paperlayer.ai summary of FVAttn, section 3 "FVAttn Design", Sparse-routing
 * frontend), one of:
 *  - token_order == NULL: 3D tiles of tile_t x tile_y x tile_x tokens in
 *    raster order over the tile grid: block b = (it*nY + iy)*nX + ix with
 *    nT = ceil(grid_t/tile_t), nY = ceil(grid_y/tile_y), nX =
 *    ceil(grid_x/tile_x).  A tile on the far edge of an axis that is not a
 *    multiple of the tile size holds only the tokens that exist; missing
 *    tokens are never keys and produce no output.  Nq = Nk = nT*nY*nX.
 *  - token_order != NULL: device int32 [N], 4-byte aligned, a permutation of
 *    the token indices (for instance the Hilbert-curve order from
 *    fva_hilbert_order); block b is entries 128*b .. min(128*b + 128, N) - 1,
 *    so every block is full except possibly the last.  Nq = Nk = ceil(N/128);
 *    tile_* are ignored.  Entries are clamped into [0, N): a malformed array
 *    gives wrong results but never an access outside q, k, v or o.  The
 *    array must stay unchanged while calls that use it run.
 *
 * Supported: head_dim in {64, 128}; dtype FVA_BF16 or FVA_F32;
 * tile volume tile_t*tile_y*tile_x <= 128; batch*heads*Nq*Nk < 2^31.
 * batch == 0 or heads == 0 is a valid empty problem (every call is a no-op).
 */
typedef struct {
    int32_t batch, heads, head_dim;
    int32_t grid_t, grid_y, grid_x;
    int32_t tile_t, tile_y, tile_x;
    int32_t dtype;                 /* fva_dtype */
    int64_t stride_b, stride_h, stride_n;
    const int32_t *token_order;    /* NULL: tile blocks; else block token order (device) */
} fva_problem;

/*
 * Slack budget of the augmentation step, per (batch, head), where K_h is the
 * head's block count after Top-p and the floor:
 *   NONE      B_h = K_h (no augmentation);
 *   FRAC      B_h = min(Nq*Nk, K_h + floor(frac*K_h)), frac >= 0, computed in
 *             IEEE double;
 *   MATCH_MAX B_h = max over heads h' of the same batch item of K_h'.
 */
typedef enum { FVA_BUDGET_NONE = 0, FVA_BUDGET_FRAC = 1, FVA_BUDGET_MATCH_MAX = 2 } fva_budget_mode;
typedef struct {
    int32_t mode;                  /* fva_budget_mode */
    double frac;
} fva_budget;

/*
 * Block lists: one CSR row per (batch, head, query block), rows in
 * (b, h, i) order, each row's kept key blocks in ascending order.
 * All device int32 buffers owned by the caller.
 */
typedef struct {
    int32_t *row_ptr;     /* [batch*heads*Nq + 1], required */
    int32_t *col_idx;     /* [fva_lists_capacity()], required; entries past row_ptr[last] undefined */
    int32_t *base_count;  /* [batch*heads*Nq] kept blocks before augmentation; may be NULL */
    int32_t *head_kept;   /* [batch*heads] final kept blocks per head (= B_h); may be NULL */
    uint32_t *mask;       /* [batch*heads*Nq*ceil(Nk/32)] bit j of row r = block j kept; may be NULL */
} fva_lists;

#define FVA_ATTN_PREPARED 1
#define FVA_ATTN_NO_ROW_PAIRS 2

/* Balancer options for fva_sparse_attn; pass NULL for the defaults (all 0). */
typedef struct {
    /* Split rows into work items of at most this many key blocks:
     *  0  automatic: C = max(16, ceil(total kept blocks / (8 * num_ctas)));
     *  <0 never split (one work item per row);
     *  >0 this chunk size. */
    int32_t chunk_blocks;
    /* Persistent workgroups; 0 = automatic: as many as fit on the current
     * device at once (two per compute unit for bf16 d=128, else one). */
    int32_t num_ctas;
    /* FVA_ATTN_PREPARED: the workspace already holds the K/V copies that
     * fva_attn_prepare wrote for the same problem, k, v and options, so
     * fva_sparse_attn skips them.
     * FVA_ATTN_NO_ROW_PAIRS: do not pair query blocks (see fva_sparse_attn).
     * No other bit may be set. */
    int32_t flags;
    int32_t reserved;     /* must be 0 */
    /* Optional caller-owned hipEvent_t pair (both or neither): recorded on
     * `stream` right before and right after the launch of the attention
     * kernel proper (after its K/V copies, before the merge of split rows),
     * so that the caller can time that one kernel. */
    void *kernel_events[2];
} fva_attn_options;

/* Written by the device into the optional stats buffer of fva_sparse_attn. */
typedef struct {
    int32_t n_items;       /* work items executed */
    int32_t chunk_blocks;  /* chunk size the plan used (INT32_MAX = no split) */
    int32_t n_split_rows;  /* rows split into more than one item */
    int32_t n_partials;    /* partial results merged by the combine step */
    int64_t total_blocks;  /* kept (query block, key block) pairs */
    int32_t num_ctas;      /* persistent workgroups launched */
    int32_t n_row_pairs;   /* work items that ran two query blocks together */
    /* Kept valid token pairs: the sum over kept (query block i, key block j)
     * of n_i * n_j, with n the blocks' token counts.  4 * head_dim times this
     * is the attention's useful flop count. */
    int64_t kept_pairs;
    /* The plan's predicted load balance: the work items, in queue order, each
     * given to the workgroup with the least work so far (ties to the lower
     * workgroup), cost = key blocks of the item; the largest workgroup load
     * over the mean (0 when more than 1,024 workgroups run). */
    float predicted_imbalance;
    int32_t reserved;      /* 0 */
} fva_plan_info;

typedef struct {
    uint32_t hw_id;        /* raw HW_ID register of the workgroup's first wave */
    uint32_t xcc_id;       /* raw XCC_ID register (accelerator complex die) */
    uint32_t items;        /* work items this workgroup processed */
    uint32_t blocks;       /* key blocks this workgroup processed */
    uint64_t t_start;      /* constant-rate (100 MHz) device clock at start */
    uint64_t t_end;        /* ... and after its last item */
} fva_cta_stat;

/*
 * Host only: the tokens of a grid_t x grid_y x grid_x grid in the order of a
 * 3D Hilbert curve, for token_order (paperlayer.ai summary of FVAttn,
 * section 3 "FVAttn Design", Sparse-routing frontend: a Hilbert-curve
 * reordering keeps tokens that are close in the video in nearby blocks).
 * The curve is J. Skilling's construction ("Programming the Hilbert curve",
 * 2004) on the smallest cube of side 2^m that holds the grid, axes (t, y, x),
 * starting at token 0; points outside the grid are skipped.  order: host
 * int32 [grid_t*grid_y*grid_x], written in full.  FVA_ERR_INVALID_ARG for a
 * NULL order, a side < 1, N >= 2^31 or a side above 2^21.
 */
fva_status fva_hilbert_order(int32_t grid_t, int32_t grid_y, int32_t grid_x, int32_t *order);

/* Number of query and key blocks of a problem.  Host only; FVA_ERR_* on an
 * invalid or unsupported problem. */
fva_status fva_num_blocks(const fva_problem *prob, int32_t *nq, int32_t *nk);

/* Host only: the valid token count of every block (the block organisation
 * of `prob`: tile extents clipped at the grid's far edges, or 128-token runs
 * of the token order with the remainder in the last), in block order.
 * sizes: host int32 [Nq].  prob->token_order is only tested against NULL.
 * FVA_ERR_* on an invalid or unsupported problem or a NULL sizes. */
fva_status fva_block_sizes(const fva_problem *prob, int32_t *sizes);

/* col_idx capacity in entries: batch*heads*Nq*Nk (0 if the problem is invalid). */
size_t fva_lists_capacity(const fva_problem *prob);

/* Workspace bytes fva_route needs (0 if the problem is invalid). */
size_t fva_route_workspace_bytes(const fva_problem *prob);

/*
 * Routing front end.  q, k: device, layout of `prob`.  p in (0, 1]: Top-p
 * mass (p = 1 keeps every block); kmin >= 0: Top-k floor (clamped to Nk).
 * Scores, softmax and cumulative masses are computed in float64; key blocks
 * are ranked by mass descending with ties to the lower block index.
 * Writes `out`'s buffers; ws: device workspace of at least
 * fva_route_workspace_bytes(prob) bytes.
 */
fva_status fva_route(const fva_problem *prob, const void *q, const void *k, double p, int32_t kmin,
                     fva_budget budget, const fva_lists *out, void *ws, size_t ws_bytes, void *stream);

/*
 * fva_route without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and checks as fva_route;
 * the scratch is instead a static device array of FVA_STATIC_SCRATCH_BYTES
 * that the library holds on every device it runs on until the process ends
 * (a one-GPU head shard of the 720p layer, 5 heads x 660 blocks, needs
 * 33 MB).  Problems with fva_route_workspace_bytes(prob) above that size
 * return FVA_ERR_SCRATCH before anything is launched.  Nothing is allocated:
 * no hipMalloc, hipFree or allocating library call.  All calls on one device
 * share its array (every buffer in it is fully rewritten by each call), so
 * calls that overlap on one device race: order them, e.g. on one stream.
 */
#define FVA_STATIC_SCRATCH_BYTES (64u << 20)
fva_status fva_route_static(const fva_problem *prob, const void *q, const void *k, double p, int32_t kmin,
                            fva_budget budget, const fva_lists *out, void *stream);

/* Workspace bytes fva_sparse_attn needs for these options (NULL = defaults).
 * With num_ctas == 0 this queries the current device (0 if that fails). */
size_t fva_attn_workspace_bytes(const fva_problem *prob, const fva_attn_options *opts);

/* Bytes of the stats buffer: one fva_plan_info then one fva_cta_stat per
 * persistent workgroup (0 if the problem or options are invalid).  Passing a
 * stats buffer adds two small launches before the attention kernel (the
 * pair count and the plan's load prediction). */
size_t fva_attn_stats_bytes(const fva_problem *prob, const fva_attn_options *opts);

/*
 * Block-sparse attention: for every query token t of block i,
 *   o_t = sum_u softmax_u(q_t . k_u / sqrt(head_dim)) v_u
 * over the tokens u of row i's kept key blocks (lists->row_ptr/col_idx as
 * written by fva_route, or any CSR with ascending or unordered, in-range,
 * duplicate-free columns).  q, k, v, o: device, layout of `prob`, o in the
 * input dtype.  bf16 inputs use bf16 MFMA with float32 accumulation and an
 * online softmax; float32 inputs use float32 arithmetic throughout.  A row
 * with no kept block yields zeros.  stats: NULL or a device buffer of
 * fva_attn_stats_bytes(prob, opts) bytes.  Only row_ptr and col_idx of
 * `lists` are read.
 *
 * Balancing (the one-GPU counterpart of the pages' Runtime Load Balancing,
 * paperlayer.ai summary of FVAttn, section 3 "FVAttn Design": attention
 * latency follows the largest workload): rows are cut into work items that
 * persistent workgroups pull from queues (opts->chunk_blocks).  For bf16 and
 * head_dim 128, unless FVA_ATTN_NO_ROW_PAIRS is set or chunk_blocks > 0, two
 * neighbouring query blocks of one head that each hold at most 64 tokens
 * (edge tiles) run as one work item over the union of their key lists, each
 * block attending only to its own kept blocks, in ascending block order; such
 * items are never split.  The results are those of the unpaired run up to
 * the rounding of the probabilities to bf16, which each run does against its
 * own softmax offsets.
 */
fva_status fva_sparse_attn(const fva_problem *prob, const void *q, const void *k, const void *v,
                           const fva_lists *lists, void *o, void *ws, size_t ws_bytes, void *stats,
                           const fva_attn_options *opts, void *stream);

/*
 * The part of fva_sparse_attn that does not depend on the block lists: the
 * block-major K and V^T copies that the bf16 head_dim-128 kernel streams
 * from (for other problems there is nothing to do and this returns FVA_OK).
 * Writing them ahead lets a caller run this on a second stream while
 * fva_route runs, and synchronise only where the data meet (paperlayer.ai
 * summary of FVAttn, section 3 "FVAttn Design", Overlap/Opt.: runtime work
 * is issued asynchronously and waits only on true data dependencies).
 * Then call fva_sparse_attn with the same prob, k, v, ws and options plus
 * FVA_ATTN_PREPARED in opts->flags, on a stream ordered after this call.
 * k, v: device, layout of `prob`.  ws, ws_bytes: the attention workspace
 * (fva_attn_workspace_bytes(prob, opts) bytes).  opts: as for
 * fva_sparse_attn (its flags are ignored here).  The copies are only ever
 * read inside the workspace, so a missing or stale preparation gives wrong
 * numbers, never an out-of-bounds access.
 */
fva_status fva_attn_prepare(const fva_problem *prob, const void *k, const void *v, void *ws, size_t ws_bytes,
                            const fva_attn_options *opts, void *stream);

/* Workspace bytes fva_layer needs for these options (NULL = defaults): the
 * routing workspace followed by the attention workspace (0 if the problem or
 * options are invalid). */
size_t fva_layer_workspace_bytes(const fva_problem *prob, const fva_attn_options *opts);

/*
 * One attention layer's whole hot path in one call: fva_route into `lists`,
 * then fva_sparse_attn on those lists into `o`, on `stream`, with the
 * arguments, checks and results of the two calls (paperlayer.ai summary of
 * FVAttn, section 3 "FVAttn Design", Pipeline: routing, then sparse
 * attention on the routed blocks).  For bf16 and head_dim 128 the two share
 * one prologue kernel that reads each of Q, K and V once, for the routing's
 * pooled block means and the attention's block-major K/V copies; lists and
 * output are bit for bit those of the separate calls.  ws: device, at least
 * fva_layer_workspace_bytes(prob, opts) bytes, 256-byte aligned.
 * opts->flags must not hold FVA_ATTN_PREPARED; kernel_events, when given,
 * bracket the attention kernel as in fva_sparse_attn.  budget: host pointer
 * (the slack budget of fva_route; passed by address in this call).
 */
fva_status fva_layer(const fva_problem *prob, const void *q, const void *k, const void *v, double p, int32_t kmin,
                     const fva_budget *budget, const fva_lists *lists, void *o, void *ws, size_t ws_bytes,
                     void *stats, const fva_attn_options *opts, void *stream);

/* Static string naming a status code. */
const char *fva_status_string(fva_status s);

#ifdef __cplusplus
}
#endif
#endif /* FVATTN_H */
