// Host side of the C ABI declared in include/fvattn.h: argument validation,
// workspace carving and kernel sequencing on the caller's stream.  No host
// synchronisation and no device allocation happen here.
#include <limits.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <utility>
#include <vector>

#include "common.h"

namespace fva {
namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxBlocks = 2048;   // key blocks per row the routing sort holds

inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool aligned16(const void *p) { return p && ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return p && ((uintptr_t)p & 3u) == 0; }

fva_status make_geo(const fva_problem *p, Geo *g) {
    if (!p) return FVA_ERR_INVALID_ARG;
    if (p->batch < 0 || p->heads < 0) return FVA_ERR_INVALID_ARG;
    if (p->grid_t < 1 || p->grid_y < 1 || p->grid_x < 1) return FVA_ERR_INVALID_ARG;
    const bool ordered = p->token_order != nullptr;
    if (ordered && ((uintptr_t)p->token_order & 3u)) return FVA_ERR_INVALID_ARG;
    if (!ordered) {
        if (p->tile_t < 1 || p->tile_y < 1 || p->tile_x < 1) return FVA_ERR_INVALID_ARG;
    }
    if (p->dtype != FVA_BF16 && p->dtype != FVA_F32) return FVA_ERR_UNSUPPORTED;
    if (p->head_dim != 64 && p->head_dim != 128) return FVA_ERR_UNSUPPORTED;
    if (!ordered) {
        const int64_t vol = (int64_t)p->tile_t * p->tile_y * p->tile_x;
        if (vol > kMaxSlots) return FVA_ERR_UNSUPPORTED;
    }
    const int64_t N = (int64_t)p->grid_t * p->grid_y * p->grid_x;
    if (N >= INT32_MAX) return FVA_ERR_INVALID_ARG;
    if (p->stride_n < p->head_dim || (p->stride_n % 8) || p->stride_h < 0 || (p->stride_h % 8) ||
        p->stride_b < 0 || (p->stride_b % 8))
        return FVA_ERR_INVALID_ARG;
    const int64_t elem = (p->dtype == FVA_BF16) ? 2 : 4;
    if (N * p->stride_n * elem >= INT32_MAX) return FVA_ERR_UNSUPPORTED;   // one head's rows span < 2 GiB
    const int64_t nT = ordered ? 0 : (p->grid_t + p->tile_t - 1) / p->tile_t;
    const int64_t nY = ordered ? 0 : (p->grid_y + p->tile_y - 1) / p->tile_y;
    const int64_t nX = ordered ? 0 : (p->grid_x + p->tile_x - 1) / p->tile_x;
    const int64_t Nb = ordered ? (N + kMaxSlots - 1) / kMaxSlots : nT * nY * nX;
    if (Nb > kMaxBlocks) return FVA_ERR_UNSUPPORTED;
    const int64_t BH = (int64_t)p->batch * p->heads;
    if (BH * Nb * Nb >= INT32_MAX) return FVA_ERR_INVALID_ARG;
    g->B = p->batch; g->H = p->heads; g->D = p->head_dim;
    g->T = p->grid_t; g->Y = p->grid_y; g->X = p->grid_x;
    g->tt = p->tile_t; g->ty = p->tile_y; g->tx = p->tile_x;
    g->nT = (int)nT; g->nY = (int)nY; g->nX = (int)nX;
    g->Nb = (int)Nb;
    g->N = (int)N;
    g->BH = (int)BH;
    g->sb = p->stride_b; g->sh = p->stride_h; g->sn = p->stride_n;
    g->dtype = p->dtype;
    g->order = p->token_order;
    return FVA_OK;
}

// Position of point (a0, a1, a2) along the 3D Hilbert curve of a 2^bits cube,
// after J. Skilling, "Programming the Hilbert curve" (AIP Conf. Proc. 707,
// 2004): undo the per-level reflections and axis exchanges from the top bit
// down, Gray-encode the axes into the transposed index, then read its bits
// plane by plane, axis 0 first.
uint64_t hilbert_key3(uint32_t a0, uint32_t a1, uint32_t a2, int bits) {
    uint32_t X[3] = {a0, a1, a2};
    const uint32_t top = 1u << (bits - 1);
    for (uint32_t Q = top; Q > 1; Q >>= 1) {
        const uint32_t low = Q - 1;
        for (int i = 0; i < 3; ++i) {
            if (X[i] & Q) {
                X[0] ^= low;
            } else {
                const uint32_t t = (X[0] ^ X[i]) & low;
                X[0] ^= t;
                X[i] ^= t;
            }
        }
    }
    X[1] ^= X[0];
    X[2] ^= X[1];
    uint32_t mask = 0;
    for (uint32_t Q = top; Q > 1; Q >>= 1)
        if (X[2] & Q) mask ^= Q - 1;
    uint64_t h = 0;
    for (int b = bits - 1; b >= 0; --b)
        for (int i = 0; i < 3; ++i) h = (h << 1) | (((X[i] ^ mask) >> b) & 1u);
    return h;
}

// Per-device CU count cache (the library's only global state).
std::mutex g_dev_mu;
int g_dev_cus[64] = {0};

int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        g_dev_cus[dev] = n;
    }
    return g_dev_cus[dev];
}

// ------------------------------------------- static routing scratch
// Scratch of fva_route_static: one array per device, sized for a one-GPU
// head shard of the 720p layer (5 heads x 660 blocks need 33 MB).  The
// array's name is a host-side stand-in; kernels get the device address that
// hipGetSymbolAddress returns for the current device, fetched once per
// device and kept.
__device__ __align__(256) static char scratch[FVA_STATIC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64] = {nullptr};

fva_status static_scratch(void **ptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FVA_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FVA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return FVA_OK;
}

// ------------------------------------------------------ route workspace
struct RouteWs {
    size_t qbar, kbar, sp, order, base, add, head_kept, total;
};

RouteWs route_layout(const Geo &g) {
    RouteWs w;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
    const size_t R = (size_t)g.BH * g.Nb;
    w.qbar = take(R * g.D * 8);
    w.kbar = take(R * g.D * 8);
    w.sp = take(R * g.Nb * 8);
    w.order = take(R * g.Nb * 4);
    w.base = take(R * 4);
    w.add = take(R * 4);
    w.head_kept = take((size_t)g.BH * 4);
    w.total = off;
    return w;
}

// -------------------------------------------------------- attn workspace
struct AttnPlanSizes {
    int num_ctas, cap_items, cap_parts, cap_splits;
    int max_pairs;   // query-block pairs per (batch, head) the workspace holds
};

// Query blocks with at most kPairTokens tokens, from the block geometry (the
// device pairs at most half of them).  Tiles: per axis, n - 1 tiles of the
// tile's extent and a last one of the remaining extent.
int64_t small_query_blocks(const Geo &g) {
    if (g.order) return (g.N - (int64_t)(g.Nb - 1) * kMaxSlots) <= kPairTokens ? 1 : 0;
    const int G[3] = {g.T, g.Y, g.X}, E[3] = {g.tt, g.ty, g.tx}, n[3] = {g.nT, g.nY, g.nX};
    int64_t cnt[3][2], ext[3][2];
    for (int a = 0; a < 3; ++a) {
        cnt[a][0] = n[a] - 1;
        ext[a][0] = E[a];
        cnt[a][1] = 1;
        ext[a][1] = G[a] - (int64_t)(n[a] - 1) * E[a];
    }
    int64_t small = 0;
    for (int t = 0; t < 2; ++t)
        for (int y = 0; y < 2; ++y)
            for (int x = 0; x < 2; ++x)
                if (ext[0][t] * ext[1][y] * ext[2][x] <= kPairTokens) small += cnt[0][t] * cnt[1][y] * cnt[2][x];
    return small;
}

fva_status attn_sizes(const Geo &g, const fva_attn_options *opts, AttnPlanSizes *s) {
    int chunk = 0, ctas = 0;
    if (opts) {
        if (opts->reserved != 0 || (opts->flags & ~(FVA_ATTN_PREPARED | FVA_ATTN_NO_ROW_PAIRS)) != 0)
            return FVA_ERR_INVALID_ARG;
        if ((opts->kernel_events[0] == nullptr) != (opts->kernel_events[1] == nullptr)) return FVA_ERR_INVALID_ARG;
        chunk = opts->chunk_blocks;
        ctas = opts->num_ctas;
        if (ctas < 0) return FVA_ERR_INVALID_ARG;
    }
    if (ctas == 0) {
        const int cus = device_cus();
        if (cus <= 0) return FVA_ERR_HIP;
        ctas = cus * attention_ctas_per_cu(g);
    }
    const int64_t R = (int64_t)g.BH * g.Nb;
    int64_t parts;
    if (chunk < 0) parts = 0;
    else if (chunk == 0) parts = 16LL * ctas;        // automatic chunks: <= 2 * total / C <= 16 * ctas
    else parts = R * ((g.Nb + chunk - 1) / chunk);   // fixed chunks
    if (parts > INT32_MAX / 2) return FVA_ERR_INVALID_ARG;
    // Room for the row pairs whatever the options, so that the layout (and
    // the K/V copies of fva_attn_prepare) does not depend on them.
    int64_t pairs = uses_packed_kv(g) ? small_query_blocks(g) / 2 : 0;
    if ((int64_t)g.BH * pairs * g.Nb > INT32_MAX / 2) pairs = 0;
    s->max_pairs = (int)pairs;
    s->num_ctas = ctas;
    s->cap_parts = (int)parts;
    s->cap_splits = (int)(parts / 2);
    s->cap_items = (int)(R + parts);
    return FVA_OK;
}

struct AttnWs {
    size_t tok, bsize, hdr, items, splits, part_o, part_ml, kp, vt;
    size_t role, first, n_pairs, ucol, ulen, hc, total;
};

AttnWs attn_layout(const Geo &g, const AttnPlanSizes &s) {
    AttnWs w;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
    w.tok = take((size_t)g.Nb * kMaxSlots * 4);
    w.bsize = take((size_t)g.Nb * 4);
    w.hdr = take(sizeof(PlanHeader));
    w.items = take((size_t)s.cap_items * sizeof(WorkItem));
    w.splits = take((size_t)(s.cap_splits > 0 ? s.cap_splits : 1) * sizeof(SplitRow));
    w.part_o = take((size_t)s.cap_parts * kMaxSlots * g.D * 4);
    w.part_ml = take((size_t)s.cap_parts * kMaxSlots * 2 * 4);
    w.kp = take(packed_kv_bytes(g));
    w.vt = take(packed_kv_bytes(g));
    w.role = take((size_t)g.Nb * 4);
    w.first = take((size_t)(s.max_pairs > 0 ? s.max_pairs : 1) * 4);
    w.n_pairs = take(4);
    w.ucol = take((size_t)g.BH * s.max_pairs * g.Nb * 4);
    w.ulen = take((size_t)g.BH * s.max_pairs * 4);
    w.hc = take((size_t)g.BH * 8 * 4);           // the plan's per-head counts
    w.total = off;
    return w;
}

#define FVA_TRY_HIP(expr)                                  \
    do {                                                   \
        if ((expr) != hipSuccess) return FVA_ERR_HIP;      \
    } while (0)

}  // namespace
}  // namespace fva

using namespace fva;

extern "C" {

fva_status fva_num_blocks(const fva_problem *prob, int32_t *nq, int32_t *nk) {
    Geo g;
    const fva_status st = make_geo(prob, &g);
    if (st != FVA_OK) return st;
    if (!nq || !nk) return FVA_ERR_INVALID_ARG;
    *nq = g.Nb;
    *nk = g.Nb;
    return FVA_OK;
}

fva_status fva_hilbert_order(int32_t grid_t, int32_t grid_y, int32_t grid_x, int32_t *order) {
    if (!order || grid_t < 1 || grid_y < 1 || grid_x < 1) return FVA_ERR_INVALID_ARG;
    const int64_t N = (int64_t)grid_t * grid_y * grid_x;
    if (N >= INT32_MAX) return FVA_ERR_INVALID_ARG;
    const int side = std::max(grid_t, std::max(grid_y, grid_x));
    int bits = 1;
    while ((1 << bits) < side) ++bits;
    if (bits > 21) return FVA_ERR_INVALID_ARG;       // 3 * bits must fit the 64-bit key
    std::vector<std::pair<uint64_t, int32_t>> key((size_t)N);
    int32_t n = 0;
    for (int32_t t = 0; t < grid_t; ++t)
        for (int32_t y = 0; y < grid_y; ++y)
            for (int32_t x = 0; x < grid_x; ++x, ++n) key[n] = {hilbert_key3(t, y, x, bits), n};
    std::sort(key.begin(), key.end());           // keys are distinct: the curve is a bijection
    for (int64_t i = 0; i < N; ++i) order[i] = key[i].second;
    return FVA_OK;
}

fva_status fva_block_sizes(const fva_problem *prob, int32_t *sizes) {
    Geo g;
    const fva_status st = make_geo(prob, &g);
    if (st != FVA_OK) return st;
    if (!sizes) return FVA_ERR_INVALID_ARG;
    for (int j = 0; j < g.Nb; ++j) {
        if (g.order) {
            sizes[j] = std::min(kMaxSlots, g.N - j * kMaxSlots);
            continue;
        }
        const int it = j / (g.nY * g.nX), iy = (j / g.nX) % g.nY, ix = j % g.nX;
        sizes[j] = std::min(g.tt, g.T - it * g.tt) * std::min(g.ty, g.Y - iy * g.ty) * std::min(g.tx, g.X - ix * g.tx);
    }
    return FVA_OK;
}

size_t fva_lists_capacity(const fva_problem *prob) {
    Geo g;
    if (make_geo(prob, &g) != FVA_OK) return 0;
    return (size_t)g.BH * g.Nb * g.Nb;
}

size_t fva_route_workspace_bytes(const fva_problem *prob) {
    Geo g;
    if (make_geo(prob, &g) != FVA_OK) return 0;
    return route_layout(g).total;
}

}  // extern "C"

namespace fva {
namespace {

// Argument checks of fva_route and fva_route_static (everything but the
// workspace).
fva_status route_args(const fva_problem *prob, const void *q, const void *k, double p, int32_t kmin,
                      fva_budget budget, const fva_lists *out, Geo *gout) {
    Geo &g = *gout;
    fva_status st = make_geo(prob, &g);
    if (st != FVA_OK) return st;
    if (!(p > 0.0 && p <= 1.0)) return FVA_ERR_INVALID_ARG;
    if (kmin < 0) return FVA_ERR_INVALID_ARG;
    if (budget.mode != FVA_BUDGET_NONE && budget.mode != FVA_BUDGET_FRAC && budget.mode != FVA_BUDGET_MATCH_MAX)
        return FVA_ERR_INVALID_ARG;
    if (budget.mode == FVA_BUDGET_FRAC && !(budget.frac >= 0.0 && budget.frac <= 1e6)) return FVA_ERR_INVALID_ARG;
    if (!out || !aligned4(out->row_ptr) || !aligned4(out->col_idx)) return FVA_ERR_INVALID_ARG;
    if (out->base_count && !aligned4(out->base_count)) return FVA_ERR_INVALID_ARG;
    if (out->head_kept && !aligned4(out->head_kept)) return FVA_ERR_INVALID_ARG;
    if (out->mask && !aligned4(out->mask)) return FVA_ERR_INVALID_ARG;
    if (g.BH != 0 && (!aligned16(q) || !aligned16(k))) return FVA_ERR_INVALID_ARG;
    return FVA_OK;
}

// The routing launches on a checked problem and a large enough workspace.
fva_status route_launch(const Geo &g, const void *q, const void *k, double p, int32_t kmin, fva_budget budget,
                        const fva_lists *out, void *ws, hipStream_t s, bool pooled = false) {
    const bool empty = (g.BH == 0);
    const RouteWs L = route_layout(g);
    char *W = static_cast<char *>(ws);
    double *qbar = (double *)(W + L.qbar), *kbar = (double *)(W + L.kbar), *SP = (double *)(W + L.sp);
    int32_t *order = (int32_t *)(W + L.order), *base = (int32_t *)(W + L.base), *add = (int32_t *)(W + L.add);
    int32_t *head_kept = out->head_kept ? out->head_kept : (int32_t *)(W + L.head_kept);
    if (!empty) {
        if (!pooled) {
            FVA_TRY_HIP(launch_pool(g, q, qbar, s));
            FVA_TRY_HIP(launch_pool(g, k, kbar, s));
        }
        FVA_TRY_HIP(launch_scores(g, qbar, kbar, SP, s));
        FVA_TRY_HIP(launch_row_select(g, SP, order, base, p, kmin, s));
        FVA_TRY_HIP(launch_augment(g, SP, base, add, head_kept, budget.mode, budget.frac, s));
    }
    FVA_TRY_HIP(launch_csr(g, order, base, add, head_kept, out->row_ptr, out->col_idx, out->base_count, out->mask,
                           s));
    return FVA_OK;
}

}  // namespace
}  // namespace fva

extern "C" {

fva_status fva_route(const fva_problem *prob, const void *q, const void *k, double p, int32_t kmin,
                     fva_budget budget, const fva_lists *out, void *ws, size_t ws_bytes, void *stream) {
    Geo g;
    const fva_status st = route_args(prob, q, k, p, kmin, budget, out, &g);
    if (st != FVA_OK) return st;
    if (!ws || ws_bytes < route_layout(g).total || ((uintptr_t)ws % kAlign)) return FVA_ERR_WORKSPACE;
    return route_launch(g, q, k, p, kmin, budget, out, ws, (hipStream_t)stream);
}

fva_status fva_route_static(const fva_problem *prob, const void *q, const void *k, double p, int32_t kmin,
                            fva_budget budget, const fva_lists *out, void *stream) {
    Geo g;
    fva_status st = route_args(prob, q, k, p, kmin, budget, out, &g);
    if (st != FVA_OK) return st;
    if (route_layout(g).total > FVA_STATIC_SCRATCH_BYTES) return FVA_ERR_SCRATCH;
    void *ws = nullptr;
    st = static_scratch(&ws);
    if (st != FVA_OK) return st;
    return route_launch(g, q, k, p, kmin, budget, out, ws, (hipStream_t)stream);
}

size_t fva_attn_workspace_bytes(const fva_problem *prob, const fva_attn_options *opts) {
    Geo g;
    if (make_geo(prob, &g) != FVA_OK) return 0;
    AttnPlanSizes sz;
    if (attn_sizes(g, opts, &sz) != FVA_OK) return 0;
    return attn_layout(g, sz).total;
}

size_t fva_attn_stats_bytes(const fva_problem *prob, const fva_attn_options *opts) {
    Geo g;
    if (make_geo(prob, &g) != FVA_OK) return 0;
    AttnPlanSizes sz;
    if (attn_sizes(g, opts, &sz) != FVA_OK) return 0;
    return sizeof(fva_plan_info) + (size_t)sz.num_ctas * sizeof(fva_cta_stat);
}

}  // extern "C"

namespace fva {
namespace {

// The attention launches on a checked problem and a large enough workspace
// (everything of fva_sparse_attn after its checks); prepared: the K/V copies
// are already in the workspace.
fva_status attn_launch(const Geo &g, const AttnPlanSizes &sz, const void *q, const void *k, const void *v,
                       const fva_lists *lists, void *o, void *ws, void *stats, const fva_attn_options *opts,
                       bool prepared, hipStream_t s) {
    const AttnWs L = attn_layout(g, sz);
    char *W = static_cast<char *>(ws);
    int32_t *tok = (int32_t *)(W + L.tok), *bsize = (int32_t *)(W + L.bsize);
    PlanHeader *hdr = (PlanHeader *)(W + L.hdr);
    WorkItem *items = (WorkItem *)(W + L.items);
    SplitRow *splits = (SplitRow *)(W + L.splits);
    float *part_o = (float *)(W + L.part_o), *part_ml = (float *)(W + L.part_ml);
    const int chunk = opts ? opts->chunk_blocks : 0;
    if (!prepared) FVA_TRY_HIP(launch_pack_kv(g, k, v, (uint16_t *)(W + L.kp), (uint16_t *)(W + L.vt), s));
    // Pairs of small query blocks, unless fixed chunks or the flag say otherwise.
    const bool pair_rows = sz.max_pairs > 0 && chunk <= 0 && !(opts && (opts->flags & FVA_ATTN_NO_ROW_PAIRS));
    const RowPairs rp{pair_rows ? sz.max_pairs : 0, (int32_t *)(W + L.role), (int32_t *)(W + L.first),
                      (int32_t *)(W + L.n_pairs), (int32_t *)(W + L.ucol), (int32_t *)(W + L.ulen)};
    FVA_TRY_HIP(launch_slot_table(g, tok, bsize, s));
    FVA_TRY_HIP(launch_row_pairs(g, bsize, lists->row_ptr, lists->col_idx, rp, s));
    FVA_TRY_HIP(launch_plan(g, lists->row_ptr, chunk, sz.num_ctas, sz.cap_items, sz.cap_parts, rp, hdr, items, splits,
                            (int32_t *)(W + L.hc), s));
    if (stats) FVA_TRY_HIP(launch_plan_stats(g, lists->row_ptr, lists->col_idx, bsize, sz.num_ctas, items, hdr, s));
    hipEvent_t ev0 = opts ? (hipEvent_t)opts->kernel_events[0] : nullptr;
    hipEvent_t ev1 = opts ? (hipEvent_t)opts->kernel_events[1] : nullptr;
    FVA_TRY_HIP(launch_attention(g, q, k, v, o, lists->row_ptr, lists->col_idx, rp.ucol, tok, bsize, hdr, items,
                                 part_o, part_ml,
                                 (fva_cta_stat *)stats, (uint16_t *)(W + L.kp), (uint16_t *)(W + L.vt), sz.num_ctas,
                                 ev0, ev1, s));
    FVA_TRY_HIP(launch_combine(g, o, tok, bsize, hdr, splits, part_o, part_ml, sz.cap_splits, s));
    return FVA_OK;
}

// Argument checks of fva_sparse_attn and fva_layer on the attention side
// (everything but the workspace).
fva_status attn_args(const Geo &g, const void *q, const void *k, const void *v, const fva_lists *lists, void *o,
                     void *stats) {
    if (!lists || !aligned4(lists->row_ptr) || !aligned4(lists->col_idx)) return FVA_ERR_INVALID_ARG;
    if (g.BH == 0) return FVA_OK;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FVA_ERR_INVALID_ARG;
    if (stats && ((uintptr_t)stats & 7u)) return FVA_ERR_INVALID_ARG;
    return FVA_OK;
}

// fva_layer's workspace: the routing workspace, then the attention's.
struct LayerWs {
    size_t route, attn, total;
};

LayerWs layer_layout(const Geo &g, const AttnPlanSizes &sz) {
    LayerWs w;
    w.route = 0;
    w.attn = align_up(route_layout(g).total);
    w.total = w.attn + attn_layout(g, sz).total;
    return w;
}

}  // namespace
}  // namespace fva

extern "C" {

fva_status fva_sparse_attn(const fva_problem *prob, const void *q, const void *k, const void *v,
                           const fva_lists *lists, void *o, void *ws, size_t ws_bytes, void *stats,
                           const fva_attn_options *opts, void *stream) {
    Geo g;
    fva_status st = make_geo(prob, &g);
    if (st != FVA_OK) return st;
    AttnPlanSizes sz;
    st = attn_sizes(g, opts, &sz);
    if (st != FVA_OK) return st;
    st = attn_args(g, q, k, v, lists, o, stats);
    if (st != FVA_OK || g.BH == 0) return st;
    if (!ws || ws_bytes < attn_layout(g, sz).total || ((uintptr_t)ws % kAlign)) return FVA_ERR_WORKSPACE;
    return attn_launch(g, sz, q, k, v, lists, o, ws, stats, opts, opts && (opts->flags & FVA_ATTN_PREPARED),
                       (hipStream_t)stream);
}

size_t fva_layer_workspace_bytes(const fva_problem *prob, const fva_attn_options *opts) {
    Geo g;
    if (make_geo(prob, &g) != FVA_OK) return 0;
    AttnPlanSizes sz;
    if (attn_sizes(g, opts, &sz) != FVA_OK) return 0;
    return layer_layout(g, sz).total;
}

fva_status fva_layer(const fva_problem *prob, const void *q, const void *k, const void *v, double p, int32_t kmin,
                     const fva_budget *budget_ptr, const fva_lists *lists, void *o, void *ws, size_t ws_bytes,
                     void *stats, const fva_attn_options *opts, void *stream) {
    if (!budget_ptr) return FVA_ERR_INVALID_ARG;
    const fva_budget budget = *budget_ptr;
    Geo g;
    fva_status st = route_args(prob, q, k, p, kmin, budget, lists, &g);
    if (st != FVA_OK) return st;
    AttnPlanSizes sz;
    st = attn_sizes(g, opts, &sz);
    if (st != FVA_OK) return st;
    if (opts && (opts->flags & FVA_ATTN_PREPARED)) return FVA_ERR_INVALID_ARG;
    st = attn_args(g, q, k, v, lists, o, stats);
    if (st != FVA_OK) return st;
    const LayerWs L = layer_layout(g, sz);
    if (!ws || ws_bytes < L.total || ((uintptr_t)ws % kAlign)) return FVA_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    char *W = static_cast<char *>(ws);
    void *rws = W + L.route, *aws = W + L.attn;
    // bf16, d = 128: one prologue reads Q, K and V once for the routing's
    // pooled means and the attention's K/V copies; otherwise the two calls'
    // own steps, back to back.
    const bool fused = uses_packed_kv(g) && g.BH > 0;
    if (fused) {
        const RouteWs R = route_layout(g);
        const AttnWs A = attn_layout(g, sz);
        char *RW = static_cast<char *>(rws), *AW = static_cast<char *>(aws);
        FVA_TRY_HIP(launch_prologue(g, q, k, v, (double *)(RW + R.qbar), (double *)(RW + R.kbar),
                                    (uint16_t *)(AW + A.kp), (uint16_t *)(AW + A.vt), s));
    }
    st = route_launch(g, q, k, p, kmin, budget, lists, rws, s, fused);
    if (st != FVA_OK || g.BH == 0) return st;
    return attn_launch(g, sz, q, k, v, lists, o, aws, stats, opts, fused, s);
}

fva_status fva_attn_prepare(const fva_problem *prob, const void *k, const void *v, void *ws, size_t ws_bytes,
                            const fva_attn_options *opts, void *stream) {
    Geo g;
    fva_status st = make_geo(prob, &g);
    if (st != FVA_OK) return st;
    AttnPlanSizes sz;
    st = attn_sizes(g, opts, &sz);
    if (st != FVA_OK) return st;
    if (g.BH == 0 || !uses_packed_kv(g)) return FVA_OK;
    if (!aligned16(k) || !aligned16(v)) return FVA_ERR_INVALID_ARG;
    const AttnWs L = attn_layout(g, sz);
    if (!ws || ws_bytes < L.total || ((uintptr_t)ws % kAlign)) return FVA_ERR_WORKSPACE;
    char *W = static_cast<char *>(ws);
    FVA_TRY_HIP(launch_pack_kv(g, k, v, (uint16_t *)(W + L.kp), (uint16_t *)(W + L.vt), (hipStream_t)stream));
    return FVA_OK;
}

const char *fva_status_string(fva_status s) {
    switch (s) {
        case FVA_OK: return "FVA_OK";
        case FVA_ERR_INVALID_ARG: return "FVA_ERR_INVALID_ARG: invalid argument";
        case FVA_ERR_UNSUPPORTED: return "FVA_ERR_UNSUPPORTED: unsupported head_dim, dtype, tile volume or block count";
        case FVA_ERR_WORKSPACE: return "FVA_ERR_WORKSPACE: workspace missing, misaligned or too small";
        case FVA_ERR_HIP: return "FVA_ERR_HIP: HIP runtime error";
        case FVA_ERR_SCRATCH:
            return "FVA_ERR_SCRATCH: the problem needs more than FVA_STATIC_SCRATCH_BYTES of routing scratch";
    }
    return "unknown fva_status";
}

}  // extern "C"
