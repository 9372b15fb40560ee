// Internal definitions shared by the HIP kernels and the host ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fvattn.h"

namespace fva {

constexpr int kMaxSlots = 128;   // tokens per block (tile volume) the kernels hold

// Geometry derived from an fva_problem on the host and passed by value.
struct Geo {
    int B, H, D;
    int T, Y, X;
    int tt, ty, tx;
    int nT, nY, nX;
    int Nb;          // Nq = Nk
    int N;           // tokens per (batch, head)
    int BH;
    int64_t sb, sh, sn;
    int dtype;
    const int32_t *order;   // token order of the blocks (device), or null for 3D tiles
};

// One unit of attention work: query-block row `row` (= (b*H + h)*Nb + i),
// key-block range [kb_begin, kb_end) of col_idx, partial slot or -1.  A
// paired item (part = -2 - i2) runs query blocks i and i2 of the same head
// together over [kb_begin, kb_end) of the pair's union list.
struct WorkItem {
    int32_t row, kb_begin, kb_end, part;
};

// Query blocks of at most kPairTokens tokens fill only two of the four
// 32-query waves of the bf16 d = 128 kernel; neighbouring ones are paired
// into one work item.  Per geometry: role[i] = pair index p for the first
// block of pair p, -2 for its second block, -1 for an unpaired block;
// first[p] = first block of pair p; *n_pairs.  Per (batch, head) and pair:
// the union of the two rows' kept blocks, ascending, at
// ucol + ((b*H + h) * max_pairs + p) * Nb, entry = j | member bits << 16
// (bit 0: in the first block's list, bit 1: in the second's), length ulen.
// max_pairs = 0: no pairing.
constexpr int kPairTokens = 64;
struct RowPairs {
    int max_pairs;
    int32_t *role, *first, *n_pairs, *ucol, *ulen;
};

// Split row bookkeeping for the combine step.
struct SplitRow {
    int32_t row, part_begin, n_parts, pad;
};

// Device-written plan header followed by the work queue counters (one
// general queue, or one per XCD for the bf16 d=128 kernel).
struct PlanHeader {
    fva_plan_info info;
    int32_t queue[8];
};

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Token layout of one block.  Tile blocks: the first token t0, the extent
// (et, ey, ex) of the (possibly clipped) tile and the token count n; slot
// r < n is token t0 + (dt*Y + dy)*X + dx with (dt, dy, dx) the raster position
// of r in the tile.  Order blocks: slot r < n is ord[r] (clamped into the
// grid, so a malformed order cannot address outside the tensors).  Slots at
// or past n stand for the block's first token.
struct BlockTokens {
    int t0, ey, ex, n, Y, X, N;
    const int32_t *ord;
    __device__ inline int token(int r) const {
        if (ord) return min(max(ord[r < n ? r : 0], 0), N - 1);
        if (r >= n) return t0;
        const int exy = ey * ex;
        const int dt = r / exy, rem = r - dt * exy, dy = rem / ex, dx = rem - dy * ex;
        return t0 + (dt * Y + dy) * X + dx;
    }
};

__device__ inline BlockTokens block_tokens(const Geo &g, int j) {
    BlockTokens b;
    b.Y = g.Y;
    b.X = g.X;
    b.N = g.N;
    if (g.order) {
        b.ord = g.order + (int64_t)j * kMaxSlots;
        b.n = min(kMaxSlots, g.N - j * kMaxSlots);
        b.t0 = 0; b.ey = 1; b.ex = 1;
        return b;
    }
    b.ord = nullptr;
    const int it = j / (g.nY * g.nX), iy = (j / g.nX) % g.nY, ix = j % g.nX;
    const int et = min(g.tt, g.T - it * g.tt);
    b.ey = min(g.ty, g.Y - iy * g.ty);
    b.ex = min(g.tx, g.X - ix * g.tx);
    b.n = et * b.ey * b.ex;
    b.t0 = ((it * g.tt) * g.Y + iy * g.ty) * g.X + ix * g.tx;
    return b;
}

// ---------------------------------------------------------------- launches
// Routing (route.hip)
hipError_t launch_slot_table(const Geo &g, int32_t *tok, int32_t *bsize, hipStream_t s);
hipError_t launch_pool(const Geo &g, const void *x, double *out, hipStream_t s);
hipError_t launch_scores(const Geo &g, const double *qbar, const double *kbar, double *S, hipStream_t s);
hipError_t launch_row_select(const Geo &g, double *SP, int32_t *order, int32_t *base, double p,
                             int kmin, hipStream_t s);
hipError_t launch_augment(const Geo &g, const double *SP, const int32_t *base, int32_t *add,
                          int32_t *head_kept, int mode, double frac, hipStream_t s);
hipError_t launch_csr(const Geo &g, const int32_t *order, const int32_t *base, const int32_t *add,
                      const int32_t *head_kept, int32_t *row_ptr, int32_t *col_idx, int32_t *base_out,
                      uint32_t *mask, hipStream_t s);

// Attention (attn.hip)
hipError_t launch_row_pairs(const Geo &g, const int32_t *bsize, const int32_t *row_ptr, const int32_t *col_idx,
                           const RowPairs &rp, hipStream_t s);
hipError_t launch_plan(const Geo &g, const int32_t *row_ptr, int chunk_mode, int num_ctas,
                       int cap_items, int cap_parts, const RowPairs &rp, PlanHeader *hdr, WorkItem *items,
                       SplitRow *splits, int32_t *head_counts, hipStream_t s);
hipError_t launch_plan_stats(const Geo &g, const int32_t *row_ptr, const int32_t *col_idx, const int32_t *bsize,
                             int num_ctas, const WorkItem *items, PlanHeader *hdr, hipStream_t s);
hipError_t launch_attention(const Geo &g, const void *q, const void *k, const void *v, void *o,
                            const int32_t *row_ptr, const int32_t *col_idx, const int32_t *ucol, const int32_t *tok,
                            const int32_t *bsize,
                            PlanHeader *hdr, const WorkItem *items, float *part_o, float *part_ml,
                            fva_cta_stat *stats, uint16_t *kp, uint16_t *vt, int num_ctas, hipEvent_t ev0,
                            hipEvent_t ev1, hipStream_t s);
size_t packed_kv_bytes(const Geo &g);
bool uses_packed_kv(const Geo &g);
hipError_t launch_pack_kv(const Geo &g, const void *k, const void *v, uint16_t *kp, uint16_t *vt, hipStream_t s);
hipError_t launch_prologue(const Geo &g, const void *q, const void *k, const void *v, double *qbar, double *kbar,
                           uint16_t *kp, uint16_t *vt, hipStream_t s);
hipError_t launch_combine(const Geo &g, void *o, const int32_t *tok, const int32_t *bsize,
                          const PlanHeader *hdr, const SplitRow *splits, const float *part_o,
                          const float *part_ml, int cap_splits, hipStream_t s);
int attention_ctas_per_cu(const Geo &g);

}  // namespace fva
