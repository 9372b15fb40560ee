// Block-sparse attention of FVAttn on gfx950: exact softmax attention over
// the kept key blocks only (paperlayer.ai summary of FVAttn, section 2
// "Background and Related Work": dynamic block-sparse attention; section 3
// "FVAttn Design": Pipeline), plus the work-list balancer that is the one-GPU
// counterpart of the pages' Runtime Load Balancing (section 3: attention
// latency follows the largest workload, so long work is spread out).
//
//   pair_table_kernel     per geometry: pairs of neighbouring query blocks of
//                         at most 64 tokens (two of the four waves each)
//   pair_union_kernel     per pair and head: the union of the two rows' kept
//                         blocks, with a member bit per row
//   plan_kernel           rows -> work items, heads densest first; rows longer
//                         than a chunk size are split so that no item
//                         dominates a compute unit's share; a pair whose union
//                         fits the chunk size is one item
//   pack_kv_kernel        block-major K and group-major V^T copies (bf16, d = 128)
//   attn_bf16_d128_kernel bf16, d = 128: two persistent workgroups per CU
//                         pull items from per-XCD queues (runs of 8 items
//                         dealt round robin to the 8 XCDs); per item (one
//                         query block, or a pair on waves 0-1 and 2-3) an
//                         online-softmax flash loop over the valid keys of
//                         the kept blocks, 64 keys per step (a step may span
//                         blocks), K/V^T streamed by LDS-DMA, bf16
//                         MFMA (v_mfma_f32_32x32x16_bf16) for Q K^T and P V
//   attn_bf16_kernel      the same for d = 64 (K/V staged through registers)
//   attn_f32_kernel       the same contract in float32 arithmetic
//   combine_kernel        log-sum-exp merge of a split row's partial results
//
// MFMA data layout (32x32x16, wave64): the kernel computes S^T = K Q^T so that
// each lane owns one query (column) and 16 keys per 32-key subtile.  The K
// rows are fed to the MFMA in the order that makes a lane's 16 scores the
// keys 16*(r/8) + 8*half + (r%8), i.e. two runs of 8 consecutive keys; those
// 8 values, rounded to bf16, are exactly the B operand of O^T = V^T P^T for a
// 16-key step.  Row max and row sum are therefore in-lane, plus one exchange
// between the two half-waves.  V is stored transposed in LDS so its A operand
// is one 16-byte read.  Both LDS tiles use an XOR swizzle of 16-byte chunks so
// the MFMA operand reads and the tile writes are bank-conflict free.
#include <float.h>
#include <math.h>

#include "common.h"

namespace fva {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// Two floats -> two bf16 (round to nearest even) in one dword, low half first.
__device__ inline uint32_t pack_bf16(float a, float b) {
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Read-only tables written by earlier launches (lists, block sizes, work
// items) are read through the constant address space so that wave-uniform
// reads become scalar loads.
typedef const int32_t __attribute__((address_space(4))) *cptr_i32;

struct AttnArgs {
    Geo g;
    const void *q, *k, *v;
    void *o;
    const int32_t *row_ptr, *col_idx, *ucol, *tok, *bsize;
    PlanHeader *hdr;
    const WorkItem *items;
    float *part_o, *part_ml;
    fva_cta_stat *stats;
    float scale_log2;   // log2(e) / sqrt(D)
};

__device__ inline uint32_t hw_id_reg() {
    uint32_t v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(v));
    return v;
}
__device__ inline uint32_t xcc_id_reg() {
    uint32_t v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
    return v;
}

__device__ inline void write_stats(const AttnArgs &a, uint64_t t0, uint32_t items, uint32_t blocks) {
    if (!a.stats || threadIdx.x != 0) return;
    const uint64_t t1 = wall_clock64();
    fva_cta_stat st;
    st.hw_id = hw_id_reg();
    st.xcc_id = xcc_id_reg();
    st.items = items;
    st.blocks = blocks;
    st.t_start = t0;
    st.t_end = t1;
    fva_cta_stat *rec = reinterpret_cast<fva_cta_stat *>(reinterpret_cast<char *>(a.stats) + sizeof(fva_plan_info));
    rec[blockIdx.x] = st;
    if (blockIdx.x == 0) *reinterpret_cast<fva_plan_info *>(a.stats) = a.hdr->info;
}

// Pull the next work item; every thread of the workgroup gets the same index.
__device__ inline int next_item(PlanHeader *hdr, int *s_item) {
    if (threadIdx.x == 0) *s_item = atomicAdd(&hdr->queue[0], 1);
    __syncthreads();
    const int it = *s_item;
    __syncthreads();
    return it;
}

// Per-XCD queues.  The item list is dealt to the 8 queues in runs of kRun
// consecutive items: queue q holds runs q, q + 8, q + 16, ...  A workgroup
// serves the queue of its own XCD first, so each run of neighbouring rows
// (which keep many of the same key blocks) shares one L2, while all XCDs
// move through the list, and hence through the same heads, together, so a
// head's keys and values are shared in the Infinity Cache.  A workgroup
// whose queue is empty moves on to the next one.  cur_q: the queue this
// workgroup is draining (starts at its XCD).
constexpr int kRun = 8;

__device__ inline int next_item_xcd(PlanHeader *hdr, int n_items, int &cur_q, int *s_item) {
    if (threadIdx.x == 0) {
        int *qs = hdr->queue;
        int it = n_items;
        const int rounds = n_items / (8 * kRun), rest = n_items - rounds * 8 * kRun;
        for (int k = 0; k < 8; ++k) {
            const int q = cur_q & 7;
            // items of queue q: (m * 8 + q) * kRun + w, w < kRun, below n_items
            const int cnt = rounds * kRun + min(kRun, max(0, rest - q * kRun));
            const int t = atomicAdd(&qs[q], 1);
            if (t < cnt) {
                it = ((t / kRun) * 8 + q) * kRun + t % kRun;
                break;
            }
            ++cur_q;
        }
        *s_item = it;
    }
    __syncthreads();
    const int it = *s_item;
    __syncthreads();
    return it;
}

// Swap bits 2 and 3 of a 5-bit MFMA row index: the K row fed to row x.
__device__ inline int krow_of(int x) { return (x & 0x13) | ((x & 4) << 1) | ((x & 8) >> 1); }

// Per-thread share of one key block: 8 consecutive slots (group g8) of one
// 16-byte chunk c of the head dimension, for K and for V.
struct TokRegs {
    int off[8];   // byte offset of the slot's chunk within the head (padding slots repeat a valid token)
    int n;        // valid tokens of the block
};

template <int D>
struct TileRegs {
    u32x4 k[8];
    u32x4 v[8];
};

__device__ __forceinline__ void load_tok(TokRegs &r, const int32_t *tok, const int32_t *bsize, int j, int g8,
                                         int row_bytes, int cbytes) {
    const int4 a = *reinterpret_cast<const int4 *>(tok + j * kMaxSlots + 8 * g8);
    const int4 b = *reinterpret_cast<const int4 *>(tok + j * kMaxSlots + 8 * g8 + 4);
    r.off[0] = a.x * row_bytes + cbytes; r.off[1] = a.y * row_bytes + cbytes;
    r.off[2] = a.z * row_bytes + cbytes; r.off[3] = a.w * row_bytes + cbytes;
    r.off[4] = b.x * row_bytes + cbytes; r.off[5] = b.y * row_bytes + cbytes;
    r.off[6] = b.z * row_bytes + cbytes; r.off[7] = b.w * row_bytes + cbytes;
    r.n = ((cptr_i32)bsize)[j];
}

// Raw buffer descriptor over one head's rows (gfx9 family dword 3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void *base, int64_t bytes) {
    const int n = bytes < 0x7fffffffLL ? (int)bytes : 0x7fffffff;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

// Global -> registers for one key block; no guards (see the slot table).
template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D> &tr, const TokRegs &tk, __amdgpu_buffer_rsrc_t rk,
                                          __amdgpu_buffer_rsrc_t rv) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        tr.k[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, tk.off[s], 0, 0));
        tr.v[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, tk.off[s], 0, 0));
    }
}

// Position (in 16-byte chunks) of chunk c of K row `slot`: an XOR swizzle that
// keeps both the tile writes (16 lanes: slots 8*g + s) and the MFMA operand
// reads (16 lanes: 16 distinct slots of one 32-key subtile) bank-conflict free.
template <int CH>
__device__ __forceinline__ int kswz(int slot, int c) { return c ^ ((slot ^ (slot >> 3)) & (CH - 1)); }

// Registers -> LDS.  K: row-major [slot][D] with the swizzle above.
// V: transposed [D][128 slots], 16-byte group g (8 slots) of row dd stored at
// group g ^ (dd % 16).
template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D> &tr, uint16_t *Kt, uint16_t *Vt, int c, int g8) {
    constexpr int CH = D / 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const int slot = 8 * g8 + s;
        *reinterpret_cast<u32x4 *>(Kt + slot * D + (kswz<CH>(slot, c) << 3)) = tr.k[s];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int dd = 8 * c + e;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        u32x4 out;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            out[w] = __builtin_amdgcn_perm(tr.v[2 * w + 1][e >> 1], tr.v[2 * w][e >> 1], sel);
        *reinterpret_cast<u32x4 *>(Vt + dd * kMaxSlots + ((g8 ^ (dd & 15)) << 3)) = out;
    }
}

// One key block for one wave's 32 queries.  FULL: all 128 slots are valid
// keys (no masking); otherwise keys at or past n_j get zero probability.
template <int D, bool FULL>
__device__ __forceinline__ void compute_tile(const uint16_t *Kt, const uint16_t *Vt, int n_j, const bf16x8 *qf,
                                             f32x16 *acc, float &m_run, float &l_run, float c, int h, int l32) {
    constexpr int CH = D / 8, KS = D / 16, NU = D / 32;
    const int krow = krow_of(l32);
    f32x16 sacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[t][r] = 0.f;
    // k-step outer, subtile inner: four independent operand reads in flight
    // ahead of four independent accumulations.
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        bf16x8 kf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int slot = 32 * t + krow;
            kf[t] = *reinterpret_cast<const bf16x8 *>(Kt + slot * D + (kswz<CH>(slot, 2 * s + h) << 3));
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t], qf[s], sacc[t], 0, 0, 0);
    }
    if (!FULL) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = 32 * t + 16 * (r >> 3) + 8 * h + (r & 7);
                if (key >= n_j) sacc[t][r] = -INFINITY;
            }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sacc[t][r]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float mnew = fmaxf(m_run, mloc);
    const float alpha = __builtin_amdgcn_exp2f((m_run - mnew) * c);
    m_run = mnew;
    const float mc = mnew * c;
    l_run *= alpha;
    if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[u][r] *= alpha;
    }
    bf16x8 pf[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // the denominator sums the bf16-rounded weights that P V uses
                const __bf16 pb = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[t][8 * hf + e], c, -mc));
                l_run += (float)pb;
                pf[2 * t + hf][e] = pb;
            }
        }
    }
#pragma unroll
    for (int sg = 0; sg < 8; ++sg) {
        bf16x8 vf[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int dd = 32 * u + l32;
            vf[u] = *reinterpret_cast<const bf16x8 *>(Vt + dd * kMaxSlots + (((2 * sg + h) ^ (dd & 15)) << 3));
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[u], pf[sg], acc[u], 0, 0, 0);
    }
}

template <int D>
__global__ __launch_bounds__(256, 1) void attn_bf16_kernel(AttnArgs a) {
    constexpr int KS = D / 16, NU = D / 32;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kMaxSlots * D];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][D * kMaxSlots];
    __shared__ int s_item;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
    // Tile loading role: chunk lc of the head dimension for slots 8*g8..8*g8+7
    // (all 256 threads for D = 128, the first 128 for D = 64).
    const int lc = tid >> 4, g8 = tid & 15;
    const bool ldr = tid < (D / 8) * 16;
    const Geo &g = a.g;
    const float c = a.scale_log2;
    const uint64_t t0 = wall_clock64();
    uint32_t n_done = 0, blocks_done = 0;
    const int n_items = a.hdr->info.n_items;
    const uint16_t *Q = static_cast<const uint16_t *>(a.q);
    const uint16_t *K = static_cast<const uint16_t *>(a.k);
    const uint16_t *V = static_cast<const uint16_t *>(a.v);
    uint16_t *O = static_cast<uint16_t *>(a.o);

    for (;;) {
        // Work-item fields are wave-uniform: keep them in scalar registers so
        // the per-block index reads below are scalar loads (lgkmcnt), not
        // vector loads that would queue behind the K/V data loads (vmcnt).
        const int it = __builtin_amdgcn_readfirstlane(next_item(a.hdr, &s_item));
        if (it >= n_items) break;
        WorkItem wi;
        {
            const cptr_i32 ip = (cptr_i32)a.items + 4 * it;
            wi.row = ip[0]; wi.kb_begin = ip[1]; wi.kb_end = ip[2]; wi.part = ip[3];
        }
        const int bh = wi.row / g.Nb, i = wi.row - (wi.row / g.Nb) * g.Nb;
        const int64_t boff = (int64_t)(bh / g.H) * g.sb + (int64_t)(bh % g.H) * g.sh;
        const int n_i = ((cptr_i32)a.bsize)[i];
        const bool active = (w * 32) < n_i;
        const int qslot = w * 32 + l32;
        const bool qvalid = qslot < n_i;
        const int qtok = a.tok[i * kMaxSlots + qslot];
        bf16x8 qf[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const u32x4 raw = *reinterpret_cast<const u32x4 *>(Q + boff + (int64_t)qtok * g.sn + 16 * s + 8 * h);
            qf[s] = __builtin_bit_cast(bf16x8, raw);
        }
        f32x16 acc[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[u][r] = 0.f;
        float m_run = -INFINITY, l_run = 0.f;
        const int nkb = wi.kb_end - wi.kb_begin;
        const cptr_i32 cols = (cptr_i32)a.col_idx + wi.kb_begin;
        if (nkb > 0) {
            // Software pipeline: token indices two blocks ahead, K/V data one
            // block ahead (registers), LDS double buffer for the block in use.
            const int64_t head_bytes = (int64_t)g.N * g.sn * 2;
            const __amdgpu_buffer_rsrc_t rk = head_rsrc(K + boff, head_bytes);
            const __amdgpu_buffer_rsrc_t rv = head_rsrc(V + boff, head_bytes);
            const int row_bytes = (int)(g.sn * 2), cbytes = lc * 16;
            TokRegs tnext;
            TileRegs<D> tr;
            load_tok(tnext, a.tok, a.bsize, cols[0], g8, row_bytes, cbytes);
            if (ldr) load_tile<D>(tr, tnext, rk, rv);
            int n_cur = tnext.n;
            if (nkb > 1) load_tok(tnext, a.tok, a.bsize, cols[1], g8, row_bytes, cbytes);
            if (ldr) store_tile<D>(tr, Ks[0], Vs[0], lc, g8);
            __syncthreads();
            for (int jj = 0; jj < nkb; ++jj) {
                const int buf = jj & 1;
                const int n_next = tnext.n;
                if (jj + 1 < nkb && ldr) load_tile<D>(tr, tnext, rk, rv);
                if (jj + 2 < nkb) load_tok(tnext, a.tok, a.bsize, cols[jj + 2], g8, row_bytes, cbytes);
                if (active) {
                    if (n_cur == kMaxSlots)
                        compute_tile<D, true>(Ks[buf], Vs[buf], n_cur, qf, acc, m_run, l_run, c, h, l32);
                    else
                        compute_tile<D, false>(Ks[buf], Vs[buf], n_cur, qf, acc, m_run, l_run, c, h, l32);
                }
                if (jj + 1 < nkb && ldr) store_tile<D>(tr, Ks[buf ^ 1], Vs[buf ^ 1], lc, g8);
                __syncthreads();
                n_cur = n_next;
            }
        }
        const float l = l_run + __shfl_xor(l_run, 32, 64);
        if (active && qvalid) {
            if (wi.part < 0) {
                const float inv = (l > 0.f) ? 1.f / l : 0.f;
                uint16_t *orow = O + boff + (int64_t)qtok * g.sn;
#pragma unroll
                for (int u = 0; u < NU; ++u) {
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const int dd = 32 * u + 8 * rg + 4 * h;
                        uint32_t w01 = pack_bf16(acc[u][4 * rg] * inv, acc[u][4 * rg + 1] * inv);
                        uint32_t w23 = pack_bf16(acc[u][4 * rg + 2] * inv, acc[u][4 * rg + 3] * inv);
                        *reinterpret_cast<uint2 *>(orow + dd) = make_uint2(w01, w23);
                    }
                }
            } else {
                float *po = a.part_o + ((int64_t)wi.part * kMaxSlots + qslot) * D;
#pragma unroll
                for (int u = 0; u < NU; ++u)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const int dd = 32 * u + 8 * rg + 4 * h;
                        *reinterpret_cast<float4 *>(po + dd) =
                            make_float4(acc[u][4 * rg], acc[u][4 * rg + 1], acc[u][4 * rg + 2], acc[u][4 * rg + 3]);
                    }
                if (h == 0) {
                    float *pm = a.part_ml + ((int64_t)wi.part * kMaxSlots + qslot) * 2;
                    pm[0] = m_run * c;
                    pm[1] = l;
                }
            }
        }
        ++n_done;
        blocks_done += nkb;
    }
    write_stats(a, t0, n_done, blocks_done);
}

// ----------------------------------------------------------------------
// Head dimension 128, bf16: the production kernel.
//
// Two workgroups per CU (two waves per SIMD), so one wave's softmax overlaps
// the other wave's matrix work.  Keys are consumed in 64-key chunks held in a
// two-stage LDS ring (2 x (16 KB K + 16 KB V^T) per workgroup), filled by
// LDS-DMA buffer loads issued one chunk ahead from the block-major K and
// group-major V^T copies that pack_kv_kernel writes (every DMA address is a per-lane
// constant plus a wave-uniform block offset, with no per-lane index loads).
// Work items come from per-XCD queues (next_item_xcd).  The softmax offset
// of a row (log2 units) is lazy: a chunk's probabilities are first
// formed against the current offset, and only when one of them could exceed
// 2^16 (a lane's sum of them does; always true on an item's first half,
// where the offset is -inf) is the offset raised to the exact running max,
// the accumulator rescaled and the chunk recomputed.  The row max is thus
// computed on a few chunks per row instead of on every chunk, and no
// probability exceeds 2^16.  Any offset is exact, since numerator and
// denominator use the same one; the denominator sums the bf16-rounded
// probabilities that P V uses, so that the two see identical weights.
constexpr int kChunk = 64;                       // keys per step
constexpr float kLazyBound = 65536.0f;           // largest probability the fast path admits

// Lane l and lane l ^ 32 (the two halves of one query's keys) combined by a
// commutative operation, so both lanes get the same bits.
__device__ __forceinline__ float max_halves(float x) { return fmaxf(x, __shfl_xor(x, 32, 64)); }
__device__ __forceinline__ float sum_halves(float x) { return x + __shfl_xor(x, 32, 64); }

// Probabilities of one wave's 64-key chunk against the offset m:
// p = exp2(s * c - m), rounded to bf16 into the B operands of P V; returns
// this lane's sum of the ROUNDED values (v_dot2 with a pair of ones, two
// partial sums).
__device__ __forceinline__ float half_probs(const f32x16 *sacc, float c, float m, bf16x8 *pf) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float a = __builtin_amdgcn_exp2f(fmaf(sacc[t][8 * hf + e], c, -m));
                const float b = __builtin_amdgcn_exp2f(fmaf(sacc[t][8 * hf + e + 1], c, -m));
                const bf16x2 pr = {(__bf16)a, (__bf16)b};
                pf[2 * t + hf][e] = pr[0];
                pf[2 * t + hf][e + 1] = pr[1];
                if (hf == 0) s0 = __builtin_amdgcn_fdot2_f32_bf16(pr, one, s0, false);
                else s1 = __builtin_amdgcn_fdot2_f32_bf16(pr, one, s1, false);
            }
    return s0 + s1;
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// K stage: [64 keys][128] bf16, 16-byte chunk c of row s at c ^ f(s).
__device__ __forceinline__ int kpos128(int slot, int c) { return c ^ ((slot ^ (slot >> 3)) & 15); }

// V stage: [8 key groups][128 dd][8 keys] bf16 (V^T per group of 8 keys, the
// layout of the packed copy), so that an 8-key group is 2 KB contiguous in
// both places.

// A chunk is 64 consecutive keys of the item's stream: the valid keys of its
// kept blocks in list order, each block rounded up to whole 8-key groups
// (the keys of the round-up are masked).  Wave w fetches groups 2w and 2w + 1
// of a chunk: K rows 16w .. 16w + 15 (four 1 KB pieces of 4 rows) and the V
// groups (four 1 KB pieces of 64 dd rows).  A group never spans two blocks,
// so every piece is one contiguous run of one block's packed copy: a per-lane
// constant offset plus a wave-uniform base.
struct DmaLane {
    int k[4];     // K piece p: source row 4 (p & 1) + lane / 16 of the group, chunk swizzled for LDS row 16w + 4p + lane / 16
    int v;        // V pieces: 16 bytes per lane (64 dd rows of 8 keys)
};

__device__ __forceinline__ DmaLane dma_lane(int w, int lane) {
    DmaLane d;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int row = 16 * w + 4 * p + (lane >> 4);
        const int ck = (lane & 15) ^ ((row ^ (row >> 3)) & 15);
        d.k[p] = (4 * (p & 1) + (lane >> 4)) * 256 + ck * 16;
    }
    d.v = lane * 16;
    return d;
}

// The chunk to fetch: destination stages (this wave's 4 KB share of each)
// and the byte offsets, in the head's packed K and V copies, of this wave's
// two groups.
struct DmaChunk {
    uint32_t kst, vst;
    __amdgpu_buffer_rsrc_t rkp, rvg;
    int sk[2], sv[2];
};

// One 1 KB LDS-DMA (16 bytes per lane), issued through inline assembly so
// that the compiler does not track it: with the builtin, the compiler's own
// waits for these loads were conservative (all outstanding loads) wherever
// it could not tell the stages apart.  The kernel waits explicitly (vmcnt(0)
// and a barrier) before any wave reads a stage, and makes Q resident before
// the first DMA of an item.  M0 carries the wave-uniform LDS address; nothing
// else in the kernel keeps a value in M0 (the clobber is declared, and the
// warning that M0 is reserved is silenced for this statement only).
__device__ __forceinline__ void dma16(uint32_t m0v, int voff, int soff, __amdgpu_buffer_rsrc_t rsrc) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(m0v), "v"(voff), "s"(rsrc), "s"(soff)
                 : "m0");
#pragma clang diagnostic pop
}

// Piece i < 4: K rows 4i .. 4i + 3 of the wave's 16; i >= 4: V group
// (i - 4) / 2, dd rows 64 ((i - 4) % 2) .. + 63.
__device__ __forceinline__ void dma_piece(const DmaChunk &d, const DmaLane &dl, int i) {
    if (i < 4)
        dma16(d.kst + i * 1024, dl.k[i], d.sk[i >> 1], d.rkp);
    else
        dma16(d.vst + (i - 4) * 1024, dl.v, d.sv[(i - 4) >> 1] + ((i - 4) & 1) * 1024, d.rvg);
}

__device__ __forceinline__ void dma_chunk(const DmaChunk &d, const DmaLane &dl) {
#pragma unroll
    for (int i = 0; i < 8; ++i) dma_piece(d, dl, i);
}

// Per-lane LDS byte offsets of the MFMA operand reads, fixed for the whole
// kernel.  K: the subtile t and the stage add immediates; the chunk order of
// k-step s for subtile 1 is that of step s ^ 2 for subtile 0 (the swizzle of
// row 32 + x is the swizzle of row x with bit 2 flipped).  V: key step sg
// reads group 2 sg + h, dd row 32 u + lane % 32 (u adds an immediate).
struct OperandAddr {
    uint32_t k[8];    // K row krow(l32), chunk for k-step s, subtile 0
    uint32_t v[4];    // V group 2 sg + h, dd row l32
};

__device__ __forceinline__ OperandAddr operand_addr(int lane) {
    OperandAddr o;
    const int h = lane >> 5, l32 = lane & 31;
    const int krow = krow_of(l32);
#pragma unroll
    for (int s = 0; s < 8; ++s) o.k[s] = (uint32_t)(krow * 256 + (kpos128(krow, 2 * s + h) << 4));
#pragma unroll
    for (int sg = 0; sg < 4; ++sg) o.v[sg] = (uint32_t)((2 * sg + h) * 2048 + l32 * 16);
    return o;
}

__device__ __forceinline__ bf16x8 lds_read16(const uint16_t *base, uint32_t byte_off) {
    return *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const char *>(base) + byte_off);
}

// One 64-key chunk for one wave's 32 queries; keys whose bit is clear in the
// 64-bit mask (mlo, mhi) get zero probability.
// The DMA of the next chunk `dn` is issued one piece per k-step of
// Q K^T, so the loads are spread over the MFMA stream instead of arriving in
// one burst; the scheduling groups below keep six operand reads in flight
// ahead of the MFMAs and put one DMA piece in each group.
__device__ __forceinline__ void chunk_tile(const uint16_t *Kt, const uint16_t *Vt, uint32_t mlo, uint32_t mhi,
                                          const bf16x8 *qf, f32x16 *acc, float &m_run, float &l_run, float c,
                                          int h, const OperandAddr &oa, const DmaChunk &dn, const DmaLane &dl) {
    f32x16 sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[t][r] = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const bf16x8 k0 = lds_read16(Kt, oa.k[s]);
        const bf16x8 k1 = lds_read16(Kt + 32 * 128, oa.k[s ^ 2]);
        dma_piece(dn, dl, s);
        sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[s], sacc[0], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[s], sacc[1], 0, 0, 0);
    }
    // The V operands of the first key step, read now so that their LDS
    // latency passes during the softmax.
    bf16x8 vf[2][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) vf[0][u] = lds_read16(Vt + u * 32 * 8, oa.v[0]);
    // Scheduling groups (masks: 0x100 LDS read, 0x020 VMEM read, 0x008
    // MFMA): ten K operand reads ahead of the first MFMA, then per pair of
    // MFMAs one DMA piece and the next reads (the V reads in the last ones).
    __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        if (s < 3) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        else if (s < 7) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    // The softmax runs at raised wave priority: while one wave of a SIMD
    // works through it, the other's MFMAs still fill the matrix core, and
    // this wave's vector work is not held back behind them.
    __builtin_amdgcn_s_setprio(1);
    if ((mlo & mhi) != 0xffffffffu) {
        // key 32t + 16(r/8) + 8h + r%8 is masked unless its bit is set
        // (bits 0-31 in mlo, 32-63 in mhi); this lane's bits are those of
        // h = 0 shifted down by 8h
        const uint32_t l0 = mlo >> (8 * h), l1 = mhi >> (8 * h);
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (!(((t ? l1 : l0) >> (16 * (r >> 3) + (r & 7))) & 1u)) sacc[t][r] = -INFINITY;
    }
    bf16x8 pf[4];
    float hs = half_probs(sacc, c, m_run, pf);
    // Slow path (wave-uniform): some lane's probabilities may exceed the
    // bound, or are not numbers (the offset was -inf, or a masked key met an
    // infinite offset): raise the offset to the exact running max and redo
    // the half.  Afterwards every probability is at most 1.
    if (__any(!(hs <= kLazyBound))) {
        float mloc = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, sacc[t][r]);
        mloc = max_halves(mloc) * c;
        const float mnew = fmaxf(m_run, mloc);
        const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
        m_run = mnew;
        l_run *= alpha;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[u][r] *= alpha;
        hs = half_probs(sacc, c, m_run, pf);
    }
    l_run += hs;
    __builtin_amdgcn_s_setprio(0);
    // P V, the operands of key step sg + 1 read while step sg multiplies
    // (two register sets, so no read waits for an MFMA to release its
    // registers).
#pragma unroll
    for (int sg = 0; sg < 4; ++sg) {
        if (sg < 3) {
#pragma unroll
            for (int u = 0; u < 4; ++u) vf[(sg + 1) & 1][u] = lds_read16(Vt + u * 32 * 8, oa.v[sg + 1]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[sg & 1][u], pf[sg], acc[u], 0, 0, 0);
    }
    // masks: 0x100 LDS read, 0x008 MFMA
#pragma unroll
    for (int sg = 0; sg < 3; ++sg)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

__global__ __launch_bounds__(256, 2) void attn_bf16_d128_kernel(AttnArgs a, const uint16_t *Kp_all,
                                                                  const uint16_t *Vt_all) {
    // Two LDS stages as distinct objects, so the compiler can see that the
    // DMA into one stage does not alias the reads of the other.
    __shared__ __attribute__((aligned(16))) uint16_t Ks0[kChunk * 128];
    __shared__ __attribute__((aligned(16))) uint16_t Vs0[kChunk * 128];
    __shared__ __attribute__((aligned(16))) uint16_t Ks1[kChunk * 128];
    __shared__ __attribute__((aligned(16))) uint16_t Vs1[kChunk * 128];
    __shared__ int s_item;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, l32 = lane & 31;
    const Geo &g = a.g;
    const float c = a.scale_log2;
    const uint64_t t0 = wall_clock64();
    uint32_t n_done = 0, blocks_done = 0;
    const int n_items = a.hdr->info.n_items;
    const uint16_t *Q = static_cast<const uint16_t *>(a.q);
    const uint16_t *K = static_cast<const uint16_t *>(a.k);
    uint16_t *O = static_cast<uint16_t *>(a.o);
    const OperandAddr oa = operand_addr(lane);
    int cur_q = (int)(xcc_id_reg() & 7);
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const DmaLane dl = dma_lane(wu, lane);
    const uint32_t seg0 = (uint32_t)wu * 4096u;   // this wave's 4 KB share of a stage

    for (;;) {
        const int it = __builtin_amdgcn_readfirstlane(next_item_xcd(a.hdr, n_items, cur_q, &s_item));
        if (it >= n_items) break;
        WorkItem wi;
        {
            const cptr_i32 ip = (cptr_i32)a.items + 4 * it;
            wi.row = ip[0]; wi.kb_begin = ip[1]; wi.kb_end = ip[2]; wi.part = ip[3];
        }
        const int bh = wi.row / g.Nb;
        const int64_t boff = (int64_t)(bh / g.H) * g.sb + (int64_t)(bh % g.H) * g.sh;
        // A paired item runs two query blocks of at most 64 tokens: waves 0-1
        // take the first (block i of the row), waves 2-3 the second; each
        // wave pair computes only the blocks of the union list that carry
        // its member bit.
        const bool paired = wi.part <= -2;
        const int grp = paired ? (wu >> 1) : 0;
        const int i = grp ? -2 - wi.part : wi.row - bh * g.Nb;
        const int part = paired ? -1 : wi.part;
        const int qw = paired ? (wu & 1) : wu;      // this wave's 32-query group within its block
        const int n_i = ((cptr_i32)a.bsize)[i];
        const bool active = (qw * 32) < n_i;
        const int qslot = qw * 32 + l32;
        const bool qvalid = qslot < n_i;
        const int qtok = a.tok[i * kMaxSlots + qslot];
        bf16x8 qf[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const u32x4 raw = *reinterpret_cast<const u32x4 *>(Q + boff + (int64_t)qtok * g.sn + 16 * s + 8 * h);
            qf[s] = __builtin_bit_cast(bf16x8, raw);
        }
        // Q is resident before the stream starts, so that no compiler wait
        // for these loads lands behind the untracked DMA.
#pragma unroll
        for (int s = 0; s < 8; ++s) asm volatile("" : "+v"(qf[s]));
        f32x16 acc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[u][r] = 0.f;
        float m_run = -INFINITY, l_run = 0.f;
        const int nkb = wi.kb_end - wi.kb_begin;
        const cptr_i32 cols = (cptr_i32)(paired ? a.ucol : a.col_idx) + wi.kb_begin;
        // list entry -> block index; whether this wave pair computes it
        const int mshift = 16 + grp;
        auto mine = [&](int e) { return !paired || ((e >> mshift) & 1); };
        if (nkb > 0) {
            const int64_t head_packed = (int64_t)bh * g.Nb * kMaxSlots * 128;
            const __amdgpu_buffer_rsrc_t rkp = head_rsrc(Kp_all + head_packed, (int64_t)g.Nb * kMaxSlots * 256);
            const __amdgpu_buffer_rsrc_t rvg = head_rsrc(Vt_all + head_packed, (int64_t)g.Nb * kMaxSlots * 256);
            const cptr_i32 bsz = (cptr_i32)a.bsize;
            auto lds_addr = [](const uint16_t *p) { return (uint32_t)(uintptr_t)(const lds_ptr_t)p; };
            // Chunk stream over the kept blocks.  Cursor: list position p,
            // key offset o (a multiple of 8) in that block.  Block entries
            // are read two positions ahead and sizes one ahead (scalar
            // loads): e0/n0 at p, e1/n1 at p + 1, e2 at p + 2.
            int p = 0, o = 0;
            int e0 = cols[0], n0 = bsz[e0 & 0xffff];
            int e1 = (nkb > 1) ? cols[1] : 0;
            int n1 = (nkb > 1) ? bsz[e1 & 0xffff] : 0;
            int e2 = (nkb > 2) ? cols[2] : 0;
            // Describe the next chunk and advance the cursor past it: this
            // wave's two group sources (block 0 of the head for groups past
            // the end: valid memory, masked keys) and this wave pair's key
            // mask (valid, owned keys).  Returns false when the stream ended.
            auto advance = [&]() {
                ++p;
                o = 0;
                e0 = e1; n0 = n1;
                if (p + 1 < nkb) { e1 = e2; n1 = bsz[e2 & 0xffff]; }
                if (p + 2 < nkb) e2 = cols[p + 2];
            };
            auto walk = [&](DmaChunk &d, uint32_t &mlo, uint32_t &mhi) -> bool {
                d.sk[0] = d.sk[1] = d.sv[0] = d.sv[1] = 0;
                mlo = mhi = 0u;
                if (p >= nkb) return false;
                if (o + kChunk <= n0) {
                    // the common case: 64 valid keys of block p
                    const int j = e0 & 0xffff;
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const int slot = o + 16 * wu + 8 * t;
                        d.sk[t] = (j * kMaxSlots + slot) * 256;
                        d.sv[t] = (j * 16 + (slot >> 3)) * 2048;
                    }
                    mlo = mhi = mine(e0) ? 0xffffffffu : 0u;
                    o += kChunk;
                    if (o >= ((n0 + 7) & ~7)) advance();
                    return true;
                }
                int x0 = 0;
                while (x0 < kChunk && p < nkb) {
                    const int j = e0 & 0xffff;
                    const int n8 = (n0 + 7) & ~7;
                    const int L = min(n8 - o, kChunk - x0);
                    const int nv = min(L, n0 - o);
                    if (mine(e0)) {
                        const uint64_t bits = (nv >= 64 ? ~0ull : ((1ull << nv) - 1ull)) << x0;
                        mlo |= (uint32_t)bits;
                        mhi |= (uint32_t)(bits >> 32);
                    }
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const int xg = 16 * wu + 8 * t;        // this wave's group t within the chunk
                        if (xg >= x0 && xg < x0 + L) {
                            const int slot = o + xg - x0;
                            d.sk[t] = (j * kMaxSlots + slot) * 256;
                            d.sv[t] = (j * 16 + (slot >> 3)) * 2048;
                        }
                    }
                    x0 += L;
                    o += L;
                    if (o >= n8) advance();
                }
                return true;
            };
            DmaChunk dc, dn;
            uint32_t cl, ch, nl, nh;
            walk(dc, cl, ch);
            dc.kst = lds_addr(Ks0) + seg0; dc.vst = lds_addr(Vs0) + seg0; dc.rkp = rkp; dc.rvg = rvg;
            dma_chunk(dc, dl);
            bool more = walk(dn, nl, nh);
            // One step of the stream: wait for the current stage, start the
            // DMA of the next chunk into the other stage, compute the
            // current one, describe the chunk after.  Unrolled by two so both
            // stages are fixed objects in each step.  After the last chunk
            // the DMA reloads the current one into the free stage (harmless,
            // and it keeps the k-step loop free of branches).
            auto step = [&](uint16_t *Kc, uint16_t *Vc, uint16_t *Kn, uint16_t *Vn) -> bool {
                __builtin_amdgcn_s_waitcnt(0x0f70);       // vmcnt(0): this wave's DMA for the current chunk landed
                __syncthreads();                          // ... and every wave's; the other stage is free again
                DmaChunk df = more ? dn : dc;
                df.kst = lds_addr(Kn) + seg0; df.vst = lds_addr(Vn) + seg0; df.rkp = rkp; df.rvg = rvg;
                if (active && (cl | ch)) chunk_tile(Kc, Vc, cl, ch, qf, acc, m_run, l_run, c, h, oa, df, dl);
                else dma_chunk(df, dl);
                if (!more) return false;
                dc = dn; cl = nl; ch = nh;
                more = walk(dn, nl, nh);
                return true;
            };
            while (step(Ks0, Vs0, Ks1, Vs1) && step(Ks1, Vs1, Ks0, Vs0)) {
            }
            __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): the last (reload) DMA has landed
            __syncthreads();       // all waves done with both stages before the next item's DMA
        }
        const float l = sum_halves(l_run);
        if (active && qvalid) {
            if (part < 0) {
                const float inv = (l > 0.f) ? 1.f / l : 0.f;
                uint16_t *orow = O + boff + (int64_t)qtok * g.sn;
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const int dd = 32 * u + 8 * rg + 4 * h;
                        *reinterpret_cast<uint2 *>(orow + dd) =
                            make_uint2(pack_bf16(acc[u][4 * rg] * inv, acc[u][4 * rg + 1] * inv),
                                       pack_bf16(acc[u][4 * rg + 2] * inv, acc[u][4 * rg + 3] * inv));
                    }
            } else {
                float *po = a.part_o + ((int64_t)part * kMaxSlots + qslot) * 128;
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const int dd = 32 * u + 8 * rg + 4 * h;
                        *reinterpret_cast<float4 *>(po + dd) =
                            make_float4(acc[u][4 * rg], acc[u][4 * rg + 1], acc[u][4 * rg + 2], acc[u][4 * rg + 3]);
                    }
                if (h == 0) {
                    float *pm = a.part_ml + ((int64_t)part * kMaxSlots + qslot) * 2;
                    pm[0] = m_run;
                    pm[1] = l;
                }
            }
        }
        ++n_done;
        // kept (query block, key block) pairs: a pair's two rows, else the range
        blocks_done += paired ? ((cptr_i32)a.row_ptr)[wi.row + 2] - ((cptr_i32)a.row_ptr)[wi.row] : nkb;
    }
    write_stats(a, t0, n_done, blocks_done);
}

// Block-major copies for the d=128 kernel, one workgroup per (block,
// batch*head): Kp[(bh*Nb + j)*128 + slot][128] and, per 8-slot group g,
// Vg[((bh*Nb + j)*16 + g)*128 + dd][8 slots] (V^T of the group, 2 KB
// contiguous); the slots of a block's last group past its tokens are zero,
// and groups wholly past its tokens are never written.  Every global access is
// a 256-byte row moved by 16 lanes (K, V reads; K writes) or 16-byte
// chunks consecutive across lanes (V^T writes): V goes through LDS, where
// thread t builds chunks t, t + 256, ... of the block's V^T from eight
// 2-byte reads of one column each (the 64 lanes of a wave read 64
// consecutive columns of one row: no bank conflicts).
// Slots past the block's tokens re-read its first token (loads stay
// unconditional, so they are all in flight at once); every consumer masks
// them by the block's token count.
__device__ __forceinline__ void load_rows(u32x4 *x, const uint16_t *T, const BlockTokens &bt, int64_t hoff,
                                          int64_t sn, int c16, int hi) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
        x[m] = *reinterpret_cast<const u32x4 *>(T + hoff + (int64_t)bt.token(hi + 16 * m) * sn + c16 * 8);
}

__device__ __forceinline__ void stage_rows(uint16_t *vs, const u32x4 *x, int c16, int hi) {
#pragma unroll
    for (int m = 0; m < 8; ++m) *reinterpret_cast<u32x4 *>(vs + (hi + 16 * m) * 128 + c16 * 8) = x[m];
}

// Rows of the block's tokens, and zero rows up to the next multiple of 8:
// the attention reads whole 8-slot groups of a block's tokens and nothing
// past them, so later groups are left unwritten.
__device__ __forceinline__ void write_k_rows(uint16_t *Kp_blk, u32x4 *x, int n, int c16, int hi) {
    const int n8 = (n + 7) & ~7;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int slot = hi + 16 * m;
        if (slot >= n) x[m] = u32x4{0, 0, 0, 0};
        if (slot < n8) *reinterpret_cast<u32x4 *>(Kp_blk + slot * 128 + c16 * 8) = x[m];
    }
}

// After a barrier behind stage_rows: the block's V^T chunks from LDS, for
// the 8-slot groups that hold tokens (slots past the tokens zero).
__device__ __forceinline__ void write_vt_groups(uint16_t *Vt_blk, const uint16_t *vs, int n) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = threadIdx.x + 256 * i;          // chunk (g, dd) = (c / 128, c % 128)
        const int r0 = 8 * (c >> 7), dd = c & 127;
        if (r0 >= n) continue;
        u32x4 o;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t lo = (r0 + 2 * w < n) ? vs[(r0 + 2 * w) * 128 + dd] : 0u;
            const uint32_t hi = (r0 + 2 * w + 1 < n) ? vs[(r0 + 2 * w + 1) * 128 + dd] : 0u;
            o[w] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4 *>(Vt_blk + c * 8) = o;
    }
}

__global__ __launch_bounds__(256) void pack_kv_kernel(Geo g, const uint16_t *K, const uint16_t *V,
                                                      uint16_t *Kp, uint16_t *Vt) {
    __shared__ __attribute__((aligned(16))) uint16_t vs[kMaxSlots * 128];
    const int j = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
    const BlockTokens bt = block_tokens(g, j);
    const int64_t hoff = (int64_t)(bh / g.H) * g.sb + (int64_t)(bh % g.H) * g.sh;
    const int64_t pblk = ((int64_t)bh * g.Nb + j) * kMaxSlots * 128;
    const int c16 = tid & 15, hi = tid >> 4;
    u32x4 kx[8], vx[8];
    load_rows(kx, K, bt, hoff, g.sn, c16, hi);
    load_rows(vx, V, bt, hoff, g.sn, c16, hi);
    stage_rows(vs, vx, c16, hi);
    write_k_rows(Kp + pblk, kx, bt.n, c16, hi);
    __syncthreads();
    write_vt_groups(Vt + pblk, vs, bt.n);
}

// The layer's prologue for bf16, d = 128, one workgroup per (block,
// batch*head): the float64 means of Q and K over the block's tokens (the
// pooling of the routing front end) and the copies of pack_kv_kernel, from a
// single read of each tensor.  The means are summed in the order of the
// routing's own pooling (thread (c, g) adds rows g, g + 16, ... of 16-byte
// chunk c, then the 16 row groups in order), so they are bit for bit the
// same.
__device__ __forceinline__ void add_rows_f64(double *acc, const u32x4 *x, int hi, int n) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        if (hi + 16 * m < n) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] += (double)__uint_as_float(x[m][i] << 16);
                acc[2 * i + 1] += (double)__uint_as_float(x[m][i] & 0xffff0000u);
            }
        }
    }
}

__device__ __forceinline__ void reduce_mean(double *red, const double *acc, int c16, int hi, int n, double *out) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[hi * 128 + c16 * 8 + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < 128) {
        double sum = 0.0;
        for (int q = 0; q < 16; ++q) sum += red[q * 128 + threadIdx.x];
        out[threadIdx.x] = sum / (double)n;
    }
    __syncthreads();
}

// 32 KB of LDS and at most 128 registers, so that four workgroups share a
// compute unit: the V^T staging area holds the two reductions' partial sums
// first (16 KB), then V.
__global__ __launch_bounds__(256, 4) void prologue_kernel(Geo g, const uint16_t *Q, const uint16_t *K,
                                                          const uint16_t *V, double *qbar, double *kbar, uint16_t *Kp,
                                                          uint16_t *Vt) {
    __shared__ __attribute__((aligned(16))) uint16_t vs[kMaxSlots * 128];
    double *red = reinterpret_cast<double *>(vs);
    const int j = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
    const BlockTokens bt = block_tokens(g, j);
    const int n = bt.n;
    const int64_t hoff = (int64_t)(bh / g.H) * g.sb + (int64_t)(bh % g.H) * g.sh;
    const int64_t pblk = ((int64_t)bh * g.Nb + j) * kMaxSlots * 128;
    const int c16 = tid & 15, hi = tid >> 4;
    u32x4 qx[8], kx[8], vx[8];
    load_rows(qx, Q, bt, hoff, g.sn, c16, hi);
    load_rows(kx, K, bt, hoff, g.sn, c16, hi);
    load_rows(vx, V, bt, hoff, g.sn, c16, hi);
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    add_rows_f64(acc, qx, hi, n);
    reduce_mean(red, acc, c16, hi, n, qbar + ((int64_t)bh * g.Nb + j) * 128);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    add_rows_f64(acc, kx, hi, n);
    reduce_mean(red, acc, c16, hi, n, kbar + ((int64_t)bh * g.Nb + j) * 128);   // ends with a barrier: red is free
    stage_rows(vs, vx, c16, hi);
    write_k_rows(Kp + pblk, kx, n, c16, hi);
    __syncthreads();
    write_vt_groups(Vt + pblk, vs, n);
}

// Float32 path: one thread per query slot, K/V tiles of one key block in LDS.
template <int D>
__global__ __launch_bounds__(kMaxSlots, 1) void attn_f32_kernel(AttnArgs a) {
    constexpr int D4 = D / 4;
    __shared__ __attribute__((aligned(16))) float Ks[kMaxSlots * D];
    __shared__ __attribute__((aligned(16))) float Vs[kMaxSlots * D];
    __shared__ int s_item;
    const int tid = threadIdx.x;
    const Geo &g = a.g;
    const float c = a.scale_log2;
    const uint64_t t0 = wall_clock64();
    uint32_t n_done = 0, blocks_done = 0;
    const int n_items = a.hdr->info.n_items;
    const float *Q = static_cast<const float *>(a.q);
    const float *K = static_cast<const float *>(a.k);
    const float *V = static_cast<const float *>(a.v);
    float *O = static_cast<float *>(a.o);

    for (;;) {
        const int it = next_item(a.hdr, &s_item);
        if (it >= n_items) break;
        const WorkItem wi = a.items[it];
        const int bh = wi.row / g.Nb, i = wi.row - (wi.row / g.Nb) * g.Nb;
        const int64_t boff = (int64_t)(bh / g.H) * g.sb + (int64_t)(bh % g.H) * g.sh;
        const int n_i = a.bsize[i];
        const bool qvalid = tid < n_i;
        const int qtok = a.tok[i * kMaxSlots + tid];
        float qv[D], ov[D];
#pragma unroll
        for (int e = 0; e < D; ++e) {
            qv[e] = qvalid ? Q[boff + (int64_t)qtok * g.sn + e] : 0.f;
            ov[e] = 0.f;
        }
        float m = -INFINITY, l = 0.f;
        const int nkb = wi.kb_end - wi.kb_begin;
        for (int jj = 0; jj < nkb; ++jj) {
            const int j = a.col_idx[wi.kb_begin + jj];
            const int n_j = a.bsize[j];
            __syncthreads();
            for (int e = tid; e < n_j * D4; e += kMaxSlots) {
                const int slot = e / D4, c4 = e - (e / D4) * D4;
                const int t = a.tok[j * kMaxSlots + slot];
                reinterpret_cast<float4 *>(Ks)[e] = reinterpret_cast<const float4 *>(K + boff + (int64_t)t * g.sn)[c4];
                reinterpret_cast<float4 *>(Vs)[e] = reinterpret_cast<const float4 *>(V + boff + (int64_t)t * g.sn)[c4];
            }
            __syncthreads();
            for (int key = 0; key < n_j; ++key) {
                float s = 0.f;
#pragma unroll
                for (int e = 0; e < D; ++e) s = fmaf(qv[e], Ks[key * D + e], s);
                s *= c;
                if (s > m) {
                    const float al = exp2f(m - s);
                    l *= al;
#pragma unroll
                    for (int e = 0; e < D; ++e) ov[e] *= al;
                    m = s;
                }
                const float p = exp2f(s - m);
                l += p;
#pragma unroll
                for (int e = 0; e < D; ++e) ov[e] = fmaf(p, Vs[key * D + e], ov[e]);
            }
        }
        if (qvalid) {
            if (wi.part < 0) {
                const float inv = (l > 0.f) ? 1.f / l : 0.f;
                float *orow = O + boff + (int64_t)qtok * g.sn;
#pragma unroll
                for (int e = 0; e < D; e += 4)
                    *reinterpret_cast<float4 *>(orow + e) = make_float4(ov[e] * inv, ov[e + 1] * inv, ov[e + 2] * inv, ov[e + 3] * inv);
            } else {
                float *po = a.part_o + ((int64_t)wi.part * kMaxSlots + tid) * D;
#pragma unroll
                for (int e = 0; e < D; e += 4) *reinterpret_cast<float4 *>(po + e) = make_float4(ov[e], ov[e + 1], ov[e + 2], ov[e + 3]);
                float *pm = a.part_ml + ((int64_t)wi.part * kMaxSlots + tid) * 2;
                pm[0] = m;
                pm[1] = l;
            }
        }
        ++n_done;
        blocks_done += nkb;
    }
    write_stats(a, t0, n_done, blocks_done);
}

// ------------------------------------------------------------- row pairs
constexpr int kPairThreads = 1024;   // two blocks per thread: Nb <= 2048

// Inclusive scan of v[0 .. 2 * kPairThreads) under a commutative op with
// identity `id`, entries 2t and 2t + 1 on thread t; tmp: kPairThreads ints.
template <typename Op>
__device__ inline void scan2(int *v, int *tmp, Op op, int id) {
    const int t = threadIdx.x;
    const int a = v[2 * t], b = op(a, v[2 * t + 1]);
    tmp[t] = b;
    __syncthreads();
    for (int off = 1; off < kPairThreads; off <<= 1) {
        const int y = (t >= off) ? tmp[t - off] : id;
        __syncthreads();
        tmp[t] = op(tmp[t], y);
        __syncthreads();
    }
    const int before = (t > 0) ? tmp[t - 1] : id;
    __syncthreads();
    v[2 * t] = op(before, a);
    v[2 * t + 1] = op(before, b);
    __syncthreads();
}

// Single workgroup.  In every run of consecutive query blocks of at most
// kPairTokens tokens, blocks (s, s + 1), (s + 2, s + 3), ... from the run's
// first block s are paired (an odd run leaves its last block alone), up to
// `cap` pairs.  Writes role, first and n_pairs (see RowPairs).
__global__ __launch_bounds__(kPairThreads) void pair_table_kernel(int Nb, int cap, const int32_t *bsize,
                                                                  int32_t *role, int32_t *first, int32_t *n_pairs) {
    __shared__ int small[2 * kPairThreads];
    __shared__ int start[2 * kPairThreads];
    __shared__ int rank[2 * kPairThreads];
    __shared__ int tmp[kPairThreads];
    const int t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int e = 2 * t + k;
        small[e] = (e < Nb && bsize[e] <= kPairTokens) ? 1 : 0;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int e = 2 * t + k;
        start[e] = (small[e] && (e == 0 || !small[e - 1])) ? e : -1;
    }
    __syncthreads();
    // for a small block: the first block of its run (the last run start at or before it)
    scan2(start, tmp, [](int x, int y) { return max(x, y); }, -1);
    auto leads = [&](int e) {
        return e >= 0 && e + 1 < Nb && small[e] && small[e + 1] && ((e - start[e]) & 1) == 0;
    };
#pragma unroll
    for (int k = 0; k < 2; ++k) rank[2 * t + k] = leads(2 * t + k) ? 1 : 0;
    __syncthreads();
    scan2(rank, tmp, [](int x, int y) { return x + y; }, 0);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int e = 2 * t + k;
        if (e >= Nb) continue;
        const int p = rank[e] - 1;   // pair index of e if it leads, else of the last leader before it
        int rl = -1;
        if (leads(e)) {
            if (p < cap) {
                rl = p;
                first[p] = e;
            }
        } else if (leads(e - 1) && p < cap) {
            rl = -2;
        }
        role[e] = rl;
    }
    if (t == 0) *n_pairs = min(rank[2 * kPairThreads - 1], cap);
}

// One wave per (pair, batch*head): the ascending union of the two rows' kept
// blocks with their member bits, through one bitmap per row in LDS (64
// words: Nb <= 2048); lane l emits the blocks of word l.
__global__ __launch_bounds__(64) void pair_union_kernel(int Nb, int max_pairs, const int32_t *row_ptr,
                                                        const int32_t *col_idx, const int32_t *first,
                                                        const int32_t *n_pairs, int32_t *ucol, int32_t *ulen) {
    __shared__ uint32_t bm[2][64];
    const int p = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
    if (p >= *n_pairs) return;
    bm[0][lane] = 0u;
    bm[1][lane] = 0u;
    __syncthreads();
    const int r0 = bh * Nb + first[p];
    for (int m = 0; m < 2; ++m) {
        const int b0 = row_ptr[r0 + m], b1 = row_ptr[r0 + m + 1];
        for (int e = b0 + lane; e < b1; e += 64) {
            const int j = col_idx[e];
            atomicOr(&bm[m][j >> 5], 1u << (j & 31));
        }
    }
    __syncthreads();
    const uint32_t a = bm[0][lane], b = bm[1][lane];
    uint32_t u = a | b;
    const int c = __popc(u);
    int incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
    }
    const int slot = bh * max_pairs + p;
    int32_t *dst = ucol + (int64_t)slot * Nb;
    int o = incl - c;
    while (u) {
        const int bit = __ffs(u) - 1;
        u &= u - 1;
        dst[o++] = (lane * 32 + bit) | (int)(((a >> bit) & 1u) << 16) | (int)(((b >> bit) & 1u) << 17);
    }
    if (lane == 63) ulen[slot] = incl;
}

// ------------------------------------------------------------------ plan
// The plan, one workgroup per (batch, head) in two launches.  Cost of a row =
// its kept key blocks.  Chunk C: fixed, none (INT_MAX) or automatic
// max(16, ceil(total / (8 * num_ctas))), which keeps every item at most 1/8 of
// a workgroup's average share; a longer row is cut into ceil(cnt / C)
// near-equal chunks, each a work item with its own partial slot.  Heads are
// emitted densest first (by kept blocks, ties to the lower (b, h); in (b, h)
// order when there are more than kPlanOrderMax heads), rows of a head in
// order: the long items of dense heads start early and the short items of
// sparse heads fill the end of the queues, and concurrently running
// workgroups read the same head's keys and values.  With row pairs (role !=
// null), a pair whose union list holds at most C blocks is one item over that
// list, emitted at the place of its first block and never split; a longer
// pair runs as two rows, so that they can still be split.  If the items or
// partial slots of C overrun the workspace, C becomes INT_MAX (cannot happen
// for the automatic size).
//   plan_count_kernel: each head's items, partial slots, split rows and pairs,
//     for C and for INT_MAX (eight counts per head);
//   plan_emit_kernel: each head settles C from all heads' counts, finds its
//     place in the emission order and the counts of the heads before it, and
//     writes its rows' items (a workgroup scan gives each thread's offsets).
constexpr int kPlanThreads = 256;
constexpr int kPlanOrderMax = 1024;        // heads ordered by density up to this many
constexpr int kPlanMaxRows = 2048;         // query blocks per head
constexpr int kPlanMaxPairs = 1024;

__device__ inline int chunks_of(int cnt, int C) { return (cnt > C) ? (cnt + C - 1) / C : 1; }

__device__ inline int plan_chunk(int chunk_mode, int64_t total, int num_ctas) {
    if (chunk_mode < 0) return INT32_MAX;
    if (chunk_mode > 0) return chunk_mode;
    return (int)max((int64_t)16, (total + 8LL * num_ctas - 1) / (8LL * num_ctas));
}

// Exclusive scan of four per-thread counts over the workgroup (wave scans by
// lane shuffles, then the wave totals through LDS): x becomes the sum over the
// threads before this one, tot the sum over all.
__device__ inline void plan_scan4(int *x, int *tot, int (*wsum)[4]) {
    constexpr int NW = kPlanThreads / 64;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    int incl[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) incl[c] = x[c];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int y = __shfl_up(incl[c], off, 64);
            if (lane >= off) incl[c] += y;
        }
    __syncthreads();
    if (lane == 63)
#pragma unroll
        for (int c = 0; c < 4; ++c) wsum[w][c] = incl[c];
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        int before = 0, all = 0;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int v = wsum[i][c];
            before += (i < w) ? v : 0;
            all += v;
        }
        tot[c] = all;
        x[c] = before + incl[c] - x[c];
    }
}

// One head's plan inputs in LDS: its Nb + 1 row_ptr entries, the pair roles
// and its union lengths.
struct PlanHead {
    int rp[kPlanMaxRows + 1];
    int role[kPlanMaxRows];
    int ulen[kPlanMaxPairs];
};

__device__ inline void stage_head(PlanHead &ph, int hb, int Nb, const int32_t *row_ptr, const int32_t *role,
                                  const int32_t *ulen, int max_pairs) {
    for (int x = threadIdx.x; x <= Nb; x += kPlanThreads) ph.rp[x] = row_ptr[(int64_t)hb * Nb + x];
    if (role) {
        for (int x = threadIdx.x; x < Nb; x += kPlanThreads) ph.role[x] = role[x];
        for (int x = threadIdx.x; x < max_pairs; x += kPlanThreads) ph.ulen[x] = ulen[(int64_t)hb * max_pairs + x];
    }
    __syncthreads();
}

// Role of query block i under chunk C: -1 alone, -2 second of a pair, p >= 0
// first of pair p.
__device__ inline int plan_role(const PlanHead &ph, bool pairs, int i, int C) {
    if (!pairs) return -1;
    const int rl = ph.role[i];
    const int p = (rl >= 0) ? rl : (rl == -2 ? ph.role[i - 1] : -1);
    if (p < 0 || ph.ulen[p] > C) return -1;
    return rl;
}

// This thread's rows [i0, i1) of the head: items, partial slots, split rows, pairs.
__device__ inline void plan_count_rows(const PlanHead &ph, bool pairs, int i0, int i1, int C, int *c4) {
    int li = 0, lp = 0, ls = 0, lq = 0;
    for (int i = i0; i < i1; ++i) {
        const int rl = plan_role(ph, pairs, i, C);
        const int n = (rl < 0) ? chunks_of(ph.rp[i + 1] - ph.rp[i], C) : 0;
        li += (rl >= 0) ? 1 : (rl == -1 ? n : 0);
        lq += (rl >= 0) ? 1 : 0;
        lp += (rl == -1 && n > 1) ? n : 0;
        ls += (rl == -1 && n > 1) ? 1 : 0;
    }
    c4[0] = li; c4[1] = lp; c4[2] = ls; c4[3] = lq;
}

__global__ __launch_bounds__(kPlanThreads) void plan_count_kernel(int BH, int Nb, const int32_t *row_ptr,
                                                                  int chunk_mode, int num_ctas, const int32_t *role,
                                                                  const int32_t *ulen, int max_pairs, int32_t *hc) {
    __shared__ PlanHead ph;
    __shared__ int wsum[kPlanThreads / 64][4];
    const int hb = blockIdx.x;
    stage_head(ph, hb, Nb, row_ptr, role, ulen, max_pairs);
    const int C = plan_chunk(chunk_mode, (int64_t)row_ptr[(int64_t)BH * Nb] - row_ptr[0], num_ctas);
    const int seg = (Nb + kPlanThreads - 1) / kPlanThreads;
    const int i0 = min(Nb, (int)threadIdx.x * seg), i1 = min(Nb, i0 + seg);
    int c4[4], tot[4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        plan_count_rows(ph, role != nullptr, i0, i1, k ? INT32_MAX : C, c4);
        plan_scan4(c4, tot, wsum);
        if (threadIdx.x == 0)
#pragma unroll
            for (int c = 0; c < 4; ++c) hc[(int64_t)hb * 8 + 4 * k + c] = tot[c];
    }
}

__global__ __launch_bounds__(kPlanThreads) void plan_emit_kernel(int BH, int Nb, const int32_t *row_ptr,
                                                                 int chunk_mode, int num_ctas, int cap_items,
                                                                 int cap_parts, const int32_t *role,
                                                                 const int32_t *ulen, int max_pairs,
                                                                 const int32_t *hc, PlanHeader *hdr, WorkItem *items,
                                                                 SplitRow *splits) {
    __shared__ PlanHead ph;
    __shared__ int wsum[kPlanThreads / 64][4];
    const int hb = blockIdx.x, tid = threadIdx.x;
    const int64_t total = (int64_t)row_ptr[(int64_t)BH * Nb] - row_ptr[0];
    // C for all heads, then the heads emitted before this one (their items,
    // partial slots and split rows) and the totals.
    int a4[4] = {0, 0, 0, 0};
    for (int h2 = tid; h2 < BH; h2 += kPlanThreads) {
        a4[0] += hc[(int64_t)h2 * 8 + 0];
        a4[1] += hc[(int64_t)h2 * 8 + 1];
    }
    int t4[4];
    plan_scan4(a4, t4, wsum);
    const int C0 = plan_chunk(chunk_mode, total, num_ctas);
    const bool wide = t4[0] > cap_items || t4[1] > cap_parts;     // never overrun the workspace
    const int C = wide ? INT32_MAX : C0;
    const int k = wide ? 4 : 0;
    const bool by_density = BH <= kPlanOrderMax;
    const int mine = row_ptr[(int64_t)(hb + 1) * Nb] - row_ptr[(int64_t)hb * Nb];
    int b4[4] = {0, 0, 0, 0}, all4[4] = {0, 0, 0, 0};
    for (int h2 = tid; h2 < BH; h2 += kPlanThreads) {
        bool before = h2 < hb;
        if (by_density) {
            const int t2 = row_ptr[(int64_t)(h2 + 1) * Nb] - row_ptr[(int64_t)h2 * Nb];
            before = t2 > mine || (t2 == mine && h2 < hb);
        }
        const int32_t *c = hc + (int64_t)h2 * 8 + k;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            b4[q] += before ? c[q] : 0;
            all4[q] += c[q];
        }
        all4[3] += c[3];
    }
    int s4[4], n4[4];
    plan_scan4(b4, s4, wsum);          // s4: the heads emitted before this one
    plan_scan4(all4, n4, wsum);        // n4: all heads (items, partial slots, split rows, pairs)
    stage_head(ph, hb, Nb, row_ptr, role, ulen, max_pairs);
    const bool pairs = role != nullptr;
    const int seg = (Nb + kPlanThreads - 1) / kPlanThreads;
    const int i0 = min(Nb, tid * seg), i1 = min(Nb, i0 + seg);
    int c4[4], tot[4];
    plan_count_rows(ph, pairs, i0, i1, C, c4);
    plan_scan4(c4, tot, wsum);
    int item = s4[0] + c4[0], part = s4[1] + c4[1], spl = s4[2] + c4[2];
    const int r0 = hb * Nb;
    for (int i = i0; i < i1; ++i) {
        const int r = r0 + i;
        const int rl = plan_role(ph, pairs, i, C);
        if (rl == -2) continue;
        if (rl >= 0) {
            const int slot = hb * max_pairs + rl;
            items[item++] = WorkItem{r, slot * Nb, slot * Nb + ph.ulen[rl], -2 - (i + 1)};
            continue;
        }
        const int b0 = ph.rp[i], cnt = ph.rp[i + 1] - b0;
        const int n = chunks_of(cnt, C);
        if (n == 1) {
            items[item++] = WorkItem{r, b0, b0 + cnt, -1};
        } else {
            splits[spl++] = SplitRow{r, part, n, 0};
            for (int q = 0; q < n; ++q) {
                const int sb = b0 + (int)((int64_t)cnt * q / n);
                const int e = b0 + (int)((int64_t)cnt * (q + 1) / n);
                items[item++] = WorkItem{r, sb, e, part++};
            }
        }
    }
    if (hb == 0 && tid == 0) {
        hdr->info.n_items = n4[0];
        hdr->info.chunk_blocks = C;
        hdr->info.n_split_rows = n4[2];
        hdr->info.n_partials = n4[1];
        hdr->info.total_blocks = total;
        hdr->info.num_ctas = num_ctas;
        hdr->info.n_row_pairs = n4[3];
        hdr->info.kept_pairs = 0;
        hdr->info.predicted_imbalance = 0.f;
        hdr->info.reserved = 0;
        for (int q = 0; q < 8; ++q) hdr->queue[q] = 0;
    }
}

// ----------------------------------------------------------- plan stats
// Only when the caller asks for stats.  One wave per row: n_i times the sum
// of n_j over the row's kept blocks, added into the plan header.
__global__ __launch_bounds__(256) void kept_pairs_kernel(int R, int Nb, const int32_t *row_ptr, const int32_t *col_idx,
                                                         const int32_t *bsize, PlanHeader *hdr) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= R) return;
    const int b0 = row_ptr[r], b1 = row_ptr[r + 1];
    long long s = 0;
    for (int e = b0 + lane; e < b1; e += 64) s += bsize[col_idx[e]];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (lane == 0 && s != 0)
        atomicAdd(reinterpret_cast<unsigned long long *>(&hdr->info.kept_pairs),
                  (unsigned long long)(s * bsize[r % Nb]));
}

// One wave: the items in queue order, each to the workgroup with the least
// work so far (ties to the lower index), cost = the item's key blocks; the
// loads stay in registers (kMaxPredict / 64 per lane) and each step is an
// argmin over the wave.  Writes max load / mean load.
constexpr int kMaxPredict = 1024;   // workgroups the prediction handles (16 loads per lane)
__global__ __launch_bounds__(64) void predict_kernel(int num_ctas, const WorkItem *items, PlanHeader *hdr) {
    constexpr int PER = kMaxPredict / 64;
    const int lane = threadIdx.x;
    const int n_items = hdr->info.n_items;
    float load[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) load[u] = (u * 64 + lane < num_ctas) ? 0.f : INFINITY;
    double total = 0.0;
    for (int it = 0; it < n_items; ++it) {
        const WorkItem wi = items[it];
        const float cost = (float)(wi.kb_end - wi.kb_begin);
        total += cost;
        float best = load[0];
        int bi = 0;
#pragma unroll
        for (int u = 1; u < PER; ++u) {
            const bool lt = load[u] < best;
            best = lt ? load[u] : best;
            bi = lt ? u : bi;
        }
        int widx = bi * 64 + lane;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ob = __shfl_xor(best, o, 64);
            const int ow = __shfl_xor(widx, o, 64);
            const bool take = (ob < best) || (ob == best && ow < widx);
            best = take ? ob : best;
            widx = take ? ow : widx;
        }
#pragma unroll
        for (int u = 0; u < PER; ++u)
            if (u * 64 + lane == widx) load[u] += cost;
    }
    float mx = 0.f;
#pragma unroll
    for (int u = 0; u < PER; ++u) mx = (u * 64 + lane < num_ctas) ? fmaxf(mx, load[u]) : mx;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if (lane == 0) {
        const double mean = total / num_ctas;
        hdr->info.predicted_imbalance = mean > 0.0 ? (float)(mx / mean) : 1.f;
    }
}

// --------------------------------------------------------------- combine
template <typename OutT>
__device__ inline void store4(OutT *p, float4 v);
template <>
__device__ inline void store4<float>(float *p, float4 v) { *reinterpret_cast<float4 *>(p) = v; }
template <>
__device__ inline void store4<uint16_t>(uint16_t *p, float4 v) {
    const uint32_t a = pack_bf16(v.x, v.y);
    const uint32_t b = pack_bf16(v.z, v.w);
    *reinterpret_cast<uint2 *>(p) = make_uint2(a, b);
}

// Workgroups per split row, each merging 16 of its query slots: the merge of
// one element is a short chain of dependent loads, so a row spread over
// eight workgroups finishes in two such chains per thread instead of 16.
constexpr int kCombineSlices = 8;

template <typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(Geo g, OutT *O, const int32_t *tok, const int32_t *bsize,
                                                      const PlanHeader *hdr, const SplitRow *splits,
                                                      const float *part_o, const float *part_ml) {
    const int n_split = hdr->info.n_split_rows;
    const int D4 = g.D / 4;
    constexpr int kSlotsPerSlice = kMaxSlots / kCombineSlices;
    for (int wi = blockIdx.x; wi < n_split * kCombineSlices; wi += gridDim.x) {
        const int sidx = wi / kCombineSlices, q0 = (wi % kCombineSlices) * kSlotsPerSlice;
        const SplitRow sr = splits[sidx];
        const int bh = sr.row / g.Nb, i = sr.row - (sr.row / g.Nb) * g.Nb;
        const int64_t boff = (int64_t)(bh / g.H) * g.sb + (int64_t)(bh % g.H) * g.sh;
        const int nq = min(bsize[i] - q0, kSlotsPerSlice);
        for (int e = threadIdx.x; e < nq * D4; e += 256) {
            const int q = q0 + e / D4, c4 = e - (e / D4) * D4;
            float M = -INFINITY;
            for (int p = 0; p < sr.n_parts; ++p)
                M = fmaxf(M, part_ml[((int64_t)(sr.part_begin + p) * kMaxSlots + q) * 2]);
            float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
            float den = 0.f;
            for (int p = 0; p < sr.n_parts; ++p) {
                const int64_t pq = (int64_t)(sr.part_begin + p) * kMaxSlots + q;
                const float mp = part_ml[pq * 2], lp = part_ml[pq * 2 + 1];
                const float wgt = (mp == -INFINITY) ? 0.f : exp2f(mp - M);
                const float4 ov = reinterpret_cast<const float4 *>(part_o + pq * g.D)[c4];
                num.x += wgt * ov.x; num.y += wgt * ov.y; num.z += wgt * ov.z; num.w += wgt * ov.w;
                den += wgt * lp;
            }
            const float inv = (den > 0.f) ? 1.f / den : 0.f;
            const int t = tok[i * kMaxSlots + q];
            store4<OutT>(O + boff + (int64_t)t * g.sn + 4 * c4,
                         make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv));
        }
    }
}

}  // namespace

// ---------------------------------------------------------------- launches
int attention_ctas_per_cu(const Geo &g) { return (g.dtype == FVA_BF16 && g.D == 128) ? 2 : 1; }

size_t packed_kv_bytes(const Geo &g) {
    return (g.dtype == FVA_BF16 && g.D == 128) ? (size_t)g.BH * g.Nb * kMaxSlots * 128 * 2 : 0;
}

hipError_t launch_plan(const Geo &g, const int32_t *row_ptr, int chunk_mode, int num_ctas, int cap_items,
                       int cap_parts, const RowPairs &rp, PlanHeader *hdr, WorkItem *items, SplitRow *splits,
                       int32_t *head_counts, hipStream_t s) {
    const bool pairs = rp.max_pairs > 0;
    if (g.Nb > kPlanMaxRows || rp.max_pairs > kPlanMaxPairs || g.BH <= 0) return hipErrorInvalidValue;
    const int32_t *role = pairs ? rp.role : nullptr, *ulen = pairs ? rp.ulen : nullptr;
    hipLaunchKernelGGL(plan_count_kernel, dim3(g.BH), dim3(kPlanThreads), 0, s, g.BH, g.Nb, row_ptr, chunk_mode,
                       num_ctas, role, ulen, rp.max_pairs, head_counts);
    hipLaunchKernelGGL(plan_emit_kernel, dim3(g.BH), dim3(kPlanThreads), 0, s, g.BH, g.Nb, row_ptr, chunk_mode,
                       num_ctas, cap_items, cap_parts, role, ulen, rp.max_pairs, head_counts, hdr, items, splits);
    return hipGetLastError();
}

hipError_t launch_plan_stats(const Geo &g, const int32_t *row_ptr, const int32_t *col_idx, const int32_t *bsize,
                             int num_ctas, const WorkItem *items, PlanHeader *hdr, hipStream_t s) {
    const int R = g.BH * g.Nb;
    if (R > 0)
        hipLaunchKernelGGL(kept_pairs_kernel, dim3((R + 3) / 4), dim3(256), 0, s, R, g.Nb, row_ptr, col_idx, bsize,
                           hdr);
    if (num_ctas <= kMaxPredict) hipLaunchKernelGGL(predict_kernel, dim3(1), dim3(64), 0, s, num_ctas, items, hdr);
    return hipGetLastError();
}

hipError_t launch_row_pairs(const Geo &g, const int32_t *bsize, const int32_t *row_ptr, const int32_t *col_idx,
                           const RowPairs &rp, hipStream_t s) {
    if (rp.max_pairs <= 0) return hipSuccess;
    hipLaunchKernelGGL(pair_table_kernel, dim3(1), dim3(kPairThreads), 0, s, g.Nb, rp.max_pairs, bsize, rp.role,
                       rp.first, rp.n_pairs);
    hipLaunchKernelGGL(pair_union_kernel, dim3(rp.max_pairs, g.BH), dim3(64), 0, s, g.Nb, rp.max_pairs, row_ptr,
                       col_idx, rp.first, rp.n_pairs, rp.ucol, rp.ulen);
    return hipGetLastError();
}

bool uses_packed_kv(const Geo &g) { return g.dtype == FVA_BF16 && g.D == 128; }

hipError_t launch_pack_kv(const Geo &g, const void *k, const void *v, uint16_t *kp, uint16_t *vt, hipStream_t s) {
    if (!uses_packed_kv(g) || g.BH == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_kv_kernel, dim3(g.Nb, g.BH), dim3(256), 0, s, g, (const uint16_t *)k,
                       (const uint16_t *)v, kp, vt);
    return hipGetLastError();
}

hipError_t launch_attention(const Geo &g, const void *q, const void *k, const void *v, void *o,
                            const int32_t *row_ptr, const int32_t *col_idx, const int32_t *ucol, const int32_t *tok,
                            const int32_t *bsize,
                            PlanHeader *hdr,
                            const WorkItem *items, float *part_o, float *part_ml, fva_cta_stat *stats,
                            uint16_t *kp, uint16_t *vt, int num_ctas, hipEvent_t ev0, hipEvent_t ev1,
                            hipStream_t s) {
    AttnArgs a;
    a.g = g;
    a.q = q; a.k = k; a.v = v; a.o = o;
    a.row_ptr = row_ptr; a.col_idx = col_idx; a.ucol = ucol; a.tok = tok; a.bsize = bsize;
    a.hdr = hdr; a.items = items;
    a.part_o = part_o; a.part_ml = part_ml;
    a.stats = stats;
    a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)g.D));
    const bool d128 = uses_packed_kv(g);
    if (ev0) {
        hipError_t e = hipEventRecord(ev0, s);
        if (e != hipSuccess) return e;
    }
    if (d128)
        hipLaunchKernelGGL(attn_bf16_d128_kernel, dim3(num_ctas), dim3(256), 0, s, a, kp, vt);
    else if (g.dtype == FVA_BF16)
        hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(num_ctas), dim3(256), 0, s, a);
    else if (g.D == 128)
        hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(num_ctas), dim3(kMaxSlots), 0, s, a);
    else
        hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(num_ctas), dim3(kMaxSlots), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev1) e = hipEventRecord(ev1, s);
    return e;
}

hipError_t launch_prologue(const Geo &g, const void *q, const void *k, const void *v, double *qbar, double *kbar,
                           uint16_t *kp, uint16_t *vt, hipStream_t s) {
    if (!uses_packed_kv(g) || g.BH == 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(prologue_kernel, dim3(g.Nb, g.BH), dim3(256), 0, s, g, (const uint16_t *)q,
                       (const uint16_t *)k, (const uint16_t *)v, qbar, kbar, kp, vt);
    return hipGetLastError();
}

hipError_t launch_combine(const Geo &g, void *o, const int32_t *tok, const int32_t *bsize, const PlanHeader *hdr,
                          const SplitRow *splits, const float *part_o, const float *part_ml, int cap_splits,
                          hipStream_t s) {
    if (cap_splits <= 0) return hipSuccess;
    const int64_t want = (int64_t)cap_splits * kCombineSlices;
    const int grid = want < 2048 ? (int)want : 2048;
    if (g.dtype == FVA_BF16)
        hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3(grid), dim3(256), 0, s, g, (uint16_t *)o, tok, bsize, hdr,
                           splits, part_o, part_ml);
    else
        hipLaunchKernelGGL(combine_kernel<float>, dim3(grid), dim3(256), 0, s, g, (float *)o, tok, bsize, hdr,
                           splits, part_o, part_ml);
    return hipGetLastError();
}

}  // namespace fva
