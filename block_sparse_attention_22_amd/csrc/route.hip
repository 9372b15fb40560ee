// Sparse-routing front end of FVAttn on gfx950: blocks that follow the
// video's 3D layout, a Top-p cut per query block with a minimum block count,
// and per-head augmentation (FVAttn abstract; paperlayer.ai summary,
// section 3 "FVAttn Design": Sparse-routing frontend and Slack-Aware Sparse
// Augmentation).
//
// Kernels, in launch order:
//   pool         mean of Q / K over each block's tokens, float64
//   scores       s_ij = qbar_i . kbar_j / sqrt(d), float64 tiled GEMM
//   row_select   one wave per query block: softmax, register bitonic sort by
//                (mass desc, index asc), prefix sums, Top-p cut, Top-k floor
//   augment      per head: base total and budget, then the not-yet-kept
//                blocks with the largest mass (ties to lower (i, j)) found by
//                a radix search over the sorted row tails
//   csr          per row: its offset, and ascending col_idx from a bitmask
// All routing arithmetic is float64 so the lists are deterministic and match
// an independent float64 evaluation except at cumulative masses within
// rounding of p.
#include <float.h>
#include <math.h>

#include "common.h"

namespace fva {

namespace {

__device__ inline double bits_to_double(uint64_t b) { return __longlong_as_double((long long)b); }
__device__ inline uint64_t double_bits(double x) { return (uint64_t)__double_as_longlong(x); }

template <typename T>
__device__ inline T wave_sum(T x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

__device__ inline double wave_max(double x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o, 64));
    return x;
}

__device__ inline int wave_min(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o, 64));
    return x;
}

// Block reductions for blockDim.x = NT (multiple of 64).  `red` holds NT/64
// entries; the result is returned to every thread.
template <int NT, typename T, typename Op>
__device__ inline T block_reduce(T x, T *red, Op op) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = op(x, __shfl_xor(x, o, 64));
    __syncthreads();
    if (lane == 0) red[w] = x;
    __syncthreads();
    T r = red[0];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) r = op(r, red[i]);
    return r;
}

// Exclusive block scan (sum) for blockDim.x = NT; `tmp` holds NT entries.
template <int NT, typename T>
__device__ inline T block_exclusive_scan(T x, T *tmp, T *total) {
    const int t = threadIdx.x;
    __syncthreads();
    tmp[t] = x;
    __syncthreads();
    for (int off = 1; off < NT; off <<= 1) {
        T y = (t >= off) ? tmp[t - off] : T(0);
        __syncthreads();
        tmp[t] += y;
        __syncthreads();
    }
    T incl = tmp[t];
    *total = tmp[NT - 1];
    return incl - x;
}

// ------------------------------------------------------------ slot table
// Used by the attention call (query loads and output stores).
// tok[b*128 + r] = token index of slot r of block b (BlockTokens: a tile's
// existing tokens in (t, y, x) raster order, or the block's run of the token
// order); slots at or past bsize[b] repeat the block's first token so that
// loads never need a guard (their scores are masked and their values
// multiplied by zero probability).
__global__ __launch_bounds__(kMaxSlots) void slot_table_kernel(Geo g, int32_t *tok, int32_t *bsize) {
    const int b = blockIdx.x, r = threadIdx.x;
    const BlockTokens bt = block_tokens(g, b);
    tok[b * kMaxSlots + r] = bt.token(r);
    if (r == 0) bsize[b] = bt.n;
}

// ------------------------------------------------------------------ pool
__device__ inline void load8(const uint16_t *p, float *f) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ inline void load8(const float *p, float *f) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// One workgroup per (block, batch*head); out[(bh*Nb + b)*D + c] = mean.
// Token indices come from the block geometry (or the token order), so every
// load is independent.
template <typename T>
__global__ __launch_bounds__(256) void pool_kernel(Geo g, const T *x, double *out) {
    __shared__ double red[256 * 8];
    const int b = blockIdx.x, bh = blockIdx.y;
    const int CH = g.D / 8, G = 256 / CH;
    const int c = threadIdx.x % CH, grp = threadIdx.x / CH;
    const T *base = x + (int64_t)(bh / g.H) * g.sb + (int64_t)(bh % g.H) * g.sh + c * 8;
    const BlockTokens bt = block_tokens(g, b);
    const int n = bt.n;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // rows grp, grp + G, ... below n (G >= 16, so at most kMaxSlots / 16 of
    // them): all loads first, then the sums in row order; rows past n load
    // the block's first token and add nothing
    constexpr int kRowsPerThread = kMaxSlots / 16;
    float f[kRowsPerThread][8];
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
        const int r = grp + u * G;
        load8(base + (int64_t)bt.token(r < n ? r : 0) * g.sn, f[u]);
    }
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
        if (grp + u * G < n) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += (double)f[u][e];
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[grp * g.D + c * 8 + e] = acc[e];
    __syncthreads();
    for (int dd = threadIdx.x; dd < g.D; dd += 256) {
        double s = 0.0;
        for (int q = 0; q < G; ++q) s += red[q * g.D + dd];
        out[((int64_t)bh * g.Nb + b) * g.D + dd] = s / (double)n;
    }
}

// ---------------------------------------------------------------- scores
// 64x64 output tile per workgroup, S[bh][i][j] = (qbar_i . kbar_j) / sqrt(D),
// on the fp64 matrix cores: each wave owns a 32x32 quarter as 2x2 tiles of
// v_mfma_f64_16x16x4f64 (A row i = lane%16, k = lane/16; B likewise; result
// register r of a lane is row lane/16 + 4r, column lane%16), fed from LDS in
// chunks of 16 along d.  Small chunks (17 KB of LDS) and at most ~100
// registers let five workgroups share a compute unit, which measured faster
// (136 -> 113 us at 720p) than chunks of 32 at three workgroups.
typedef __attribute__((ext_vector_type(4))) double f64x4;

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void scores_kernel(Geo g, const double *qbar,
                                                                                             const double *kbar,
                                                                                             double *S) {
    __shared__ double qs[64][17];
    __shared__ double ks[64][17];
    const int j0 = blockIdx.x * 64, i0 = blockIdx.y * 64, bh = blockIdx.z;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wy = w >> 1, wx = w & 1;
    const int l16 = lane & 15, kq = lane >> 4;
    const int Nb = g.Nb;
    const double *qb = qbar + (int64_t)bh * Nb * g.D;
    const double *kb = kbar + (int64_t)bh * Nb * g.D;
    f64x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
    // chunk d0 of both tiles: element e = threadIdx.x + 256 m is row e / 16,
    // column e % 16; the next chunk is loaded into registers while the
    // current one is multiplied
    double qr[4], kr[4];
    auto load_chunk = [&](int d0) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = threadIdx.x + 256 * m, r = e >> 4, cc = e & 15;
            qr[m] = (i0 + r < Nb) ? qb[(int64_t)(i0 + r) * g.D + d0 + cc] : 0.0;
            kr[m] = (j0 + r < Nb) ? kb[(int64_t)(j0 + r) * g.D + d0 + cc] : 0.0;
        }
    };
    load_chunk(0);
    for (int d0 = 0; d0 < g.D; d0 += 16) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = threadIdx.x + 256 * m, r = e >> 4, cc = e & 15;
            qs[r][cc] = qr[m];
            ks[r][cc] = kr[m];
        }
        __syncthreads();
        if (d0 + 16 < g.D) load_chunk(d0 + 16);
#pragma unroll
        for (int kk = 0; kk < 16; kk += 4) {
            double av[2], bv[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) av[a] = qs[32 * wy + 16 * a + l16][kk + kq];
#pragma unroll
            for (int b = 0; b < 2; ++b) bv[b] = ks[32 * wx + 16 * b + l16][kk + kq];
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
        }
        __syncthreads();
    }
    const double rsq = 1.0 / sqrt((double)g.D);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int j = j0 + 32 * wx + 16 * b + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = i0 + 32 * wy + 16 * a + kq + 4 * r;
                if (i < Nb && j < Nb) S[((int64_t)bh * Nb + i) * Nb + j] = acc[a][b][r] * rsq;
            }
        }
}

// ------------------------------------------------------------ row_select
// One wave per (query block, batch*head) row, four rows per workgroup.  The
// row (padded to a power of two NKP = 64*E with mass +0 and indices >= Nk,
// which therefore sort after every real entry) lives in registers, E entries
// per lane, entry e = lane*E + r.  A bitonic network orders it by (mass desc,
// index asc): strides below E exchange registers inside a lane, larger
// strides exchange with lane ^ (stride/E).  The first launch sorts one
// 64-bit integer key per entry (a truncated mass above the index, built in
// row_select_kernel) and checks the result against the exact masses; a row
// that fails the check is marked (base = -1) and left to a second launch
// (EXACT) that sorts only such rows on (mass, index) pairs; two launches
// keep one network per kernel.  Writes the sorted masses (in place), the
// matching key-block order and the Top-p + floor count.
__device__ inline bool before(double pa, int ia, double pb, int ib) {
    return (pa > pb) | ((pa == pb) & (ia < ib));     // bitwise: no short-circuit branch
}

constexpr int kRowsPerGroup = 4;

// The 32-bit word of lane ^ LM (LM a power of two below 64): quad
// permutations (DPP) for 1 and 2, the bit-mode lane swizzle for 4 to 16,
// an LDS permute for 32.
template <int LM>
__device__ __forceinline__ int xor_lane(int x) {
    if constexpr (LM == 1) return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    else if constexpr (LM == 2) return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    else if constexpr (LM < 32) return __builtin_amdgcn_ds_swizzle(x, (LM << 10) | 0x1F);  // and 31, xor LM
    else return __shfl_xor(x, 32, 64);
}

template <int LM>
__device__ __forceinline__ double xor_lane_d(double x) {
    const int lo = xor_lane<LM>(__double2loint(x)), hi = xor_lane<LM>(__double2hiint(x));
    return __hiloint2double(hi, lo);
}

// One bitonic stage whose partner entries live in lane ^ LM (same register).
// up: the direction of this lane's entries (the same for all of them, since
// the merge width k of a cross-lane stage is at least 2E).
template <int LM, int E>
__device__ __forceinline__ void cross_stage(double *v, int *id, int lane, bool up) {
    const bool flip = ((lane & LM) == 0) != up;
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const double ov = xor_lane_d<LM>(v[r]);
        const int oi = xor_lane<LM>(id[r]);
        const bool take = before(ov, oi, v[r], id[r]) != flip;
        v[r] = take ? ov : v[r];
        id[r] = take ? oi : id[r];
    }
}

// Compare-exchange of entries r and r + j of this lane, ascending (mass
// desc, index asc) when up.
__device__ __forceinline__ void lane_cx(double *v, int *id, int r, int j, bool up) {
    const double va = v[r], vb = v[r + j];
    const int ia = id[r], ib = id[r + j];
    const bool sw = before(vb, ib, va, ia) == up;
    v[r] = sw ? vb : va;
    v[r + j] = sw ? va : vb;
    id[r] = sw ? ib : ia;
    id[r + j] = sw ? ia : ib;
}

// The bitonic network over the whole row (see row_select_kernel).  Entry
// e = e0 + r runs in direction up = ((e & k) == 0) in the merge of width k.
// For k < E that is (r & k) == 0, a constant of the unrolled loops; for
// k >= E it is (e0 & k) == 0, the same for all of a lane's entries.
template <int E>
__device__ __forceinline__ void bitonic_row(double *v, int *id, int lane, int e0) {
    constexpr int NKP = 64 * E;
    // Exchanges are written as selects so that they compile to v_cndmask
    // rather than divergent branches.
#pragma unroll
    for (int k = 2; k < E; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j >= 1; j >>= 1)
#pragma unroll
            for (int r = 0; r < E; ++r)
                if (!(r & j)) lane_cx(v, id, r, j, (r & k) == 0);
    for (int k = E; k <= NKP; k <<= 1) {
        const bool up = (e0 & k) == 0;
        for (int j = k >> 1; j >= E; j >>= 1) {
            switch (j / E) {      // wave-uniform
                case 1: cross_stage<1, E>(v, id, lane, up); break;
                case 2: cross_stage<2, E>(v, id, lane, up); break;
                case 4: cross_stage<4, E>(v, id, lane, up); break;
                case 8: cross_stage<8, E>(v, id, lane, up); break;
                case 16: cross_stage<16, E>(v, id, lane, up); break;
                default: cross_stage<32, E>(v, id, lane, up); break;
            }
        }
#pragma unroll
        for (int j = E / 2; j >= 1; j >>= 1)
#pragma unroll
            for (int r = 0; r < E; ++r)
                if (!(r & j)) lane_cx(v, id, r, j, up);
    }
}

// The same network on one 64-bit key per entry, descending.
template <int LM>
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t x) {
    const uint32_t lo = (uint32_t)xor_lane<LM>((int)(uint32_t)x), hi = (uint32_t)xor_lane<LM>((int)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

template <int LM, int E>
__device__ __forceinline__ void cross_stage_key(uint64_t *key, int lane, bool up) {
    const bool flip = ((lane & LM) == 0) != up;
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const uint64_t ok = xor_lane_u64<LM>(key[r]);
        key[r] = ((ok > key[r]) != flip) ? ok : key[r];
    }
}

// Descending compare-exchange of two keys read as doubles: a gets the larger,
// b the smaller.  Keys are bit patterns of finite doubles >= 0 (fp64
// denormals are kept), so the double order is the key order; a lane that
// sorts ascending flips the sign bit of its keys first, which reverses the
// order.  The instructions are written out because the library maximum
// first canonicalises operands that it cannot prove are not NaN.
__device__ __forceinline__ void key_maxmin(uint64_t &a, uint64_t &b) {
    const double x = __longlong_as_double((long long)a), y = __longlong_as_double((long long)b);
    double mx, mn;
    asm("v_max_f64 %0, %1, %2" : "=v"(mx) : "v"(x), "v"(y));
    asm("v_min_f64 %0, %1, %2" : "=v"(mn) : "v"(x), "v"(y));
    a = (uint64_t)__double_as_longlong(mx);
    b = (uint64_t)__double_as_longlong(mn);
}

// The same exchange as a 64-bit compare and selects, in direction `desc`.
__device__ __forceinline__ void key_cx(uint64_t &a, uint64_t &b, bool desc) {
    const uint64_t x = a, y = b;
    const bool sw = (y > x) == desc;
    a = sw ? y : x;
    b = sw ? x : y;
}

// Inside a lane the exchanges are fp64 max/min at 32 slots per lane, and
// compares with selects below that: each form measured faster where it is
// used (1080p and 720p rows).
template <int E>
__device__ __forceinline__ void bitonic_keys(uint64_t *key, int lane, int e0) {
    constexpr int NKP = 64 * E;
    constexpr bool kMaxMin = E >= 32;
#pragma unroll
    for (int k = 2; k < E; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j >= 1; j >>= 1)
#pragma unroll
            for (int r = 0; r < E; ++r)
                if (!(r & j)) {
                    if (!kMaxMin) key_cx(key[r], key[r + j], (r & k) == 0);
                    else if ((r & k) == 0) key_maxmin(key[r], key[r + j]);
                    else key_maxmin(key[r + j], key[r]);
                }
    for (int k = E; k <= NKP; k <<= 1) {
        const bool up = (e0 & k) == 0;
        for (int j = k >> 1; j >= E; j >>= 1) {
            switch (j / E) {      // wave-uniform
                case 1: cross_stage_key<1, E>(key, lane, up); break;
                case 2: cross_stage_key<2, E>(key, lane, up); break;
                case 4: cross_stage_key<4, E>(key, lane, up); break;
                case 8: cross_stage_key<8, E>(key, lane, up); break;
                case 16: cross_stage_key<16, E>(key, lane, up); break;
                default: cross_stage_key<32, E>(key, lane, up); break;
            }
        }
        if constexpr (kMaxMin) {
            const uint64_t sgn = up ? 0 : (1ull << 63);
#pragma unroll
            for (int r = 0; r < E; ++r) key[r] ^= sgn;
#pragma unroll
            for (int j = E / 2; j >= 1; j >>= 1)
#pragma unroll
                for (int r = 0; r < E; ++r)
                    if (!(r & j)) key_maxmin(key[r], key[r + j]);
#pragma unroll
            for (int r = 0; r < E; ++r) key[r] ^= sgn;
        } else {
#pragma unroll
            for (int j = E / 2; j >= 1; j >>= 1)
#pragma unroll
                for (int r = 0; r < E; ++r)
                    if (!(r & j)) key_cx(key[r], key[r + j], up);
        }
    }
}

constexpr int kIdxMask = 2047;     // index field of the sort key: rows of up to 2,048 slots

// The first launch asks for five waves per SIMD at up to 16 slots per lane
// and three at 32: each costs a few spilled registers and measured faster
// than fewer waves.
template <int E, bool EXACT>
__global__ __launch_bounds__(64 * kRowsPerGroup) __attribute__((amdgpu_waves_per_eu(EXACT ? 1 : (E >= 32 ? 3 : 5)))) void row_select_kernel(Geo g, double *SP, int32_t *order,
                                                                        int32_t *base, double p, int kmin) {
    static_assert(64 * E <= kIdxMask + 1, "slot indices must fit the key's index field");
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerGroup + (threadIdx.x >> 6);
    if (row >= (int64_t)g.BH * g.Nb) return;
    if (EXACT && base[row] >= 0) return;      // sorted by the first launch
    const int Nk = g.Nb;
    double *srow = SP + row * Nk;
    const int e0 = lane * E;

    // Before the sort, entry r of a lane holds slot r * 64 + lane, so each
    // load is 64 consecutive scores; the network orders by (mass, slot), so
    // where an entry starts does not matter.  After the sort, entry r of a
    // lane is sorted position e0 + r.
    double v[E];
    int id[E];
    double mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const int sl = r * 64 + lane;
        const double x = srow[min(sl, Nk - 1)];
        v[r] = (sl < Nk) ? x : -INFINITY;
        id[r] = sl;
        mx = fmax(mx, v[r]);
    }
    mx = wave_max(mx);
    double sum = 0.0;
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const double ex = exp(v[r] - mx);    // exp(-inf) = 0 for the padding
        v[r] = ex;
        sum += ex;
    }
    sum = wave_sum(sum);
    int32_t *orow = order + row * Nk;
    if (!isfinite(sum)) {
        // A score that is not a finite number (from a non-finite q or k
        // token) leaves the row's masses undefined, so no prefix reaches p:
        // the row keeps every key block, in block order, and offers no
        // augmentation candidate.  The sort never sees such a row (a NaN
        // key would break the network's permutation).  Wave-uniform.
#pragma unroll
        for (int r = 0; r < E; ++r) {
            const int sl = r * 64 + lane;
            if (sl < Nk) {
                srow[sl] = 0.0;
                orow[sl] = sl;
            }
        }
        if (lane == 0) base[row] = Nk;
        return;
    }
    const double inv = 1.0 / sum;
#pragma unroll
    for (int r = 0; r < E; ++r) v[r] = (id[r] < Nk) ? v[r] * inv : 0.0;   // padding: +0, index >= Nk

    if (EXACT) {
        bitonic_row<E>(v, id, lane, e0);
    } else {
        // Key = the mass's bit pattern with its low 11 bits replaced by the
        // complemented index (entries < 64 * E <= 2048): the sign, exponent
        // and 41 mantissa bits order masses >= 0 with no underflow, so one
        // integer compare per exchange orders by (truncated mass desc, index
        // asc).  The low 11 bits of each mass wait in LDS, so the exact mass
        // is the key's high bits with them put back.  Two neighbours of the result
        // whose masses agree above the low 11 bits can still be out of exact
        // order; a row with any such pair is left to the exact launch.
        __shared__ uint16_t pl[kRowsPerGroup][64 * E];
        uint16_t *prow = pl[threadIdx.x >> 6];
        uint64_t key[E];
#pragma unroll
        for (int r = 0; r < E; ++r) {
            const uint64_t bits = (uint64_t)__double_as_longlong(v[r]);
            prow[id[r]] = (uint16_t)(bits & kIdxMask);
            key[r] = (bits & ~(uint64_t)kIdxMask) | (uint32_t)(kIdxMask - id[r]);
        }
        bitonic_keys<E>(key, lane, e0);
#pragma unroll
        for (int r = 0; r < E; ++r) {
            id[r] = kIdxMask - (int)((uint32_t)key[r] & kIdxMask);
            v[r] = __longlong_as_double((long long)((key[r] & ~(uint64_t)kIdxMask) | prow[id[r]]));
        }
        // Equal exact masses already sit in index order (the low word), so
        // the only misorder is a smaller mass before a larger one.
        bool bad = false;
#pragma unroll
        for (int r = 0; r + 1 < E; ++r) bad |= v[r] < v[r + 1];
        const double nv = __shfl_down(v[0], 1, 64);
        bad |= (lane < 63) & (v[E - 1] < nv);
        if (__any(bad)) {
            if (lane == 0) base[row] = -1;
            return;
        }
    }

    // Inclusive prefix sums in sorted order: lane totals, then a wave scan.
    double local = 0.0;
#pragma unroll
    for (int r = 0; r < E; ++r) local += (e0 + r < Nk) ? v[r] : 0.0;
    double incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double y = __shfl_up(incl, o, 64);
        incl = (lane >= o) ? incl + y : incl;
    }
    double run = incl - local;
    int first = Nk;
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const bool in = e0 + r < Nk;
        run += in ? v[r] : 0.0;
        first = (in && run >= p && first == Nk) ? e0 + r + 1 : first;
    }
    first = wave_min(first);
    const int m_p = (p >= 1.0) ? Nk : first;
    const int m = min(Nk, max(m_p, kmin));

    // A lane whose E entries all lie in the row writes them as 16-byte
    // stores when row * Nk is a multiple of 4 (the row's masses and order
    // then start 16-byte aligned; the same for the whole wave).
    bool stored = false;
    if constexpr (E >= 4) {
        if (e0 + E <= Nk && ((row * Nk) & 3) == 0) {
#pragma unroll
            for (int r = 0; r < E; r += 2)
                *reinterpret_cast<double2 *>(srow + e0 + r) = make_double2(v[r], v[r + 1]);
#pragma unroll
            for (int r = 0; r < E; r += 4)
                *reinterpret_cast<int4 *>(orow + e0 + r) = make_int4(id[r], id[r + 1], id[r + 2], id[r + 3]);
            stored = true;
        }
    }
    if (!stored) {
#pragma unroll
        for (int r = 0; r < E; ++r) {
            if (e0 + r < Nk) {
                srow[e0 + r] = v[r];
                orow[e0 + r] = id[r];
            }
        }
    }
    if (lane == 0) base[row] = m;
}

// --------------------------------------------------------------- augment
constexpr int kAugThreads = 1024;
constexpr int kAugRows = 2;            // rows per thread: Nb <= 2048

// Augmentation resolves kAugBits bits of tau's bit pattern per round, with
// one threshold per nonzero digit value.  Each threshold costs every row a
// binary search on the one compute unit that serves the head, whose memory
// pipeline is the limit: one bit per round (one search, more rounds) measured
// fastest, ahead of 2, 3 and 4 bits (720p: 73, 76, 91 and 133 us).
constexpr int kAugBits = 1;
constexpr int kAugDigits = 1 << kAugBits;

// For the thresholds t_v = x | (v << sh), v = 1 .. kAugDigits - 1: the first position
// in [lo, hi) of a descending sorted row whose bit pattern is below t_v
// (every position before it holds a value >= t_v), written to pos[v].  The
// bracket's first entry (its largest) and last entry (its smallest) settle
// every threshold outside their range without a search; the rest run as
// binary searches side by side, each halving one round of loads (only the
// open searches load).
__device__ inline void first_below_digits(const double *row, int lo, int hi, uint64_t x, int sh, int *pos) {
    int a[kAugDigits], c[kAugDigits];
    uint64_t top = 0, bot = 0;
    if (lo < hi) {
        top = double_bits(row[lo]);
        bot = double_bits(row[hi - 1]);
    }
#pragma unroll
    for (int v = 1; v < kAugDigits; ++v) {
        const uint64_t t = x | ((uint64_t)v << sh);
        if (lo >= hi || top < t) {
            a[v] = c[v] = lo;            // no entry at or above t
        } else if (bot >= t) {
            a[v] = c[v] = hi;            // every entry at or above t
        } else {
            a[v] = lo + 1;               // row[lo] >= t > row[hi - 1]
            c[v] = hi - 1;
        }
    }
    // each step leaves a bracket of n entries with at most floor(n / 2)
    for (int len = hi - lo; len > 0; len >>= 1) {
        bool any = false;
#pragma unroll
        for (int v = 1; v < kAugDigits; ++v) any |= a[v] < c[v];
        if (!any) break;
        uint64_t bits[kAugDigits];
#pragma unroll
        for (int v = 1; v < kAugDigits; ++v) bits[v] = (a[v] < c[v]) ? double_bits(row[(a[v] + c[v]) >> 1]) : 0;
        // Every open load leaves before the first compare waits: without
        // this the scheduler interleaved them with the compares in groups,
        // several dependent round trips per halving instead of one.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int v = 1; v < kAugDigits; ++v) {
            const int mid = (a[v] + c[v]) >> 1;
            const bool open = a[v] < c[v];
            const bool above = bits[v] >= (x | ((uint64_t)v << sh));
            a[v] = (open && above) ? mid + 1 : a[v];
            c[v] = (open && !above) ? mid : c[v];
        }
    }
#pragma unroll
    for (int v = 1; v < kAugDigits; ++v) pos[v] = a[v];
}

// First positions in [lo, hi) of a descending sorted row whose bit pattern
// is below t0 and below t1: two binary searches side by side, so each
// halving waits for one round of loads.
__device__ inline void first_below2(const double *row, int lo, int hi, uint64_t t0, uint64_t t1, int *p0,
                                    int *p1) {
    int a0 = lo, c0 = hi, a1 = lo, c1 = hi;
    const int last = max(lo, hi - 1);
    for (int len = hi - lo; len > 0; len >>= 1) {
        const int m0 = (a0 + c0) >> 1, m1 = (a1 + c1) >> 1;
        const uint64_t b0 = double_bits(row[min(m0, last)]);
        const uint64_t b1 = double_bits(row[min(m1, last)]);
        __builtin_amdgcn_sched_barrier(0);
        if (a0 < c0) {
            if (b0 >= t0) a0 = m0 + 1;
            else c0 = m0;
        }
        if (a1 < c1) {
            if (b1 >= t1) a1 = m1 + 1;
            else c1 = m1;
        }
    }
    *p0 = a0;
    *p1 = a1;
}

constexpr int kAugGather = 512;    // bracket size from which tau is picked directly

// One workgroup per (batch, head).  Chooses the A_h candidates (positions
// r >= base_i of each row's sorted masses) with the largest mass, ties to
// lower (i, j): a radix search over the IEEE bit pattern of the masses
// (kAugBits bits per round) narrows a per-row bracket around
// the A_h-th largest mass tau; once the brackets hold at most kAugGather
// entries together, tau is picked among them directly (rank counting in
// LDS) and each row is re-bracketed to its entries equal to tau.  Rows take
// everything above tau, and the entries equal to tau go to the lowest rows
// first (each row's equal entries are already in ascending j).
__global__ __launch_bounds__(kAugThreads) void augment_kernel(Geo g, const double *SP, const int32_t *base,
                                                              int32_t *add, int32_t *head_kept, int mode,
                                                              double frac) {
    __shared__ int cnt[kAugDigits];
    __shared__ int tmp[kAugThreads];
    __shared__ int ired[kAugThreads / 64];
    __shared__ uint64_t gat[kAugGather];
    __shared__ uint64_t tau_s;
    const int bh = blockIdx.x, tid = threadIdx.x;
    const int b = bh / g.H;
    const int Nb = g.Nb;
    const int64_t NN = (int64_t)Nb * Nb;
    // K = the head's kept blocks before augmentation (the sum of its rows'
    // base counts); for match-max also the largest K among the heads of
    // batch b, each wave summing whole heads.
    int ks = 0;
    for (int i = tid; i < Nb; i += kAugThreads) ks += base[(int64_t)bh * Nb + i];
    const int K = block_reduce<kAugThreads>(ks, ired, [](int x, int y) { return x + y; });
    int64_t Bh = K;
    if (mode == FVA_BUDGET_FRAC) {
        Bh = K + (int64_t)floor(frac * (double)K);
        if (Bh > NN) Bh = NN;
    } else if (mode == FVA_BUDGET_MATCH_MAX) {
        const int lane = tid & 63;
        int kmax = 0;
        for (int hh = tid >> 6; hh < g.H; hh += kAugThreads / 64) {
            const int32_t *hb = base + (int64_t)(b * g.H + hh) * Nb;
            int s = 0;
            for (int i = lane; i < Nb; i += 64) s += hb[i];
            kmax = max(kmax, wave_sum(s));
        }
        Bh = max(Bh, (int64_t)block_reduce<kAugThreads>(kmax, ired, [](int x, int y) { return max(x, y); }));
    }
    const int A = (int)(Bh - K);
    if (tid == 0) head_kept[bh] = (int)Bh;
    const int32_t *hbase = base + (int64_t)bh * Nb;
    int32_t *hadd = add + (int64_t)bh * Nb;
    if (A <= 0) {
        for (int i = tid; i < Nb; i += kAugThreads) hadd[i] = 0;
        return;
    }
    // Contiguous rows per thread so the tie scan runs in row order.
    const int seg = (Nb + kAugThreads - 1) / kAugThreads;
    const int r0 = min(Nb, tid * seg);
    const int nr = min(Nb, r0 + seg) - r0;
    int lo[kAugRows], hi[kAugRows], m[kAugRows];
#pragma unroll
    for (int q = 0; q < kAugRows; ++q) {
        m[q] = (q < nr) ? hbase[r0 + q] : 0;
        lo[q] = m[q];
        hi[q] = (q < nr) ? Nb : 0;
    }
    // Every candidate mass lies between the largest (the first entry of some
    // row's tail) and the smallest (the last entry of some row), so all of
    // them share the leading bits on which those two agree (bit patterns of
    // masses >= 0 order like the masses).  The search starts at the digit
    // that holds their first difference, with x = the shared bits above it:
    // the digits the rounds before it would have chosen.
    __shared__ uint64_t ured[kAugThreads / 64];
    uint64_t cmax = 0, cmin = ~0ull;
#pragma unroll
    for (int q = 0; q < kAugRows; ++q) {
        if (q < nr && m[q] < Nb) {
            const double *row = SP + ((int64_t)bh * Nb + r0 + q) * Nb;
            cmax = max(cmax, double_bits(row[m[q]]));
            cmin = min(cmin, double_bits(row[Nb - 1]));
        }
    }
    cmax = block_reduce<kAugThreads>(cmax, ured, [](uint64_t a, uint64_t c) { return max(a, c); });
    cmin = block_reduce<kAugThreads>(cmin, ured, [](uint64_t a, uint64_t c) { return min(a, c); });
    const uint64_t diff = cmax ^ cmin;
    const int sh0 = diff ? ((63 - __clzll((long long)diff)) / kAugBits) * kAugBits : 0;
    uint64_t x = (sh0 + kAugBits >= 64) ? 0 : (cmax >> (sh0 + kAugBits)) << (sh0 + kAugBits);
    bool direct = false;
    for (int sh = sh0; sh >= 0; sh -= kAugBits) {
        if (tid < kAugDigits) cnt[tid] = 0;
        __syncthreads();
        int pos[kAugRows][kAugDigits];
#pragma unroll
        for (int q = 0; q < kAugRows; ++q) {
            pos[q][0] = hi[q];
            const double *row = SP + ((int64_t)bh * Nb + (q < nr ? r0 + q : 0)) * Nb;
            // rows past nr have lo = hi = 0: no step runs and every pos is 0
            first_below_digits(row, lo[q], hi[q], x, sh, pos[q]);
        }
#pragma unroll
        for (int v = 1; v < kAugDigits; ++v) {
            int c = 0;
#pragma unroll
            for (int q = 0; q < kAugRows; ++q) c += (q < nr) ? pos[q][v] - m[q] : 0;
            c = wave_sum(c);
            if ((tid & 63) == 0) atomicAdd(&cnt[v], c);
        }
        __syncthreads();
        int vs = 0;
        for (int v = kAugDigits - 1; v >= 1; --v)
            if (cnt[v] >= A) { vs = v; break; }
        x |= (uint64_t)vs << sh;
#pragma unroll
        for (int q = 0; q < kAugRows; ++q) {
            int nlo = lo[q], nhi = hi[q];
#pragma unroll
            for (int v = 0; v < kAugDigits; ++v) {
                if (v == vs) nhi = pos[q][v];
                if (v == vs + 1) nlo = pos[q][v];
            }
            hi[q] = nhi;
            lo[q] = nlo;
        }
        __syncthreads();
        int br = 0;
#pragma unroll
        for (int q = 0; q < kAugRows; ++q) br += hi[q] - lo[q];
        if (sh > 0 && block_reduce<kAugThreads>(br, ired, [](int a, int c) { return a + c; }) <= kAugGather) {
            direct = true;
            break;
        }
    }
    if (direct) {
        // tau is the (A - above)-th largest of the bracketed entries
        int above = 0, inb = 0;
#pragma unroll
        for (int q = 0; q < kAugRows; ++q) {
            above += (q < nr) ? lo[q] - m[q] : 0;
            inb += hi[q] - lo[q];
        }
        const int rank_tau = A - block_reduce<kAugThreads>(above, ired, [](int a, int c) { return a + c; }) - 1;
        if (tid == 0) tau_s = 0;     // overwritten below by the entry of rank rank_tau
        int n_in;
        int o = block_exclusive_scan<kAugThreads>(inb, tmp, &n_in);
#pragma unroll
        for (int q = 0; q < kAugRows; ++q) {
            const double *row = SP + ((int64_t)bh * Nb + (q < nr ? r0 + q : 0)) * Nb;
            // four loads in flight per step (the last one repeated past hi)
            for (int pp = lo[q]; pp < hi[q]; pp += 4) {
                uint64_t b[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) b[u] = double_bits(row[min(pp + u, hi[q] - 1)]);
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (pp + u < hi[q]) gat[o++] = b[u];
            }
        }
        __syncthreads();
        // rank of entry e in (bits desc, e asc): unique, so one entry has rank_tau
        for (int e = tid; e < n_in; e += kAugThreads) {
            const uint64_t ve = gat[e];
            int rk = 0;
            for (int f = 0; f < n_in; ++f) {
                const uint64_t vf = gat[f];
                rk += (vf > ve) | ((vf == ve) & (f < e));
            }
            if (rk == rank_tau) tau_s = ve;
        }
        __syncthreads();
        const uint64_t tau = tau_s;
#pragma unroll
        for (int q = 0; q < kAugRows; ++q) {
            if (q < nr) {
                const double *row = SP + ((int64_t)bh * Nb + r0 + q) * Nb;
                // first entry <= tau, first entry < tau
                first_below2(row, lo[q], hi[q], tau + 1, tau, &lo[q], &hi[q]);
            }
        }
    }
    // lo..hi now brackets the entries equal to tau; before lo: above tau.
    int gt = 0, eq = 0;
#pragma unroll
    for (int q = 0; q < kAugRows; ++q)
        if (q < nr) { gt += lo[q] - m[q]; eq += hi[q] - lo[q]; }
    const int n_gt = block_reduce<kAugThreads>(gt, ired, [](int a, int c) { return a + c; });
    int rem = A - n_gt;
    int tot;
    int pre = block_exclusive_scan<kAugThreads>(eq, tmp, &tot);
#pragma unroll
    for (int q = 0; q < kAugRows; ++q) {
        if (q < nr) {
            const int e = hi[q] - lo[q];
            const int take = min(e, max(0, rem - pre));
            pre += e;
            hadd[r0 + q] = (lo[q] - m[q]) + take;
        }
    }
}

// ------------------------------------------------------------ scan / csr
// No rows: the CSR is row_ptr[0] = 0 (a kernel rather than a memset, so
// that a captured graph replays it reliably).
__global__ void empty_csr_kernel(int32_t *row_ptr) {
    if (threadIdx.x == 0) row_ptr[0] = 0;
}

// One wave per row: the row's offset (the kept blocks of the heads before
// it, which augmentation wrote, plus those of the head's rows before it),
// then a bitmask of the first count entries of the row's order, and the set
// bits emitted in ascending order.  The last row also writes row_ptr[R].
__global__ __launch_bounds__(64) void csr_kernel(Geo g, const int32_t *order, const int32_t *base,
                                                 const int32_t *add, const int32_t *head_kept, int32_t *row_ptr,
                                                 int32_t *col_idx, int32_t *base_out, uint32_t *mask) {
    __shared__ uint32_t bits[64];
    const int i = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
    const int Nk = g.Nb;
    const int64_t row = (int64_t)bh * g.Nb + i, r0 = (int64_t)bh * g.Nb;
    int before = 0;
    for (int h = lane; h < bh; h += 64) before += head_kept[h];
    for (int x = lane; x < i; x += 64) before += base[r0 + x] + add[r0 + x];
    const int start = wave_sum(before);
    const int cnt = base[row] + add[row];
    if (lane == 0) {
        row_ptr[row] = start;
        if (row + 1 == (int64_t)g.BH * g.Nb) row_ptr[row + 1] = start + cnt;
        if (base_out) base_out[row] = base[row];
    }
    const int W = (Nk + 31) / 32;
    bits[lane] = 0;
    __syncthreads();
    const int32_t *ord = order + row * Nk;
    for (int r = lane; r < cnt; r += 64) {
        const int j = ord[r];
        if ((unsigned)j < (unsigned)Nk) atomicOr(&bits[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    const uint32_t word = (lane < W) ? bits[lane] : 0u;
    const int pc = __popc(word);
    int pre = pc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(pre, o, 64);
        if (lane >= o) pre += y;
    }
    pre -= pc;
    int pos = start + pre;
    uint32_t wv = word;
    while (wv) {
        const int bit = __ffs(wv) - 1;
        col_idx[pos++] = lane * 32 + bit;
        wv &= wv - 1;
    }
    if (mask && lane < W) mask[row * W + lane] = word;
}

}  // namespace

// ---------------------------------------------------------------- launches
hipError_t launch_slot_table(const Geo &g, int32_t *tok, int32_t *bsize, hipStream_t s) {
    hipLaunchKernelGGL(slot_table_kernel, dim3(g.Nb), dim3(kMaxSlots), 0, s, g, tok, bsize);
    return hipGetLastError();
}

hipError_t launch_pool(const Geo &g, const void *x, double *out, hipStream_t s) {
    const dim3 grid(g.Nb, g.BH);
    if (g.dtype == FVA_BF16)
        hipLaunchKernelGGL(pool_kernel<uint16_t>, grid, dim3(256), 0, s, g, (const uint16_t *)x, out);
    else
        hipLaunchKernelGGL(pool_kernel<float>, grid, dim3(256), 0, s, g, (const float *)x, out);
    return hipGetLastError();
}

hipError_t launch_scores(const Geo &g, const double *qbar, const double *kbar, double *S, hipStream_t s) {
    const dim3 grid(ceil_div(g.Nb, 64), ceil_div(g.Nb, 64), g.BH);
    hipLaunchKernelGGL(scores_kernel, grid, dim3(256), 0, s, g, qbar, kbar, S);
    return hipGetLastError();
}

hipError_t launch_row_select(const Geo &g, double *SP, int32_t *order, int32_t *base, double p, int kmin,
                             hipStream_t s) {
    const int64_t R = (int64_t)g.BH * g.Nb;
    if (R == 0) return hipSuccess;
    const dim3 grid((unsigned)((R + kRowsPerGroup - 1) / kRowsPerGroup)), block(64 * kRowsPerGroup);
    // the sort on the truncated-mass keys, then the exact sort of the rows it marked
    for (int pass = 0; pass < 2; ++pass) {
        auto go = [&](auto fast, auto exact) {
            hipLaunchKernelGGL(pass == 0 ? fast : exact, grid, block, 0, s, g, SP, order, base, p, kmin);
        };
        if (g.Nb <= 64) go(row_select_kernel<1, false>, row_select_kernel<1, true>);
        else if (g.Nb <= 128) go(row_select_kernel<2, false>, row_select_kernel<2, true>);
        else if (g.Nb <= 256) go(row_select_kernel<4, false>, row_select_kernel<4, true>);
        else if (g.Nb <= 512) go(row_select_kernel<8, false>, row_select_kernel<8, true>);
        else if (g.Nb <= 1024) go(row_select_kernel<16, false>, row_select_kernel<16, true>);
        else go(row_select_kernel<32, false>, row_select_kernel<32, true>);
    }
    return hipGetLastError();
}

hipError_t launch_augment(const Geo &g, const double *SP, const int32_t *base, int32_t *add, int32_t *head_kept,
                          int mode, double frac, hipStream_t s) {
    hipLaunchKernelGGL(augment_kernel, dim3(g.BH), dim3(kAugThreads), 0, s, g, SP, base, add, head_kept, mode,
                       frac);
    return hipGetLastError();
}

hipError_t launch_csr(const Geo &g, const int32_t *order, const int32_t *base, const int32_t *add,
                      const int32_t *head_kept, int32_t *row_ptr, int32_t *col_idx, int32_t *base_out,
                      uint32_t *mask, hipStream_t s) {
    const int R = g.BH * g.Nb;
    if (R == 0) {
        // no rows: only row_ptr[0] = 0
        hipLaunchKernelGGL(empty_csr_kernel, dim3(1), dim3(64), 0, s, row_ptr);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(csr_kernel, dim3(g.Nb, g.BH), dim3(64), 0, s, g, order, base, add, head_kept, row_ptr,
                       col_idx, base_out, mask);
    return hipGetLastError();
}

}  // namespace fva
