// isg_attention: one flash-style attention over the exact and sampled columns of
// every query group.
//
// Pages: InstaGen, acceptodds.com page, abstract (exact blocks and sampled
// tokens go through one attention kernel, the sampled scores adjusted to stand
// for every skipped key); thelatestinai.com page, Figure 3(d) (one key set per
// query group, so the work is dense blocks).
//
// Structure:
//   1. columns_kernel   per query group: the column list (row of K_p/V_p, offset
//                       in score units, i.e. divided by the softmax scale, so it
//                       can start the K Q^T accumulator) = rows of the exact
//                       groups in ascending group order (offset 0), then the
//                       samples, padded to a multiple of 64 with offset -inf.
//   2. tile_table_kernel per head: (group, first row, end row) of every 128-row
//                       query tile; the launch walks tiles in an XCD-aware order
//                       so the tiles of one group share an L2.
//   3. attn_pp_kernel   (d = 128) two 128-row query tiles per work-group of 8
//                       waves, run one slot apart so that on each SIMD one wave
//                       issues matrix products while the other computes weights;
//                       K/V tiles of 64 columns are gathered row by row straight
//                       into LDS; S^T = K Q^T and O^T += V^T P^T on
//                       v_mfma_f32_32x32x16_bf16 so each lane owns one query and
//                       the weights stay in registers; V is read through the LDS
//                       transpose read.  All weights use one fixed reference per
//                       query; tiles whose row sums underflow are flagged.
//      attn_bf16_kernel 4 waves x 32 query rows, one tile per work-group, the
//                       same products: the fast kernel for d = 64, and (with a
//                       running maximum) the fallback for flagged tiles.
//      attn_f32_kernel  fp32 inputs: plain VALU version of the same loop.
#include <algorithm>
#include <cmath>

#include "isg_internal.h"

namespace {

constexpr int kTK = 64;          // columns per K/V tile
constexpr int kTQ = 128;         // query rows per bf16 work-group
constexpr int kTQ32 = 64;        // query rows per fp32 work-group
constexpr int kMaxGroups = 1024;
constexpr float kLog2e = 1.4426950408889634f;
// The fixed per-row reference sits this far (log2 units) below the
// Cauchy-Schwarz bound of the row's logits: weights are at most 2^64.
constexpr float kRefShift = 64.0f;
// 32-row query blocks per wave in the fast bf16 kernel.  Two blocks per wave
// halve the LDS fragment traffic per product but leave one wave per SIMD, whose
// single instruction stream serialises LDS latency, exponentials and products;
// measured slower on gfx950 than two single-block waves per SIMD.
constexpr int kQB = 1;
// Most work-groups of the rescaling fallback, which loops over the flagged tiles
// (64 flags per look).
constexpr int kFallbackBlocks = 512;


// ------------------------------------------------------------------ prep
__global__ __launch_bounds__(256) void columns_kernel(const int32_t *k_offsets, const int32_t *exact_groups,
                                                      const int32_t *n_exact, const int32_t *sample_idx,
                                                      const float *sample_bias, const int32_t *n_sample,
                                                      int Cq, int Ck, int m, float scale, int64_t cap, int32_t *col_row,
                                                      float *col_bias, int32_t *col_len, int32_t *col_x,
                                                      float *col_bmax)
{
    __shared__ int pref[kMaxGroups + 1];
    __shared__ int start[kMaxGroups];
    __shared__ int tmp[256];
    const int64_t gi = blockIdx.x;
    const int64_t bh = gi / Cq;
    const int32_t *ko = k_offsets + bh * (Ck + 1);
    const int ne = n_exact[gi];
    for (int e = threadIdx.x; e < ne; e += 256) {
        const int g = exact_groups[gi * Ck + e];
        start[e] = ko[g];
        pref[e] = ko[g + 1] - ko[g];
    }
    __syncthreads();
    const int X = block_exclusive_scan_int(pref, ne, tmp);
    const int ns = n_sample[gi];
    const int L = X + ns;
    const int Lpad = (L + kTK - 1) / kTK * kTK;
    int32_t *cr = col_row + gi * cap;
    float *cb = col_bias + gi * cap;
    const int32_t *si = sample_idx + gi * (int64_t)m;
    const float *sb = sample_bias + gi * (int64_t)m;
    float bmax = 0.0f;  // largest offset (log2 units) of the group, exact columns count as 0
    for (int c = threadIdx.x; c < Lpad; c += 256) {
        int row = 0;
        float bias = -INFINITY;
        if (c < X) {
            int lo = 0, hi = ne - 1;  // last e with pref[e] <= c
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (pref[mid] <= c) lo = mid; else hi = mid - 1;
            }
            row = start[lo] + (c - pref[lo]);
            bias = 0.0f;
        } else if (c < L) {
            row = si[c - X];
            bias = sb[c - X] / scale;
            bmax = fmaxf(bmax, sb[c - X] * kLog2e);
        }
        cr[c] = row;
        cb[c] = bias;
    }
    tmp[threadIdx.x] = __float_as_int(bmax);  // non-negative floats order like ints
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (threadIdx.x < off) tmp[threadIdx.x] = max(tmp[threadIdx.x], tmp[threadIdx.x + off]);
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        col_len[gi] = L;
        col_x[gi] = X;
        col_bmax[gi] = __int_as_float(tmp[0]);
    }
}

// Largest squared key norm of each head (fp32 of the bf16 rows), as float bits
// (non-negative floats order like their bits); kmax must start at 0.  D/8 lanes
// share a row, each summing one 16-byte chunk, then a butterfly over the row;
// every lane has kKU rows in flight per step.
constexpr int kKU = 4;

template <int D>
__global__ __launch_bounds__(256) void kmax_kernel(const uint16_t *k_p, int N, int *kmax)
{
    constexpr int TPR = D / 8;     // lanes per row
    constexpr int RPB = 256 / TPR;  // rows per block step
    __shared__ float red[4];
    const int bh = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ck = threadIdx.x % TPR;
    float best = 0.0f;
    for (int r0 = blockIdx.x * RPB * kKU + threadIdx.x / TPR; r0 < N; r0 += gridDim.x * RPB * kKU) {
        u32x4 w[kKU];
#pragma unroll
        for (int u = 0; u < kKU; ++u)
            if (r0 + u * RPB < N)
                w[u] = *reinterpret_cast<const u32x4 *>(k_p + ((int64_t)bh * N + r0 + u * RPB) * D + ck * 8);
#pragma unroll
        for (int u = 0; u < kKU; ++u) {
            float ss = 0.0f;
            if (r0 + u * RPB < N) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float a = __uint_as_float(w[u][q] << 16), c = __uint_as_float(w[u][q] & 0xFFFF0000u);
                    ss = fmaf(a, a, ss);
                    ss = fmaf(c, c, ss);
                }
            }
#pragma unroll
            for (int off = TPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
            best = fmaxf(best, ss);
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) best = fmaxf(best, __shfl_xor(best, off));
    if (lane == 0) red[wave] = best;
    __syncthreads();
    if (threadIdx.x == 0)
        atomicMax(&kmax[bh], __float_as_int(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))));
}

__global__ __launch_bounds__(256) void tile_table_kernel(const int32_t *q_offsets, int BH, int Cq, int tq,
                                                         int tph, int ntotal, int4 *table, int *redo, int *kmax2,
                                                         int32_t *nflag)
{
    __shared__ int cnt[kMaxGroups];
    __shared__ int tmp[256];
    const int bh = blockIdx.x;
    const int32_t *qo = q_offsets + (int64_t)bh * (Cq + 1);
    for (int i = threadIdx.x; i < Cq; i += 256) cnt[i] = (qo[i + 1] - qo[i] + tq - 1) / tq;
    __syncthreads();
    const int total = block_exclusive_scan_int(cnt, Cq, tmp);
    int4 *tb = table + (int64_t)bh * tph;
    for (int i = threadIdx.x; i < Cq; i += 256) {
        const int a = qo[i], z = qo[i + 1];
        int s = cnt[i];
        for (int r = a; r < z; r += tq, ++s) tb[s] = make_int4(i, r, min(z, r + tq), bh);
    }
    for (int s = total + threadIdx.x; s < tph; s += 256) tb[s] = make_int4(-1, 0, 0, bh);
    if (bh == BH - 1)
        for (int s = BH * tph + threadIdx.x; s < ntotal; s += 256) table[s] = make_int4(-1, 0, 0, bh);
    // clear the per-tile redo flags (indexed by logical tile) and this head's key-norm maximum
    for (int s = bh * tph + threadIdx.x; s < (bh + 1) * tph; s += 256) redo[s] = 0;
    if (bh == BH - 1)
        for (int s = BH * tph + threadIdx.x; s < ntotal; s += 256) redo[s] = 0;
    if (threadIdx.x == 0) kmax2[bh] = 0;
    if (nflag && bh == 0 && threadIdx.x == 0) *nflag = 0;  // tiles the fallback will recompute
}

// ------------------------------------------------------------------ bf16 MFMA kernel
// K tile in LDS: 64 unpadded rows, the 16-byte chunks of row r XOR-swizzled by
// r mod (chunks per row) so that 8 lanes reading one chunk of 8 rows hit 8
// distinct bank groups.
template <int D>
__device__ __forceinline__ int kswz(int row, int chunk)
{
    constexpr int CPR = D / 8;
    return row * CPR + (chunk ^ (row & (CPR - 1)));
}

// V tile in LDS: row-major (key rows of D elements) with the 16-byte chunks of each
// row XOR-swizzled.  The P.V product reads it with the LDS transpose read
// (ds_read_b64_tr_b16): inside each group of 16 lanes, lane j supplies the address
// of 4 elements of key row k0 + j/4 at column d0 + 4 (j mod 4), and lane i
// receives column d0 + i of the four rows k0 .. k0+3.  The 32 lanes that share a
// cycle read 4 rows x 4 consecutive chunks; the swizzle puts those 16 chunks in
// 16 distinct 16-byte bank slots (a 256-byte bank cycle): rows r mod 4 move by
// 4 r chunks for D = 128 (16 chunks a row); for D = 64 (8 chunks, so two rows
// share a bank cycle) rows 2 and 3 of each group of 4 move by 4.
template <int D>
__device__ __forceinline__ int vswz_mask(int row)
{
    return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

template <int D>
__device__ __forceinline__ int vswz(int row, int chunk)
{
    constexpr int CPR = D / 8;
    return row * CPR + (chunk ^ vswz_mask<D>(row));
}

// Tile rows go straight from memory into LDS (global_load_lds_dwordx4: lane l of a
// wave writes 16 bytes at M0 + 16 l); each lane fetches the chunk that belongs at
// its swizzled position.  `base` is the head's first row and rows[] holds row
// indices.
template <int D, int NW, bool ISV>
__device__ __forceinline__ void tile_direct(uint8_t *buf, const uint8_t *base, const int *rows, int wave, int lane)
{
    constexpr int CPR = D / 8;
    constexpr int ROUNDS = kTK * CPR / (64 * NW);
#pragma unroll
    for (int it = 0; it < ROUNDS; ++it) {
        const int blk = it * NW + wave;  // 64-chunk (1 KB) block of the tile
        const int P = blk * 64 + lane;
        const int row = P / CPR;
        const int c = ISV ? (P % CPR) ^ vswz_mask<D>(row) : (P % CPR) ^ (row & (CPR - 1));
        const uint16_t *src = reinterpret_cast<const uint16_t *>(base) + (uint32_t)rows[row] * (uint32_t)D + (uint32_t)(c * 8);
        __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)src,
                                         (void __attribute__((address_space(3))) *)(buf + blk * 1024), 16, 0, 0);
    }
}

// Split form of tile_direct for the ping-pong kernel.  tile_rows reads the row
// indices of this wave's chunks (for a tile past the end of the column list the
// caller passes a row of zeros: the instruction count stays fixed); tile_issue
// then starts the loads, addressed as a uniform base plus a 32-bit byte offset.
// Reading the indices of both tiles before issuing any load lets one LDS wait
// cover all of them.  The LDS destination is hidden from the compiler:
// it then does not tie these loads to a buffer and inserts no waits before reads
// of the other buffers -- the caller's own waits and barriers order every read
// after the load that fills it.
template <int D, int NW>
struct TileRows {
    static constexpr int ROUNDS = kTK * (D / 8) / (64 * NW);
    uint32_t r[ROUNDS];
};

template <int D, int NW>
__device__ __forceinline__ TileRows<D, NW> tile_rows(const int *rows, int wave, int lane)
{
    constexpr int CPR = D / 8;
    TileRows<D, NW> t;
#pragma unroll
    for (int it = 0; it < TileRows<D, NW>::ROUNDS; ++it) {
        const int P = (it * NW + wave) * 64 + lane;
        t.r[it] = (uint32_t)rows[P / CPR];
    }
    return t;
}

template <int D, int NW, bool ISV>
__device__ __forceinline__ void tile_issue(uint8_t *buf, const uint8_t *base, const TileRows<D, NW> &t, int wave,
                                           int lane)
{
    constexpr int CPR = D / 8;
#pragma unroll
    for (int it = 0; it < TileRows<D, NW>::ROUNDS; ++it) {
        const int blk = it * NW + wave;
        const int P = blk * 64 + lane;
        const int row = P / CPR;
        const int c = ISV ? (P % CPR) ^ vswz_mask<D>(row) : (P % CPR) ^ (row & (CPR - 1));
        const uint8_t *src = base + (t.r[it] * (uint32_t)(2 * D) + (uint32_t)(c * 16));
        auto *dst = (void __attribute__((address_space(3))) *)(buf + blk * 1024);
        asm volatile("" : "+s"(dst));
        __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)src, dst, 16, 0, 0);
    }
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Byte offset, inside a V tile, of the 8 bytes this lane supplies to the transpose
// read of d-block db (32 columns) for key rows 4 hl + (j/4) (+16 s, +8 later).
template <int D>
__device__ __forceinline__ int v_tr_offset(int db, int lane)
{
    const int j = lane & 15, x = (lane >> 4) & 1, hl = lane >> 5;
    const int row = 4 * hl + (j >> 2);
    const int dcol = db * 32 + 16 * x + 4 * (j & 3);
    return vswz<D>(row, dcol >> 3) * 16 + ((dcol >> 2) & 1) * 8;
}

// One tile step of the attention loop for a wave holding QB blocks of 32 query
// rows: multiply the 64 columns of tile t held in (kcur, vcur) while tile t+1 is
// being fetched into (knext, vnext).  The four buffers are distinct LDS objects,
// so the compiler can see that reading the current tile does not depend on the
// direct loads filling the next one.  Each K or V fragment read from LDS feeds
// QB matrix products.
template <int D, bool FIXED, int QB>
__device__ __forceinline__ void tile_step(int t, int T, int X, const uint8_t *kcur, const uint8_t *vcur,
                                          uint8_t *knext, uint8_t *vnext, const uint8_t *kbase,
                                          const uint8_t *vbase, const int32_t *crow, const float *cbias,
                                          int (*idx_row)[kTK], float (*idx_bias)[kTK], const bf16x8 (*qf)[D / 16],
                                          f32x16 (*oacc)[D / 32], float *l_run, float *m_run, const int *vtr,
                                          float scale_log2, bool wave_active, int wave, int lane, int hl, int l32)
{
    constexpr int NW = 4 / QB;
    constexpr int NDS = D / 16;
    constexpr int NDB = D / 32;
    constexpr int RSTR = D * 2;  // bytes per V row
    const bool more = t + 1 < T;
    if (more) {
        tile_direct<D, NW, false>(knext, kbase, idx_row[(t + 1) % 3], wave, lane);
        tile_direct<D, NW, true>(vnext, vbase, idx_row[(t + 1) % 3], wave, lane);
    }
    int32_t nrow = 0;
    float nbias = 0.0f;
    const bool fetch2 = wave == 0 && t + 2 < T;
    if (fetch2) {
        nrow = crow[(int64_t)(t + 2) * kTK + lane];
        nbias = cbias[(int64_t)(t + 2) * kTK + lane];
    }
    if (wave_active) {
        // The K Q^T accumulator starts at the column offsets (score units): lane
        // holds keys k2*32 + 8g + 4hl + e (e = 0..3) of its query.  Tiles of exact
        // columns only have offset 0.
        const int slot = t % 3;
        const bool exact_tile = (t + 1) * kTK <= X;
        f32x16 sacc[QB][2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 bv = exact_tile ? f32x4{0.0f, 0.0f, 0.0f, 0.0f}
                                            : *reinterpret_cast<const f32x4 *>(&idx_bias[slot][k2 * 32 + g * 8 + hl * 4]);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sacc[qb][k2][4 * g + e] = bv[e];
            }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < NDS; ++s) {
            const int c = s * 2 + hl;
            const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(kcur + kswz<D>(l32, c) * 16);
            const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(kcur + kswz<D>(32 + l32, c) * 16);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                sacc[qb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[qb][s], sacc[qb][0], 0, 0, 0);
                sacc[qb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[qb][s], sacc[qb][1], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
        // logits in log2 units: (score + offset) * scale * log2 e
        const float cf = scale_log2;
        if (!FIXED) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                float mr = sacc[qb][0][0];
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mr = fmaxf(mr, sacc[qb][k2][r]);
                float mx = mr * cf;
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                // lazy rescale: O and l stay relative to m_run until some lane's
                // maximum exceeds it by more than 8 (weights up to 2^8 are safe)
                if (__any(mx > m_run[qb] + 8.0f)) {
                    const float m_new = fmaxf(m_run[qb], mx);
                    const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
                    l_run[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
                    m_run[qb] = m_new;
                }
            }
        }
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        // raised wave priority while this wave issues MFMAs lets another wave on
        // the SIMD fill the VALU slots; s_setprio also bounds the scheduling
        // region, so it brackets the whole loop (the exponentials of chunk s+1
        // interleave with the products of chunk s)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 pb[QB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float mneg = -m_run[qb];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pb[qb][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[qb][s >> 1][8 * (s & 1) + e], cf, mneg));
                // row sum of the rounded weights, the same ones P.V uses
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const bf16x2 pp = {pb[qb][e], pb[qb][e + 1]};
                    l_run[qb] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run[qb], false);
                }
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                // keys 16 s + 4 hl + 0..3 and 16 s + 8 + 4 hl + 0..3 of column db*32 + l32
                const uint8_t *vp = vcur + vtr[db] + s * 16 * RSTR;
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)vp);
                const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(vp + 8 * RSTR));
                const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[qb], oacc[qb][db], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    }
    if (fetch2) {
        idx_row[(t + 2) % 3][lane] = nrow;
        idx_bias[(t + 2) % 3][lane] = nbias;
    }
    __builtin_amdgcn_s_waitcnt(0);  // direct K and V loads of the next tile have landed
    __syncthreads();
}

// One work-group = 128 query rows of one query group: 4/QB waves, each holding
// QB blocks of 32 rows.  S^T = K Q^T and O^T += V^T P^T on
// v_mfma_f32_32x32x16_bf16, so each lane owns one query per block: its weights
// stay in registers and feed P.V directly.  QB = 2 halves the LDS fragment
// traffic per product (one wave per SIMD, up to 512 registers); QB = 1 runs two
// waves per SIMD.
//
// FIXED = true (the fast kernel): every row uses the fixed reference
//   m_ref = scale log2(e) |q| max|k| + max(offsets, 0) - kRefShift,
// where the first terms bound every logit of the row (Cauchy-Schwarz), so
// weights exp2(l - m_ref) never exceed 2^kRefShift and O, l need no rescaling.
// The shift only has to keep sums of such weights (times values) inside the
// fp32 range; lowering the reference lets rows whose logits sit far below the
// bound (a wide spread of |q| |k|) keep normal weights.  If a row's weight sum
// ends below 2^-80 (its logits more than ~80 + kRefShift below the bound),
// weights may have underflowed, and if a sum or an output is not finite (values
// beyond ~2^40), something overflowed: either way the tile is flagged in `redo`.
// FIXED = false (the fallback): running maximum with rescaling; it processes
// only the flagged tiles.
template <int D, bool FIXED, int QB>
__global__ __launch_bounds__(256 / QB) __attribute__((amdgpu_waves_per_eu(3 - QB, 3 - QB))) void attn_bf16_kernel(
    const uint16_t *__restrict__ q_p, const uint16_t *__restrict__ k_p, const uint16_t *__restrict__ v_p,
    int N, int Cq, const int4 *__restrict__ table, int nblocks, const int32_t *__restrict__ col_row,
    const float *__restrict__ col_bias, const int32_t *__restrict__ col_len, const int32_t *__restrict__ col_x,
    const float *__restrict__ col_bmax, const int *__restrict__ kmax2, int64_t cap, float scale_log2,
    uint16_t *__restrict__ o_p, float *__restrict__ lse_p, const int32_t *__restrict__ perm_q,
    int *__restrict__ redo, int32_t *__restrict__ nflag)
{
    constexpr int NDS = D / 16;          // 16-wide d steps of S^T = K Q^T
    constexpr int NDB = D / 32;          // 32-row d blocks of O^T
    constexpr int KBYTES = kTK * D * 2;
    constexpr int VBYTES = kTK * D * 2;
    constexpr int WROWS = 32 * QB;       // query rows per wave
    __shared__ __attribute__((aligned(1024))) uint8_t kb0[KBYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t kb1[KBYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t vb0[VBYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t vb1[VBYTES];
    __shared__ int idx_row[3][kTK];
    __shared__ __attribute__((aligned(16))) float idx_bias[3][kTK];

    // One query tile; the exits below leave a tile (a wave that has no rows, or
    // a flagged tile, skips only the epilogue, which has no barrier).
    auto run_tile = [&](const int lb) {
        const int4 te = table[lb];
        if (te.x < 0) return;
        const int i = te.x, r0 = te.y, r1 = te.z, bh = te.w;
        const int64_t gi = (int64_t)bh * Cq + i;
        const int L = col_len[gi];
        const int X = col_x[gi];
        const int T = (L + kTK - 1) / kTK;
        const int32_t *crow = col_row + gi * cap;
        const float *cbias = col_bias + gi * cap;
        const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
        const uint8_t *kbase = reinterpret_cast<const uint8_t *>(k_p + (int64_t)bh * N * D);
        const uint8_t *vbase = reinterpret_cast<const uint8_t *>(v_p + (int64_t)bh * N * D);

        // Q^T fragments (B operand of S^T = K Q^T): lane owns query row l32 of each block.
        const bool wave_active = r0 + wave * WROWS < r1;
        bf16x8 qf[QB][NDS];
        float m_run[QB], l_run[QB];
    #pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int qrow = min(r0 + wave * WROWS + qb * 32 + l32, r1 - 1);
            const uint16_t *qsrc = q_p + ((int64_t)bh * N + qrow) * D + hl * 8;
            float qss = 0.0f;
    #pragma unroll
            for (int s = 0; s < NDS; ++s) {
                qf[qb][s] = *reinterpret_cast<const bf16x8 *>(qsrc + s * 16);
                if (FIXED) {
    #pragma unroll
                    for (int e = 0; e < 8; ++e) qss = fmaf((float)qf[qb][s][e], (float)qf[qb][s][e], qss);
                }
            }
            m_run[qb] = -INFINITY;
            l_run[qb] = 0.0f;
            if (FIXED) {
                qss += __shfl_xor(qss, 32);
                const float kmx = sqrtf(__int_as_float(kmax2[bh]));
                m_run[qb] = fmaf(scale_log2 * sqrtf(qss) * kmx, 1.0f + 1e-5f, col_bmax[gi]) + 1e-6f - kRefShift;
            }
        }

        // column list of tiles 0 and 1 into the index ring
        if (wave == 0) {
            idx_row[0][lane] = crow[lane];
            idx_bias[0][lane] = cbias[lane];
            if (T > 1) {
                idx_row[1][lane] = crow[kTK + lane];
                idx_bias[1][lane] = cbias[kTK + lane];
            }
        }
        __syncthreads();
        constexpr int NW = 4 / QB;
        tile_direct<D, NW, false>(kb0, kbase, idx_row[0], wave, lane);
        tile_direct<D, NW, true>(vb0, vbase, idx_row[0], wave, lane);
        int vtr[NDB];
    #pragma unroll
        for (int db = 0; db < NDB; ++db) vtr[db] = v_tr_offset<D>(db, lane);
        __builtin_amdgcn_s_waitcnt(0);  // direct K and V loads have landed in LDS
        __syncthreads();

        f32x16 oacc[QB][NDB];
    #pragma unroll
        for (int qb = 0; qb < QB; ++qb)
    #pragma unroll
            for (int db = 0; db < NDB; ++db)
    #pragma unroll
                for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.0f;

        for (int t = 0; t < T; t += 2) {
            tile_step<D, FIXED, QB>(t, T, X, kb0, vb0, kb1, vb1, kbase, vbase, crow, cbias, idx_row, idx_bias, qf,
                                    oacc, l_run, m_run, vtr, scale_log2, wave_active, wave, lane, hl, l32);
            if (t + 1 < T)
                tile_step<D, FIXED, QB>(t + 1, T, X, kb1, vb1, kb0, vb0, kbase, vbase, crow, cbias, idx_row, idx_bias,
                                        qf, oacc, l_run, m_run, vtr, scale_log2, wave_active, wave, lane, hl, l32);
        }

        if (!wave_active) return;
        float l_tot[QB];
        bool low = false;
    #pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            l_tot[qb] = l_run[qb] + __shfl_xor(l_run[qb], 32);
            const int qrow_raw = r0 + wave * WROWS + qb * 32 + l32;
            // 2^-80: weights may have underflowed; not finite: something overflowed
            bool bad = !(l_tot[qb] >= 8.271806e-25f) || !(l_tot[qb] < INFINITY);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) bad = bad || !(fabsf(oacc[qb][db][r]) < INFINITY);
            low = low || (qrow_raw < r1 && bad);
        }
        if (FIXED && __any(low)) {
            if (lane == 0) redo[lb] = 1;
            return;
        }
    #pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int qrow_raw = r0 + wave * WROWS + qb * 32 + l32;
            if (qrow_raw < r1) {
                const float inv = 1.0f / l_tot[qb];
                // token order when a permutation is given (the un-permute step fused)
                const int orow_i = perm_q ? perm_q[(int64_t)bh * N + qrow_raw] : qrow_raw;
                uint16_t *orow = o_p + ((int64_t)bh * N + orow_i) * D;
    #pragma unroll
                for (int db = 0; db < NDB; ++db)
    #pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int d0 = db * 32 + g * 8 + hl * 4;
                        const uint32_t lo = (uint32_t)f32_to_bf16_bits(oacc[qb][db][4 * g] * inv) |
                                            ((uint32_t)f32_to_bf16_bits(oacc[qb][db][4 * g + 1] * inv) << 16);
                        const uint32_t hi = (uint32_t)f32_to_bf16_bits(oacc[qb][db][4 * g + 2] * inv) |
                                            ((uint32_t)f32_to_bf16_bits(oacc[qb][db][4 * g + 3] * inv) << 16);
                        *reinterpret_cast<u32x2 *>(orow + d0) = u32x2{lo, hi};
                    }
                if (lse_p && hl == 0)
                    lse_p[(int64_t)bh * N + orow_i] = (m_run[qb] + log2f(l_tot[qb])) * 0.6931471805599453f;
            }
        }
    };
    if constexpr (FIXED) {
        run_tile(xcd_logical_block(blockIdx.x, nblocks));
    } else {
        // the fallback: each work-group reads the flags of 64 tiles at once (every
        // wave the same 64, so the ballot is uniform) and runs the flagged ones
        const int lane = threadIdx.x & 63;
        for (int base = blockIdx.x * 64; base < nblocks; base += gridDim.x * 64) {
            uint64_t mask = __ballot(base + lane < nblocks && redo[base + lane] != 0);
            if (nflag && mask && threadIdx.x == 0) atomicAdd(nflag, (int32_t)__popcll(mask));
            while (mask) {
                const int bit = __ffsll((unsigned long long)mask) - 1;
                mask &= mask - 1;
                run_tile(base + bit);
                __syncthreads();  // LDS tiles and index rows free for the next tile
            }
        }
    }
}

// ------------------------------------------------------------------ ping-pong bf16 kernel
// Two independent 128-row query tiles share a work-group of 8 waves: waves 0-3
// hold tile A, waves 4-7 tile B (the hardware places waves w and w+4 of a
// work-group on the same SIMD).  A tile is processed as a sequence of slots --
// slot 2t: the P.V product of tile t-1 and the S = K Q^T product of tile t (MFMA);
// slot 2t+1: the weights of tile t (VALU) -- and tile B runs one slot behind tile
// A.  One barrier per phase keeps the halves in step, so while one wave of a SIMD
// issues matrix products the other computes weights.  K and V tiles are loaded
// straight into LDS three phases before their products (issued in the weight
// slot two tiles ahead), and a phase ends waiting only for loads issued in the
// current slot.  Weights as in attn_bf16_kernel<D, true, 1> (fixed reference);
// the row sums come from an extra product instead of VALU additions.
constexpr int kPPWaves = 8;
// The paired-tile kernel lowers each row's fixed reference to at most this far
// (log2 units) above the largest logit of the row's first column tile.  With the
// bound kRefShift above it, a row's reference is min(bound - kRefShift, first
// tile's maximum + kAnchor): the largest weight is then >= 2^-kAnchor (no
// underflow), and weights exceed 2^kRefShift only where a later logit beats the
// first tile's maximum by more than kAnchor + kRefShift, far beyond realistic
// data (the non-finite check catches an actual overflow).
constexpr float kAnchor = 72.0f;
constexpr bool kUsePingPong = true;
constexpr int kPPAhead = 4;  // products whose operands are in flight ahead of use
constexpr int kPPRing = 8;   // column-index ring: tiles u .. u+4 are live in weight slot u

// Wait for LDS traffic and for all but the newest `keep` vector-memory operations
// of this wave, then barrier.  The empty asm statements stop the compiler from
// moving memory accesses across the barrier; the explicit wait replaces the full
// drain a release fence would emit, so direct loads stay in flight across phases.
template <int KEEP>
__device__ __forceinline__ void pp_barrier()
{
    static_assert(KEEP >= 0 && KEEP < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((KEEP & 0xF) | (0x7 << 4));  // vmcnt(KEEP), expcnt off, lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Barrier that waits for LDS traffic only (a product slot issues no vector-memory
// operations, and everything older than the previous slot's direct loads has
// already been waited for).
__device__ __forceinline__ void pp_barrier_lds()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt and expcnt at their maxima, lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int D>
struct PPTile {
    int T, r0, r1, bh, lb;
    const int32_t *crow;
    const float *cbias;
    bool active;
};

// K Q^T accumulators set to a tile's column offsets: lane holds keys
// k2*32 + 8g + 4hl + e (e = 0..3) of its query.
__device__ __forceinline__ void load_offsets(f32x16 *sacc, const float *bias, int hl)
{
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 bv = *reinterpret_cast<const f32x4 *>(&bias[k2 * 32 + g * 8 + hl * 4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) sacc[k2][4 * g + e] = bv[e];
        }
}

// One phase of one half.  SLOT parity and buffer parities are compile-time
// functions of (J, HALF); the tile index is runtime.  m_ref is the row's fixed
// reference, lowered once to the first tile's largest logit + kAnchor, or (RUN,
// the rescaling pass over flagged tiles) the row's running maximum.
template <int D, bool RUN, int HALF, int J>
__device__ __forceinline__ void pp_phase(int c, const PPTile<D> &tt, uint8_t *k0, uint8_t *k1, uint8_t *v0,
                                         uint8_t *v1, int (*ring_row)[kTK], float (*ring_bias)[kTK],
                                         const uint16_t *kh, const uint16_t *vh, const bf16x8 *qf, f32x16 *oacc,
                                         f32x16 *sacc, bf16x8 *pb, f32x4 &lacc, const bf16x8 &ones_a,
                                         const int *zrow, float &m_ref, const int *vtr, float scale_log2,
                                         bool wave_active, int wq, int lane, int hl, int l32)
{
    constexpr int NDS = D / 16;
    constexpr int NDB = D / 32;
    constexpr int RSTR = D * 2;
    constexpr int NDMA = kTK * (D / 8) / 256;  // direct-load instructions per wave per tile (K or V)
    constexpr int K = J - HALF;                // slot index relative to 4c (may be -1)
    constexpr bool GEMM = ((K % 2) + 2) % 2 == 0;
    const int slot = 4 * c + K;
    const bool live = tt.active && slot >= 0 && slot <= 2 * tt.T;
    if (GEMM) {
        if (live && wave_active) {
            // P.V of tile t-1 (weights pb, V buffer (t-1) % 2) and S = K Q^T of tile
            // t (K buffer t % 2) as one list of 32 products, P.V and K Q^T
            // alternating so that consecutive products feed different accumulators,
            // plus one row-sum product per key step.
            // Operands are read kPPAhead products ahead of use, and scheduling
            // fences keep that order, so each product waits only for reads issued
            // several products earlier.  For t = 0 the P.V terms multiply zero
            // weights by a zero buffer; for t = T the S tile is never used.
            constexpr int QP = ((K / 2) % 2 + 2) % 2;   // t % 2 (4c is even)
            const uint8_t *kc = QP == 0 ? k0 : k1;
            const uint8_t *vc = QP == 0 ? v1 : v0;      // tile t-1
            constexpr int NJ = 2 * NDS + 4 * NDB;       // 32 products for D = 128
            static_assert(2 * NDS == 4 * NDB, "P.V and K Q^T lists alternate");
            constexpr int R = kPPAhead + 1;
            bf16x8 opnd[R];
            auto load = [&](int j, bf16x8 &dst) {
                const int i = j >> 1;
                if ((j & 1) == 0) {  // P.V: d block i % NDB, key step i / NDB
                    const int db = i % NDB, s = i / NDB;
                    const uint8_t *vp = vc + vtr[db] + s * 16 * RSTR;
                    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)vp);
                    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(vp + 8 * RSTR));
                    dst = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                } else {             // K Q^T: key half i % 2, d step i / 2
                    const int k2 = i & 1, s = i >> 1;
                    dst = *reinterpret_cast<const bf16x8 *>(kc + kswz<D>(k2 * 32 + l32, s * 2 + hl) * 16);
                }
            };
            // the K Q^T accumulator already holds tile t's column offsets (read at the
            // end of this wave's previous weight slot, or in the prologue for t = 0)
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int j = 0; j < kPPAhead; ++j) load(j, opnd[j]);
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                // fences keep the reads of product j + kPPAhead ahead of product j
                __builtin_amdgcn_sched_barrier(0);
                if (j + kPPAhead < NJ) load(j + kPPAhead, opnd[(j + kPPAhead) % R]);
                __builtin_amdgcn_sched_barrier(0);
                const int i = j >> 1;
                if ((j & 1) == 0) {
                    const int db = i % NDB, s = i / NDB;
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[j % R], pb[s], oacc[db], 0, 0, 0);
                } else {
                    const int k2 = i & 1, s = i >> 1;
                    sacc[k2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[j % R], qf[s], sacc[k2], 0, 0, 0);
                }
                // row sums of the weights: the 16 keys x 32 queries of pb[s], read as the
                // B operand of a 16x16x32 product, hold queries n and n + 16 in
                // alternate 8-key blocks; an A with ones in those blocks for rows 0 and
                // 1 sums both at half the cost of a 32x32x16 product
                if ((j & 7) == 7)
                    lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_a, pb[j >> 3], lacc, 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
        }
        pp_barrier_lds();
    } else {
        // The barrier sits in the same branch as the direct loads, so the compiler's
        // count of outstanding loads matches the wait on every path.
        if (live) {
            const int u = (slot - 1) / 2;  // weights of tile u
            constexpr int UP = (((K - 1) / 2) % 2 + 2) % 2;  // u % 2
            // column indices and offsets of tile u+4 straight into the ring: each
            // wave of the half loads 16 entries (lanes 0-15).  They are first read
            // two exponential slots later, after a barrier that has waited for them.
            {
                const int ent = wq * 16 + lane;
                const int64_t src = (int64_t)(u + 4 < tt.T ? u + 4 : 0) * kTK + ent;
                auto *drow = (void __attribute__((address_space(3))) *)&ring_row[(u + 4) % kPPRing][wq * 16];
                auto *dbias = (void __attribute__((address_space(3))) *)&ring_bias[(u + 4) % kPPRing][wq * 16];
                asm volatile("" : "+s"(drow));
                asm volatile("" : "+s"(dbias));
                if (lane < 16) {
                    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)(tt.crow + src),
                                                     drow, 4, 0, 0);
                    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)(tt.cbias + src),
                                                     dbias, 4, 0, 0);
                }
            }
            // K of tile u+2 into buffer u % 2, V of tile u+1 into buffer (u+1) % 2;
            // past the end these load row 0 into buffers no later slot reads
            const TileRows<D, 4> kr = tile_rows<D, 4>(u + 2 < tt.T ? ring_row[(u + 2) % kPPRing] : zrow, wq, lane);
            const TileRows<D, 4> vr = tile_rows<D, 4>(u + 1 < tt.T ? ring_row[(u + 1) % kPPRing] : zrow, wq, lane);
            tile_issue<D, 4, false>(UP == 0 ? k0 : k1, reinterpret_cast<const uint8_t *>(kh), kr, wq, lane);
            tile_issue<D, 4, true>(UP == 0 ? v1 : v0, reinterpret_cast<const uint8_t *>(vh), vr, wq, lane);
            if (wave_active) {
                if constexpr (RUN) {
                    // the largest logit of tile u in this lane's query (the lane holds
                    // half of the 64 keys, lane l ^ 32 the other half); the maximum is
                    // raised lazily, only when the tile exceeds it by more than 8, so
                    // weights stay below 2^8 and O and the row sums (which hold the
                    // tiles before u) are rescaled rarely
                    float mx = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
                    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(sacc[0][r], sacc[1][r]));
                    mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;
                    if (__any(mx > m_ref + 8.0f)) {
                        const float m_new = fmaxf(m_ref, mx);
                        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);  // 0 before the first tile
#pragma unroll
                        for (int db = 0; db < NDB; ++db)
#pragma unroll
                            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
                        // row sums: lane l < 16 holds queries l (element 0) and l + 16 (element 1)
                        const float a16 = __shfl(alpha, (lane & 15) + 16);
                        lacc[0] *= alpha;
                        lacc[1] *= a16;
                        m_ref = m_new;
                    }
                } else if (u == 0) {
                    // anchor: the first tile's largest logit of this lane's query (the
                    // lane holds half of the 64 keys, lane l ^ 32 the other half) bounds
                    // the row's maximum from below, so a reference at most kAnchor above
                    // it keeps the largest weight >= 2^-kAnchor (no underflow)
                    float mx = fmaxf(sacc[0][0], sacc[1][0]);
#pragma unroll
                    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(sacc[0][r], sacc[1][r]));
                    mx = fmaxf(mx, __shfl_xor(mx, 32));
                    m_ref = fminf(m_ref, fmaf(mx, scale_log2, kAnchor));
                }
                // logits in log2 units: (score + offset) * scale * log2 e
                const float mneg = -m_ref;
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        pb[s][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[s >> 1][8 * (s & 1) + e], scale_log2, mneg));
            }
            // the next product slot's K Q^T accumulator starts at tile u+1's column
            // offsets (score units), read here where the slot has time to spare
            // instead of ahead of its first product
            load_offsets(sacc, ring_bias[(u + 1) % kPPRing], hl);
            // this slot's direct loads stay in flight; everything older has landed
            pp_barrier<2 * NDMA + 2>();
        } else {
            // before a half's first product slot this is tile 0's offsets; after its
            // last one the value is not used
            load_offsets(sacc, ring_bias[0], hl);
            pp_barrier<0>();
        }
    }
}

template <int D, bool RUN, int HALF>
__device__ __forceinline__ void pp_chunks(int nchunks, const PPTile<D> &tt, uint8_t *k0, uint8_t *k1, uint8_t *v0,
                                          uint8_t *v1, int (*ring_row)[kTK], float (*ring_bias)[kTK],
                                          int *zrow, const uint16_t *kh, const uint16_t *vh, const bf16x8 *qf,
                                          f32x16 *oacc, f32x4 &lacc, float &m_ref, const int *vtr, float scale_log2,
                                          bool wave_active, int wq, int lane, int hl, int l32)
{
    constexpr int KB = kTK * D * 2;
    // column indices of tiles 0..3, then K of tiles 0 and 1 and V of tile 0; the
    // second V buffer starts at zero (the first product slot multiplies it by zero
    // weights)
    if (wq == 0 && tt.active) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
            if (t < tt.T) {
                ring_row[t][lane] = tt.crow[t * kTK + lane];
                ring_bias[t][lane] = tt.cbias[t * kTK + lane];
            }
    }
    for (int x = wq * 64 + lane; x < KB / 16; x += 256) *reinterpret_cast<u32x4 *>(v1 + 16 * x) = u32x4{0, 0, 0, 0};
    if (wq == 0) zrow[lane] = 0;  // both halves write the same zeros
    __syncthreads();
    if (tt.active) {
        tile_direct<D, 4, false>(k0, reinterpret_cast<const uint8_t *>(kh), ring_row[0], wq, lane);
        tile_issue<D, 4, false>(k1, reinterpret_cast<const uint8_t *>(kh),
                                tile_rows<D, 4>(tt.T > 1 ? ring_row[1] : zrow, wq, lane), wq, lane);
        tile_direct<D, 4, true>(v0, reinterpret_cast<const uint8_t *>(vh), ring_row[0], wq, lane);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    f32x16 sacc[2];
    bf16x8 pb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[s][e] = (__bf16)0.0f;
    // the first product slot's K Q^T accumulator starts at tile 0's offsets
    load_offsets(sacc, ring_bias[0], hl);
    // A operand of the row-sum product (16x16x32: lane l holds row l % 16, k block
    // l / 16): row 0 is one on k blocks 0 and 2 (query n of the 32x32x16 B layout),
    // row 1 on blocks 1 and 3 (query n + 16)
    bf16x8 ones_a;
    const bool one = (lane & 15) == ((lane >> 4) & 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) ones_a[e] = (__bf16)(one ? 1.0f : 0.0f);
    for (int c = 0; c < nchunks; ++c) {
        pp_phase<D, RUN, HALF, 0>(c, tt, k0, k1, v0, v1, ring_row, ring_bias, kh, vh, qf, oacc, sacc, pb, lacc, ones_a,
                             zrow, m_ref, vtr, scale_log2, wave_active, wq, lane, hl, l32);
        pp_phase<D, RUN, HALF, 1>(c, tt, k0, k1, v0, v1, ring_row, ring_bias, kh, vh, qf, oacc, sacc, pb, lacc, ones_a,
                             zrow, m_ref, vtr, scale_log2, wave_active, wq, lane, hl, l32);
        pp_phase<D, RUN, HALF, 2>(c, tt, k0, k1, v0, v1, ring_row, ring_bias, kh, vh, qf, oacc, sacc, pb, lacc, ones_a,
                             zrow, m_ref, vtr, scale_log2, wave_active, wq, lane, hl, l32);
        pp_phase<D, RUN, HALF, 3>(c, tt, k0, k1, v0, v1, ring_row, ring_bias, kh, vh, qf, oacc, sacc, pb, lacc, ones_a,
                             zrow, m_ref, vtr, scale_log2, wave_active, wq, lane, hl, l32);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the last (unused) direct loads have landed
}

// RUN = false: the fast pass over every tile pair of the table (fixed, anchored
// reference; tiles whose sums leave the fp32 range are flagged in `redo`).
// RUN = true: the rescaling pass, over the flagged tiles only (flist holds their
// ids in ascending order, *nflag their number), with a running maximum per row.
template <int D, bool RUN>
__global__ __launch_bounds__(64 * kPPWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_pp_kernel(
    const uint16_t *__restrict__ q_p, const uint16_t *__restrict__ k_p, const uint16_t *__restrict__ v_p, int N,
    int Cq, const int4 *__restrict__ table, int nblocks, const int32_t *__restrict__ col_row,
    const float *__restrict__ col_bias, const int32_t *__restrict__ col_len, const int32_t *__restrict__ col_x,
    const float *__restrict__ col_bmax, const int *__restrict__ kmax2, int64_t cap, float scale_log2,
    uint16_t *__restrict__ o_p, float *__restrict__ lse_p, const int32_t *__restrict__ perm_q,
    int *__restrict__ redo, const int *__restrict__ flist, const int *__restrict__ nflag)
{
    constexpr int NDS = D / 16;
    constexpr int NDB = D / 32;
    constexpr int KB = kTK * D * 2;
    __shared__ __attribute__((aligned(1024))) uint8_t ka0[KB];
    __shared__ __attribute__((aligned(1024))) uint8_t ka1[KB];
    __shared__ __attribute__((aligned(1024))) uint8_t va0[KB];
    __shared__ __attribute__((aligned(1024))) uint8_t va1[KB];
    __shared__ __attribute__((aligned(1024))) uint8_t kb0[KB];
    __shared__ __attribute__((aligned(1024))) uint8_t kb1[KB];
    __shared__ __attribute__((aligned(1024))) uint8_t vb0[KB];
    __shared__ __attribute__((aligned(1024))) uint8_t vb1[KB];
    __shared__ int ring_row[2][kPPRing][kTK];
    __shared__ __attribute__((aligned(16))) float ring_bias[2][kPPRing][kTK];
    __shared__ int zrow[kTK];

    const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = wave >> 2, wq = wave & 3;
    // one tile pair per work-group: pairs of the table (fast pass) or of the list
    // of flagged tiles (rescaling pass; work-groups past its end exit at once)
    const int lp = xcd_logical_block(blockIdx.x, gridDim.x);
    const int nlist = RUN ? *nflag : nblocks;
    if (2 * lp >= nlist) return;
    // both halves' tiles (every wave reads both, so the phase count is uniform)
    int Th[2];
    int4 teh[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int pos = 2 * lp + h;
        const int tile = pos < nlist ? (RUN ? flist[pos] : pos) : nblocks;
        teh[h] = tile < nblocks ? table[tile] : make_int4(-1, 0, 0, 0);
        Th[h] = teh[h].x >= 0 ? (col_len[(int64_t)teh[h].w * Cq + teh[h].x] + kTK - 1) / kTK : 0;
    }
    if (teh[0].x < 0 && teh[1].x < 0) return;
    // phases: half h runs slot k in phase k + h; the last slot of a tile sequence is 2T
    const int nphase = max(2 * Th[0], 2 * Th[1] + 1) + 1;
    const int nchunks = (nphase + 3) / 4;

    const int4 te = half ? teh[1] : teh[0];  // selects, not an indexed private array
    PPTile<D> tt;
    tt.T = half ? Th[1] : Th[0];
    tt.active = te.x >= 0 && tt.T > 0;
    const int i = tt.active ? te.x : 0, bh = tt.active ? te.w : 0;
    tt.r0 = te.y;
    tt.r1 = te.z;
    tt.bh = bh;
    tt.lb = RUN ? 0 : 2 * lp + half;  // the flag slot (the fast pass only)
    const int64_t gi = (int64_t)bh * Cq + i;
    tt.crow = col_row + gi * cap;
    tt.cbias = col_bias + gi * cap;
    const uint16_t *kh = k_p + (int64_t)bh * N * D;
    const uint16_t *vh = v_p + (int64_t)bh * N * D;

    // Q^T fragments of this wave's 32 rows and the row's reference: fixed (lowered
    // to the first tile's maximum + kAnchor in the first weight slot), or the
    // running maximum (RUN; -inf before the first tile).  A tile with an empty
    // column list does no products and is flagged below (zero row sums), as in
    // the single-tile kernel
    const bool wave_active = te.x >= 0 && tt.r0 + wq * 32 < tt.r1;
    bf16x8 qf[NDS];
    float m_ref = -INFINITY;
    {
        const int qrow = tt.active ? min(tt.r0 + wq * 32 + l32, tt.r1 - 1) : 0;
        const uint16_t *qsrc = q_p + ((int64_t)bh * N + qrow) * D + hl * 8;
#pragma unroll
        for (int s = 0; s < NDS; ++s) qf[s] = *reinterpret_cast<const bf16x8 *>(qsrc + s * 16);
        if constexpr (!RUN) {
            float qss = 0.0f;
#pragma unroll
            for (int s = 0; s < NDS; ++s)
#pragma unroll
                for (int e = 0; e < 8; ++e) qss = fmaf((float)qf[s][e], (float)qf[s][e], qss);
            qss += __shfl_xor(qss, 32);
            const float kmx = sqrtf(__int_as_float(kmax2[bh]));
            m_ref = fmaf(scale_log2 * sqrtf(qss) * kmx, 1.0f + 1e-5f, tt.active ? col_bmax[gi] : 0.0f) + 1e-6f -
                    kRefShift;
        }
    }
    int vtr[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) vtr[db] = v_tr_offset<D>(db, lane);

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
    f32x4 lacc = {0.0f, 0.0f, 0.0f, 0.0f};
    // each half names its own buffers, so the compiler sees which LDS object every
    // direct load writes and every product reads; both paths pass 4 * nchunks barriers
    if (half == 0)
        pp_chunks<D, RUN, 0>(nchunks, tt, ka0, ka1, va0, va1, ring_row[0], ring_bias[0], zrow, kh, vh, qf, oacc, lacc, m_ref,
                        vtr, scale_log2, wave_active, wq, lane, hl, l32);
    else
        pp_chunks<D, RUN, 1>(nchunks, tt, kb0, kb1, vb0, vb1, ring_row[1], ring_bias[1], zrow, kh, vh, qf, oacc, lacc, m_ref,
                        vtr, scale_log2, wave_active, wq, lane, hl, l32);

    if (wave_active) {
        // rows 0 and 1 of the row-sum product live in lanes 0-15: the sums of queries
        // 0-15 and 16-31
        const float ls0 = __shfl(lacc[0], l32 & 15), ls1 = __shfl(lacc[1], l32 & 15);
        const float l_tot = l32 < 16 ? ls0 : ls1;
        const int qrow_raw = tt.r0 + wq * 32 + l32;
        // 2^-80: weights may have underflowed; not finite: something overflowed.
        // Either hands the tile to the rescaling pass.
        bool bad = !(l_tot >= 8.271806e-25f) || !(l_tot < INFINITY);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) bad = bad || !(fabsf(oacc[db][r]) < INFINITY);
        if (!RUN && __any(qrow_raw < tt.r1 && bad)) {
            if (lane == 0) redo[tt.lb] = 1;
        } else if (qrow_raw < tt.r1) {
            const float inv = 1.0f / l_tot;
            // token order when a permutation is given (the un-permute step fused)
            const int orow_i = perm_q ? perm_q[(int64_t)bh * N + qrow_raw] : qrow_raw;
            uint16_t *orow = o_p + ((int64_t)bh * N + orow_i) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d0 = db * 32 + g * 8 + hl * 4;
                    const uint32_t lo = (uint32_t)f32_to_bf16_bits(oacc[db][4 * g] * inv) |
                                        ((uint32_t)f32_to_bf16_bits(oacc[db][4 * g + 1] * inv) << 16);
                    const uint32_t hi = (uint32_t)f32_to_bf16_bits(oacc[db][4 * g + 2] * inv) |
                                        ((uint32_t)f32_to_bf16_bits(oacc[db][4 * g + 3] * inv) << 16);
                    *reinterpret_cast<u32x2 *>(orow + d0) = u32x2{lo, hi};
                }
            if (lse_p && hl == 0) lse_p[(int64_t)bh * N + orow_i] = (m_ref + log2f(l_tot)) * 0.6931471805599453f;
        }
    }
}

// ------------------------------------------------------------------ fp32 VALU kernel
template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(const float *__restrict__ q_p, const float *__restrict__ k_p,
                                                       const float *__restrict__ v_p, int N, int Cq,
                                                       const int4 *__restrict__ table, int nblocks,
                                                       const int32_t *__restrict__ col_row,
                                                       const float *__restrict__ col_bias,
                                                       const int32_t *__restrict__ col_len, int64_t cap,
                                                       float scale_log2, float *__restrict__ o_p,
                                                       float *__restrict__ lse_p,
                                                       const int32_t *__restrict__ perm_q)
{
    constexpr int DQ = D / 4;
    constexpr int TKF = 32;
    __shared__ float ks[TKF][D];
    __shared__ float vs[TKF][D];
    __shared__ float bs[TKF];
    const int lb = xcd_logical_block(blockIdx.x, nblocks);
    const int4 te = table[lb];
    if (te.x < 0) return;
    const int i = te.x, r0 = te.y, r1 = te.z, bh = te.w;
    const int64_t gi = (int64_t)bh * Cq + i;
    const int L = col_len[gi];
    const int32_t *crow = col_row + gi * cap;
    const float *cbias = col_bias + gi * cap;
    const int tid = threadIdx.x, qi = tid >> 2, part = tid & 3;
    const int qrow_raw = r0 + qi;
    const int qrow = min(qrow_raw, r1 - 1);
    const float *kh = k_p + (int64_t)bh * N * D;
    const float *vh = v_p + (int64_t)bh * N * D;
    float q[DQ], o[DQ];
#pragma unroll
    for (int e = 0; e < DQ; ++e) {
        q[e] = q_p[((int64_t)bh * N + qrow) * D + part * DQ + e];
        o[e] = 0.0f;
    }
    float m_run = -INFINITY, l_run = 0.0f;
    for (int c0 = 0; c0 < L; c0 += TKF) {
        __syncthreads();
        for (int e = tid; e < TKF * D; e += 256) {
            const int kk = e / D, dd = e % D;
            const int c = c0 + kk;
            const int row = crow[c];  // padded to a multiple of 64: always in the list
            ks[kk][dd] = kh[(int64_t)row * D + dd];
            vs[kk][dd] = vh[(int64_t)row * D + dd];
        }
        if (tid < TKF) bs[tid] = cbias[c0 + tid];
        __syncthreads();
        const int nk = min(TKF, L - c0);
        for (int kk = 0; kk < nk; ++kk) {
            float s = 0.0f;
#pragma unroll
            for (int e = 0; e < DQ; ++e) s = fmaf(q[e], ks[kk][part * DQ + e], s);
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            const float xl = (s + bs[kk]) * scale_log2;
            const float m_new = fmaxf(m_run, xl);
            const float a = exp2f(m_run - m_new);
            const float p = exp2f(xl - m_new);
            l_run = l_run * a + p;
#pragma unroll
            for (int e = 0; e < DQ; ++e) o[e] = fmaf(o[e], a, p * vs[kk][part * DQ + e]);
            m_run = m_new;
        }
    }
    if (qrow_raw < r1) {
        const float inv = 1.0f / l_run;
        const int orow_i = perm_q ? perm_q[(int64_t)bh * N + qrow_raw] : qrow_raw;
#pragma unroll
        for (int e = 0; e < DQ; ++e) o_p[((int64_t)bh * N + orow_i) * D + part * DQ + e] = o[e] * inv;
        if (lse_p && part == 0) lse_p[(int64_t)bh * N + orow_i] = (m_run + log2f(l_run)) * 0.6931471805599453f;
    }
}

// The flagged tiles' logical ids in ascending order (flist) and their number
// (*nlist, and *nflag when given).  One work-group of 1024 threads: each thread
// counts the flags of 32 consecutive tiles, a block scan of the counts gives
// every thread its first list position, and the ids follow in order (chunks of
// 32768 tiles).
constexpr int kListPer = 32;

__global__ __launch_bounds__(1024) void list_flags_kernel(const int *redo, int ntotal, int *flist, int *nlist,
                                                          int32_t *nflag)
{
    __shared__ int wtot[16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int base = 0;
    for (int c0 = 0; c0 < ntotal; c0 += 1024 * kListPer) {
        const int t0 = c0 + threadIdx.x * kListPer;
        uint32_t bits = 0;
#pragma unroll
        for (int u = 0; u < kListPer; ++u)
            if (t0 + u < ntotal && redo[t0 + u] != 0) bits |= 1u << u;
        const int cnt = __popc(bits);
        const int incl = wave_inclusive_scan(cnt);
        if (lane == 63) wtot[wave] = incl;
        __syncthreads();
        int before = base, add = 0;
        for (int w = 0; w < 16; ++w) {
            const int v = wtot[w];
            if (w < wave) before += v;
            add += v;
        }
        int pos = before + incl - cnt;
        while (bits) {
            const int u = __ffs(bits) - 1;
            bits &= bits - 1;
            flist[pos++] = t0 + u;
        }
        base += add;
        __syncthreads();  // wtot is rewritten by the next chunk
    }
    if (threadIdx.x == 0) {
        *nlist = base;
        if (nflag) *nflag = base;
    }
}

struct Layout {
    int64_t cap;       // columns per group in the column map
    int tph;           // tile slots per head
    int ntotal;        // launched blocks (multiple of 8)
    size_t off_row, off_bias, off_len, off_x, off_bmax, off_kmax, off_redo, off_table, off_flist, off_nlist, total;
};

Layout layout(int B, int H, int N, int Cq, int m, int tq)
{
    Layout L;
    const int64_t G = (int64_t)B * H * Cq;
    L.cap = ((int64_t)N + m + kTK - 1) / kTK * kTK;
    L.tph = (N + tq - 1) / tq + Cq;
    const int64_t nt = (int64_t)B * H * L.tph;
    L.ntotal = (int)((nt + 7) / 8 * 8);
    size_t o = 0;
    L.off_row = o; o += isg_align256((size_t)G * L.cap * sizeof(int32_t));
    L.off_bias = o; o += isg_align256((size_t)G * L.cap * sizeof(float));
    L.off_len = o; o += isg_align256((size_t)G * sizeof(int32_t));
    L.off_x = o; o += isg_align256((size_t)G * sizeof(int32_t));
    L.off_bmax = o; o += isg_align256((size_t)G * sizeof(float));
    L.off_kmax = o; o += isg_align256((size_t)B * H * sizeof(int));
    L.off_redo = o; o += isg_align256((size_t)L.ntotal * sizeof(int));
    L.off_table = o; o += isg_align256((size_t)L.ntotal * sizeof(int4));
    L.off_flist = o; o += isg_align256((size_t)L.ntotal * sizeof(int));
    L.off_nlist = o; o += isg_align256(sizeof(int));
    L.total = o;
    return L;
}

// Fast kernel (fixed per-row reference), then the rescaling kernel on the tiles
// the fast one flagged (rows whose logits all sit far below the bound).  Both
// walk the same 128-row tile table; the rare fallback keeps one query block per
// wave, where its running-maximum state fits the registers.
template <int D, int QB>
void launch_bf16(hipStream_t st, const Layout &Lq, const void *q_p, const void *k_p, const void *v_p, int N, int Cq,
                 const int4 *table, const int32_t *col_row, const float *col_bias, const int32_t *col_len,
                 const int32_t *col_x, const float *col_bmax, const int *kmax2, float scale_log2, void *o_p,
                 float *lse_p, const int32_t *perm_q, int *redo, int *flist, int *nlist, int32_t *nflag)
{
    if constexpr (D == 128 && kUsePingPong) {
        // fast pass over every tile pair, then the flagged tiles (listed in
        // ascending order) again with a running maximum, two per work-group like
        // the fast pass; work-groups past the list's end exit at once
        const int npairs = (Lq.ntotal / 2 + 7) / 8 * 8;
        attn_pp_kernel<D, false><<<npairs, 64 * kPPWaves, 0, st>>>(
            (const uint16_t *)q_p, (const uint16_t *)k_p, (const uint16_t *)v_p, N, Cq, table, Lq.ntotal, col_row,
            col_bias, col_len, col_x, col_bmax, kmax2, Lq.cap, scale_log2, (uint16_t *)o_p, lse_p, perm_q, redo,
            nullptr, nullptr);
        list_flags_kernel<<<1, 1024, 0, st>>>(redo, Lq.ntotal, flist, nlist, nflag);
        attn_pp_kernel<D, true><<<npairs, 64 * kPPWaves, 0, st>>>(
            (const uint16_t *)q_p, (const uint16_t *)k_p, (const uint16_t *)v_p, N, Cq, table, Lq.ntotal, col_row,
            col_bias, col_len, col_x, col_bmax, kmax2, Lq.cap, scale_log2, (uint16_t *)o_p, lse_p, perm_q, redo,
            flist, nlist);
    } else {
        (void)flist;
        (void)nlist;
        attn_bf16_kernel<D, true, QB><<<Lq.ntotal, 256 / QB, 0, st>>>(
            (const uint16_t *)q_p, (const uint16_t *)k_p, (const uint16_t *)v_p, N, Cq, table, Lq.ntotal, col_row,
            col_bias, col_len, col_x, col_bmax, kmax2, Lq.cap, scale_log2, (uint16_t *)o_p, lse_p, perm_q, redo,
            nullptr);
        attn_bf16_kernel<D, false, 1><<<std::min((Lq.ntotal + 63) / 64, kFallbackBlocks), 256, 0, st>>>(
            (const uint16_t *)q_p, (const uint16_t *)k_p, (const uint16_t *)v_p, N, Cq, table, Lq.ntotal, col_row,
            col_bias, col_len, col_x, col_bmax, kmax2, Lq.cap, scale_log2, (uint16_t *)o_p, lse_p, perm_q, redo,
            nflag);
    }
}

}  // namespace

extern "C" size_t isg_attention_workspace_size(int B, int H, int N, int Cq, int Ck, int m)
{
    (void)Ck;
    if (B < 1 || H < 1 || N < 1 || Cq < 1 || m < 0 || m > N) return 0;
    // the column map holds up to N exact columns plus the m samples per query group
    return layout(B, H, N, Cq, m, kTQ32).total;
}

extern "C" isg_status isg_attention(void *stream, const void *q_p, const void *k_p, const void *v_p,
                                    isg_dtype dt, int B, int H, int N, int d, int Cq, int Ck,
                                    const int32_t *q_offsets, const int32_t *k_offsets,
                                    const int32_t *exact_groups, const int32_t *n_exact,
                                    const int32_t *sample_idx, const float *sample_bias,
                                    const int32_t *n_sample, int m, float scale,
                                    const float *k_max_sqnorm, void *o_p, float *lse_p,
                                    const int32_t *perm_q, int32_t *n_fallback_tiles, void *workspace,
                                    size_t ws_bytes)
{
    ISG_REQUIRE(q_p && k_p && v_p && q_offsets && k_offsets && exact_groups && n_exact && n_sample && o_p,
                ISG_E_ARG, "isg_attention: null pointer argument");
    ISG_REQUIRE(m == 0 || (sample_idx && sample_bias), ISG_E_ARG,
                "isg_attention: sample_idx / sample_bias required when m > 0");
    ISG_REQUIRE(B >= 1 && H >= 1 && N >= 1, ISG_E_ARG, "isg_attention: B, H, N must be >= 1");
    ISG_REQUIRE((int64_t)B * H <= 65535, ISG_E_ARG, "isg_attention: B*H must be <= 65535 (got %lld)",
                (long long)B * H);
    ISG_REQUIRE(dt == ISG_F32 || dt == ISG_BF16, ISG_E_DTYPE, "isg_attention: dtype %d", (int)dt);
    ISG_REQUIRE(d == 64 || d == 128, ISG_E_UNSUPPORTED, "isg_attention: d=%d not built (64, 128)", d);
    ISG_REQUIRE(Cq >= 1 && Cq <= kMaxGroups && Ck >= 1 && Ck <= kMaxGroups, ISG_E_ARG,
                "isg_attention: Cq, Ck must be in [1, %d]", kMaxGroups);
    ISG_REQUIRE(m >= 0 && m <= N, ISG_E_ARG, "isg_attention: need 0 <= m <= N");
    ISG_REQUIRE((int64_t)N * d * 4 <= 0x7fffffff, ISG_E_ARG,
                "isg_attention: N*d too large for 32-bit row offsets (N=%d, d=%d)", N, d);
    ISG_REQUIRE(std::isfinite(scale) && scale > 0.0f, ISG_E_ARG,
                "isg_attention: scale must be finite and > 0 (the fixed per-row reference bounds the logits only "
                "for a positive scale)");
    ISG_REQUIRE(((uintptr_t)q_p & 15) == 0 && ((uintptr_t)k_p & 15) == 0 && ((uintptr_t)v_p & 15) == 0 &&
                    ((uintptr_t)o_p & 15) == 0,
                ISG_E_ARG, "isg_attention: q_p, k_p, v_p, o_p must be 16-byte aligned");
    const int tq = dt == ISG_BF16 ? kTQ : kTQ32;
    const Layout Lq = layout(B, H, N, Cq, m, tq);
    const size_t need = isg_attention_workspace_size(B, H, N, Cq, Ck, m);
    ISG_REQUIRE(workspace && ws_bytes >= need, ISG_E_WORKSPACE, "isg_attention: workspace %zu < %zu bytes",
                workspace ? ws_bytes : (size_t)0, need);
    const int64_t G = (int64_t)B * H * Cq;
    ISG_REQUIRE(G <= 0x7fffffff && (int64_t)B * H <= 0x7fffffff, ISG_E_ARG, "isg_attention: too many groups");
    hipStream_t st = (hipStream_t)stream;
    uint8_t *ws = (uint8_t *)workspace;
    int32_t *col_row = (int32_t *)(ws + Lq.off_row);
    float *col_bias = (float *)(ws + Lq.off_bias);
    int32_t *col_len = (int32_t *)(ws + Lq.off_len);
    int32_t *col_x = (int32_t *)(ws + Lq.off_x);
    float *col_bmax = (float *)(ws + Lq.off_bmax);
    int *kmax2 = (int *)(ws + Lq.off_kmax);
    // the per-head largest squared key norm: the caller's (from isg_cluster of K),
    // else the key-norm pass below fills the workspace copy
    const int *kmx = k_max_sqnorm ? reinterpret_cast<const int *>(k_max_sqnorm) : kmax2;
    int *redo = (int *)(ws + Lq.off_redo);
    int *flist = (int *)(ws + Lq.off_flist);
    int *nlist = (int *)(ws + Lq.off_nlist);
    int4 *table = (int4 *)(ws + Lq.off_table);
    columns_kernel<<<(unsigned)G, 256, 0, st>>>(k_offsets, exact_groups, n_exact, sample_idx, sample_bias,
                                               n_sample, Cq, Ck, m, scale, Lq.cap, col_row, col_bias, col_len, col_x,
                                               col_bmax);
    tile_table_kernel<<<B * H, 256, 0, st>>>(q_offsets, B * H, Cq, tq, Lq.tph, Lq.ntotal, table, redo, kmax2,
                                             n_fallback_tiles);
    const float scale_log2 = (float)((double)scale * 1.4426950408889634);
    if (dt == ISG_BF16) {
        const dim3 kgrid((unsigned)std::min((N + 255) / 256, 128), (unsigned)(B * H));
        if (d == 128) {
            if (!k_max_sqnorm) kmax_kernel<128><<<kgrid, 256, 0, st>>>((const uint16_t *)k_p, N, kmax2);
            launch_bf16<128, kQB>(st, Lq, q_p, k_p, v_p, N, Cq, table, col_row, col_bias, col_len, col_x, col_bmax,
                                  kmx, scale_log2, o_p, lse_p, perm_q, redo, flist, nlist, n_fallback_tiles);
        } else {
            if (!k_max_sqnorm) kmax_kernel<64><<<kgrid, 256, 0, st>>>((const uint16_t *)k_p, N, kmax2);
            launch_bf16<64, kQB>(st, Lq, q_p, k_p, v_p, N, Cq, table, col_row, col_bias, col_len, col_x, col_bmax,
                                 kmx, scale_log2, o_p, lse_p, perm_q, redo, flist, nlist, n_fallback_tiles);
        }
    } else {
        if (d == 128)
            attn_f32_kernel<128><<<Lq.ntotal, 256, 0, st>>>((const float *)q_p, (const float *)k_p,
                                                           (const float *)v_p, N, Cq, table, Lq.ntotal, col_row,
                                                           col_bias, col_len, Lq.cap, scale_log2, (float *)o_p,
                                                           lse_p, perm_q);
        else
            attn_f32_kernel<64><<<Lq.ntotal, 256, 0, st>>>((const float *)q_p, (const float *)k_p,
                                                          (const float *)v_p, N, Cq, table, Lq.ntotal, col_row,
                                                          col_bias, col_len, Lq.cap, scale_log2, (float *)o_p,
                                                          lse_p, perm_q);
    }
    return isg_check_launch("isg_attention");
}
