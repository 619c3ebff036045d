// isg_attention: one flash-style attention over the exact and sampled columns of
// every query group.
//
// Pages: InstaGen, acceptodds.com page, abstract (the sampled tokens are computed
// together with the top blocks in a single attention kernel, their scores
// reweighted for the whole skipped region); thelatestinai.com page, Figure 3(d)
// (the queries of a group share keys, so attention runs over dense blocks).
//
// Structure:
//   1. columns_kernel   per query group: the column list (row of K_p/V_p, offset
//                       in log2 units) = rows of the exact groups in ascending
//                       group order, then the samples, padded to a multiple of
//                       64 with offset -inf.
//   2. tile_table_kernel per head: (group, first row, end row) of every 128-row
//                       query tile; the launch walks tiles in an XCD-aware order
//                       so the tiles of one group share an L2.
//   3. attn_bf16_kernel 4 waves x 32 query rows; K/V tiles of 64 columns are
//                       gathered row by row into LDS (double buffered, one tile
//                       prefetched in registers); S^T = K Q^T and O^T += V^T P^T
//                       on v_mfma_f32_32x32x16_bf16 so each lane owns one query
//                       and the online softmax stays in registers.
//      attn_f32_kernel  fp32 inputs: plain VALU version of the same loop.
#include <cmath>

#include "isg_internal.h"

namespace {

constexpr int kTK = 64;          // columns per K/V tile
constexpr int kTQ = 128;         // query rows per bf16 work-group
constexpr int kTQ32 = 64;        // query rows per fp32 work-group
constexpr int kMaxGroups = 1024;
constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------------ prep
__global__ __launch_bounds__(256) void columns_kernel(const int32_t *k_offsets, const int32_t *exact_groups,
                                                      const int32_t *n_exact, const int32_t *sample_idx,
                                                      const float *sample_bias, const int32_t *n_sample,
                                                      int Cq, int Ck, int m, int64_t cap, int32_t *col_row,
                                                      float *col_bias, int32_t *col_len, int32_t *col_x)
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
            bias = sb[c - X] * kLog2e;
        }
        cr[c] = row;
        cb[c] = bias;
    }
    if (threadIdx.x == 0) {
        col_len[gi] = L;
        col_x[gi] = X;
    }
}

__global__ __launch_bounds__(256) void tile_table_kernel(const int32_t *q_offsets, int BH, int Cq, int tq,
                                                         int tph, int ntotal, int4 *table)
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
}

// ------------------------------------------------------------------ bf16 MFMA kernel
// Position of key k (0..63) inside a transposed V row: bits 2 and 3 swapped, so
// that the 8 keys one lane feeds to the P.V product are contiguous.
__device__ __forceinline__ int vt_pos(int k)
{
    return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// K/V rows of one 64-column tile held in registers between the global load and
// the LDS store (a struct passed by value so it stays in VGPRs).
template <int KIT> struct KVRegs {
    u32x4 k[KIT];
    u32x4 v[4];
};

template <int D, int KIT, int VTASK>
__device__ __forceinline__ KVRegs<KIT> kv_gload(const uint16_t *kh, const uint16_t *vh, const int *rows, int tid,
                                                 int vquad, int vchunk)
{
    constexpr int CPR = D / 8;
    KVRegs<KIT> r;
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
        const int e = it * 256 + tid;
        const int key = e / CPR, ch = e % CPR;
        r.k[it] = *reinterpret_cast<const u32x4 *>(kh + (int64_t)rows[key] * D + ch * 8);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) r.v[kk] = u32x4{0, 0, 0, 0};
    if (tid < VTASK) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            r.v[kk] = *reinterpret_cast<const u32x4 *>(vh + (int64_t)rows[vquad * 4 + kk] * D + vchunk * 8);
    }
    return r;
}

// K rows go to LDS as they are (rows padded to KSTR bytes); V goes transposed, one
// row per d, keys at swizzled positions, four keys (8 bytes) per store.
template <int D, int KIT, int VTASK>
__device__ __forceinline__ void kv_sstore(const KVRegs<KIT> &r, uint8_t *kb, int tid, int vquad, int vchunk)
{
    constexpr int CPR = D / 8;
    constexpr int KSTR = D * 2 + 16;
    constexpr int VSTR = kTK * 2 + 16;
    uint8_t *vb = kb + kTK * KSTR;
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
        const int e = it * 256 + tid;
        const int key = e / CPR, ch = e % CPR;
        *reinterpret_cast<u32x4 *>(kb + key * KSTR + ch * 16) = r.k[it];
    }
    if (tid < VTASK) {
        const uint32_t w0[4] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w};
        const uint32_t w1[4] = {r.v[1].x, r.v[1].y, r.v[1].z, r.v[1].w};
        const uint32_t w2[4] = {r.v[2].x, r.v[2].y, r.v[2].z, r.v[2].w};
        const uint32_t w3[4] = {r.v[3].x, r.v[3].y, r.v[3].z, r.v[3].w};
        const int pos = vt_pos(vquad * 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int w = e >> 1;
            uint32_t lo, hi;
            if (e & 1) {
                lo = (w0[w] >> 16) | (w1[w] & 0xFFFF0000u);
                hi = (w2[w] >> 16) | (w3[w] & 0xFFFF0000u);
            } else {
                lo = (w0[w] & 0xFFFFu) | (w1[w] << 16);
                hi = (w2[w] & 0xFFFFu) | (w3[w] << 16);
            }
            *reinterpret_cast<u32x2 *>(vb + (vchunk * 8 + e) * VSTR + pos * 2) = u32x2{lo, hi};
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bf16_kernel(
    const uint16_t *__restrict__ q_p, const uint16_t *__restrict__ k_p, const uint16_t *__restrict__ v_p,
    int N, int Cq, const int4 *__restrict__ table, int nblocks, const int32_t *__restrict__ col_row,
    const float *__restrict__ col_bias, const int32_t *__restrict__ col_len, const int32_t *__restrict__ col_x,
    int64_t cap, float scale_log2, uint16_t *__restrict__ o_p, float *__restrict__ lse_p)
{
    constexpr int NDS = D / 16;          // 16-wide d steps of S^T = K Q^T
    constexpr int NDB = D / 32;          // 32-row d blocks of O^T
    constexpr int KSTR = D * 2 + 16;     // bytes per K row in LDS
    constexpr int VSTR = kTK * 2 + 16;   // bytes per transposed V row (one d) in LDS
    constexpr int KBYTES = kTK * KSTR;
    constexpr int VBYTES = D * VSTR;
    constexpr int BUF = KBYTES + VBYTES;
    constexpr int CPR = D / 8;           // 16-byte chunks per row
    constexpr int KIT = kTK * CPR / 256; // K chunks per thread per tile
    constexpr int VTASK = 16 * CPR;      // (key quad, chunk) tasks per tile
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * BUF];
    __shared__ int idx_row[3][kTK];
    __shared__ __attribute__((aligned(16))) float idx_bias[3][kTK];

    const int lb = xcd_logical_block(blockIdx.x, nblocks);
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
    const uint16_t *kh = k_p + (int64_t)bh * N * D;
    const uint16_t *vh = v_p + (int64_t)bh * N * D;

    // Q^T fragment (B operand of S^T = K Q^T): lane owns query row l32 of its wave.
    const int qrow_raw = r0 + wave * 32 + l32;
    const int qrow = min(qrow_raw, r1 - 1);
    const bool wave_active = r0 + wave * 32 < r1;
    bf16x8 qf[NDS];
    {
        const uint16_t *qsrc = q_p + ((int64_t)bh * N + qrow) * D + hl * 8;
#pragma unroll
        for (int s = 0; s < NDS; ++s) qf[s] = *reinterpret_cast<const bf16x8 *>(qsrc + s * 16);
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

    const int vquad = tid & 15, vchunk = tid >> 4;
    KVRegs<KIT> kv = kv_gload<D, KIT, VTASK>(kh, vh, idx_row[0], tid, vquad, vchunk);
    kv_sstore<D, KIT, VTASK>(kv, smem, tid, vquad, vchunk);
    __syncthreads();

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    for (int t = 0; t < T; ++t) {
        const int cur = t & 1;
        const bool more = t + 1 < T;
        if (more) kv = kv_gload<D, KIT, VTASK>(kh, vh, idx_row[(t + 1) % 3], tid, vquad, vchunk);
        int32_t nrow = 0;
        float nbias = 0.0f;
        const bool fetch2 = wave == 0 && t + 2 < T;
        if (fetch2) {
            nrow = crow[(int64_t)(t + 2) * kTK + lane];
            nbias = cbias[(int64_t)(t + 2) * kTK + lane];
        }
        if (wave_active) {
            const uint8_t *kb = smem + cur * BUF;
            const uint8_t *vb = kb + KBYTES;
            f32x16 sacc[2];
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb2][r] = 0.0f;
#pragma unroll
            for (int s = 0; s < NDS; ++s) {
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kb + (kb2 * 32 + l32) * KSTR + s * 32 + hl * 16);
                    sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb2], 0, 0, 0);
                }
            }
            // Logits in log2 units; lane holds keys kb2*32 + 8g + 4hl + e (e = 0..3) of
            // its query.  A tile made only of exact columns has no offsets.
            const int slot = t % 3;
            const bool exact_tile = (t + 1) * kTK <= X;
            float mx;
            if (exact_tile) {
                float mr = sacc[0][0];
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mr = fmaxf(mr, sacc[kb2][r]);
                mx = mr * scale_log2;
            } else {
                mx = -INFINITY;
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 bv = *reinterpret_cast<const f32x4 *>(&idx_bias[slot][kb2 * 32 + g * 8 + hl * 4]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float v = fmaf(sacc[kb2][4 * g + e], scale_log2, bv[e]);
                            sacc[kb2][4 * g + e] = v;
                            mx = fmaxf(mx, v);
                        }
                    }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            // Lazy rescale: O and l stay relative to m_run until some lane's maximum
            // exceeds it by more than 8 (weights up to 2^8 are safe in bf16 and fp32).
            if (__any(mx > m_run + 8.0f)) {
                const float m_new = fmaxf(m_run, mx);
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
                m_run = m_new;
            }
            const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8 pb;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v = sacc[s >> 1][8 * (s & 1) + e];
                    const float p = exact_tile ? __builtin_amdgcn_exp2f(fmaf(v, scale_log2, -m_run))
                                               : __builtin_amdgcn_exp2f(v - m_run);
                    pb[e] = (__bf16)p;
                }
                // row sum of the rounded weights, the same ones P.V uses
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const bf16x2 pp = {pb[e], pb[e + 1]};
                    l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run, false);
                }
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vb + (db * 32 + l32) * VSTR + (s * 16 + hl * 8) * 2);
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[db], 0, 0, 0);
                }
            }
        }
        if (more) kv_sstore<D, KIT, VTASK>(kv, smem + (cur ^ 1) * BUF, tid, vquad, vchunk);
        if (fetch2) {
            idx_row[(t + 2) % 3][lane] = nrow;
            idx_bias[(t + 2) % 3][lane] = nbias;
        }
        __syncthreads();
    }

    if (!wave_active) return;
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.0f / l_tot;
    if (qrow_raw < r1) {
        uint16_t *orow = o_p + ((int64_t)bh * N + qrow_raw) * D;
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
        if (lse_p && hl == 0) lse_p[(int64_t)bh * N + qrow_raw] = (m_run + log2f(l_tot)) * 0.6931471805599453f;
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
                                                       float *__restrict__ lse_p)
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
            const float xl = fmaf(s, scale_log2, bs[kk]);
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
#pragma unroll
        for (int e = 0; e < DQ; ++e) o_p[((int64_t)bh * N + qrow_raw) * D + part * DQ + e] = o[e] * inv;
        if (lse_p && part == 0) lse_p[(int64_t)bh * N + qrow_raw] = (m_run + log2f(l_run)) * 0.6931471805599453f;
    }
}

struct Layout {
    int64_t cap;       // columns per group in the column map
    int tph;           // tile slots per head
    int ntotal;        // launched blocks (multiple of 8)
    size_t off_row, off_bias, off_len, off_x, off_table, total;
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
    L.off_table = o; o += isg_align256((size_t)L.ntotal * sizeof(int4));
    L.total = o;
    return L;
}

}  // namespace

extern "C" size_t isg_attention_workspace_size(int B, int H, int N, int Cq, int Ck)
{
    (void)Ck;
    if (B < 1 || H < 1 || N < 1 || Cq < 1) return 0;
    // the column map is sized for m = N (the largest sample a call may ask for)
    return layout(B, H, N, Cq, N, kTQ32).total;
}

extern "C" isg_status isg_attention(void *stream, const void *q_p, const void *k_p, const void *v_p,
                                    isg_dtype dt, int B, int H, int N, int d, int Cq, int Ck,
                                    const int32_t *q_offsets, const int32_t *k_offsets,
                                    const int32_t *exact_groups, const int32_t *n_exact,
                                    const int32_t *sample_idx, const float *sample_bias,
                                    const int32_t *n_sample, int m, float scale, void *o_p, float *lse_p,
                                    void *workspace, size_t ws_bytes)
{
    ISG_REQUIRE(q_p && k_p && v_p && q_offsets && k_offsets && exact_groups && n_exact && n_sample && o_p,
                ISG_E_ARG, "isg_attention: null pointer argument");
    ISG_REQUIRE(m == 0 || (sample_idx && sample_bias), ISG_E_ARG,
                "isg_attention: sample_idx / sample_bias required when m > 0");
    ISG_REQUIRE(B >= 1 && H >= 1 && N >= 1, ISG_E_ARG, "isg_attention: B, H, N must be >= 1");
    ISG_REQUIRE(dt == ISG_F32 || dt == ISG_BF16, ISG_E_DTYPE, "isg_attention: dtype %d", (int)dt);
    ISG_REQUIRE(d == 64 || d == 128, ISG_E_UNSUPPORTED, "isg_attention: d=%d not built (64, 128)", d);
    ISG_REQUIRE(Cq >= 1 && Cq <= kMaxGroups && Ck >= 1 && Ck <= kMaxGroups, ISG_E_ARG,
                "isg_attention: Cq, Ck must be in [1, %d]", kMaxGroups);
    ISG_REQUIRE(m >= 0 && m <= N, ISG_E_ARG, "isg_attention: need 0 <= m <= N");
    ISG_REQUIRE(std::isfinite(scale), ISG_E_ARG, "isg_attention: scale must be finite");
    ISG_REQUIRE(((uintptr_t)q_p & 15) == 0 && ((uintptr_t)k_p & 15) == 0 && ((uintptr_t)v_p & 15) == 0 &&
                    ((uintptr_t)o_p & 15) == 0,
                ISG_E_ARG, "isg_attention: q_p, k_p, v_p, o_p must be 16-byte aligned");
    const int tq = dt == ISG_BF16 ? kTQ : kTQ32;
    const Layout Lq = layout(B, H, N, Cq, m, tq);
    const size_t need = isg_attention_workspace_size(B, H, N, Cq, Ck);
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
    int4 *table = (int4 *)(ws + Lq.off_table);
    columns_kernel<<<(unsigned)G, 256, 0, st>>>(k_offsets, exact_groups, n_exact, sample_idx, sample_bias,
                                               n_sample, Cq, Ck, m, Lq.cap, col_row, col_bias, col_len, col_x);
    tile_table_kernel<<<B * H, 256, 0, st>>>(q_offsets, B * H, Cq, tq, Lq.tph, Lq.ntotal, table);
    const float scale_log2 = (float)((double)scale * 1.4426950408889634);
    if (dt == ISG_BF16) {
        if (d == 128)
            attn_bf16_kernel<128><<<Lq.ntotal, 256, 0, st>>>(
                (const uint16_t *)q_p, (const uint16_t *)k_p, (const uint16_t *)v_p, N, Cq, table, Lq.ntotal,
                col_row, col_bias, col_len, col_x, Lq.cap, scale_log2, (uint16_t *)o_p, lse_p);
        else
            attn_bf16_kernel<64><<<Lq.ntotal, 256, 0, st>>>(
                (const uint16_t *)q_p, (const uint16_t *)k_p, (const uint16_t *)v_p, N, Cq, table, Lq.ntotal,
                col_row, col_bias, col_len, col_x, Lq.cap, scale_log2, (uint16_t *)o_p, lse_p);
    } else {
        if (d == 128)
            attn_f32_kernel<128><<<Lq.ntotal, 256, 0, st>>>((const float *)q_p, (const float *)k_p,
                                                           (const float *)v_p, N, Cq, table, Lq.ntotal, col_row,
                                                           col_bias, col_len, Lq.cap, scale_log2, (float *)o_p,
                                                           lse_p);
        else
            attn_f32_kernel<64><<<Lq.ntotal, 256, 0, st>>>((const float *)q_p, (const float *)k_p,
                                                          (const float *)v_p, N, Cq, table, Lq.ntotal, col_row,
                                                          col_bias, col_len, Lq.cap, scale_log2, (float *)o_p,
                                                          lse_p);
    }
    return isg_check_launch("isg_attention");
}
