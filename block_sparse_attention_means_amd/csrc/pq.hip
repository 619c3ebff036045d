// isg_pq_votes: product-quantised per-query voting for the exact set.
//
// Pages: InstaGen, acceptodds.com page, abstract (queries and keys are product-
// quantised so that block scores are cheap enough for every query rather than
// only the centroid; each query votes for its top blocks; the cluster attends to
// the blocks with the most votes).  The pages give no formula; the reading:
//   Kbar_{j,s} = mean over the keys of group j of their subspace-s codeword
//                (fp64 sum in permuted row order, one division, rounded to fp32),
//   M_s[a][j]  = scale * <cw^q_{s,a}, Kbar_{j,s}>   (fp32 fma chain over the dims),
//   score(q,j) = sum_s M_s[code_s(q)][j]            (fp32, s ascending),
//   every query takes the exact-set rule over its own ranking (score desc, j asc)
//   and votes for the groups it takes; votes[i][j] counts the votes of group i.
// Codes come from isg_cluster on each d/P-dim subspace (Cc codewords).
//
// The per-query rule is evaluated without sorting: with C(u) = sum of n_j over
// groups whose order-preserving score bits are >= u, the groups strictly above
// u* = max{u : C(u) > E} are all taken (their total is <= E), and the groups at
// u* are then taken in ascending j while the running count stays <= E (the first
// group of the ranking always).  u* is found by bisection over the 32-bit key
// space with one wave-wide sum per step.
#include <cmath>

#include "isg_internal.h"

namespace {

constexpr int kMaxGroups = 1024;
constexpr int kChunk = 256;  // rows staged per round in pq_kbar_kernel

// One block per (key group, head); thread e owns element e of Kbar.  Rows are
// summed in permuted order, exactly as the definition reads.
__global__ __launch_bounds__(256) void pq_kbar_kernel(const int32_t *k_codes, const float *k_cb,
                                                      const int32_t *perm_k, const int32_t *k_offsets, int B,
                                                      int H, int N, int P, int Cc, int ds, int Ck, float *kbar)
{
    __shared__ int codes[kChunk * 16];  // [P][kChunk], P <= 16 when d <= 256 and ds >= 16... see launch check
    const int j = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
    const int d = P * ds, tid = threadIdx.x;
    const int32_t *ko = k_offsets + (int64_t)bh * (Ck + 1);
    const int r0 = ko[j], r1 = ko[j + 1];
    const int s = tid / ds, ee = tid % ds;
    const float *cb = k_cb + (((int64_t)s * B + b) * H + h) * (int64_t)Cc * ds + ee;
    double acc = 0.0;
    for (int c0 = r0; c0 < r1; c0 += kChunk) {
        const int nc = min(kChunk, r1 - c0);
        __syncthreads();
        for (int x = tid; x < nc * P; x += blockDim.x) {
            const int ss = x / nc, rr = x % nc;
            const int t = perm_k[(int64_t)bh * N + c0 + rr];
            codes[ss * kChunk + rr] = k_codes[(((int64_t)ss * B + b) * H + h) * N + t];
        }
        __syncthreads();
        if (tid < d) {
#pragma unroll 8
            for (int rr = 0; rr < nc; ++rr) acc += (double)cb[(int64_t)codes[s * kChunk + rr] * ds];
        }
    }
    if (tid < d) kbar[((int64_t)bh * Ck + j) * d + tid] = r1 > r0 ? (float)(acc / (double)(r1 - r0)) : 0.0f;
}

__global__ __launch_bounds__(256) void pq_tables_kernel(const float *q_cb, const float *kbar, int B, int H, int P,
                                                        int Cc, int ds, int Ck, float scale, float *tables)
{
    const int sa = blockIdx.y;  // s * Cc + a
    const int bh = blockIdx.z, b = bh / H, h = bh % H;
    const int s = sa / Cc, a = sa % Cc;
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= Ck) return;
    const int d = P * ds;
    const float *cw = q_cb + ((((int64_t)s * B + b) * H + h) * Cc + a) * ds;
    const float *kb = kbar + ((int64_t)bh * Ck + j) * d + s * ds;
    float acc = 0.0f;
    for (int e = 0; e < ds; ++e) acc = __fmaf_rn(cw[e], kb[e], acc);
    tables[(((int64_t)bh * P + s) * Cc + a) * Ck + j] = __fmul_rn(acc, scale);
}

// The same tables for subspaces of at most 32 dims: a thread keeps its key group's
// Kbar slice in registers and walks the codewords, staged 64 at a time in LDS, so
// every Kbar element is read once and the table rows are written coalesced.
template <int DS>
__global__ __launch_bounds__(256) void pq_tables_tiled_kernel(const float *q_cb, const float *kbar, int B, int H,
                                                              int P, int Cc, int Ck, float scale, float *tables)
{
    constexpr int AT = 64;  // codewords per LDS tile
    __shared__ float cws[AT][DS];
    const int s = blockIdx.y, bh = blockIdx.z, b = bh / H, h = bh % H;
    const int j = blockIdx.x * 256 + threadIdx.x;
    const int d = P * DS;
    float kb[DS];
#pragma unroll
    for (int e = 0; e < DS; ++e) kb[e] = j < Ck ? kbar[((int64_t)bh * Ck + j) * d + s * DS + e] : 0.0f;
    const float *cwb = q_cb + (((int64_t)s * B + b) * H + h) * (int64_t)Cc * DS;
    float *out = tables + ((int64_t)bh * P + s) * (int64_t)Cc * Ck;
    for (int a0 = 0; a0 < Cc; a0 += AT) {
        const int na = min(AT, Cc - a0);
        __syncthreads();
        for (int x = threadIdx.x; x < na * DS; x += 256) cws[x / DS][x % DS] = cwb[(int64_t)a0 * DS + x];
        __syncthreads();
        if (j < Ck) {
            for (int a = 0; a < na; ++a) {
                float acc = 0.0f;
#pragma unroll
                for (int e = 0; e < DS; ++e) acc = __fmaf_rn(cws[a][e], kb[e], acc);
                out[(int64_t)(a0 + a) * Ck + j] = __fmul_rn(acc, scale);
            }
        }
    }
}

// Order-preserving bits of a float (+0 and -0 map to the same key).
__device__ __forceinline__ uint32_t orderable(float f)
{
    const uint32_t u = f == 0.0f ? 0u : __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Sum over the 64 lanes: DPP inside each row of 16, then the four row totals.
__device__ __forceinline__ int wave_sum(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
    return __builtin_amdgcn_readlane(v, 15) + __builtin_amdgcn_readlane(v, 31) +
           __builtin_amdgcn_readlane(v, 47) + __builtin_amdgcn_readlane(v, 63);
}

// One wave per query; lane owns key groups j = k*64 + lane, k < KPL.  The 8
// waves of a block share a query group, and logical blocks are laid out so that
// one XCD works on consecutive query groups of the same head: an XCD then holds
// about one head's groups at a time, so the head's tables (P*Cc*Ck fp32, 4 MB at
// 8 x 256 x 500) stay in its L2.
constexpr int kVoteWaves = 8;
constexpr int kPBatch = 8;  // subspaces whose table rows are in flight together

template <int KPL>
__global__ __launch_bounds__(64 * kVoteWaves) void pq_votes_kernel(const int32_t *q_codes, const float *tables,
                                                       const int32_t *perm_q, const int32_t *q_offsets,
                                                       const int32_t *k_offsets, int B, int H, int N, int P,
                                                       int Cc, int Cq, int Ck, int exact_keys, int nblocks,
                                                       int32_t *votes)
{
    __shared__ int cnt[KPL * 64];
    __shared__ int nsz[KPL * 64];
    const int nb8 = gridDim.x;
    const int lb = xcd_logical_block(blockIdx.x, nb8);
    if (lb >= nblocks) return;
    const int i = lb % Cq, bh = lb / Cq, b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int32_t *ko = k_offsets + (int64_t)bh * (Ck + 1);
    for (int j = tid; j < KPL * 64; j += 64 * kVoteWaves) {
        cnt[j] = 0;
        nsz[j] = j < Ck ? ko[j + 1] - ko[j] : 0;
    }
    __syncthreads();
    int nk[KPL], vk[KPL];
    int part = 0;
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
        nk[k] = nsz[k * 64 + lane];
        vk[k] = 0;
        part += nk[k];
    }
    const int total = wave_sum(part);
    const int E = exact_keys;
    const int32_t *qo = q_offsets + (int64_t)bh * (Cq + 1);
    const float *tb = tables + (int64_t)bh * P * Cc * Ck;
    const int r_end = qo[i + 1];
    if (total <= E) {  // every non-empty group fits every query's budget
        for (int r = qo[i] + wave; r < r_end; r += kVoteWaves)
#pragma unroll
            for (int k = 0; k < KPL; ++k) vk[k] += nk[k] > 0;
    }
    const int32_t *qcode = q_codes + ((int64_t)b * H + h) * N;  // + s*B*H*N + t
    const int64_t sstride = (int64_t)B * H * N;
    // codes of the next query are fetched while the current one runs its bisection
    int codes[kPBatch];
    int r = qo[i] + wave;
    if (total > E && r < r_end) {
        const int t = perm_q[(int64_t)bh * N + r];
#pragma unroll
        for (int s = 0; s < kPBatch; ++s) codes[s] = s < P ? qcode[s * sstride + t] : 0;
    }
    for (; total > E && r < r_end; r += kVoteWaves) {
        // this query's table rows, all issued before any is added (rows of the
        // first kPBatch subspaces; further subspaces in batches of kPBatch)
        float sc[KPL];
#pragma unroll
        for (int k = 0; k < KPL; ++k) sc[k] = 0.0f;
        for (int s0 = 0; s0 < P; s0 += kPBatch) {
            if (s0 > 0) {
                const int t = perm_q[(int64_t)bh * N + r];
#pragma unroll
                for (int s = 0; s < kPBatch; ++s) codes[s] = s0 + s < P ? qcode[(s0 + s) * sstride + t] : 0;
            }
            float rv[kPBatch][KPL];
#pragma unroll
            for (int s = 0; s < kPBatch; ++s) {
                const float *row = tb + ((int64_t)(s0 + s) * Cc + codes[s]) * Ck + lane;
#pragma unroll
                for (int k = 0; k < KPL; ++k)
                    rv[s][k] = (s0 + s < P && k * 64 + lane < Ck) ? row[k * 64] : 0.0f;
            }
#pragma unroll
            for (int s = 0; s < kPBatch; ++s)
                if (s0 + s < P) {
#pragma unroll
                    for (int k = 0; k < KPL; ++k)
                        if (k * 64 + lane < Ck) sc[k] = __fadd_rn(sc[k], rv[s][k]);
                }
        }
        if (r + kVoteWaves < r_end) {
            const int tn = perm_q[(int64_t)bh * N + r + kVoteWaves];
#pragma unroll
            for (int s = 0; s < kPBatch; ++s) codes[s] = s < P ? qcode[s * sstride + tn] : 0;
        }
        uint32_t ok[KPL];
#pragma unroll
        for (int k = 0; k < KPL; ++k) ok[k] = orderable(sc[k]);
        // bisection: lo keeps C(lo) > E, hi keeps C(hi) <= E (C(2^32) = 0)
        uint32_t lo = 0;
        uint64_t hi = 1ull << 32;
        int above = 0;  // C(hi)
        for (int it = 0; it < 32; ++it) {
            const uint32_t mid = lo + (uint32_t)((hi - lo) >> 1);
            int p = 0;
#pragma unroll
            for (int k = 0; k < KPL; ++k) p += ok[k] >= mid ? nk[k] : 0;
            const int c = wave_sum(p);
            if (c > E) {
                lo = mid;
            } else {
                hi = mid;
                above = c;
            }
        }
        uint64_t take[KPL], tie[KPL];
#pragma unroll
        for (int k = 0; k < KPL; ++k) {
            take[k] = __ballot(nk[k] > 0 && ok[k] > lo);
            tie[k] = __ballot(nk[k] > 0 && ok[k] == lo);
        }
        int cum = above;
        bool first = above == 0;  // nothing taken yet
        for (;;) {
            int j = -1;
#pragma unroll
            for (int k = 0; k < KPL; ++k)
                if (j < 0 && tie[k] != 0) j = k * 64 + __builtin_ctzll(tie[k]);
            if (j < 0) break;
            const int nj = nsz[j];
            if (!first && cum + nj > E) break;
            cum += nj;
            first = false;
#pragma unroll
            for (int k = 0; k < KPL; ++k)
                if (k == (j >> 6)) {
                    take[k] |= 1ull << (j & 63);
                    tie[k] &= ~(1ull << (j & 63));
                }
        }
#pragma unroll
        for (int k = 0; k < KPL; ++k) vk[k] += (int)((take[k] >> lane) & 1ull);
    }
#pragma unroll
    for (int k = 0; k < KPL; ++k)
        if (vk[k]) atomicAdd(&cnt[k * 64 + lane], vk[k]);
    __syncthreads();
    for (int j = tid; j < Ck; j += 64 * kVoteWaves) votes[((int64_t)bh * Cq + i) * Ck + j] = cnt[j];
}

template <int KPL>
void launch_votes(hipStream_t st, const int32_t *q_codes, const float *tables, const int32_t *perm_q,
                  const int32_t *q_offsets, const int32_t *k_offsets, int B, int H, int N, int P, int Cc, int Cq,
                  int Ck, int E, int32_t *votes)
{
    const int nblocks = B * H * Cq;
    const int nb8 = (nblocks + 7) & ~7;
    pq_votes_kernel<KPL><<<nb8, 64 * kVoteWaves, 0, st>>>(q_codes, tables, perm_q, q_offsets, k_offsets, B, H, N, P, Cc, Cq,
                                              Ck, E, nblocks, votes);
}

}  // namespace

extern "C" isg_status isg_pq_votes(void *stream, const int32_t *q_codes, const float *q_codebooks,
                                   const int32_t *k_codes, const float *k_codebooks, const int32_t *perm_q,
                                   const int32_t *q_offsets, const int32_t *perm_k, const int32_t *k_offsets,
                                   int B, int H, int N, int d, int P, int Cc, int Cq, int Ck, int exact_keys,
                                   float scale, float *kbar, float *tables, int32_t *votes)
{
    ISG_REQUIRE(q_codes && q_codebooks && k_codes && k_codebooks && perm_q && q_offsets && perm_k && k_offsets &&
                    kbar && tables && votes,
                ISG_E_ARG, "isg_pq_votes: null pointer argument");
    ISG_REQUIRE(B >= 1 && H >= 1 && N >= 1, ISG_E_ARG, "isg_pq_votes: B, H, N must be >= 1");
    ISG_REQUIRE(d >= 1 && d <= 256 && P >= 1 && P <= 16 && d % P == 0, ISG_E_ARG,
                "isg_pq_votes: need d <= 256, 1 <= P <= 16, P | d (got d=%d P=%d)", d, P);
    ISG_REQUIRE(Cc >= 1 && Cc <= 4096, ISG_E_ARG, "isg_pq_votes: Cc must be in [1, 4096] (got %d)", Cc);
    ISG_REQUIRE(Cq >= 1 && Cq <= kMaxGroups && Ck >= 1 && Ck <= kMaxGroups, ISG_E_ARG,
                "isg_pq_votes: Cq, Ck must be in [1, %d]", kMaxGroups);
    ISG_REQUIRE(exact_keys >= 0, ISG_E_ARG, "isg_pq_votes: exact_keys must be >= 0");
    ISG_REQUIRE(std::isfinite(scale), ISG_E_ARG, "isg_pq_votes: scale must be finite");
    const int64_t BH = (int64_t)B * H;
    ISG_REQUIRE(BH <= 65535 && (int64_t)P * Cc <= 65535 && BH * Cq <= (1 << 30), ISG_E_ARG,
                "isg_pq_votes: grid too large");
    hipStream_t st = (hipStream_t)stream;
    const int ds = d / P;
    const int kthreads = (d + 63) & ~63;
    pq_kbar_kernel<<<dim3(Ck, (unsigned)BH), kthreads, 0, st>>>(k_codes, k_codebooks, perm_k, k_offsets, B, H, N, P,
                                                               Cc, ds, Ck, kbar);
    const dim3 tgrid((Ck + 255) / 256, P, (unsigned)BH);
    if (ds == 16)
        pq_tables_tiled_kernel<16><<<tgrid, 256, 0, st>>>(q_codebooks, kbar, B, H, P, Cc, Ck, scale, tables);
    else if (ds == 8)
        pq_tables_tiled_kernel<8><<<tgrid, 256, 0, st>>>(q_codebooks, kbar, B, H, P, Cc, Ck, scale, tables);
    else if (ds == 32)
        pq_tables_tiled_kernel<32><<<tgrid, 256, 0, st>>>(q_codebooks, kbar, B, H, P, Cc, Ck, scale, tables);
    else
        pq_tables_kernel<<<dim3((Ck + 255) / 256, P * Cc, (unsigned)BH), 256, 0, st>>>(q_codebooks, kbar, B, H, P,
                                                                                      Cc, ds, Ck, scale, tables);
    if (Ck <= 64)
        launch_votes<1>(st, q_codes, tables, perm_q, q_offsets, k_offsets, B, H, N, P, Cc, Cq, Ck, exact_keys, votes);
    else if (Ck <= 128)
        launch_votes<2>(st, q_codes, tables, perm_q, q_offsets, k_offsets, B, H, N, P, Cc, Cq, Ck, exact_keys, votes);
    else if (Ck <= 256)
        launch_votes<4>(st, q_codes, tables, perm_q, q_offsets, k_offsets, B, H, N, P, Cc, Cq, Ck, exact_keys, votes);
    else if (Ck <= 512)
        launch_votes<8>(st, q_codes, tables, perm_q, q_offsets, k_offsets, B, H, N, P, Cc, Cq, Ck, exact_keys, votes);
    else
        launch_votes<16>(st, q_codes, tables, perm_q, q_offsets, k_offsets, B, H, N, P, Cc, Cq, Ck, exact_keys,
                         votes);
    return isg_check_launch("isg_pq_votes");
}
