// isg_pq_votes: product-quantised per-query voting for the exact set.
//
// Pages: InstaGen, acceptodds.com page, abstract (product-quantised Q and K make
// block scores affordable for every query, not only the centroid; each query
// picks its own top blocks and the group keeps the blocks picked most often).  The pages give no formula; the reading:
//   Kbar_{j,s} = mean over the keys of group j of their subspace-s codeword
//                (fp64 sum in permuted row order, one division, rounded to fp32),
//   M_s[a][j]  = scale * <cw^q_{s,a}, Kbar_{j,s}>   (fp32 fma chain over the dims),
//   score(q,j) = sum_s M_s[code_s(q)][j]            (fp32, s ascending),
//   every query takes the exact-set rule over its own ranking (score desc, j asc)
//   and votes for the groups it takes; votes[i][j] counts the votes of group i.
// Codes come from isg_pq_codebooks: k-means of each d/P-dim subspace (Cc codewords).
//
// The per-query rule is evaluated without sorting: with C(u) = sum of n_j over
// groups whose order-preserving score bits are >= u, the groups strictly above
// u* = max{u : C(u) > E} are all taken (their total is <= E), and the groups at
// u* are then taken in ascending j while the running count stays <= E (the first
// group of the ranking always).  u* is found by a radix selection over the 32-bit
// keys (radix_threshold below).
#include <algorithm>
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

// Work split: a work-group takes kVoteChunk consecutive queries of one head in
// the permuted (query-group) order, kVoteChunk / kVoteWaves per wave, so every
// work-group does the same work however unequal the query groups are.  A wave
// keeps its votes per lane (lane owns key groups j = k*64 + lane, k < KPL) for
// the query group it is in and adds them to votes[i][j] with integer atomics
// when its queries move to the next group and at its end (integer sums: the
// result does not depend on the order).  Logical blocks are laid out so that one
// XCD works on consecutive chunks of the same head: an XCD then holds about one
// head at a time, so the head's tables (P*Cc*Ck fp32, 4 MB at 8 x 256 x 500)
// stay in its L2.
constexpr int kVoteWaves = 8;
constexpr int kVoteQPW = 16;  // queries per wave
constexpr int kVoteChunk = kVoteWaves * kVoteQPW;
constexpr int kPBatch = 8;  // subspaces whose codes are fetched together
constexpr int kRowSplit = 2;  // parts of a batch whose table rows are in flight together

__device__ __forceinline__ uint32_t wave_min(uint32_t v)
{
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
    return min(min((uint32_t)__builtin_amdgcn_readlane(v, 15), (uint32_t)__builtin_amdgcn_readlane(v, 31)),
               min((uint32_t)__builtin_amdgcn_readlane(v, 47), (uint32_t)__builtin_amdgcn_readlane(v, 63)));
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
    return max(max((uint32_t)__builtin_amdgcn_readlane(v, 15), (uint32_t)__builtin_amdgcn_readlane(v, 31)),
               max((uint32_t)__builtin_amdgcn_readlane(v, 47), (uint32_t)__builtin_amdgcn_readlane(v, 63)));
}

constexpr int kCountBits = 20;  // sizes below 2^20, counts up to 1024: sums stay below 2^31
constexpr int kCountMask = (1 << kCountBits) - 1;

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t *p, int64_t n)
{
    for (int64_t e = blockIdx.x * 256ll + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) p[e] = 0;
}

// The exact-set threshold of one query: with C(u) = sum of n_j over the
// non-empty groups whose order-preserving score key is >= u, find u* = max{u :
// C(u) > E} (C(min key) = total > E) and C(u* + 1).  Radix selection from the
// highest bit in which the keys differ, 8 bits a pass: each pass sums n_j per
// digit over the groups that still match the digits chosen so far (LDS atomics
// into this wave's 256-bin histogram), and the digit taken is the largest whose
// suffix sum, plus the sizes already above, exceeds E -- so the chosen prefix is
// always the largest u with C(u) > E among the keys decided so far.  With packed
// sizes (total < 2^kCountBits) every bin also counts its groups, and a pass that
// leaves one group in the chosen bin ends the search: u* is that group's key.
template <int KPL>
__device__ __forceinline__ void radix_threshold(const uint32_t (&ok)[KPL], const int (&nk)[KPL],
                                                const int (&nkp)[KPL], bool packed, int E, int *hist, int lane,
                                                uint32_t &thr, int &above)
{
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int k = 0; k < KPL; ++k)
        if (nk[k] > 0) {
            kmin = min(kmin, ok[k]);
            kmax = max(kmax, ok[k]);
        }
    kmin = wave_min(kmin);
    kmax = wave_max(kmax);
    const uint32_t diff = kmin ^ kmax;
    int pos = diff == 0u ? 0 : 32 - __builtin_clz(diff);  // bits [0, pos) are undecided
    uint32_t prefix = pos == 32 ? 0u : (kmin >> pos) << pos;
    int ab = 0;  // packed sum of the groups above the prefix's range
    while (pos > 0) {
        const int nb = min(8, pos), shift = pos - nb;
        // clear, count (one wave: its LDS operations take effect in program order)
        *reinterpret_cast<int4 *>(&hist[4 * lane]) = make_int4(0, 0, 0, 0);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int k = 0; k < KPL; ++k) {
            const bool alive = nk[k] > 0 && ((uint64_t)ok[k] >> pos) == ((uint64_t)prefix >> pos);
            if (alive) atomicAdd(&hist[(ok[k] >> shift) & ((1u << nb) - 1u)], nkp[k]);
        }
        __builtin_amdgcn_wave_barrier();
        const int4 h = *reinterpret_cast<const int4 *>(&hist[4 * lane]);
        // suffix sums over the bins: s_i = bins >= 4 lane + i of this lane, plus the lanes above
        const int s3 = h.w, s2 = s3 + h.z, s1 = s2 + h.y, s0 = s1 + h.x;
        const int incl = wave_inclusive_scan(s0);
        const int rest = __builtin_amdgcn_readlane(incl, 63) - incl;  // bins of the lanes above
        const int c0 = ab + rest + s0, c1 = ab + rest + s1, c2 = ab + rest + s2, c3 = ab + rest + s3;
        auto wt = [&](int v) { return packed ? (v & kCountMask) : v; };
        // C is non-increasing in the digit, so the digits with C > E are 0 .. d*
        const int dstar = __popcll(__ballot(wt(c0) > E)) + __popcll(__ballot(wt(c1) > E)) +
                          __popcll(__ballot(wt(c2) > E)) + __popcll(__ballot(wt(c3) > E)) - 1;
        // C(prefix . d*) and C(prefix . (d* + 1)) (the latter is ab when d* is the last bin)
        const int ls = dstar >> 2, is = dstar & 3;
        const int cs = is == 0 ? __builtin_amdgcn_readlane(c0, ls) : is == 1 ? __builtin_amdgcn_readlane(c1, ls)
                     : is == 2 ? __builtin_amdgcn_readlane(c2, ls) : __builtin_amdgcn_readlane(c3, ls);
        const int ln = (dstar + 1) >> 2, in = (dstar + 1) & 3;
        int cn = ab;
        if (dstar + 1 < (1 << nb))
            cn = in == 0 ? __builtin_amdgcn_readlane(c0, ln) : in == 1 ? __builtin_amdgcn_readlane(c1, ln)
               : in == 2 ? __builtin_amdgcn_readlane(c2, ln) : __builtin_amdgcn_readlane(c3, ln);
        prefix |= (uint32_t)dstar << shift;
        ab = cn;
        pos = shift;
        if (packed && pos > 0 && ((cs - cn) >> kCountBits) == 1) {
            // one group left in the chosen bin: its key is the threshold
#pragma unroll
            for (int k = 0; k < KPL; ++k) {
                const uint64_t m = __ballot(nk[k] > 0 && ((uint64_t)ok[k] >> pos) == ((uint64_t)prefix >> pos));
                if (m) prefix = __builtin_amdgcn_readlane(ok[k], __builtin_ctzll(m));
            }
            pos = 0;
        }
    }
    thr = prefix;
    above = packed ? (ab & kCountMask) : ab;
}

template <int KPL>
__device__ __forceinline__ void flush_votes(int32_t *row, int Ck, int lane, int (&vk)[KPL])
{
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
        if (vk[k] != 0 && k * 64 + lane < Ck) atomicAdd(row + k * 64 + lane, vk[k]);
        vk[k] = 0;
    }
}

template <int KPL>
__global__ __launch_bounds__(64 * kVoteWaves) void pq_votes_kernel(const int32_t *q_codes, const float *tables,
                                                       const int32_t *perm_q, const int32_t *q_offsets,
                                                       const int32_t *k_offsets, int B, int H, int N, int P,
                                                       int Cc, int Cq, int Ck, int exact_keys, int chunks,
                                                       int nblocks, int32_t *votes)
{
    __shared__ int nsz[KPL * 64];
    __shared__ __attribute__((aligned(16))) int vhist[kVoteWaves][256];  // one radix histogram per wave
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    if (lb >= nblocks) return;
    const int bh = lb / chunks, b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int32_t *ko = k_offsets + (int64_t)bh * (Ck + 1);
    for (int j = tid; j < KPL * 64; j += 64 * kVoteWaves) nsz[j] = j < Ck ? ko[j + 1] - ko[j] : 0;
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
    // packed per-group term of the threshold search's sums: size in the low
    // kCountBits bits, one count per non-empty group above them (needs total <
    // 2^kCountBits)
    const bool packed = total < (1 << kCountBits);
    int nkp[KPL];
#pragma unroll
    for (int k = 0; k < KPL; ++k) nkp[k] = nk[k] + (packed && nk[k] > 0 ? (1 << kCountBits) : 0);
    const int E = exact_keys;
    const int32_t *qo = q_offsets + (int64_t)bh * (Cq + 1);
    const float *tb = tables + (int64_t)bh * P * Cc * Ck;
    int32_t *vb = votes + (int64_t)bh * Cq * Ck;
    // this wave's queries: rows [r, r_stop) of the permuted order
    int r = (lb % chunks) * kVoteChunk + wave * kVoteQPW;
    const int r_stop = min(N, r + kVoteQPW);
    if (r >= r_stop) return;
    // query group of row r: the largest i with qo[i] <= r (groups may be empty)
    int i = 0;
    {
        int lo = 0, hi = Cq;  // qo[lo] <= r < qo[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (qo[mid] <= r) lo = mid; else hi = mid;
        }
        i = lo;
    }
    int g_end = qo[i + 1];
    const int32_t *qcode = q_codes + ((int64_t)b * H + h) * N;  // + s*B*H*N + t
    const int64_t sstride = (int64_t)B * H * N;
    if (total <= E) {  // every non-empty group fits every query's budget
        for (; r < r_stop; ++r) {
            while (r >= g_end) {
                flush_votes<KPL>(vb + (int64_t)i * Ck, Ck, lane, vk);
                ++i;
                g_end = qo[i + 1];
            }
#pragma unroll
            for (int k = 0; k < KPL; ++k) vk[k] += nk[k] > 0;
        }
        flush_votes<KPL>(vb + (int64_t)i * Ck, Ck, lane, vk);
        return;
    }
    // codes of the next query are fetched while the current one runs its threshold search
    int codes[kPBatch];
    {
        const int t = perm_q[(int64_t)bh * N + r];
#pragma unroll
        for (int s = 0; s < kPBatch; ++s) codes[s] = s < P ? qcode[s * sstride + t] : 0;
    }
    for (; r < r_stop; ++r) {
        while (r >= g_end) {
            flush_votes<KPL>(vb + (int64_t)i * Ck, Ck, lane, vk);
            ++i;
            g_end = qo[i + 1];
        }
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
            // rows in kRowSplit parts of kPBatch / kRowSplit subspaces: fewer
            // registers in flight, so more waves per SIMD hide the latency; each
            // part is issued after the one before is summed
#pragma unroll
            for (int hb = 0; hb < kRowSplit; ++hb) {
                constexpr int HB = kPBatch / kRowSplit;
                float rv[HB][KPL];
#pragma unroll
                for (int s = 0; s < HB; ++s) {
                    const int ss = hb * HB + s;
                    const float *row = tb + ((int64_t)(s0 + ss) * Cc + codes[ss]) * Ck + lane;
#pragma unroll
                    for (int k = 0; k < KPL; ++k)
                        rv[s][k] = (s0 + ss < P && k * 64 + lane < Ck) ? row[k * 64] : 0.0f;
                }
#pragma unroll
                for (int s = 0; s < HB; ++s)
                    if (s0 + hb * HB + s < P) {
#pragma unroll
                        for (int k = 0; k < KPL; ++k)
                            if (k * 64 + lane < Ck) sc[k] = __fadd_rn(sc[k], rv[s][k]);
                    }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (r + 1 < r_stop) {
            const int tn = perm_q[(int64_t)bh * N + r + 1];
#pragma unroll
            for (int s = 0; s < kPBatch; ++s) codes[s] = s < P ? qcode[s * sstride + tn] : 0;
        }
        uint32_t ok[KPL];
#pragma unroll
        for (int k = 0; k < KPL; ++k) ok[k] = orderable(sc[k]);
        uint32_t lo = 0;  // the threshold: the largest key u with C(u) > E
        int above = 0;    // C(lo + 1): the size of the groups strictly above it
        radix_threshold<KPL>(ok, nk, nkp, packed, E, vhist[wave], lane, lo, above);
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
    flush_votes<KPL>(vb + (int64_t)i * Ck, Ck, lane, vk);
}

template <int KPL>
void launch_votes(hipStream_t st, const int32_t *q_codes, const float *tables, const int32_t *perm_q,
                  const int32_t *q_offsets, const int32_t *k_offsets, int B, int H, int N, int P, int Cc, int Cq,
                  int Ck, int E, int32_t *votes)
{
    const int64_t nv = (int64_t)B * H * Cq * Ck;
    zero_i32_kernel<<<(unsigned)std::min<int64_t>((nv + 255) / 256, 4096), 256, 0, st>>>(votes, nv);
    const int chunks = (N + kVoteChunk - 1) / kVoteChunk;
    const int nblocks = B * H * chunks;
    const int nb8 = (nblocks + 7) & ~7;
    pq_votes_kernel<KPL><<<nb8, 64 * kVoteWaves, 0, st>>>(q_codes, tables, perm_q, q_offsets, k_offsets, B, H, N, P,
                                                          Cc, Cq, Ck, E, chunks, nblocks, votes);
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
    ISG_REQUIRE(std::isfinite(scale) && scale > 0.0f, ISG_E_ARG, "isg_pq_votes: scale must be finite and > 0");
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
