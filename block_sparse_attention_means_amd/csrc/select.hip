// isg_probs and isg_select_sample.
//
// Pages: InstaGen, thelatestinai.com page, Figure 3(b)-(c) (centroid scores
// turned into a per-(query group, key group) probability pi; the best key group
// never dropped; other keys drawn with probability pi and weight 1/pi); Paper
// Reading AI Learner page, abstract (an exactly computed set of high-scoring
// keys, the rest estimated from a sample drawn by estimated attention, each term
// divided by its draw probability, one sample per query cluster);
// acceptodds.com page, abstract (the number of sampled tokens is the budget).
//
// Everything that decides an integer (scores, ranking, proposal weights, draws)
// uses explicitly rounded fp32 operations or integers, so the lists and sample
// indices are reproducible bit for bit by any implementation of the same
// definition.  This file is compiled with -ffp-contract=off.
#include <cmath>

#include "isg_internal.h"

namespace {

constexpr int kMaxGroups = 1024;
constexpr int kThreads = 256;

// S_ij = fma-chain(cq_i . ck_j) * scale (fp32, k ascending); pi from S in fp64.
// A work-group takes kQB query centroids of one head, so each key centroid's row
// is read once for kQB chains; per row i the reductions are those of a one-row
// work-group (thread t takes j = t, t + 256, ...), so the results do not depend
// on kQB.
constexpr int kQB = 4;
__global__ __launch_bounds__(kThreads) void probs_kernel(const float *cq, const float *ck,
                                                         const int32_t *k_offsets, int Cq, int Ck, int d,
                                                         float scale, float *scores, float *pi)
{
    extern __shared__ float qs[];  // kQB rows of d floats
    __shared__ double red[kThreads];
    __shared__ float redf[kThreads];
    const int nqb = (Cq + kQB - 1) / kQB;
    const int64_t bh = blockIdx.x / nqb;
    const int i0 = (int)(blockIdx.x % nqb) * kQB;
    const int nq = min(kQB, Cq - i0);
    const float *qi = cq + (bh * Cq + i0) * d;
    for (int k = threadIdx.x; k < kQB * d; k += kThreads) qs[k] = k < nq * d ? qi[k] : 0.0f;
    __syncthreads();
    const int32_t *ko = k_offsets + bh * (Ck + 1);
    float lmax[kQB];
#pragma unroll
    for (int r = 0; r < kQB; ++r) lmax[r] = -INFINITY;
    for (int j = threadIdx.x; j < Ck; j += kThreads) {
        const float *kj = ck + (bh * Ck + j) * d;
        float acc[kQB];
#pragma unroll
        for (int r = 0; r < kQB; ++r) acc[r] = 0.0f;
        for (int k = 0; k < d; ++k) {
            const float kv = kj[k];
#pragma unroll
            for (int r = 0; r < kQB; ++r) acc[r] = __fmaf_rn(qs[r * d + k], kv, acc[r]);
        }
        const bool nonempty = ko[j + 1] > ko[j];
#pragma unroll
        for (int r = 0; r < kQB; ++r)
            if (r < nq) {
                const float s = __fmul_rn(acc[r], scale);
                scores[(bh * Cq + i0 + r) * Ck + j] = s;
                if (nonempty) lmax[r] = fmaxf(lmax[r], s);
            }
    }
    if (!pi) return;
#pragma unroll
    for (int r = 0; r < kQB; ++r) {
        if (r >= nq) break;  // uniform over the work-group
        const int64_t gi = bh * Cq + i0 + r;
        const float *S = scores + gi * Ck;
        redf[threadIdx.x] = lmax[r];
        __syncthreads();
        for (int off = kThreads / 2; off > 0; off >>= 1) {
            if (threadIdx.x < off) redf[threadIdx.x] = fmaxf(redf[threadIdx.x], redf[threadIdx.x + off]);
            __syncthreads();
        }
        const double mx = (double)redf[0];
        double part = 0.0;
        for (int j = threadIdx.x; j < Ck; j += kThreads) {
            const int nj = ko[j + 1] - ko[j];
            if (nj > 0) part += (double)nj * exp((double)S[j] - mx);
        }
        red[threadIdx.x] = part;
        __syncthreads();
        for (int off = kThreads / 2; off > 0; off >>= 1) {
            if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
            __syncthreads();
        }
        const double tot = red[0];
        for (int j = threadIdx.x; j < Ck; j += kThreads) {
            const int nj = ko[j + 1] - ko[j];
            pi[gi * Ck + j] = nj > 0 ? (float)((double)nj * exp((double)S[j] - mx) / tot) : 0.0f;
        }
    }
}

struct ProposalTable {
    uint32_t v[256];
};

// Philox4x64-10 (Salmon et al., SC'11): per round, products of words 0 and 2
// with the two multipliers; new words (hi1^w1^k0, lo1, hi0^w3^k1, lo0); Weyl key
// bump between rounds.
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1)
{
    const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
    const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
        const uint64_t hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
        const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
        k0 += W0; k1 += W1;
    }
}

// floor((hi * 2^64 + lo) * T / 2^128)
__device__ __forceinline__ uint64_t scale128(uint64_t hi, uint64_t lo, uint64_t T)
{
    const uint64_t a1 = __umul64hi(hi, T), a0 = hi * T;
    const uint64_t b1 = __umul64hi(lo, T);
    const uint64_t mid = a0 + b1;
    return a1 + (mid < a0 ? 1 : 0);
}

// Per-work-group arrays in dynamic LDS, each P2 long (Ck rounded up to a power of
// two), plus block-scan and reduction scratch.
struct SelShared {
    uint64_t *W;       // rank keys, then compacted skipped weights -> exclusive prefix
    uint64_t *tmp64;
    int *order;
    int *n;
    float *S;
    float *P;          // pi (top-p rule), then 1/u per skipped group
    int *votes;        // votes, then the log weight per skipped group
    int *flag;         // 1 = exact
    int *buf;          // scan scratch (ints)
    int *tmp;
    int *sk_group;     // compacted skipped group ids (ascending)
    uint32_t *sk_u;
    float *red_f;
    int *red_i;
};

__host__ __device__ inline int sel_p2(int Ck)
{
    int P2 = 1;
    while (P2 < Ck) P2 <<= 1;
    return P2;
}

__host__ __device__ inline size_t sel_lds_bytes(int Ck)
{
    const size_t P2 = (size_t)sel_p2(Ck);
    return P2 * 8 + kThreads * 8 + 9 * P2 * 4 + 3 * kThreads * 4;
}

__device__ inline SelShared sel_carve(uint8_t *base, int P2)
{
    SelShared sh;
    uint8_t *p = base;
    auto take = [&](size_t bytes) { uint8_t *r = p; p += bytes; return r; };
    sh.W = reinterpret_cast<uint64_t *>(take((size_t)P2 * 8));
    sh.tmp64 = reinterpret_cast<uint64_t *>(take(kThreads * 8));
    sh.order = reinterpret_cast<int *>(take((size_t)P2 * 4));
    sh.n = reinterpret_cast<int *>(take((size_t)P2 * 4));
    sh.S = reinterpret_cast<float *>(take((size_t)P2 * 4));
    sh.P = reinterpret_cast<float *>(take((size_t)P2 * 4));
    sh.votes = reinterpret_cast<int *>(take((size_t)P2 * 4));
    sh.flag = reinterpret_cast<int *>(take((size_t)P2 * 4));
    sh.buf = reinterpret_cast<int *>(take((size_t)P2 * 4));
    sh.sk_group = reinterpret_cast<int *>(take((size_t)P2 * 4));
    sh.sk_u = reinterpret_cast<uint32_t *>(take((size_t)P2 * 4));
    sh.tmp = reinterpret_cast<int *>(take(kThreads * 4));
    sh.red_f = reinterpret_cast<float *>(take(kThreads * 4));
    sh.red_i = reinterpret_cast<int *>(take(kThreads * 4));
    return sh;
}

// Ranking of non-empty groups: (S desc, j asc); (votes desc, S desc, j asc) in
// votes mode; (pi desc, j asc) under the top-p rule.  Empty groups sort last.
__device__ __forceinline__ bool rank_before(const SelShared &sh, int a, int b, int mode, bool topp, int Ck)
{
    const bool ea = a < Ck && sh.n[a] > 0, eb = b < Ck && sh.n[b] > 0;
    if (ea != eb) return ea;
    if (!ea) return a < b;
    if (topp) {
        if (sh.P[a] != sh.P[b]) return sh.P[a] > sh.P[b];
        return a < b;
    }
    if (mode == ISG_SAMPLE_VOTES && sh.votes[a] != sh.votes[b]) return sh.votes[a] > sh.votes[b];
    if (sh.S[a] != sh.S[b]) return sh.S[a] > sh.S[b];
    return a < b;
}

// The same ranking as one ascending 64-bit key, for the rankings without votes:
// bit 63 marks an empty (or padding) group, bits 62..31 hold the complement of
// the score's order-preserving bits (scores descending; -0 counts as +0, as in
// the float comparison), bits 30..0 the group id (ascending on ties).  Scores
// are finite.
__device__ __forceinline__ uint64_t rank_key(float v, int j, bool nonempty)
{
    if (!nonempty) return (1ull << 63) | (uint64_t)j;
    const uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v);
    const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)(~ord) << 31) | (uint64_t)j;
}

// floor(diff / u) for u >= 1 and a quotient below 2^32: an fp32 estimate from
// rcp ~ 1/u, one fp32 step on the remainder, then exact integer correction.
__device__ __forceinline__ uint64_t div_floor(uint64_t diff, uint32_t u, float rcp)
{
    uint64_t q = (uint64_t)((float)diff * rcp);
    int64_t r = (int64_t)(diff - q * (uint64_t)u);
    q += (uint64_t)(int64_t)floorf((float)r * rcp);
    r = (int64_t)(diff - q * (uint64_t)u);
    while (r < 0) { --q; r += u; }
    while (r >= (int64_t)u) { ++q; r -= u; }
    return q;
}

// Exact set, then the shared sample.  Budget rule (pi == nullptr): the first
// group of the ranking always, then groups while the running key count stays
// <= exact_keys.  Top-p rule (pi given): groups in (pi desc, j asc) order until
// the fp64 running sum of pi, added in that order by one lane, reaches top_p.
__global__ __launch_bounds__(kThreads) void select_sample_kernel(
    const float *scores, const float *pi, double top_p, const int32_t *k_offsets, const int32_t *votes, int H,
    int Cq, int Ck, int exact_keys, int m, int mode, uint64_t seed, uint64_t call_id, ProposalTable tbl,
    int32_t *exact_groups, int32_t *n_exact, int32_t *sample_idx, float *sample_bias, int32_t *n_sample)
{
    const bool topp = pi != nullptr;
    extern __shared__ __attribute__((aligned(16))) uint8_t sel_lds[];
    const int tid = threadIdx.x;
    const int64_t gi = blockIdx.x;
    const int64_t bh = gi / Cq;
    const int i = (int)(gi % Cq), h = (int)(bh % H), b = (int)(bh / H);
    const int32_t *ko = k_offsets + bh * (Ck + 1);
    const int P2 = sel_p2(Ck);
    const SelShared sh = sel_carve(sel_lds, P2);
    for (int j = tid; j < P2; j += kThreads) {
        sh.order[j] = j;
        if (j < Ck) {
            sh.n[j] = ko[j + 1] - ko[j];
            sh.S[j] = scores[gi * Ck + j];
            sh.P[j] = topp ? pi[gi * Ck + j] : 0.0f;
            sh.votes[j] = votes ? votes[gi * Ck + j] : 0;
            sh.flag[j] = 0;
        }
    }
    __syncthreads();
    if (mode == ISG_SAMPLE_VOTES && !topp) {
        // bitonic sort of group ids by rank_before
        for (int size = 2; size <= P2; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int p = tid; p < P2 / 2; p += kThreads) {
                    const int lo = 2 * p - (p & (stride - 1));
                    const int hi = lo + stride;
                    const bool up = (lo & size) == 0;
                    const int a = sh.order[lo], c = sh.order[hi];
                    const bool swap =
                        up ? rank_before(sh, c, a, mode, topp, Ck) : rank_before(sh, a, c, mode, topp, Ck);
                    if (swap) { sh.order[lo] = c; sh.order[hi] = a; }
                }
                __syncthreads();
            }
        }
    } else {
        // the same bitonic network on rank keys (sh.W is free until the sample)
        uint64_t *key = sh.W;
        for (int j = tid; j < P2; j += kThreads)
            key[j] = rank_key(topp ? sh.P[j < Ck ? j : 0] : sh.S[j < Ck ? j : 0], j, j < Ck && sh.n[j] > 0);
        __syncthreads();
        for (int size = 2; size <= P2; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int p = tid; p < P2 / 2; p += kThreads) {
                    const int lo = 2 * p - (p & (stride - 1));
                    const int hi = lo + stride;
                    const bool up = (lo & size) == 0;
                    const uint64_t a = key[lo], c = key[hi];
                    if (up ? c < a : a < c) { key[lo] = c; key[hi] = a; }
                }
                __syncthreads();
            }
        }
        for (int p = tid; p < P2; p += kThreads) sh.order[p] = (int)(key[p] & 0x7FFFFFFFu);
        __syncthreads();
    }
    if (topp) {
        if (tid == 0) {
            double mass = 0.0;
            for (int p = 0; p < Ck; ++p) {
                const int j = sh.order[p];
                if (sh.n[j] == 0) break;  // empty groups sort last
                sh.flag[j] = 1;
                mass += (double)sh.P[j];
                if (mass >= top_p) break;
            }
        }
        __syncthreads();
    } else {
        // running key count along the order; the first group is always taken
        for (int p = tid; p < Ck; p += kThreads) {
            const int j = sh.order[p];
            sh.buf[p] = sh.n[j];
        }
        __syncthreads();
        block_exclusive_scan_int(sh.buf, Ck, sh.tmp);
        for (int p = tid; p < Ck; p += kThreads) {
            const int j = sh.order[p];
            const int incl = sh.buf[p] + sh.n[j];
            if (sh.n[j] > 0 && (p == 0 || incl <= exact_keys)) sh.flag[j] = 1;
        }
        __syncthreads();
    }
    // exact groups ascending
    for (int j = tid; j < Ck; j += kThreads) sh.buf[j] = sh.flag[j];
    __syncthreads();
    const int ne = block_exclusive_scan_int(sh.buf, Ck, sh.tmp);
    int32_t *eg = exact_groups + gi * Ck;
    for (int j = tid; j < Ck; j += kThreads) {
        if (sh.flag[j]) eg[sh.buf[j]] = j;
        if (j >= ne) eg[j] = -1;
    }
    if (tid == 0) n_exact[gi] = ne;
    __syncthreads();
    // skipped groups ascending, their key count M and largest score
    for (int j = tid; j < Ck; j += kThreads) sh.buf[j] = (sh.n[j] > 0 && !sh.flag[j]) ? 1 : 0;
    __syncthreads();
    int lcount = 0;
    float lmax = -INFINITY;
    for (int j = tid; j < Ck; j += kThreads)
        if (sh.n[j] > 0 && !sh.flag[j]) { lcount += sh.n[j]; lmax = fmaxf(lmax, sh.S[j]); }
    sh.red_i[tid] = lcount;
    sh.red_f[tid] = lmax;
    __syncthreads();
    for (int off = kThreads / 2; off > 0; off >>= 1) {
        if (tid < off) {
            sh.red_i[tid] += sh.red_i[tid + off];
            sh.red_f[tid] = fmaxf(sh.red_f[tid], sh.red_f[tid + off]);
        }
        __syncthreads();
    }
    const int M = sh.red_i[0];
    const float smax = sh.red_f[0];
    const int nsk = block_exclusive_scan_int(sh.buf, Ck, sh.tmp);
    for (int j = tid; j < Ck; j += kThreads)
        if (sh.n[j] > 0 && !sh.flag[j]) sh.sk_group[sh.buf[j]] = j;
    __syncthreads();
    int32_t *si = sample_idx + gi * (int64_t)m;
    float *sb = sample_bias + gi * (int64_t)m;
    if (M == 0) {
        if (tid == 0) n_sample[gi] = 0;
        return;
    }
    if (M <= m) {
        // enumerate every skipped key once, offset 0
        for (int s = tid; s < nsk; s += kThreads) sh.buf[s] = sh.n[sh.sk_group[s]];
        __syncthreads();
        block_exclusive_scan_int(sh.buf, nsk, sh.tmp);
        for (int t = tid; t < M; t += kThreads) {
            int lo = 0, hi = nsk - 1;  // last s with buf[s] <= t
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (sh.buf[mid] <= t) lo = mid; else hi = mid - 1;
            }
            si[t] = ko[sh.sk_group[lo]] + (t - sh.buf[lo]);
            sb[t] = 0.0f;
        }
        if (tid == 0) n_sample[gi] = M;
        return;
    }
    // proposal weights W = n u, exclusive prefix in ascending group order; per
    // skipped group also 1/u and the log weight (the ranking arrays are free now)
    float *sk_rcp = sh.P;
    float *sk_bias = reinterpret_cast<float *>(sh.votes);
    for (int s = tid; s < nsk; s += kThreads) {
        const int j = sh.sk_group[s];
        uint32_t u = 1;
        if (mode != ISG_SAMPLE_UNIFORM) {
            const float diff = __fsub_rn(smax, sh.S[j]);
            const float prod = __fmul_rn(diff, 369.32993f);  // 256 * log2(e)
            int a = (int)rintf(prod);
            a = min(max(a, 0), 7936);
            const int shft = min(a >> 8, 31);
            u = tbl.v[a & 255] >> shft;
            if (u < 1) u = 1;
        }
        sh.sk_u[s] = u;
        sk_rcp[s] = 1.0f / (float)u;
        sh.W[s] = (uint64_t)sh.n[j] * u;
    }
    __syncthreads();
    const uint64_t T = block_exclusive_scan_u64(sh.W, nsk, sh.tmp64);
    const double lnT = log((double)T), lnm = log((double)m);
    for (int s = tid; s < nsk; s += kThreads) sk_bias[s] = (float)(lnT - log((double)sh.sk_u[s]) - lnm);
    __syncthreads();
    for (int t2 = 2 * tid; t2 < m; t2 += 2 * kThreads) {
        uint64_t c[4] = {(uint64_t)(t2 / 2) + 1, (uint64_t)i, (uint64_t)h, (uint64_t)b};
        philox4x64_10(c, seed, call_id);
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const int t = t2 + w;
            if (t >= m) break;
            const uint64_t z = scale128(c[2 * w], c[2 * w + 1], T);
            int lo = 0, hi = nsk - 1;  // last s with W[s] <= z
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (sh.W[mid] <= z) lo = mid; else hi = mid - 1;
            }
            const int j = sh.sk_group[lo];
            si[t] = ko[j] + (int)div_floor(z - sh.W[lo], sh.sk_u[lo], sk_rcp[lo]);
            sb[t] = sk_bias[lo];
        }
    }
    if (tid == 0) n_sample[gi] = m;
}

}  // namespace

extern "C" isg_status isg_probs(void *stream, const float *cq, const float *ck, const int32_t *k_offsets,
                                int B, int H, int Cq, int Ck, int d, float scale, float *scores, float *pi)
{
    ISG_REQUIRE(cq && ck && k_offsets && scores, ISG_E_ARG, "isg_probs: null pointer argument");
    ISG_REQUIRE(B >= 1 && H >= 1, ISG_E_ARG, "isg_probs: B, H must be >= 1");
    ISG_REQUIRE(Cq >= 1 && Cq <= kMaxGroups && Ck >= 1 && Ck <= kMaxGroups, ISG_E_ARG,
                "isg_probs: Cq, Ck must be in [1, %d] (got %d, %d)", kMaxGroups, Cq, Ck);
    ISG_REQUIRE(d >= 1 && d <= 1024, ISG_E_ARG, "isg_probs: d must be in [1, 1024]");
    ISG_REQUIRE(std::isfinite(scale) && scale > 0.0f, ISG_E_ARG, "isg_probs: scale must be finite and > 0");
    hipStream_t st = (hipStream_t)stream;
    const int64_t G = (int64_t)B * H * ((Cq + kQB - 1) / kQB);
    ISG_REQUIRE((int64_t)B * H * Cq <= 0x7fffffff, ISG_E_ARG, "isg_probs: too many groups");
    probs_kernel<<<(unsigned)G, kThreads, kQB * d * sizeof(float), st>>>(cq, ck, k_offsets, Cq, Ck, d, scale,
                                                                         scores, pi);
    return isg_check_launch("isg_probs");
}

extern "C" isg_status isg_select_sample(void *stream, const float *scores, const int32_t *k_offsets,
                                        const int32_t *votes, int B, int H, int Cq, int Ck, int N,
                                        int exact_keys, int m, int mode, uint64_t seed, uint64_t call_id,
                                        int32_t *exact_groups, int32_t *n_exact, int32_t *sample_idx,
                                        float *sample_bias, int32_t *n_sample)
{
    ISG_REQUIRE(scores && k_offsets && exact_groups && n_exact && n_sample, ISG_E_ARG,
                "isg_select_sample: null pointer argument");
    ISG_REQUIRE(m == 0 || (sample_idx && sample_bias), ISG_E_ARG,
                "isg_select_sample: sample_idx / sample_bias required when m > 0");
    ISG_REQUIRE(B >= 1 && H >= 1 && N >= 1, ISG_E_ARG, "isg_select_sample: B, H, N must be >= 1");
    ISG_REQUIRE(Cq >= 1 && Ck >= 1 && Ck <= kMaxGroups, ISG_E_ARG,
                "isg_select_sample: need Cq >= 1 and 1 <= Ck <= %d (got %d, %d)", kMaxGroups, Cq, Ck);
    ISG_REQUIRE(exact_keys >= 0, ISG_E_ARG, "isg_select_sample: exact_keys must be >= 0");
    ISG_REQUIRE(m >= 0 && m <= N, ISG_E_ARG, "isg_select_sample: need 0 <= m <= N (got m=%d, N=%d)", m, N);
    ISG_REQUIRE(mode == ISG_SAMPLE_IMPORTANCE || mode == ISG_SAMPLE_UNIFORM || mode == ISG_SAMPLE_VOTES,
                ISG_E_ARG, "isg_select_sample: unknown mode %d", mode);
    ISG_REQUIRE((mode == ISG_SAMPLE_VOTES) == (votes != nullptr), ISG_E_ARG,
                "isg_select_sample: votes must be given exactly in votes mode");
    const int64_t G = (int64_t)B * H * Cq;
    ISG_REQUIRE(G <= 0x7fffffff, ISG_E_ARG, "isg_select_sample: too many groups");
    ProposalTable tbl;
    isg_proposal_table(tbl.v);
    hipStream_t st = (hipStream_t)stream;
    select_sample_kernel<<<(unsigned)G, kThreads, sel_lds_bytes(Ck), st>>>(scores, nullptr, 0.0, k_offsets, votes, H, Cq, Ck,
                                                           exact_keys, m, mode, seed, call_id, tbl, exact_groups,
                                                           n_exact, sample_idx, sample_bias, n_sample);
    return isg_check_launch("isg_select_sample");
}

extern "C" isg_status isg_select_sample_topp(void *stream, const float *scores, const float *pi,
                                             const int32_t *k_offsets, int B, int H, int Cq, int Ck, int N,
                                             float top_p, int m, int mode, uint64_t seed, uint64_t call_id,
                                             int32_t *exact_groups, int32_t *n_exact, int32_t *sample_idx,
                                             float *sample_bias, int32_t *n_sample)
{
    ISG_REQUIRE(scores && pi && k_offsets && exact_groups && n_exact && n_sample, ISG_E_ARG,
                "isg_select_sample_topp: null pointer argument");
    ISG_REQUIRE(m == 0 || (sample_idx && sample_bias), ISG_E_ARG,
                "isg_select_sample_topp: sample_idx / sample_bias required when m > 0");
    ISG_REQUIRE(B >= 1 && H >= 1 && N >= 1, ISG_E_ARG, "isg_select_sample_topp: B, H, N must be >= 1");
    ISG_REQUIRE(Cq >= 1 && Ck >= 1 && Ck <= kMaxGroups, ISG_E_ARG,
                "isg_select_sample_topp: need Cq >= 1 and 1 <= Ck <= %d (got %d, %d)", kMaxGroups, Cq, Ck);
    ISG_REQUIRE(std::isfinite(top_p) && top_p > 0.0f, ISG_E_ARG,
                "isg_select_sample_topp: top_p must be finite and > 0");
    ISG_REQUIRE(m >= 0 && m <= N, ISG_E_ARG, "isg_select_sample_topp: need 0 <= m <= N (got m=%d, N=%d)", m, N);
    ISG_REQUIRE(mode == ISG_SAMPLE_IMPORTANCE || mode == ISG_SAMPLE_UNIFORM, ISG_E_ARG,
                "isg_select_sample_topp: mode must be importance or uniform (got %d)", mode);
    const int64_t G = (int64_t)B * H * Cq;
    ISG_REQUIRE(G <= 0x7fffffff, ISG_E_ARG, "isg_select_sample_topp: too many groups");
    ProposalTable tbl;
    isg_proposal_table(tbl.v);
    hipStream_t st = (hipStream_t)stream;
    select_sample_kernel<<<(unsigned)G, kThreads, sel_lds_bytes(Ck), st>>>(scores, pi, (double)top_p, k_offsets, nullptr, H, Cq,
                                                           Ck, 0, m, mode, seed, call_id, tbl, exact_groups,
                                                           n_exact, sample_idx, sample_bias, n_sample);
    return isg_check_launch("isg_select_sample_topp");
}
