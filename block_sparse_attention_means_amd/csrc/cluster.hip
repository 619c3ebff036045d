// isg_cluster: Lloyd k-means per head + stable counting sort + coalesced gather.
//
// Pages: InstaGen, thelatestinai.com page, Figure 3(a) (Q and K partitioned by
// clustering) and Figure 2 (Cq = 100, Ck = 500).  Reading: Euclidean
// k-means on the raw vectors, strided init, ties to the lowest index, empty
// clusters keep their centroid; the permutation is the stable sort by label.
//
// Per round: assign (labels) -> per-chunk histograms -> scan over chunks ->
// label offsets + stable scatter (perm, offsets) -> segmented fp64 mean in sorted order
// (centroids).  No float atomics: every output is deterministic.
#include <mutex>
#include <type_traits>

#include "isg_internal.h"

namespace {

constexpr int kSortChunk = 1024;  // tokens per histogram / scatter chunk
constexpr int kMaxC = 4096;
constexpr int kMaxLabelBits = 12;  // labels below kMaxC
constexpr int kPqMaxP = 64;        // subspaces per row the split kernel tracks exponents for
constexpr int kPqIntMaxC = 256;    // codewords up to which the PQ update sums integers in LDS
constexpr int kPqAccTok = 8192;    // tokens per work-group of that update
constexpr int kPqAccThreads = 256; // its threads (two per token)
constexpr int kPqPitch = 17;       // int64 words per codeword in its LDS sums (16 dims + 1)
constexpr int kAssignTile = 32;   // centroids per LDS tile in the assign kernel
// Rows per piece of the centroid update: 16 rows for each of the work-group's row
// slots (256 threads, d/8 per row), so 256 at d = 128 and 2048 at d = 16.
__host__ __device__ constexpr int piece_rows(int d) { return 16 * (256 / (d / 8)); }

struct Strides {
    int64_t b, h, t;
};

// 8 consecutive elements starting at p (p 16-byte aligned) as fp32.
__device__ __forceinline__ void load8(const float *p, float out[8])
{
    float4 a = *reinterpret_cast<const float4 *>(p);
    float4 c = *reinterpret_cast<const float4 *>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = c.x; out[5] = c.y; out[6] = c.z; out[7] = c.w;
}
// 8 elements as loaded (bf16: one 16-byte word; fp32: two), widened when used.
template <typename T>
struct Raw8;
template <>
struct Raw8<uint16_t> {
    uint4 a;
    __device__ __forceinline__ void load(const uint16_t *p) { a = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ void store(uint16_t *p) const { *reinterpret_cast<uint4 *>(p) = a; }
    __device__ __forceinline__ float get(int e) const
    {
        const uint32_t w = e < 2 ? a.x : e < 4 ? a.y : e < 6 ? a.z : a.w;
        return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
};
template <>
struct Raw8<float> {
    float4 a, c;
    __device__ __forceinline__ void load(const float *p)
    {
        a = *reinterpret_cast<const float4 *>(p);
        c = *reinterpret_cast<const float4 *>(p + 4);
    }
    __device__ __forceinline__ void store(float *p) const
    {
        *reinterpret_cast<float4 *>(p) = a;
        *reinterpret_cast<float4 *>(p + 4) = c;
    }
    __device__ __forceinline__ float get(int e) const
    {
        const float4 &f = e < 4 ? a : c;
        const int k = e & 3;
        return k == 0 ? f.x : k == 1 ? f.y : k == 2 ? f.z : f.w;
    }
};
// Copy 8 elements (16 B for bf16, 32 B for fp32).
__device__ __forceinline__ void copy8(uint16_t *dst, const uint16_t *src)
{
    *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
}
__device__ __forceinline__ void copy8(float *dst, const float *src)
{
    *reinterpret_cast<float4 *>(dst) = *reinterpret_cast<const float4 *>(src);
    *reinterpret_cast<float4 *>(dst + 4) = *reinterpret_cast<const float4 *>(src + 4);
}

template <typename T>
__global__ void init_centroids_kernel(const T *x, Strides xs, int H, int N, int C, int D, float *cent,
                                      int64_t total)
{
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        int k = (int)(e % D);
        int64_t r = e / D;
        int j = (int)(r % C);
        int64_t bh = r / C;
        int b = (int)(bh / H), h = (int)(bh % H);
        int64_t t = (int64_t)j * N / C;
        cent[e] = Elem<T>::load(x, b * xs.b + h * xs.h + t * xs.t + k);
    }
}

// labels[t] = argmin_j |x_t - c_j|^2.  fp32 distances, each a sequential fused
// sum of squared differences (relative error < (D + 2) 2^-24).  The fp32 argmin
// stands unless the runner-up lies within 4e-5 relative of the best (more than
// twice that bound); then every centroid is re-compared in fp64 with unfused
// operations in the order k = 0..D-1, ties to the lower index (a third candidate
// may be as close as the runner-up, so the rescan covers all of them).
template <typename T, int D>
__global__ __launch_bounds__(256) void assign_kernel(const T *x, Strides xs, int H, int N, int C,
                                                     const float *cent, int32_t *labels)
{
    __shared__ float cs[kAssignTile][D];
    const int bh = blockIdx.y, b = bh / H, h = bh % H;
    const int t = blockIdx.x * 256 + threadIdx.x;
    const bool valid = t < N;
    const T *xr = x + b * xs.b + h * xs.h + (int64_t)min(t, N - 1) * xs.t;
    float xv[D];
#pragma unroll
    for (int k = 0; k < D; k += 8) load8(xr + k, xv + k);
    const float *ch = cent + (int64_t)bh * C * D;
    float best = INFINITY, second = INFINITY;
    int bi = 0;
    for (int c0 = 0; c0 < C; c0 += kAssignTile) {
        const int nc = min(kAssignTile, C - c0);
        __syncthreads();
        for (int e = threadIdx.x; e < nc * D; e += 256) cs[e / D][e % D] = ch[(int64_t)c0 * D + e];
        __syncthreads();
        for (int jj = 0; jj < nc; ++jj) {
            float s = 0.0f;
#pragma unroll
            for (int k = 0; k < D; ++k) {
                float df = xv[k] - cs[jj][k];
                s = fmaf(df, df, s);
            }
            const int j = c0 + jj;
            if (s < best) {
                second = best; best = s; bi = j;
            } else if (s < second) {
                second = s;
            }
        }
    }
    if (!valid) return;
    if (C > 1 && second - best <= 4e-5f * second) {
        double bd = INFINITY;
        for (int j = 0; j < C; ++j) {
            const float *cj = ch + (int64_t)j * D;
            double dj = 0.0;
#pragma unroll
            for (int k = 0; k < D; ++k) {
                const double a = __dsub_rn((double)xv[k], (double)cj[k]);
                dj = __dadd_rn(dj, __dmul_rn(a, a));
            }
            if (dj < bd) { bd = dj; bi = j; }
        }
    }
    labels[(int64_t)bh * N + t] = bi;
}

__global__ __launch_bounds__(256) void hist_kernel(const int32_t *labels, int N, int C, int nchunks,
                                                   int32_t *hist)
{
    __shared__ int hs[kMaxC];
    const int chunk = blockIdx.x, bh = blockIdx.y;
    for (int c = threadIdx.x; c < C; c += 256) hs[c] = 0;
    // the chunk's labels, all loads in flight before the first count
    constexpr int kPer = kSortChunk / 256;
    int lab[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int t = chunk * kSortChunk + u * 256 + threadIdx.x;
        lab[u] = t < N ? labels[(int64_t)bh * N + t] : -1;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPer; ++u)
        if (lab[u] >= 0) atomicAdd(&hs[lab[u]], 1);
    __syncthreads();
    int32_t *out = hist + ((int64_t)bh * nchunks + chunk) * C;
    for (int c = threadIdx.x; c < C; c += 256) out[c] = hs[c];
}

// hist[bh][chunk][c] -> number of tokens with label c in the chunks before this
// one; tot[bh][c] = number of tokens with label c.  One lane per label: the four
// waves of a work-group take consecutive quarters of the chunks, sum them, and
// each then rewrites its quarter starting from the sum of the quarters before.
__global__ __launch_bounds__(256) void scan_kernel(int32_t *hist, int nchunks, int C, int32_t *tot)
{
    constexpr int kB = 8;  // loads in flight per lane
    __shared__ int part[4][64];
    const int bh = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = blockIdx.x * 64 + lane;
    const int q = (nchunks + 3) / 4;
    const int ch0 = min(nchunks, wave * q), ch1 = min(nchunks, ch0 + q);
    int32_t *hc = hist + (int64_t)bh * nchunks * C + c;
    int sum = 0;
    if (c < C)
        for (int a = ch0; a < ch1; a += kB) {
            int v[kB];
#pragma unroll
            for (int u = 0; u < kB; ++u) v[u] = a + u < ch1 ? hc[(int64_t)(a + u) * C] : 0;
#pragma unroll
            for (int u = 0; u < kB; ++u) sum += v[u];
        }
    part[wave][lane] = sum;
    __syncthreads();
    if (c >= C) return;
    int run = 0;
    for (int w = 0; w < wave; ++w) run += part[w][lane];
    if (wave == 3) tot[(int64_t)bh * C + c] = run + sum;
    for (int a = ch0; a < ch1; a += kB) {
        int v[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) v[u] = a + u < ch1 ? hc[(int64_t)(a + u) * C] : 0;
#pragma unroll
        for (int u = 0; u < kB; ++u)
            if (a + u < ch1) {
                hc[(int64_t)(a + u) * C] = run;
                run += v[u];
            }
    }
}

// Lanes of the wave whose label equals this lane's: those that differ from it
// in no label bit, i.e. not in the OR over the bits of (ballot of the bit) XOR
// (this lane's bit as all ones / zeros).  NB covers every label bit (bits above
// the labels' width are zero in every lane and change nothing); the bits are
// independent, so their ballots overlap instead of forming one serial chain.
template <int NB>
__device__ __forceinline__ uint64_t same_label(int lab)
{
    uint32_t dlo = 0, dhi = 0;
#pragma unroll
    for (int bt = 0; bt < NB; ++bt) {
        const uint64_t bal = __ballot((lab >> bt) & 1);
        const uint32_t own = 0u - (uint32_t)((lab >> bt) & 1);
        dlo |= (uint32_t)bal ^ own;
        dhi |= (uint32_t)(bal >> 32) ^ own;
    }
    return ~(((uint64_t)dhi << 32) | dlo);
}

// One wave per chunk.  It first turns the label counts into label offsets (the
// exclusive prefix over labels, lane l taking a contiguous run of labels) and
// adds the chunk's per-label base, so run[c] is the first sorted row of
// (chunk, c); the wave of chunk 0 also writes offsets and poff (the prefix of
// the number of prow-row pieces per group).  It then walks its tokens in order,
// 64 at a time; a token's rank among equal labels of the same step comes from
// ballots over the label bits.
__global__ __launch_bounds__(64) void scatter_kernel(const int32_t *labels, const int32_t *base,
                                                     const int32_t *tot, int N, int C, int nchunks, int bits,
                                                     int prow, int maxp, int64_t nblocks, int32_t *perm,
                                                     int32_t *offsets, int32_t *poff, int4 *ptab)
{
    extern __shared__ int run[];  // C entries (dynamic, so small C lets more waves share a CU)
    // XCD-aware order: each XCD (launch id mod 8) takes a contiguous range of
    // (head, chunk) pairs, so all chunks of a head run on one XCD.  A chunk
    // writes a short run of each label's rows (1,024 / C tokens on average);
    // the runs of neighbouring chunks are adjacent in perm, and on one L2 their
    // partial-line stores merge before they reach memory.
    const int64_t lb = (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    if (lb >= nblocks) return;
    const int chunk = (int)(lb % nchunks), bh = (int)(lb / nchunks), lane = threadIdx.x;
    const int32_t *bb = base + ((int64_t)bh * nchunks + chunk) * C;
    const int32_t *tb = tot + (int64_t)bh * C;
    // Loads in issue order: the first batch of label counts and of the chunk's
    // bases, then the chunk's labels, so that one wait covers the counts and the
    // others stay in flight through the label scan.
    constexpr int kB = 8;
    int tv[kB], bv[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
        const int c = lane + 64 * u;
        tv[u] = c < C ? tb[c] : 0;
        bv[u] = c < C ? bb[c] : 0;
    }
    const int t0 = chunk * kSortChunk;
    int labs[kSortChunk / 64];
#pragma unroll
    for (int step = 0; step < kSortChunk / 64; ++step) {
        const int t = t0 + step * 64 + lane;
        labs[step] = t < N ? labels[(int64_t)bh * N + t] : 0;
    }
#pragma unroll
    for (int u = 0; u < kB; ++u)
        if (lane + 64 * u < C) run[lane + 64 * u] = tv[u];
    for (int c0 = lane + 64 * kB; c0 < C; c0 += 64 * kB) {
        int v[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) v[u] = c0 + 64 * u < C ? tb[c0 + 64 * u] : 0;
#pragma unroll
        for (int u = 0; u < kB; ++u)
            if (c0 + 64 * u < C) run[c0 + 64 * u] = v[u];
    }
    __builtin_amdgcn_wave_barrier();  // one wave: LDS order is program order
    {
        const int S = (C + 63) / 64, l0 = min(C, lane * S), l1 = min(C, l0 + S);
        int ls = 0, lp = 0;
        for (int c = l0; c < l1; ++c) {
            const int n = run[c];
            ls += n;
            lp += (n + prow - 1) / prow;
        }
        int xs = ls, xp = lp;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int ys = __shfl_up(xs, off), yp = __shfl_up(xp, off);
            if (lane >= off) {
                xs += ys;
                xp += yp;
            }
        }
        int os = xs - ls, op = xp - lp;
        const bool first = chunk == 0;
        int32_t *ob = offsets + (int64_t)bh * (C + 1);
        int32_t *pb = poff + (int64_t)bh * (C + 1);
        int4 *pt = ptab + (int64_t)bh * maxp;
        for (int c = l0; c < l1; ++c) {
            const int n = run[c];
            run[c] = os;
            if (first) {
                ob[c] = os;
                pb[c] = op;
                // piece table: group and row range of each of the group's pieces
                for (int k = 0; k < n; k += prow) pt[op + k / prow] = make_int4(c, os + k, os + min(n, k + prow), 0);
            }
            os += n;
            op += (n + prow - 1) / prow;
        }
        // lane 63 ends on the totals (its run of labels may be empty)
        if (first && lane == 63) {
            ob[C] = os;
            pb[C] = op;
        }
    }
    __builtin_amdgcn_wave_barrier();  // one wave: LDS order is program order
#pragma unroll
    for (int u = 0; u < kB; ++u)
        if (lane + 64 * u < C) run[lane + 64 * u] += bv[u];
    for (int c0 = lane + 64 * kB; c0 < C; c0 += 64 * kB) {
        int v[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) v[u] = c0 + 64 * u < C ? bb[c0 + 64 * u] : 0;
#pragma unroll
        for (int u = 0; u < kB; ++u)
            if (c0 + 64 * u < C) run[c0 + 64 * u] += v[u];
    }
    __builtin_amdgcn_wave_barrier();  // one wave: LDS order is program order
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int step = 0; step < kSortChunk / 64; ++step) {
        const int t = t0 + step * 64 + lane;
        const bool valid = t < N;
        const int lab = labs[step];
        const uint64_t m = __ballot(valid) & (bits <= 8 ? same_label<8>(lab) : same_label<kMaxLabelBits>(lab));
        const int rank = __popcll(m & below);
        const int cnt = __popcll(m);
        int pos = 0;
        if (valid) pos = run[lab] + rank;
        // The work-group is one wave, whose LDS accesses take effect in program
        // order: the next step's reads see this step's writes with no barrier
        // (a work-group barrier here would also wait for every perm store to
        // complete, twice per step).
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            perm[(int64_t)bh * N + pos] = t;
            if (rank == cnt - 1) run[lab] = pos + 1;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// Centroid update in two passes, both in a fixed order: every group is cut into
// pieces of piece_rows(D) sorted rows; a work-group sums one piece in fp64 (rows
// strided over RP slots, then slot order) and the final pass adds the pieces of
// each group in order and divides: c_j = mean of the rows of group j, rounded
// to fp32 (an empty group keeps its centroid).
template <typename T, int D>
__global__ __launch_bounds__(256) void update_piece_kernel(const T *x, Strides xs, int H, int N, int C,
                                                           const int32_t *perm, const int32_t *poff,
                                                           const int4 *ptab, int maxp, int64_t nblocks,
                                                           double *partial, T *x_perm, float *pmax)
{
    constexpr int TPR = D / 8;     // threads per row
    constexpr int RP = 256 / TPR;  // row slots
    constexpr int PR = piece_rows(D);
    constexpr int RPT = PR / RP;   // rows per slot: all indices, then all rows, in flight at once
    __shared__ double red[RP][D];
    // At D = 16 (one head of 32-byte rows is 2.4 MB at N = 75,600) the order is
    // XCD-aware: each XCD (launch id mod 8) walks a contiguous range of (head,
    // piece) pairs, so the heads it works on at a time are few and their rows,
    // read at random positions, stay in that XCD's L2.  Wider rows do not fit an
    // L2 per head; there the launch order stays head-major (both orders time the
    // same at D = 128).
    const int64_t lb = D == 16 ? (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3)
                               : (int64_t)blockIdx.x;
    if (lb >= nblocks) return;
    const int q = (int)(lb % maxp), bh = (int)(lb / maxp), b = bh / H, h = bh % H;
    // the piece's row range comes from the table the scatter wrote (entries past
    // the head's piece count are stale and not read)
    const int npieces = poff[(int64_t)bh * (C + 1) + C];
    const int4 pt = ptab[(int64_t)bh * maxp + q];
    if (q >= npieces) return;
    const int r0 = pt.y, r1 = pt.z;
    const int rs = threadIdx.x / TPR, ck = threadIdx.x % TPR;
    const T *xb = x + b * xs.b + h * xs.h + ck * 8;
    const int32_t *pm = perm + (int64_t)bh * N;
    int idx[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int rr = r0 + rs + i * RP;
        idx[i] = rr < r1 ? pm[rr] : -1;
    }
    Raw8<T> v[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        if (idx[i] >= 0) v[i].load(xb + (int64_t)idx[i] * xs.t);
    // last k-means iteration: the rows just read are also the permuted copy (x_perm[r] = x[perm[r]])
    if (x_perm) {
        T *xp = x_perm + (int64_t)bh * N * D + ck * 8;
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            if (idx[i] >= 0) v[i].store(xp + (int64_t)(r0 + rs + i * RP) * D);
    }
    // last k-means iteration, if asked: the largest squared norm of the piece's
    // rows, in the key-norm pass's arithmetic (fp32 fma chain over a lane's 8
    // elements, then a butterfly over the row's lanes), one value per piece (the
    // final pass takes the head's maximum: no atomics on one shared line)
    if (pmax) {
        __shared__ float wmax[4];
        float best = 0.0f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            float ss = 0.0f;
            if (idx[i] >= 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(v[i].get(e), v[i].get(e), ss);
            }
#pragma unroll
            for (int off = TPR / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
            best = fmaxf(best, ss);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) best = fmaxf(best, __shfl_xor(best, off));
        if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = best;
        __syncthreads();
        if (threadIdx.x == 0)
            pmax[(int64_t)bh * maxp + q] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    }
    // fp64 sum of the slot's rows in sorted order
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        if (idx[i] >= 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += (double)v[i].get(e);
        }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rs][ck * 8 + e] = acc[e];
    __syncthreads();
    for (int k = threadIdx.x; k < D; k += 256) {
        double sum = 0.0;
        for (int rr = 0; rr < RP; ++rr) sum += red[rr][k];
        partial[((int64_t)bh * maxp + q) * D + k] = sum;
    }
}

template <int D>
__global__ __launch_bounds__(128) void update_final_kernel(int C, const int32_t *offsets, const int32_t *poff,
                                                           int maxp, const double *partial, float *cent,
                                                           const float *pmax, float *max_sqnorm)
{
    const int j = blockIdx.x, bh = blockIdx.y;
    const int32_t *pb = poff + (int64_t)bh * (C + 1);
    if (pmax && j == 0) {
        // the head's largest squared row norm: the maximum over its pieces
        __shared__ float wmax[2];
        float best = 0.0f;
        for (int q = threadIdx.x; q < pb[C]; q += 128) best = fmaxf(best, pmax[(int64_t)bh * maxp + q]);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) best = fmaxf(best, __shfl_xor(best, off));
        if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = best;
        __syncthreads();
        if (threadIdx.x == 0) max_sqnorm[bh] = fmaxf(wmax[0], wmax[1]);
    }
    // 128 / D centroids per work-group (one for D >= 128), D threads each
    constexpr int CPW = D >= 128 ? 1 : 128 / D;
    const int jc = j * CPW + (D >= 128 ? 0 : (int)threadIdx.x / D);
    if (jc >= C) return;
    const int32_t *ob = offsets + (int64_t)bh * (C + 1);
    const int n = ob[jc + 1] - ob[jc];
    if (n == 0) return;  // empty: keep the centroid
    for (int k = D >= 128 ? (int)threadIdx.x : (int)threadIdx.x % D; k < D; k += 128) {
        double sum = 0.0;
        for (int q = pb[jc]; q < pb[jc + 1]; ++q) sum += partial[((int64_t)bh * maxp + q) * D + k];
        cent[((int64_t)bh * C + jc) * D + k] = (float)(sum / (double)n);
    }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void gather_kernel(const T *x, Strides xs, const T *comp, int H, int N,
                                                     const int32_t *perm, T *x_perm, T *comp_perm,
                                                     int64_t total)
{
    constexpr int TPR = D / 8;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int ck = (int)(e % TPR);
        const int64_t row = e / TPR;  // bh*N + r
        const int64_t bh = row / N;
        const int b = (int)(bh / H), h = (int)(bh % H);
        const int64_t src = b * xs.b + h * xs.h + (int64_t)perm[row] * xs.t + ck * 8;
        if (x_perm) copy8(x_perm + row * D + ck * 8, x + src);
        if (comp_perm) copy8(comp_perm + row * D + ck * 8, comp + src);
    }
}

// ---------------------------------------------------------------- MFMA assign (bf16 x)
// Distances |x - c|^2 = |c|^2 - 2<x, c> + |x|^2 on v_mfma_f32_32x32x16_bf16.  x is
// exact in bf16; each fp32 centroid, times -2 (exact), is split into bf16 planes
// hi + lo (16 significant bits, residual <= 2^-16 |c|); padded rows have norm 1e30.
// The norms enter the same accumulation through one more k step: |c|^2 and
// |x|^2 + M are each split exactly into three bf16 parts (24 significant bits),
// paired with ones, so the accumulator holds |x - c|^2 + M itself, M a per-token
// margin above the screening error (so the accumulator stays positive).  Per
// token the best candidates are kept (four; three at D = 16); whenever a rival lies within
// tau = 1e-4 (|x|^2 + max_j |c_j|^2) -- several times the worst-case error of the
// split and of fp32 accumulation -- the decision is re-taken on fp64 distances
// (the close candidates, or every centroid when all kept candidates are close),
// ties to the lower index.  Those fp64 distances are per-lane fused sums over a
// few dims, then a fixed butterfly over 16 lanes: a different rounding order from
// the plain sequential sum of the definition, which matters only at fp64 ties.
constexpr int kCT = 32;  // centroids per MFMA tile

// Exact split of an fp32 value into three bf16 parts, largest first.
__device__ __forceinline__ void split3_bf16(float v, uint16_t *out)
{
    const uint16_t h = f32_to_bf16_bits(v);
    const float r1 = v - bf16_bits_to_f32(h);  // exact
    const uint16_t m = f32_to_bf16_bits(r1);
    const float r2 = r1 - bf16_bits_to_f32(m);  // exact; at most 8 significant bits left
    out[0] = h;
    out[1] = m;
    out[2] = f32_to_bf16_bits(r2);
}

// One wave per centroid: bf16 planes hi + lo of -2c, the squared norm (fp64 over
// the lanes, then a fixed butterfly), and the norm row of the extra k step
// (|c|^2 in three bf16 parts, then three ones); padded rows get zero planes and
// norm 1e30.
template <int D>
__global__ __launch_bounds__(256) void centroid_planes_kernel(const float *cent, int C, int Cpad, uint16_t *planes,
                                                              float *norms, uint16_t *aug)
{
    // LPC lanes per centroid (D of them for D < 64): the fp64 norm is the same
    // butterfly either way, since lanes past D only ever added zeros
    constexpr int LPC = D < 64 ? D : 64, CPB = 256 / LPC;
    const int bh = blockIdx.y, lane = threadIdx.x % LPC;
    const int j = blockIdx.x * CPB + threadIdx.x / LPC;
    if (j >= Cpad) return;
    uint16_t *hi = planes + ((int64_t)bh * 2 * Cpad + j) * D;
    uint16_t *lo = planes + ((int64_t)bh * 2 * Cpad + Cpad + j) * D;
    double nn = 0.0;
    for (int k = lane; k < D; k += LPC) {
        if (j < C) {
            const float v = cent[((int64_t)bh * C + j) * D + k];
            const uint16_t hb = f32_to_bf16_bits(-2.0f * v);
            const float r = -2.0f * v - bf16_bits_to_f32(hb);  // exact
            hi[k] = hb;
            lo[k] = f32_to_bf16_bits(r);
            nn += (double)v * (double)v;
        } else {
            hi[k] = 0;
            lo[k] = 0;
        }
    }
#pragma unroll
    for (int off = LPC / 2; off > 0; off >>= 1) nn += __shfl_xor(nn, off);
    if (lane == 0) {
        const float nf = j < C ? (float)nn : 1e30f;  // padded: never wins
        norms[(int64_t)bh * Cpad + j] = nf;
        uint16_t row[16];
        split3_bf16(nf, row);
        row[3] = row[4] = row[5] = 0x3F80;  // 1.0
#pragma unroll
        for (int e = 6; e < 16; ++e) row[e] = 0;  // k = 6..15 of the extra step
        uint16_t *ar = aug + ((int64_t)bh * Cpad + j) * 16;
#pragma unroll
        for (int e = 0; e < 16; ++e) ar[e] = row[e];
    }
}

// Candidates are kept as integer keys: the bits of a positive approximate
// distance with the low bits replaced by the centroid index.  Positive floats
// order like their bit patterns, so unsigned min/med3 on keys order by distance
// (up to the dropped bits, a resolution of 2^bits ulps) and carry the index
// along.  The K smallest keys are kept sorted: one min and K-1 med3 per
// candidate.  K = 4, or 3 at d = 16 (a codebook assign that is bound by this
// epilogue; a token with all K kept candidates inside the decision window is
// rescanned in full, about 0.1 % of tokens with three and 0.003 % with four on
// 16-dim subspaces; with two, every close pair, about 3 %, would be).
template <int K>
struct TopK {
    uint32_t k[K];
};

__device__ __forceinline__ uint32_t umed3(uint32_t a, uint32_t b, uint32_t c)
{
    return max(min(a, b), min(max(a, b), c));
}

template <int K>
__device__ __forceinline__ void top_insert(TopK<K> &t, uint32_t key)
{
    uint32_t n[K];
#pragma unroll
    for (int i = K - 1; i >= 1; --i) n[i] = umed3(t.k[i - 1], t.k[i], key);
    n[0] = min(t.k[0], key);
#pragma unroll
    for (int i = 0; i < K; ++i) t.k[i] = n[i];
}

template <int D>
constexpr int topk_of() { return D == 16 ? 3 : 4; }

// fp64 partial sum of (x_k - c_k)^2 over the DPL dims of one lane (x bf16, c fp32;
// 16-byte aligned; DPL a multiple of 8), one fused chain in the order of k.
template <int DPL>
__device__ __forceinline__ double seg_sqdist(const uint16_t *xr, const float *cr)
{
    static_assert(DPL % 8 == 0, "whole 16-byte chunks of x");
    double part = 0.0;
#pragma unroll
    for (int k0 = 0; k0 < DPL; k0 += 8) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(xr + k0);
        const f32x4 c0 = *reinterpret_cast<const f32x4 *>(cr + k0);
        const f32x4 c1 = *reinterpret_cast<const f32x4 *>(cr + k0 + 4);
        float xv[8], cv[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            xv[2 * q] = __uint_as_float(w[q] << 16);
            xv[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
            cv[q] = c0[q];
            cv[4 + q] = c1[q];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const double a = (double)xv[q] - (double)cv[q];
            part = fma(a, a, part);
        }
    }
    return part;
}

// |x - c|^2 over 16 dims in fp64: the terms in the order k = 0..15, each squared
// difference rounded before it is added (no fused multiply-add), as in the exact
// definition (x bf16, c fp32; 16-byte aligned).
__device__ __forceinline__ double seq_sqdist16(const uint16_t *xr, const float *cr)
{
#pragma clang fp contract(off)
    double s = 0.0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(xr + 8 * h);
        const f32x4 c0 = *reinterpret_cast<const f32x4 *>(cr + 8 * h);
        const f32x4 c1 = *reinterpret_cast<const f32x4 *>(cr + 8 * h + 4);
        float xv[8], cv[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            xv[2 * q] = __uint_as_float(w[q] << 16);
            xv[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
            cv[q] = c0[q];
            cv[4 + q] = c1[q];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const double a = (double)xv[e] - (double)cv[e];
            s += a * a;
        }
    }
    return s;
}

// the sum over the 4 lanes of an aligned group
__device__ __forceinline__ double sum4(double v)
{
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 1);
    return v;
}

// Centroid tile in LDS: [plane][row][16-byte chunk], the chunks of row r
// XOR-swizzled by r mod (chunks per row), loaded straight from memory.
template <int D>
__device__ __forceinline__ int cswz(int plane, int row, int chunk)
{
    constexpr int CPR = D / 8;
    return (plane * kCT + row) * CPR + (chunk ^ (row & (CPR - 1)));
}

template <int D>
__device__ __forceinline__ void planes_direct(uint8_t *buf, const uint16_t *pb, const uint16_t *ab, int Cpad,
                                              int tile, int wave, int lane)
{
    constexpr int CPR = D / 8;
    constexpr int NCH = 2 * kCT * CPR;  // chunks per tile (both planes)
    // the tile's 32 norm rows (32 B each) after the planes: one 64-lane load
    if (wave == 0)
        __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)(ab + (int64_t)tile * kCT * 16 +
                                                                                        lane * 8),
                                         (void __attribute__((address_space(3))) *)(buf + NCH * 16), 16, 0, 0);
#pragma unroll
    for (int it = 0; it < (NCH + 255) / 256; ++it) {
        const int blk = it * 4 + wave;
        if (blk * 64 < NCH) {
            const int P = blk * 64 + lane;
            const int plane = P / (kCT * CPR), rem = P % (kCT * CPR), row = rem / CPR;
            const int c = (rem % CPR) ^ (row & (CPR - 1));
            const uint16_t *src = pb + ((int64_t)plane * Cpad + tile * kCT + row) * D + c * 8;
            __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)src,
                                             (void __attribute__((address_space(3))) *)(buf + blk * 1024), 16, 0,
                                             0);
        }
    }
}

// One tile of 32 centroids against the 64 tokens of this wave: the accumulators
// end as |x - c|^2 + 1 (norm step first, then the -2 <x, c> steps), and every
// (token, centroid) key goes into the token's kept candidates.  The key's index bits
// hold the centroid's row in the tile without the half-wave's offset of 4 rows;
// the caller adds it once per token.
template <int D, bool BYTEKEY>
__device__ __forceinline__ void assign_tile(const uint8_t *cur, int tile, int C, const bf16x8 (*xf)[D / 16],
                                            const bf16x8 *xaug, uint32_t hi_mask, TopK<topk_of<D>()> *top, int hl,
                                            int l32)
{
    constexpr int NDS = D / 16;
    constexpr int NCH = 2 * kCT * (D / 8);
    f32x16 acc[2];
    const bf16x8 an = *reinterpret_cast<const bf16x8 *>(cur + NCH * 16 + (l32 * 2 + hl) * 16);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(an, xaug[tb], f32x16{}, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
        const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(cur + cswz<D>(0, l32, 2 * s + hl) * 16);
        const bf16x8 al = *reinterpret_cast<const bf16x8 *>(cur + cswz<D>(1, l32, 2 * s + hl) * 16);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xf[tb][s], acc[tb], 0, 0, 0);
            acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xf[tb][s], acc[tb], 0, 0, 0);
        }
    }
    const uint32_t jb = (uint32_t)(tile * kCT);  // wave-uniform
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const uint32_t j = jb + (r >> 2) * 8 + (r & 3);
        // rows j and j + 4 both padding: skip (a scalar branch; a padding row j + 4
        // alone is inserted, and the decisions below keep it out)
        if (j >= (uint32_t)C) continue;
        // indices below 256: the key is the distance's upper three bytes and the
        // index byte (one byte permute); else the distance with its low bits
        // replaced by the index
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
            top_insert(top[tb], BYTEKEY ? __builtin_amdgcn_perm(__float_as_uint(acc[tb][r]), j, 0x07060500u)
                                        : ((__float_as_uint(acc[tb][r]) & hi_mask) | j));
    }
}

// At D = 16 the epilogue (key packing and top-k insertion on the VALU) outweighs the
// MFMA work and hides latency only through occupancy: six waves per SIMD (80 VGPRs)
// beat four; asking for seven spills to scratch and is slower again.
template <int D, bool BYTEKEY>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 16 ? 6 : 2))) void assign_mfma_kernel(
    const uint16_t *__restrict__ x, Strides xs, int H, int N, int C, int Cpad, const uint16_t *__restrict__ planes,
    const float *__restrict__ norms, const uint16_t *__restrict__ aug, const float *__restrict__ cent,
    int32_t *__restrict__ labels)
{
    constexpr int NDS = D / 16;
    constexpr int TBYTES = 2 * kCT * D * 2 + kCT * 32;  // both planes of a tile, then its norm rows
    __shared__ __attribute__((aligned(1024))) uint8_t tb0[TBYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t tb1[TBYTES];
    const int bh = blockIdx.y, b = bh / H, h = bh % H;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
    const uint16_t *xb = x + b * xs.b + h * xs.h;

    const uint16_t *pb = planes + (int64_t)bh * 2 * Cpad * D;
    const uint16_t *ab = aug + (int64_t)bh * Cpad * 16;
    const float *nb = norms + (int64_t)bh * Cpad;
    const int ntiles = Cpad / kCT;
    // Every prologue load is issued before the first wait: tile 0's planes, the
    // token rows, then the centroid norms (for the largest, used by the decision
    // window; an index past C re-reads norm C - 1, harmless for a maximum).
    planes_direct<D>(tb0, pb, ab, Cpad, 0, wave, lane);
    int tok[2];
    bf16x8 xf[2][NDS];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int t = blockIdx.x * 256 + wave * 64 + tb * 32 + l32;
        tok[tb] = t;
        const uint16_t *row = xb + (int64_t)min(t, N - 1) * xs.t + hl * 8;
#pragma unroll
        for (int s = 0; s < NDS; ++s) xf[tb][s] = *reinterpret_cast<const bf16x8 *>(row + s * 16);
    }
    __shared__ float cm_part[4];
    float lmax = 0.0f;
    for (int j0 = 0; j0 < C; j0 += 1024) {
        float nv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) nv[u] = nb[min(j0 + u * 256 + tid, C - 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u) lmax = fmaxf(lmax, nv[u]);
    }
    float xn[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        float ss = 0.0f;
#pragma unroll
        for (int s = 0; s < NDS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = (float)xf[tb][s][e];
                ss = fmaf(v, v, ss);
            }
        xn[tb] = ss + __shfl_xor(ss, 32);
    }
    int ibits = 1;
    while ((1 << ibits) < Cpad) ++ibits;
    if (BYTEKEY) ibits = 8;  // Cpad <= 256: the index is the key's low byte
    const uint32_t imask = (1u << ibits) - 1u;
    // the key's mask lives in a vector register: with the index a scalar, the key
    // is then one v_and_or_b32 (a VOP3 reads at most one scalar operand)
    uint32_t hi_mask;
    asm volatile("v_mov_b32 %0, %1" : "=v"(hi_mask) : "s"(~imask));
    constexpr int TK = topk_of<D>();
    TopK<TK> top[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int c = 0; c < TK; ++c) top[tb].k[c] = 0xFFFFFFFFu;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, off));
    if (lane == 0) cm_part[wave] = lmax;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const float cm = fmaxf(fmaxf(cm_part[0], cm_part[1]), fmaxf(cm_part[2], cm_part[3]));
    // B operand of the norm step: [1, 1, 1, (|x|^2 + M) in three parts] in k = 0..7
    // (lanes of the first half-wave), zero in k = 8..15.  The margin
    // M = 1 + 1e-4 (|x|^2 + max|c|^2) is the same for every centroid of the token, so
    // it leaves the ranking alone; it exceeds the worst-case screening error (the
    // decision window below is built on the same bound), so every accumulator ends
    // >= 1 even where |x - c|^2 is 0 and the norms are large: keys stay positive
    // floats and order like their bits.
    bf16x8 xaug[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const float xn1 = xn[tb] + fmaf(1e-4f, xn[tb] + cm, 1.0f);
        const uint16_t h = f32_to_bf16_bits(xn1);
        const float r1 = xn1 - bf16_bits_to_f32(h);
        const uint16_t m = f32_to_bf16_bits(r1);
        const uint16_t l = f32_to_bf16_bits(r1 - bf16_bits_to_f32(m));
        const uint16_t parts[8] = {0x3F80, 0x3F80, 0x3F80, h, m, l, 0, 0};
#pragma unroll
        for (int e = 0; e < 8; ++e) xaug[tb][e] = __builtin_bit_cast(__bf16, (uint16_t)(hl ? 0 : parts[e]));
    }
    for (int tile = 0; tile < ntiles; tile += 2) {
        // tile in tb0 while tile+1 loads into tb1, then the reverse
        if (tile + 1 < ntiles) planes_direct<D>(tb1, pb, ab, Cpad, tile + 1, wave, lane);
        assign_tile<D, BYTEKEY>(tb0, tile, C, xf, xaug, hi_mask, top, hl, l32);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tile + 1 >= ntiles) break;
        if (tile + 2 < ntiles) planes_direct<D>(tb0, pb, ab, Cpad, tile + 2, wave, lane);
        assign_tile<D, BYTEKEY>(tb1, tile + 1, C, xf, xaug, hi_mask, top, hl, l32);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    // the second half-wave's candidates are 4 rows further into each group of 8
    // (slots never filled keep the empty key 0xFFFFFFFF, which must not wrap: with
    // C < 4 a half-wave inserts fewer than four keys, the padding rows being skipped)
    if (hl) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int c = 0; c < TK; ++c)
                if (top[tb].k[c] != 0xFFFFFFFFu) top[tb].k[c] += 4u;
    }

    // Decisions.  Close calls go to a work list of (token, candidate) entries whose
    // |x - c|^2 is evaluated in fp64, and the token takes the smallest (ties to the
    // lower index).  A token whose kept candidates are all within tau is rescanned
    // in fp64 over all C.  At D = 16 one lane takes a whole entry (or centroid of a
    // rescan) and sums in the exact definition's order and rounding; wider rows
    // spread an entry over 4 lanes (a fused fp64 chain over D/4 dims per lane, then
    // a butterfly), so that one pass of loads covers a work-group's entries.
    constexpr int kRQ = 3 * 256;
    constexpr int DPL = D / 4;  // dims per lane of a 4-lane distance (rows wider than 16)
    __shared__ int rq_n, full_n;
    __shared__ int rq_slot[kRQ];
    __shared__ int rq_cand[kRQ];
    __shared__ double rq_dist[kRQ];
    __shared__ int full_slot[256];
    __shared__ int full_best[256];
    __shared__ double grp_d[4];
    __shared__ int grp_j[4];
    if (tid == 0) { rq_n = 0; full_n = 0; }
    __syncthreads();
    const float *cb = cent + (int64_t)bh * C * D;
    int qpos[2] = {0, 0}, qcnt[2] = {0, 0}, fpos[2] = {-1, -1};
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        TopK<TK> &T = top[tb];
        uint32_t other[TK];
#pragma unroll
        for (int c = 0; c < TK; ++c) other[c] = __shfl_xor(T.k[c], 32);
#pragma unroll
        for (int c = 0; c < TK; ++c) top_insert(T, other[c]);
        if (hl != 0 || tok[tb] >= N) continue;
        // window: tau plus the key resolution (2^ibits ulps of the largest value compared)
        const float tau = 1e-4f * (xn[tb] + cm);
        const float d1 = __uint_as_float(T.k[0] & hi_mask);
        const float lim0 = d1 + tau;
        const float res = __uint_as_float((__float_as_uint(lim0) & 0x7F800000u)) * ldexpf(1.0f, ibits - 23);
        const float lim = lim0 + 2.0f * res;
        const int slot = wave * 64 + tb * 32 + l32;
        // The second half-wave's rows j + 4 of the last tile can be padding while
        // rows j are not; their keys (norm 1e30) lose to every real distance below
        // that, but with extreme magnitudes or infinities one could be kept first
        // or inside the window.  Such a token is rescanned over the real centroids.
        int n = 1;
        bool pad = (T.k[0] & imask) >= (uint32_t)C;
#pragma unroll
        for (int c = 1; c < TK; ++c) {
            const bool in = __uint_as_float(T.k[c] & hi_mask) < lim;
            n += in;
            pad = pad || (in && (T.k[c] & imask) >= (uint32_t)C);
        }
        if (n == TK || pad) {  // every kept candidate is close: all centroids in fp64
            const int f = atomicAdd(&full_n, 1);
            full_slot[f] = slot;
            fpos[tb] = f;
        } else if (n > 1) {
            const int pos = atomicAdd(&rq_n, n);
#pragma unroll
            for (int c = 0; c < TK - 1; ++c)
                if (c < n) {
                    rq_slot[pos + c] = slot;
                    rq_cand[pos + c] = (int)(T.k[c] & imask);
                }
            qpos[tb] = pos;
            qcnt[tb] = n;
        }
    }
    __syncthreads();
    if constexpr (D == 16) {
        const int nq = rq_n;
        for (int e = tid; e < nq; e += 256) {
            const int t = blockIdx.x * 256 + rq_slot[e];
            rq_dist[e] = seq_sqdist16(xb + (int64_t)t * xs.t, cb + (int64_t)rq_cand[e] * 16);
        }
        const int nf = full_n;
        for (int f = 0; f < nf; ++f) {
            const int t = blockIdx.x * 256 + full_slot[f];
            const uint16_t *xr = xb + (int64_t)t * xs.t;
            double bd = INFINITY;
            int bj = 0;
            for (int j = tid; j < C; j += 256) {
                const double dd = seq_sqdist16(xr, cb + (int64_t)j * 16);
                if (dd < bd) { bd = dd; bj = j; }
            }
            // smallest distance, ties to the lower index: over the wave, then the waves
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                const double od = __shfl_xor(bd, off);
                const int oj = __shfl_xor(bj, off);
                if (od < bd || (od == bd && oj < bj)) { bd = od; bj = oj; }
            }
            if (lane == 0) { grp_d[wave] = bd; grp_j[wave] = bj; }
            __syncthreads();
            if (tid == 0) {
                double b = grp_d[0];
                int jb = grp_j[0];
                for (int g = 1; g < 4; ++g)
                    if (grp_d[g] < b || (grp_d[g] == b && grp_j[g] < jb)) { b = grp_d[g]; jb = grp_j[g]; }
                full_best[f] = jb;
            }
            __syncthreads();
        }
    } else {
    const int sub = tid & 3, grp = tid >> 2;
    {
        const int nq = rq_n;
        for (int e = grp; e < nq; e += 64) {
            const int t = blockIdx.x * 256 + rq_slot[e];
            const double dd = sum4(seg_sqdist<DPL>(xb + (int64_t)t * xs.t + sub * DPL,
                                                   cb + (int64_t)rq_cand[e] * D + sub * DPL));
            if (sub == 0) rq_dist[e] = dd;
        }
    }
    const int nf = full_n;
    for (int f = 0; f < nf; ++f) {
        const int t = blockIdx.x * 256 + full_slot[f];
        const uint16_t *xr = xb + (int64_t)t * xs.t + sub * DPL;
        double bd = INFINITY;
        int bj = 0;
        for (int j = grp; j < C; j += 64) {
            const double dd = sum4(seg_sqdist<DPL>(xr, cb + (int64_t)j * D + sub * DPL));
            if (dd < bd) { bd = dd; bj = j; }
        }
        // smallest distance, ties to the lower index: over the wave, then the waves
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const double od = __shfl_xor(bd, off);
            const int oj = __shfl_xor(bj, off);
            if (od < bd || (od == bd && oj < bj)) { bd = od; bj = oj; }
        }
        if (lane == 0) { grp_d[wave] = bd; grp_j[wave] = bj; }
        __syncthreads();
        if (tid == 0) {
            double b = grp_d[0];
            int jb = grp_j[0];
            for (int g = 1; g < 4; ++g)
                if (grp_d[g] < b || (grp_d[g] == b && grp_j[g] < jb)) { b = grp_d[g]; jb = grp_j[g]; }
            full_best[f] = jb;
        }
        __syncthreads();
    }
    }
    __syncthreads();
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int t = tok[tb];
        if (hl != 0 || t >= N) continue;
        int best = (int)(top[tb].k[0] & imask);
        if (fpos[tb] >= 0) {
            best = full_best[fpos[tb]];
        } else if (qcnt[tb] > 1) {
            double bd = rq_dist[qpos[tb]];
            best = rq_cand[qpos[tb]];
            for (int q = 1; q < qcnt[tb]; ++q) {
                const double dd = rq_dist[qpos[tb] + q];
                const int j = rq_cand[qpos[tb] + q];
                if (dd < bd || (dd == bd && j < best)) { bd = dd; best = j; }
            }
        }
        labels[(int64_t)bh * N + t] = best;
    }
}

struct ClusterWs {
    size_t off_hist, off_tot, off_planes, off_norms, off_aug, off_poff, off_ptab, off_partial, off_pmax, total;
    int Cpad, maxp;
};

ClusterWs cluster_ws(int B, int H, int N, int d, int C)
{
    ClusterWs w;
    const size_t BH = (size_t)B * H;
    const size_t nchunks = ((size_t)N + kSortChunk - 1) / kSortChunk;
    w.Cpad = (C + kCT - 1) / kCT * kCT;
    w.maxp = (N + piece_rows(d) - 1) / piece_rows(d) + C;  // >= sum over groups of ceil(n_j / piece rows)
    size_t o = 0;
    w.off_hist = o; o += isg_align256(BH * nchunks * C * sizeof(int32_t));
    w.off_tot = o; o += isg_align256(BH * C * sizeof(int32_t));
    w.off_planes = o; o += isg_align256(BH * 2 * w.Cpad * d * sizeof(uint16_t));
    w.off_norms = o; o += isg_align256(BH * w.Cpad * sizeof(float));
    w.off_aug = o; o += isg_align256(BH * w.Cpad * 16 * sizeof(uint16_t));
    w.off_poff = o; o += isg_align256(BH * (C + 1) * sizeof(int32_t));
    w.off_ptab = o; o += isg_align256(BH * (size_t)w.maxp * sizeof(int4));
    w.off_partial = o; o += isg_align256(BH * (size_t)w.maxp * d * sizeof(double));
    w.off_pmax = o; o += isg_align256(BH * (size_t)w.maxp * sizeof(float));
    w.total = o;
    return w;
}

template <typename T, int D>
void launch_assign(hipStream_t st, const T *x, Strides xs, int B, int H, int N, int C, const float *cent,
                   int32_t *labels, uint8_t *ws, const ClusterWs &w)
{
    const int BH = B * H;
    if constexpr (std::is_same<T, uint16_t>::value) {
        uint16_t *planes = (uint16_t *)(ws + w.off_planes);
        float *norms = (float *)(ws + w.off_norms);
        uint16_t *aug = (uint16_t *)(ws + w.off_aug);
        centroid_planes_kernel<D><<<dim3(w.Cpad / (D < 64 ? 256 / D : 4), BH), 256, 0, st>>>(cent, C, w.Cpad, planes,
                                                                                          norms, aug);
        const dim3 grid((N + 255) / 256, BH);
        if (w.Cpad <= 256)
            assign_mfma_kernel<D, true><<<grid, 256, 0, st>>>(x, xs, H, N, C, w.Cpad, planes, norms, aug, cent,
                                                              labels);
        else
            assign_mfma_kernel<D, false><<<grid, 256, 0, st>>>(x, xs, H, N, C, w.Cpad, planes, norms, aug, cent,
                                                               labels);
    } else {
        assign_kernel<T, D><<<dim3((N + 255) / 256, BH), 256, 0, st>>>(x, xs, H, N, C, cent, labels);
    }
}

// Subspace-major copy for product quantisation: x[b][h][t][s*ds + e] ->
// out[s][b][h][t][e].  A work-group moves 64 tokens: it reads their rows whole
// (coalesced) and writes P runs of 64*ds contiguous elements, so each subspace's
// k-means then reads dense ds-element rows instead of ds-element pieces of longer
// rows (a 32-byte piece costs a 128-byte line fetch).  With wmax non-null (bf16)
// it also writes, per subspace, the largest exponent field among the work-group's
// values (sign dropped) to wmax[(s*B*H + bh) * gridDim.x + blockIdx.x]; the
// integer update scales by the maximum of these over a subspace.
template <typename T>
__global__ __launch_bounds__(256) void pq_split_kernel(const T *x, Strides xs, int B, int H, int N, int d, int ds,
                                                       T *out, int32_t *wmax)
{
    __shared__ int smax[kPqMaxP];
    const int cpr = d / 8;  // 8-element chunks per row
    const int bh = blockIdx.y, b = bh / H, h = bh % H;
    const int t0 = blockIdx.x * 64;
    const int nt = min(64, N - t0);
    const int64_t plane = (int64_t)B * H * N * ds;
    if (wmax) {
        for (int s = threadIdx.x; s < d / ds; s += 256) smax[s] = 0;
        __syncthreads();
    }
    int ps = -1;  // this thread's subspace so far and its largest exponent field
    uint32_t pm = 0;
    for (int q = threadIdx.x; q < nt * cpr; q += 256) {
        const int tt = q / cpr, c = q % cpr;
        const int s = (c * 8) / ds, e0 = (c * 8) % ds;
        const T *src = x + b * xs.b + h * xs.h + (int64_t)(t0 + tt) * xs.t + c * 8;
        T *dst = out + s * plane + ((int64_t)bh * N + t0 + tt) * ds + e0;
        if constexpr (std::is_same<T, uint16_t>::value) {
            const uint4 w = *reinterpret_cast<const uint4 *>(src);
            *reinterpret_cast<uint4 *>(dst) = w;
            if (wmax) {
                if (s != ps) {
                    if (ps >= 0) atomicMax(&smax[ps], (int)pm);
                    ps = s;
                    pm = 0;
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) pm = max(pm, max((w[k] >> 7) & 0xFFu, (w[k] >> 23) & 0xFFu));
            }
        } else {
            copy8(dst, src);
        }
    }
    if (wmax) {
        if (ps >= 0) atomicMax(&smax[ps], (int)pm);
        __syncthreads();
        for (int s = threadIdx.x; s < d / ds; s += 256)
            wmax[((int64_t)s * B * H + bh) * gridDim.x + blockIdx.x] = smax[s];
    }
}

// emax[p] = the largest of the split's per-work-group exponent fields of triple p.
__global__ __launch_bounds__(256) void pq_emax_kernel(const int32_t *wmax, int nwg, int32_t *emax)
{
    __shared__ int part[4];
    const int p = blockIdx.x;
    int m = 0;
    for (int i = threadIdx.x; i < nwg; i += 256) m = max(m, wmax[(int64_t)p * nwg + i]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = max(m, __shfl_xor(m, off));
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) emax[p] = max(max(part[0], part[1]), max(part[2], part[3]));
}

// ---------------------------------------------------------------- PQ update from integer sums
// The k-means update of 16-dim bf16 subspaces with at most kPqIntMaxC codewords
// needs no sorted order: every row is added into its codeword's sum as an exact
// integer.  A subspace whose largest exponent field is E holds values below
// 2^(E-126); times 2^s, s = 126 - E + lim, each is below 2^lim and is rounded to
// an integer (exact unless its exponent lies more than lim - 8 below E), and any
// sum of N of them stays below 2^62 (lim = min(62 - ceil(log2(N+1)), 51); 51 keeps
// the rounding trick below exact).  Integer sums do not depend on the order of
// the additions, so work-groups add a chunk of tokens each in LDS with atomics,
// and the result is the same on every run.  The mean, (sum * 2^-s) / n in fp64
// rounded to fp32, equals the sorted fp64 sum's whenever that sum is exact.
__host__ __device__ constexpr int pq_int_lim(int N)
{
    int L = 0;
    while (L < 31 && (1LL << L) <= (long long)N) ++L;  // N < 2^L
    return 62 - L < 51 ? 62 - L : 51;
}

__device__ __forceinline__ int pq_int_shift(int32_t e, int N) { return 126 - max(e, 1) + pq_int_lim(N); }

// The chunk's sums in LDS ([codeword][17]: 16 dims and a pad word, so that the
// atomics of one instruction spread over the banks) and counts; two lanes per
// token, 8 dims each.  Then the chunk's partial, [C][16] int64 and [C] int32,
// goes to acc.
__global__ __launch_bounds__(kPqAccThreads) void pq_accum16_kernel(const uint16_t *__restrict__ xc,
                                                         const int32_t *__restrict__ labels, int N, int C,
                                                         const int32_t *__restrict__ emax, int nchunk,
                                                         size_t chunk_bytes, uint8_t *__restrict__ acc)
{
    extern __shared__ __attribute__((aligned(16))) unsigned long long lsum[];
    unsigned *lcnt = reinterpret_cast<unsigned *>(lsum + C * kPqPitch);
    const int pair = blockIdx.y, chunk = blockIdx.x, tid = threadIdx.x, hl = tid & 1;
    for (int i = tid; i < C * kPqPitch; i += kPqAccThreads) lsum[i] = 0ull;
    for (int i = tid; i < C; i += kPqAccThreads) lcnt[i] = 0u;
    __syncthreads();
    const double sc = ldexp(1.0, pq_int_shift(emax[pair], N));
    const double magic = 6755399441055744.0;  // 1.5 * 2^52: adding it rounds |y| < 2^51 to an integer
    const long long mbits = __double_as_longlong(magic);
    const int t0 = chunk * kPqAccTok, t1 = min(N, t0 + kPqAccTok);
    const uint16_t *xb = xc + (int64_t)pair * N * 16 + hl * 8;
    const int32_t *lb = labels + (int64_t)pair * N;
    constexpr int U = 4;  // tokens per lane in flight
    for (int tb = t0 + (tid >> 1); tb < t1; tb += kPqAccThreads / 2 * U) {
        int lab[U];
        uint4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = tb + u * (kPqAccThreads / 2);
            lab[u] = t < t1 ? lb[t] : -1;
            if (t < t1) w[u] = *reinterpret_cast<const uint4 *>(xb + (int64_t)t * 16);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (lab[u] < 0) continue;
            unsigned long long *row = lsum + lab[u] * kPqPitch + hl * 8;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float lo = __uint_as_float(w[u][k] << 16), hi = __uint_as_float(w[u][k] & 0xFFFF0000u);
                const long long il = __double_as_longlong(fma((double)lo, sc, magic)) - mbits;
                const long long ih = __double_as_longlong(fma((double)hi, sc, magic)) - mbits;
                atomicAdd(row + 2 * k, (unsigned long long)il);
                atomicAdd(row + 2 * k + 1, (unsigned long long)ih);
            }
            if (hl == 0) atomicAdd(lcnt + lab[u], 1u);
        }
    }
    __syncthreads();
    uint8_t *dst = acc + ((int64_t)pair * nchunk + chunk) * chunk_bytes;
    unsigned long long *ds = reinterpret_cast<unsigned long long *>(dst);
    for (int i = tid; i < C * 16; i += kPqAccThreads) ds[i] = lsum[(i >> 4) * kPqPitch + (i & 15)];
    unsigned *dc = reinterpret_cast<unsigned *>(dst + (size_t)C * 16 * 8);
    for (int i = tid; i < C; i += kPqAccThreads) dc[i] = lcnt[i];
}

// Adds the chunks' partials of one (subspace, batch, head) triple and divides:
// one thread per (codeword, dim); an empty codeword keeps its value.
__global__ __launch_bounds__(256) void pq_final16_kernel(const uint8_t *__restrict__ acc, int nchunk,
                                                         size_t chunk_bytes, int N, int C,
                                                         const int32_t *__restrict__ emax, float *__restrict__ cent)
{
    const int pair = blockIdx.y, k = blockIdx.x * 256 + threadIdx.x;
    if (k >= C * 16) return;
    const int j = k >> 4;
    long long S = 0;
    long long n = 0;
    for (int c = 0; c < nchunk; ++c) {
        const uint8_t *src = acc + ((int64_t)pair * nchunk + c) * chunk_bytes;
        S += reinterpret_cast<const long long *>(src)[k];
        n += reinterpret_cast<const unsigned *>(src + (size_t)C * 16 * 8)[j];
    }
    if (n == 0) return;
    const double sum = ldexp((double)S, -pq_int_shift(emax[pair], N));
    cent[((int64_t)pair * C + j) * 16 + (k & 15)] = (float)(sum / (double)n);
}

template <typename T, int D>
isg_status run_cluster(hipStream_t st, const T *x, Strides xs, int B, int H, int N, int C, int iters,
                       int init_mode, const T *comp, float *cent, int32_t *labels, int32_t *perm,
                       int32_t *offsets, T *x_perm, T *comp_perm, float *max_sqnorm, uint8_t *ws)
{
    const int BH = B * H;
    const int nchunks = (N + kSortChunk - 1) / kSortChunk;
    const ClusterWs w = cluster_ws(B, H, N, D, C);
    int32_t *hist = (int32_t *)(ws + w.off_hist);
    int32_t *tot = (int32_t *)(ws + w.off_tot);
    int32_t *poff = (int32_t *)(ws + w.off_poff);
    int4 *ptab = (int4 *)(ws + w.off_ptab);
    double *partial = (double *)(ws + w.off_partial);
    float *pmax = (float *)(ws + w.off_pmax);
    int bits = 1;
    while ((1 << bits) < C) ++bits;
    const int64_t upd_n = (int64_t)w.maxp * BH;         // (piece, head) work-groups
    const int64_t sc_n = (int64_t)nchunks * BH;          // (chunk, head) scatter waves
    const unsigned sc_blocks = (unsigned)((sc_n + 7) & ~(int64_t)7);
    const unsigned upd_blocks = (unsigned)((upd_n + 7) & ~(int64_t)7);
    if (init_mode == 0) {
        const int64_t total = (int64_t)BH * C * D;
        const int grid = (int)std::min<int64_t>((total + 255) / 256, 65536);
        init_centroids_kernel<T><<<grid, 256, 0, st>>>(x, xs, H, N, C, D, cent, total);
    }
    for (int it = 0; it < iters; ++it) {
        const bool last_norms = max_sqnorm && it + 1 == iters;
        launch_assign<T, D>(st, x, xs, B, H, N, C, cent, labels, ws, w);
        hist_kernel<<<dim3(nchunks, BH), 256, 0, st>>>(labels, N, C, nchunks, hist);
        scan_kernel<<<dim3((C + 63) / 64, BH), 256, 0, st>>>(hist, nchunks, C, tot);
        scatter_kernel<<<sc_blocks, 64, C * sizeof(int32_t), st>>>(labels, hist, tot, N, C, nchunks, bits,
                                                                   piece_rows(D), w.maxp, sc_n, perm, offsets,
                                                                   poff, ptab);
        // the last iteration's update also writes the permuted copy of x
        update_piece_kernel<T, D><<<upd_blocks, 256, 0, st>>>(x, xs, H, N, C, perm, poff, ptab, w.maxp, upd_n,
                                                              partial, it + 1 == iters ? x_perm : nullptr,
                                                              last_norms ? pmax : nullptr);
        update_final_kernel<D><<<dim3((C + (D >= 128 ? 1 : 128 / D) - 1) / (D >= 128 ? 1 : 128 / D), BH), 128, 0, st>>>(C, offsets, poff, w.maxp, partial, cent,
                                                            last_norms ? pmax : nullptr, max_sqnorm);
    }
    if (comp_perm) {
        const int64_t total = (int64_t)BH * N * (D / 8);
        const int grid = (int)std::min<int64_t>((total + 255) / 256, 1 << 20);
        gather_kernel<T, D><<<grid, 256, 0, st>>>(x, xs, comp, H, N, perm, nullptr, comp_perm, total);
    }
    return isg_check_launch("isg_cluster");
}

// Lloyd rounds of 16-dim bf16 subspaces with at most kPqIntMaxC codewords on the
// dense subspace-major copy (PB = P*B batches): run_cluster's init and assign,
// then the integer-sum update; no sorted order is built (the codes are the last
// round's labels and the codebooks the means of those groups, as there).
isg_status run_pq16(hipStream_t st, const uint16_t *xc, int PB, int H, int N, int C, int iters,
                    const int32_t *emax, float *cent, int32_t *labels, uint8_t *acc, size_t chunk_bytes,
                    uint8_t *ws)
{
    const int pairs = PB * H;
    const Strides cs{(int64_t)H * N * 16, (int64_t)N * 16, 16};
    const ClusterWs w = cluster_ws(PB, H, N, 16, C);
    const int nchunk = (N + kPqAccTok - 1) / kPqAccTok;
    const int64_t total = (int64_t)pairs * C * 16;
    init_centroids_kernel<uint16_t><<<(int)std::min<int64_t>((total + 255) / 256, 65536), 256, 0, st>>>(
        xc, cs, H, N, C, 16, cent, total);
    const size_t lds = (size_t)C * kPqPitch * sizeof(unsigned long long) + (size_t)C * sizeof(unsigned);
    for (int it = 0; it < iters; ++it) {
        launch_assign<uint16_t, 16>(st, xc, cs, PB, H, N, C, cent, labels, ws, w);
        pq_accum16_kernel<<<dim3(nchunk, pairs), kPqAccThreads, lds, st>>>(xc, labels, N, C, emax, nchunk, chunk_bytes, acc);
        pq_final16_kernel<<<dim3((C * 16 + 255) / 256, pairs), 256, 0, st>>>(acc, nchunk, chunk_bytes, N, C, emax,
                                                                            cent);
    }
    return isg_check_launch("isg_pq_codebooks");
}

template <typename T>
isg_status dispatch_d(int d, hipStream_t st, const T *x, Strides xs, int B, int H, int N, int C,
                      int iters, int init_mode, const T *comp, float *cent, int32_t *labels,
                      int32_t *perm, int32_t *offsets, T *x_perm, T *comp_perm, float *max_sqnorm, uint8_t *ws)
{
    switch (d) {
    case 16:
        return run_cluster<T, 16>(st, x, xs, B, H, N, C, iters, init_mode, comp, cent, labels, perm,
                                  offsets, x_perm, comp_perm, max_sqnorm, ws);
    case 64:
        return run_cluster<T, 64>(st, x, xs, B, H, N, C, iters, init_mode, comp, cent, labels, perm,
                                  offsets, x_perm, comp_perm, max_sqnorm, ws);
    case 128:
        return run_cluster<T, 128>(st, x, xs, B, H, N, C, iters, init_mode, comp, cent, labels, perm,
                                   offsets, x_perm, comp_perm, max_sqnorm, ws);
    default:
        return isg_fail(ISG_E_UNSUPPORTED, "isg_cluster: d=%d not built (16, 64, 128)", d);
    }
}

// Host-side checks shared by isg_cluster and isg_cluster_noalloc (everything but
// the workspace).
isg_status check_cluster_args(const void *x, isg_dtype dt, const int64_t x_strides[3], int B, int H, int N,
                              int d, int C, int iters, int init_mode, const void *companion,
                              const float *centroids, const int32_t *labels, const int32_t *perm,
                              const int32_t *offsets, const void *x_perm, const void *companion_perm)
{
    ISG_REQUIRE(x && x_strides && centroids && labels && perm && offsets, ISG_E_ARG,
                "isg_cluster: null pointer argument");
    ISG_REQUIRE(B >= 1 && H >= 1 && N >= 1, ISG_E_ARG, "isg_cluster: B, H, N must be >= 1 (got %d, %d, %d)",
                B, H, N);
    ISG_REQUIRE((int64_t)B * H <= 65535, ISG_E_ARG, "isg_cluster: B*H must be <= 65535 (got %lld)",
                (long long)B * H);
    ISG_REQUIRE(dt == ISG_F32 || dt == ISG_BF16, ISG_E_DTYPE, "isg_cluster: dtype %d", (int)dt);
    ISG_REQUIRE(d == 16 || d == 64 || d == 128, ISG_E_UNSUPPORTED, "isg_cluster: d=%d not built (16, 64, 128)",
                d);
    ISG_REQUIRE(C >= 1 && C <= N && C <= kMaxC, ISG_E_ARG, "isg_cluster: need 1 <= C <= min(N, %d), got C=%d N=%d",
                kMaxC, C, N);
    ISG_REQUIRE(iters >= 1, ISG_E_ARG, "isg_cluster: iters must be >= 1 (got %d)", iters);
    ISG_REQUIRE(init_mode == 0 || init_mode == 1, ISG_E_ARG, "isg_cluster: init_mode must be 0 or 1");
    ISG_REQUIRE((companion == nullptr) == (companion_perm == nullptr), ISG_E_ARG,
                "isg_cluster: companion and companion_perm must both be given or both be NULL");
    for (int k = 0; k < 3; ++k)
        ISG_REQUIRE(x_strides[k] >= 0 && x_strides[k] % 8 == 0, ISG_E_ARG,
                    "isg_cluster: x_strides must be non-negative multiples of 8 elements");
    ISG_REQUIRE(x_strides[2] >= d, ISG_E_ARG, "isg_cluster: token stride %lld < d", (long long)x_strides[2]);
    ISG_REQUIRE(((uintptr_t)x & 15) == 0 && ((uintptr_t)companion & 15) == 0 && ((uintptr_t)x_perm & 15) == 0 &&
                    ((uintptr_t)companion_perm & 15) == 0,
                ISG_E_ARG, "isg_cluster: x / companion / outputs must be 16-byte aligned");
    return ISG_OK;
}

isg_status run_checked(hipStream_t st, const void *x, isg_dtype dt, const int64_t x_strides[3], int B, int H,
                       int N, int d, int C, int iters, int init_mode, const void *companion, float *centroids,
                       int32_t *labels, int32_t *perm, int32_t *offsets, void *x_perm, void *companion_perm,
                       float *max_sqnorm, uint8_t *ws)
{
    Strides xs{x_strides[0], x_strides[1], x_strides[2]};
    if (dt == ISG_F32)
        return dispatch_d<float>(d, st, (const float *)x, xs, B, H, N, C, iters, init_mode,
                                 (const float *)companion, centroids, labels, perm, offsets, (float *)x_perm,
                                 (float *)companion_perm, max_sqnorm, ws);
    return dispatch_d<uint16_t>(d, st, (const uint16_t *)x, xs, B, H, N, C, iters, init_mode,
                                (const uint16_t *)companion, centroids, labels, perm, offsets,
                                (uint16_t *)x_perm, (uint16_t *)companion_perm, max_sqnorm, ws);
}

// ---------------------------------------------------------------- scratch of isg_cluster_noalloc
// A fixed device array takes the place of the caller's workspace.  Every GPU the
// library runs on holds its own copy (allocated with the code object, kept until
// the process ends).  In host code `scratch` names a host-side stand-in, not a
// device address, so it is never passed to a kernel: its device address is looked
// up once per device and only that pointer is used.  Every call on one GPU shares
// the array; nothing in it has to start at zero (each round writes every word it
// later reads), and calls that overlap on one GPU race.
constexpr size_t kNoAllocScratchBytes = (size_t)ISG_CLUSTER_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t *g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch`, resolved on the first call
// for that device with the device current.
isg_status scratch_for_stream(hipStream_t st, uint8_t **out)
{
    int dev = 0;
    if (st) {
        hipDevice_t sd = 0;
        const hipError_t e = hipStreamGetDevice(st, &sd);
        if (e != hipSuccess) return isg_fail(ISG_E_HIP, "isg_cluster_noalloc: hipStreamGetDevice: %s",
                                             hipGetErrorString(e));
        dev = (int)sd;
    } else {
        const hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return isg_fail(ISG_E_HIP, "isg_cluster_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    }
    ISG_REQUIRE(dev >= 0 && dev < kMaxDevices, ISG_E_UNSUPPORTED, "isg_cluster_noalloc: device %d >= %d", dev,
                kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        void *p = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess || !p)
            return isg_fail(ISG_E_HIP, "isg_cluster_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                            hipGetErrorString(e));
        g_scratch_ptr[dev] = (uint8_t *)p;
    }
    *out = g_scratch_ptr[dev];
    return ISG_OK;
}

}  // namespace

extern "C" size_t isg_cluster_workspace_size(int B, int H, int N, int d, int C)
{
    if (B < 1 || H < 1 || N < 1 || C < 1 || d < 1) return 0;
    return cluster_ws(B, H, N, d, C).total;
}

extern "C" isg_status isg_cluster(void *stream, const void *x, isg_dtype dt, const int64_t x_strides[3],
                                  int B, int H, int N, int d, int C, int iters, int init_mode,
                                  const void *companion, float *centroids, int32_t *labels, int32_t *perm,
                                  int32_t *offsets, void *x_perm, void *companion_perm, float *max_sqnorm,
                                  void *workspace, size_t ws_bytes)
{
    const isg_status a = check_cluster_args(x, dt, x_strides, B, H, N, d, C, iters, init_mode, companion,
                                            centroids, labels, perm, offsets, x_perm, companion_perm);
    if (a != ISG_OK) return a;
    const size_t need = isg_cluster_workspace_size(B, H, N, d, C);
    ISG_REQUIRE(workspace && ws_bytes >= need, ISG_E_WORKSPACE, "isg_cluster: workspace %zu < %zu bytes",
                workspace ? ws_bytes : (size_t)0, need);
    return run_checked((hipStream_t)stream, x, dt, x_strides, B, H, N, d, C, iters, init_mode, companion, centroids,
                       labels, perm, offsets, x_perm, companion_perm, max_sqnorm, (uint8_t *)workspace);
}

extern "C" isg_status isg_cluster_noalloc(void *stream, const void *x, isg_dtype dt, const int64_t x_strides[3],
                                          int B, int H, int N, int d, int C, int iters, int init_mode,
                                          const void *companion, float *centroids, int32_t *labels,
                                          int32_t *perm, int32_t *offsets, void *x_perm, void *companion_perm,
                                          float *max_sqnorm)
{
    const isg_status a = check_cluster_args(x, dt, x_strides, B, H, N, d, C, iters, init_mode, companion,
                                            centroids, labels, perm, offsets, x_perm, companion_perm);
    if (a != ISG_OK) return a;
    const size_t need = isg_cluster_workspace_size(B, H, N, d, C);
    ISG_REQUIRE(need <= kNoAllocScratchBytes, ISG_E_WORKSPACE,
                "isg_cluster_noalloc: this shape needs %zu bytes of scratch, more than the %zu-byte static array "
                "(split the heads over several calls, or use isg_cluster with a workspace)",
                need, kNoAllocScratchBytes);
    hipStream_t st = (hipStream_t)stream;
    uint8_t *ws = nullptr;
    const isg_status s = scratch_for_stream(st, &ws);
    if (s != ISG_OK) return s;
    return run_checked(st, x, dt, x_strides, B, H, N, d, C, iters, init_mode, companion, centroids, labels, perm,
                       offsets, x_perm, companion_perm, max_sqnorm, ws);
}

// ---------------------------------------------------------------- product-quantisation codebooks
namespace {

// The integer-sum update serves bf16 16-dim subspaces with at most kPqIntMaxC
// codewords (its LDS sums grow with Cc); anything else runs isg_cluster's rounds.
bool pq_int_path(isg_dtype dt, int d, int P, int Cc)
{
    return dt == ISG_BF16 && d / P == 16 && P <= kPqMaxP && Cc <= kPqIntMaxC;
}

struct PqWs {
    size_t off_copy, off_perm, off_offsets, off_emax, off_wmax, off_acc, chunk_bytes, off_cluster, total;
};

PqWs pq_ws(isg_dtype dt, int B, int H, int N, int d, int P, int Cc)
{
    const int ds = d / P;
    const size_t esz = dt == ISG_F32 ? sizeof(float) : sizeof(uint16_t);
    const size_t rows = (size_t)P * B * H * N;
    const size_t pairs = (size_t)P * B * H;
    const bool ip = pq_int_path(dt, d, P, Cc);
    PqWs w;
    size_t o = 0;
    w.off_copy = o; o += isg_align256(rows * ds * esz);
    w.off_perm = o; o += ip ? 0 : isg_align256(rows * sizeof(int32_t));
    w.off_offsets = o; o += ip ? 0 : isg_align256(pairs * (Cc + 1) * sizeof(int32_t));
    w.off_emax = o; o += ip ? isg_align256(pairs * sizeof(int32_t)) : 0;
    // the split's exponent field per (triple, work-group of 64 tokens)
    w.off_wmax = o; o += ip ? isg_align256(pairs * (size_t)((N + 63) / 64) * sizeof(int32_t)) : 0;
    // per (triple, chunk of kPqAccTok tokens): Cc*16 int64 sums, then Cc int32 counts
    w.chunk_bytes = isg_align256((size_t)Cc * 16 * sizeof(int64_t) + (size_t)Cc * sizeof(int32_t));
    w.off_acc = o; o += ip ? pairs * (size_t)((N + kPqAccTok - 1) / kPqAccTok) * w.chunk_bytes : 0;
    w.off_cluster = o; o += cluster_ws(P * B, H, N, ds, Cc).total;
    w.total = o;
    return w;
}

}  // namespace

extern "C" size_t isg_pq_codebooks_workspace_size(isg_dtype dt, int B, int H, int N, int d, int P, int Cc)
{
    if (B < 1 || H < 1 || N < 1 || d < 1 || P < 1 || Cc < 1 || d % P != 0 || (dt != ISG_F32 && dt != ISG_BF16))
        return 0;
    return pq_ws(dt, B, H, N, d, P, Cc).total;
}

extern "C" isg_status isg_pq_codebooks(void *stream, const void *x, isg_dtype dt, const int64_t x_strides[3], int B,
                                       int H, int N, int d, int P, int Cc, int iters, int32_t *codes,
                                       float *codebooks, void *workspace, size_t ws_bytes)
{
    ISG_REQUIRE(x && x_strides && codes && codebooks, ISG_E_ARG, "isg_pq_codebooks: null pointer argument");
    ISG_REQUIRE(B >= 1 && H >= 1 && N >= 1, ISG_E_ARG, "isg_pq_codebooks: B, H, N must be >= 1 (got %d, %d, %d)", B,
                H, N);
    ISG_REQUIRE(dt == ISG_F32 || dt == ISG_BF16, ISG_E_DTYPE, "isg_pq_codebooks: dtype %d", (int)dt);
    ISG_REQUIRE(P >= 1 && d >= 1 && d % P == 0, ISG_E_ARG, "isg_pq_codebooks: need P >= 1 and P | d (got d=%d P=%d)",
                d, P);
    const int ds = d / P;
    ISG_REQUIRE(ds == 16 || ds == 64 || ds == 128, ISG_E_UNSUPPORTED,
                "isg_pq_codebooks: subspace dimension d/P = %d not built (16, 64, 128)", ds);
    ISG_REQUIRE((int64_t)P * B * H <= 65535, ISG_E_ARG, "isg_pq_codebooks: P*B*H must be <= 65535 (got %lld)",
                (long long)P * B * H);
    ISG_REQUIRE(Cc >= 1 && Cc <= N && Cc <= kMaxC, ISG_E_ARG,
                "isg_pq_codebooks: need 1 <= Cc <= min(N, %d), got Cc=%d N=%d", kMaxC, Cc, N);
    ISG_REQUIRE(iters >= 1, ISG_E_ARG, "isg_pq_codebooks: iters must be >= 1 (got %d)", iters);
    for (int k = 0; k < 3; ++k)
        ISG_REQUIRE(x_strides[k] >= 0 && x_strides[k] % 8 == 0, ISG_E_ARG,
                    "isg_pq_codebooks: x_strides must be non-negative multiples of 8 elements");
    ISG_REQUIRE(x_strides[2] >= d, ISG_E_ARG, "isg_pq_codebooks: token stride %lld < d", (long long)x_strides[2]);
    ISG_REQUIRE(((uintptr_t)x & 15) == 0, ISG_E_ARG, "isg_pq_codebooks: x must be 16-byte aligned");
    const PqWs w = pq_ws(dt, B, H, N, d, P, Cc);
    ISG_REQUIRE(workspace && ws_bytes >= w.total, ISG_E_WORKSPACE, "isg_pq_codebooks: workspace %zu < %zu bytes",
                workspace ? ws_bytes : (size_t)0, w.total);
    hipStream_t st = (hipStream_t)stream;
    uint8_t *ws = (uint8_t *)workspace;
    const Strides xs{x_strides[0], x_strides[1], x_strides[2]};
    const dim3 grid((N + 63) / 64, B * H);
    if (pq_int_path(dt, d, P, Cc)) {
        // subspace s of batch b is batch s*B + b of the rounds on the dense copy
        const int pairs = P * B * H;
        int32_t *emax = (int32_t *)(ws + w.off_emax), *wmax = (int32_t *)(ws + w.off_wmax);
        pq_split_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t *)x, xs, B, H, N, d, ds,
                                                        (uint16_t *)(ws + w.off_copy), wmax);
        pq_emax_kernel<<<pairs, 256, 0, st>>>(wmax, (int)grid.x, emax);
        return run_pq16(st, (const uint16_t *)(ws + w.off_copy), P * B, H, N, Cc, iters, emax, codebooks, codes,
                        ws + w.off_acc, w.chunk_bytes, ws + w.off_cluster);
    }
    if (dt == ISG_F32)
        pq_split_kernel<float><<<grid, 256, 0, st>>>((const float *)x, xs, B, H, N, d, ds, (float *)(ws + w.off_copy),
                                                     nullptr);
    else
        pq_split_kernel<uint16_t><<<grid, 256, 0, st>>>((const uint16_t *)x, xs, B, H, N, d, ds,
                                                        (uint16_t *)(ws + w.off_copy), nullptr);
    // subspace s of batch b is batch s*B + b of one clustering call on the dense copy
    const int64_t cs[3] = {(int64_t)H * N * ds, (int64_t)N * ds, ds};
    return run_checked(st, ws + w.off_copy, dt, cs, P * B, H, N, ds, Cc, iters, 0, nullptr, codebooks, codes,
                       (int32_t *)(ws + w.off_perm), (int32_t *)(ws + w.off_offsets), nullptr, nullptr, nullptr,
                       ws + w.off_cluster);
}
