// isg_cluster: Lloyd k-means per head + stable counting sort + coalesced gather.
//
// Pages: InstaGen, thelatestinai.com page, Figure 3(a) (queries and keys are
// clustered into groups) and Figure 2 (Cq = 100, Ck = 500).  Reading: Euclidean
// k-means on the raw vectors, strided init, ties to the lowest index, empty
// clusters keep their centroid; the permutation is the stable sort by label.
//
// Per round: assign (labels) -> per-chunk histograms -> scan over chunks ->
// label offsets + stable scatter (perm, offsets) -> segmented fp64 mean in sorted order
// (centroids).  No float atomics: every output is deterministic.
#include <type_traits>

#include "isg_internal.h"

namespace {

constexpr int kSortChunk = 1024;  // tokens per histogram / scatter chunk
constexpr int kMaxC = 4096;
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
__device__ __forceinline__ void load8(const uint16_t *p, float out[8])
{
    uint4 a = *reinterpret_cast<const uint4 *>(p);
    uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        out[2 * k] = __uint_as_float(w[k] << 16);
        out[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
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
// sum of squared differences (relative error < (D + 2) 2^-24); whenever the two
// best candidates are within 4e-5 relative of each other (more than twice that
// bound) they are re-compared in fp64 with unfused operations in the order
// k = 0..D-1, ties to the lower index.
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
    int bi = 0, si = 0;
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
                second = best; si = bi; best = s; bi = j;
            } else if (s < second) {
                second = s; si = j;
            }
        }
    }
    if (!valid) return;
    if (C > 1 && second - best <= 4e-5f * second) {
        double d1 = 0.0, d2 = 0.0;
        const float *c1 = ch + (int64_t)bi * D, *c2 = ch + (int64_t)si * D;
        for (int k = 0; k < D; ++k) {
            double a1 = __dsub_rn((double)xv[k], (double)c1[k]);
            double a2 = __dsub_rn((double)xv[k], (double)c2[k]);
            d1 = __dadd_rn(d1, __dmul_rn(a1, a1));
            d2 = __dadd_rn(d2, __dmul_rn(a2, a2));
        }
        if (d2 < d1 || (d2 == d1 && si < bi)) bi = si;
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

// One wave per chunk.  It first turns the label counts into label offsets (the
// exclusive prefix over labels, lane l taking a contiguous run of labels) and
// adds the chunk's per-label base, so run[c] is the first sorted row of
// (chunk, c); the wave of chunk 0 also writes offsets and poff (the prefix of
// the number of prow-row pieces per group).  It then walks its tokens in order,
// 64 at a time; a token's rank among equal labels of the same step comes from
// ballots over the label bits.
__global__ __launch_bounds__(64) void scatter_kernel(const int32_t *labels, const int32_t *base,
                                                     const int32_t *tot, int N, int C, int nchunks, int bits,
                                                     int prow, int32_t *perm, int32_t *offsets, int32_t *poff)
{
    extern __shared__ int run[];  // C entries (dynamic, so small C lets more waves share a CU)
    const int chunk = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
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
    __syncthreads();
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
        for (int c = l0; c < l1; ++c) {
            const int n = run[c];
            run[c] = os;
            if (first) {
                ob[c] = os;
                pb[c] = op;
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
    __syncthreads();
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
    __syncthreads();
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int step = 0; step < kSortChunk / 64; ++step) {
        const int t = t0 + step * 64 + lane;
        const bool valid = t < N;
        const int lab = labs[step];
        uint64_t m = __ballot(valid);
        for (int bt = 0; bt < bits; ++bt) {
            const bool one = (lab >> bt) & 1;
            const uint64_t bal = __ballot(one);
            m &= one ? bal : ~bal;
        }
        const int rank = __popcll(m & below);
        const int cnt = __popcll(m);
        int pos = 0;
        if (valid) pos = run[lab] + rank;
        __syncthreads();
        if (valid) {
            perm[(int64_t)bh * N + pos] = t;
            if (rank == cnt - 1) run[lab] = pos + 1;
        }
        __syncthreads();
    }
}

// Centroid update in two passes, both in a fixed order: every group is cut into
// pieces of piece_rows(D) sorted rows; a work-group sums one piece in fp64 (rows
// strided over RP slots, then slot order) and the final pass adds the pieces of
// each group in order and divides: c_j = mean of the rows of group j, rounded
// to fp32 (an empty group keeps its centroid).
template <typename T, int D>
__global__ __launch_bounds__(256) void update_piece_kernel(const T *x, Strides xs, int H, int N, int C,
                                                           const int32_t *perm, const int32_t *offsets,
                                                           const int32_t *poff, int maxp, double *partial,
                                                           T *x_perm, float *pmax)
{
    constexpr int TPR = D / 8;     // threads per row
    constexpr int RP = 256 / TPR;  // row slots
    constexpr int PR = piece_rows(D);
    constexpr int RPT = PR / RP;   // rows per slot: all indices, then all rows, in flight at once
    __shared__ double red[RP][D];
    __shared__ int grp;
    const int q = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
    const int32_t *pb = poff + (int64_t)bh * (C + 1);
    if (q >= pb[C]) return;
    // group of piece q: the one j with poff[j] <= q < poff[j + 1] (one parallel pass)
    for (int jj = threadIdx.x; jj < C; jj += 256)
        if (pb[jj] <= q && q < pb[jj + 1]) grp = jj;
    __syncthreads();
    const int j = grp;
    const int32_t *ob = offsets + (int64_t)bh * (C + 1);
    const int r0 = ob[j] + (q - pb[j]) * PR, r1 = min(ob[j + 1], r0 + PR);
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
    const int32_t *ob = offsets + (int64_t)bh * (C + 1);
    const int n = ob[j + 1] - ob[j];
    if (n == 0) return;  // empty: keep the centroid
    for (int k = threadIdx.x; k < D; k += 128) {
        double sum = 0.0;
        for (int q = pb[j]; q < pb[j + 1]; ++q) sum += partial[((int64_t)bh * maxp + q) * D + k];
        cent[((int64_t)bh * C + j) * D + k] = (float)(sum / (double)n);
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
// |x|^2 + 1 are each split exactly into three bf16 parts (24 significant bits),
// paired with ones, so the accumulator holds |x - c|^2 + 1 itself.  Per
// token the four best candidates are kept; whenever a rival lies within
// tau = 1e-4 (|x|^2 + max_j |c_j|^2) -- several times the worst-case error of the
// split and of fp32 accumulation -- the decision is re-taken in fp64 with the
// same unfused arithmetic as the exact definition (the close candidates, or
// every centroid when all kept candidates are close), ties to the lower index.
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
    const int bh = blockIdx.y, lane = threadIdx.x & 63;
    const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (j >= Cpad) return;
    uint16_t *hi = planes + ((int64_t)bh * 2 * Cpad + j) * D;
    uint16_t *lo = planes + ((int64_t)bh * 2 * Cpad + Cpad + j) * D;
    double nn = 0.0;
    for (int k = lane; k < D; k += 64) {
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
    for (int off = 32; off > 0; off >>= 1) nn += __shfl_xor(nn, off);
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
// along.  The K = 4 smallest keys are kept sorted: one min and K-1 med3 per
// candidate.  (Two would halve the epilogue, but at d = 16 with 256 codewords
// close pairs are common and each would cost a full rescan.)
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
constexpr int topk_of() { return 4; }

// fp64 partial sum of (x_k - c_k)^2 over the DPL dims of one lane (x bf16, c fp32;
// both 8/16-byte aligned at these offsets).
template <int DPL>
__device__ __forceinline__ double seg_sqdist(const uint16_t *xr, const float *cr)
{
    float xv[DPL], cv[DPL];
    if constexpr (DPL == 8) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(xr);
        const f32x4 c0 = *reinterpret_cast<const f32x4 *>(cr);
        const f32x4 c1 = *reinterpret_cast<const f32x4 *>(cr + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            xv[2 * q] = __uint_as_float(w[q] << 16);
            xv[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
            cv[q] = c0[q];
            cv[4 + q] = c1[q];
        }
    } else if constexpr (DPL == 4) {
        const u32x2 w = *reinterpret_cast<const u32x2 *>(xr);
        const f32x4 c0 = *reinterpret_cast<const f32x4 *>(cr);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            xv[2 * q] = __uint_as_float(w[q] << 16);
            xv[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) cv[q] = c0[q];
    } else {
#pragma unroll
        for (int q = 0; q < DPL; ++q) { xv[q] = bf16_bits_to_f32(xr[q]); cv[q] = cr[q]; }
    }
    double part = 0.0;
#pragma unroll
    for (int q = 0; q < DPL; ++q) {
        const double a = (double)xv[q] - (double)cv[q];
        part = fma(a, a, part);
    }
    return part;
}

__device__ __forceinline__ double sum16(double v)
{
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 4);
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
// (token, centroid) key goes into the token's top four.  The key's index bits
// hold the centroid's row in the tile without the half-wave's offset of 4 rows;
// the caller adds it once per token.
template <int D>
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
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const uint32_t j = (uint32_t)(tile * kCT + (r >> 2) * 8 + (r & 3));  // wave-uniform
        // rows j and j + 4 both padding (norm 1e30, never kept): skip (a scalar branch)
        if (j >= (uint32_t)C) continue;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) top_insert(top[tb], (__float_as_uint(acc[tb][r]) & hi_mask) | j);
    }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void assign_mfma_kernel(
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
    // keys hold |x|^2 + 1 + |c|^2 - 2<x,c> >= 1 (so they are positive normal floats)
    int ibits = 1;
    while ((1 << ibits) < Cpad) ++ibits;
    const uint32_t imask = (1u << ibits) - 1u, hi_mask = ~imask;
    // B operand of the norm step: [1, 1, 1, (|x|^2 + 1) in three parts] in k = 0..7
    // (lanes of the first half-wave), zero in k = 8..15
    bf16x8 xaug[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const float xn1 = xn[tb] + 1.0f;
        const uint16_t h = f32_to_bf16_bits(xn1);
        const float r1 = xn1 - bf16_bits_to_f32(h);
        const uint16_t m = f32_to_bf16_bits(r1);
        const uint16_t l = f32_to_bf16_bits(r1 - bf16_bits_to_f32(m));
        const uint16_t parts[8] = {0x3F80, 0x3F80, 0x3F80, h, m, l, 0, 0};
#pragma unroll
        for (int e = 0; e < 8; ++e) xaug[tb][e] = __builtin_bit_cast(__bf16, (uint16_t)(hl ? 0 : parts[e]));
    }
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
    for (int tile = 0; tile < ntiles; tile += 2) {
        // tile in tb0 while tile+1 loads into tb1, then the reverse
        if (tile + 1 < ntiles) planes_direct<D>(tb1, pb, ab, Cpad, tile + 1, wave, lane);
        assign_tile<D>(tb0, tile, C, xf, xaug, hi_mask, top, hl, l32);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tile + 1 >= ntiles) break;
        if (tile + 2 < ntiles) planes_direct<D>(tb0, pb, ab, Cpad, tile + 2, wave, lane);
        assign_tile<D>(tb1, tile + 1, C, xf, xaug, hi_mask, top, hl, l32);
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

    // Decisions.  Close calls go to a work list: 16 lanes per (token, candidate)
    // entry evaluate |x - c|^2 in fp64 and the token takes the smallest (ties to
    // the lower index).  A token with four candidates within tau is rescanned in
    // fp64 over all C, again 16 lanes per candidate.
    constexpr int kRQ = 3 * 256;
    constexpr int DPL = D / 16;  // dims per lane
    __shared__ int rq_n, full_n;
    __shared__ int rq_slot[kRQ];
    __shared__ int rq_cand[kRQ];
    __shared__ double rq_dist[kRQ];
    __shared__ int full_slot[256];
    __shared__ int full_best[256];
    __shared__ double grp_d[16];
    __shared__ int grp_j[16];
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
        int n = 1;
#pragma unroll
        for (int c = 1; c < TK; ++c) n += __uint_as_float(T.k[c] & hi_mask) < lim;
        if (n == TK) {  // every kept candidate is close: all centroids in fp64
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
    const int sub = tid & 15, grp = tid >> 4;
    {
        const int nq = rq_n;
        for (int e = grp; e < nq; e += 16) {
            const int t = blockIdx.x * 256 + rq_slot[e];
            const double dd = sum16(seg_sqdist<DPL>(xb + (int64_t)t * xs.t + sub * DPL,
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
        for (int j = grp; j < C; j += 16) {
            const double dd = sum16(seg_sqdist<DPL>(xr, cb + (int64_t)j * D + sub * DPL));
            if (dd < bd) { bd = dd; bj = j; }
        }
        if (sub == 0) { grp_d[grp] = bd; grp_j[grp] = bj; }
        __syncthreads();
        if (tid == 0) {
            double b = grp_d[0];
            int jb = grp_j[0];
            for (int g = 1; g < 16; ++g)
                if (grp_d[g] < b || (grp_d[g] == b && grp_j[g] < jb)) { b = grp_d[g]; jb = grp_j[g]; }
            full_best[f] = jb;
        }
        __syncthreads();
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
    size_t off_hist, off_tot, off_planes, off_norms, off_aug, off_poff, off_partial, off_pmax, total;
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
        centroid_planes_kernel<D><<<dim3(w.Cpad / 4, BH), 256, 0, st>>>(cent, C, w.Cpad, planes, norms, aug);
        assign_mfma_kernel<D><<<dim3((N + 255) / 256, BH), 256, 0, st>>>(x, xs, H, N, C, w.Cpad, planes, norms,
                                                                         aug, cent, labels);
    } else {
        assign_kernel<T, D><<<dim3((N + 255) / 256, BH), 256, 0, st>>>(x, xs, H, N, C, cent, labels);
    }
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
    double *partial = (double *)(ws + w.off_partial);
    float *pmax = (float *)(ws + w.off_pmax);
    int bits = 1;
    while ((1 << bits) < C) ++bits;
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
        scatter_kernel<<<dim3(nchunks, BH), 64, C * sizeof(int32_t), st>>>(labels, hist, tot, N, C, nchunks, bits,
                                                                           piece_rows(D), perm, offsets, poff);
        // the last iteration's update also writes the permuted copy of x
        update_piece_kernel<T, D><<<dim3(w.maxp, BH), 256, 0, st>>>(x, xs, H, N, C, perm, offsets, poff, w.maxp,
                                                                    partial, it + 1 == iters ? x_perm : nullptr,
                                                                    last_norms ? pmax : nullptr);
        update_final_kernel<D><<<dim3(C, BH), 128, 0, st>>>(C, offsets, poff, w.maxp, partial, cent,
                                                            last_norms ? pmax : nullptr, max_sqnorm);
    }
    if (comp_perm) {
        const int64_t total = (int64_t)BH * N * (D / 8);
        const int grid = (int)std::min<int64_t>((total + 255) / 256, 1 << 20);
        gather_kernel<T, D><<<grid, 256, 0, st>>>(x, xs, comp, H, N, perm, nullptr, comp_perm, total);
    }
    return isg_check_launch("isg_cluster");
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
    const size_t need = isg_cluster_workspace_size(B, H, N, d, C);
    ISG_REQUIRE(workspace && ws_bytes >= need, ISG_E_WORKSPACE, "isg_cluster: workspace %zu < %zu bytes",
                workspace ? ws_bytes : (size_t)0, need);
    hipStream_t st = (hipStream_t)stream;
    Strides xs{x_strides[0], x_strides[1], x_strides[2]};
    uint8_t *ws = (uint8_t *)workspace;
    if (dt == ISG_F32)
        return dispatch_d<float>(d, st, (const float *)x, xs, B, H, N, C, iters, init_mode,
                                 (const float *)companion, centroids, labels, perm, offsets, (float *)x_perm,
                                 (float *)companion_perm, max_sqnorm, ws);
    return dispatch_d<uint16_t>(d, st, (const uint16_t *)x, xs, B, H, N, C, iters, init_mode,
                                (const uint16_t *)companion, centroids, labels, perm, offsets,
                                (uint16_t *)x_perm, (uint16_t *)companion_perm, max_sqnorm, ws);
}
