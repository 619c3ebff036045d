// isg_cluster: Lloyd k-means per head + stable counting sort + coalesced gather.
//
// Pages: InstaGen, thelatestinai.com page, Figure 3(a) (queries and keys are
// clustered into groups) and Figure 2 (Cq = 100, Ck = 500).  Reading: Euclidean
// k-means on the raw vectors, strided init, ties to the lowest index, empty
// clusters keep their centroid; the permutation is the stable sort by label.
//
// Per round: assign (labels) -> per-chunk histograms -> per-head scan ->
// stable scatter (perm, offsets) -> segmented fp64 mean in sorted order
// (centroids).  No float atomics: every output is deterministic.
#include "isg_internal.h"

namespace {

constexpr int kSortChunk = 1024;  // tokens per histogram / scatter chunk
constexpr int kMaxC = 4096;
constexpr int kAssignTile = 32;   // centroids per LDS tile in the assign kernel

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
    __syncthreads();
    const int t0 = chunk * kSortChunk, t1 = min(N, t0 + kSortChunk);
    for (int t = t0 + threadIdx.x; t < t1; t += 256) atomicAdd(&hs[labels[(int64_t)bh * N + t]], 1);
    __syncthreads();
    int32_t *out = hist + ((int64_t)bh * nchunks + chunk) * C;
    for (int c = threadIdx.x; c < C; c += 256) out[c] = hs[c];
}

// hist[bh][chunk][c] -> first sorted row of (chunk, c); offsets = prefix of counts.
__global__ __launch_bounds__(256) void scan_kernel(int32_t *hist, int nchunks, int C, int32_t *offsets)
{
    __shared__ int cnt[kMaxC];
    __shared__ int tmp[256];
    const int bh = blockIdx.x;
    int32_t *hb = hist + (int64_t)bh * nchunks * C;
    for (int c = threadIdx.x; c < C; c += 256) {
        int run = 0;
        for (int ch = 0; ch < nchunks; ++ch) {
            int v = hb[(int64_t)ch * C + c];
            hb[(int64_t)ch * C + c] = run;
            run += v;
        }
        cnt[c] = run;
    }
    __syncthreads();
    const int total = block_exclusive_scan_int(cnt, C, tmp);
    int32_t *ob = offsets + (int64_t)bh * (C + 1);
    for (int c = threadIdx.x; c < C; c += 256) {
        ob[c] = cnt[c];
        for (int ch = 0; ch < nchunks; ++ch) hb[(int64_t)ch * C + c] += cnt[c];
    }
    if (threadIdx.x == 0) ob[C] = total;
}

// One wave per chunk walks its tokens in order, 64 at a time; a token's rank
// among equal labels of the same step comes from ballots over the label bits.
__global__ __launch_bounds__(64) void scatter_kernel(const int32_t *labels, const int32_t *base, int N,
                                                     int C, int nchunks, int bits, int32_t *perm)
{
    __shared__ int run[kMaxC];
    const int chunk = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
    const int32_t *bb = base + ((int64_t)bh * nchunks + chunk) * C;
    for (int c = lane; c < C; c += 64) run[c] = bb[c];
    __syncthreads();
    const int t0 = chunk * kSortChunk;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int step = 0; step < kSortChunk / 64; ++step) {
        const int t = t0 + step * 64 + lane;
        const bool valid = t < N;
        const int lab = valid ? labels[(int64_t)bh * N + t] : 0;
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

// c_j = mean of the rows of group j in sorted order, fp64 partial sums in a fixed
// order (rows strided over RP slots, then slot order), rounded to fp32.
template <typename T, int D>
__global__ __launch_bounds__(256) void update_kernel(const T *x, Strides xs, int H, int N, int C,
                                                     const int32_t *perm, const int32_t *offsets,
                                                     float *cent)
{
    constexpr int TPR = D / 8;     // threads per row
    constexpr int RP = 256 / TPR;  // rows in flight
    __shared__ double red[RP][D];
    const int j = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
    const int r0 = offsets[(int64_t)bh * (C + 1) + j], r1 = offsets[(int64_t)bh * (C + 1) + j + 1];
    if (r1 == r0) return;  // empty: keep the centroid
    const int rs = threadIdx.x / TPR, ck = threadIdx.x % TPR;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const T *xb = x + b * xs.b + h * xs.h + ck * 8;
    const int32_t *pb = perm + (int64_t)bh * N;
    for (int r = r0 + rs; r < r1; r += RP) {
        float v[8];
        load8(xb + (int64_t)pb[r] * xs.t, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += (double)v[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rs][ck * 8 + e] = acc[e];
    __syncthreads();
    const double n = (double)(r1 - r0);
    for (int k = threadIdx.x; k < D; k += 256) {
        double s = 0.0;
        for (int rr = 0; rr < RP; ++rr) s += red[rr][k];
        cent[((int64_t)bh * C + j) * D + k] = (float)(s / n);
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

template <typename T, int D>
isg_status run_cluster(hipStream_t st, const T *x, Strides xs, int B, int H, int N, int C, int iters,
                       int init_mode, const T *comp, float *cent, int32_t *labels, int32_t *perm,
                       int32_t *offsets, T *x_perm, T *comp_perm, int32_t *hist)
{
    const int BH = B * H;
    const int nchunks = (N + kSortChunk - 1) / kSortChunk;
    int bits = 1;
    while ((1 << bits) < C) ++bits;
    if (init_mode == 0) {
        const int64_t total = (int64_t)BH * C * D;
        const int grid = (int)std::min<int64_t>((total + 255) / 256, 65536);
        init_centroids_kernel<T><<<grid, 256, 0, st>>>(x, xs, H, N, C, D, cent, total);
    }
    for (int it = 0; it < iters; ++it) {
        assign_kernel<T, D><<<dim3((N + 255) / 256, BH), 256, 0, st>>>(x, xs, H, N, C, cent, labels);
        hist_kernel<<<dim3(nchunks, BH), 256, 0, st>>>(labels, N, C, nchunks, hist);
        scan_kernel<<<BH, 256, 0, st>>>(hist, nchunks, C, offsets);
        scatter_kernel<<<dim3(nchunks, BH), 64, 0, st>>>(labels, hist, N, C, nchunks, bits, perm);
        update_kernel<T, D><<<dim3(C, BH), 256, 0, st>>>(x, xs, H, N, C, perm, offsets, cent);
    }
    if (x_perm || comp_perm) {
        const int64_t total = (int64_t)BH * N * (D / 8);
        const int grid = (int)std::min<int64_t>((total + 255) / 256, 1 << 20);
        gather_kernel<T, D><<<grid, 256, 0, st>>>(x, xs, comp, H, N, perm, x_perm, comp_perm, total);
    }
    return isg_check_launch("isg_cluster");
}

template <typename T>
isg_status dispatch_d(int d, hipStream_t st, const T *x, Strides xs, int B, int H, int N, int C,
                      int iters, int init_mode, const T *comp, float *cent, int32_t *labels,
                      int32_t *perm, int32_t *offsets, T *x_perm, T *comp_perm, int32_t *hist)
{
    switch (d) {
    case 16:
        return run_cluster<T, 16>(st, x, xs, B, H, N, C, iters, init_mode, comp, cent, labels, perm,
                                  offsets, x_perm, comp_perm, hist);
    case 64:
        return run_cluster<T, 64>(st, x, xs, B, H, N, C, iters, init_mode, comp, cent, labels, perm,
                                  offsets, x_perm, comp_perm, hist);
    case 128:
        return run_cluster<T, 128>(st, x, xs, B, H, N, C, iters, init_mode, comp, cent, labels, perm,
                                   offsets, x_perm, comp_perm, hist);
    default:
        return isg_fail(ISG_E_UNSUPPORTED, "isg_cluster: d=%d not built (16, 64, 128)", d);
    }
}

}  // namespace

extern "C" size_t isg_cluster_workspace_size(int B, int H, int N, int d, int C)
{
    (void)d;
    if (B < 1 || H < 1 || N < 1 || C < 1) return 0;
    const size_t nchunks = ((size_t)N + kSortChunk - 1) / kSortChunk;
    return isg_align256((size_t)B * H * nchunks * C * sizeof(int32_t));
}

extern "C" isg_status isg_cluster(void *stream, const void *x, isg_dtype dt, const int64_t x_strides[3],
                                  int B, int H, int N, int d, int C, int iters, int init_mode,
                                  const void *companion, float *centroids, int32_t *labels, int32_t *perm,
                                  int32_t *offsets, void *x_perm, void *companion_perm, void *workspace,
                                  size_t ws_bytes)
{
    ISG_REQUIRE(x && x_strides && centroids && labels && perm && offsets, ISG_E_ARG,
                "isg_cluster: null pointer argument");
    ISG_REQUIRE(B >= 1 && H >= 1 && N >= 1, ISG_E_ARG, "isg_cluster: B, H, N must be >= 1 (got %d, %d, %d)",
                B, H, N);
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
    int32_t *hist = (int32_t *)workspace;
    if (dt == ISG_F32)
        return dispatch_d<float>(d, st, (const float *)x, xs, B, H, N, C, iters, init_mode,
                                 (const float *)companion, centroids, labels, perm, offsets, (float *)x_perm,
                                 (float *)companion_perm, hist);
    return dispatch_d<uint16_t>(d, st, (const uint16_t *)x, xs, B, H, N, C, iters, init_mode,
                                (const uint16_t *)companion, centroids, labels, perm, offsets,
                                (uint16_t *)x_perm, (uint16_t *)companion_perm, hist);
}
