// isg_unpermute: attention rows back to token order, o[perm_q[r]] = o_p[r].
// The attention runs over a permuted matrix (InstaGen, Paper Reading AI Learner
// page, abstract), so its output rows are in cluster order until this step.
#include "isg_internal.h"

namespace {

struct Strides {
    int64_t b, h, t;
};

// One 16-byte chunk per thread: reads are contiguous rows of o_p, writes land on
// whole (d-contiguous) rows of o.
template <typename T, int D>
__global__ __launch_bounds__(256) void unpermute_kernel(const T *o_p, const float *lse_p, const int32_t *perm,
                                                        int H, int N, T *o, Strides os, float *lse, int64_t total)
{
    constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
    constexpr int CPR = D / EPC;
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int ck = (int)(e % CPR);
        const int64_t row = e / CPR;  // bh*N + r
        const int64_t bh = row / N;
        const int b = (int)(bh / H), h = (int)(bh % H);
        const int t = perm[row];
        const uint4 v = *reinterpret_cast<const uint4 *>(o_p + row * D + ck * EPC);
        *reinterpret_cast<uint4 *>(o + b * os.b + h * os.h + (int64_t)t * os.t + ck * EPC) = v;
        if (lse && ck == 0) lse[bh * N + t] = lse_p[row];
    }
}

template <typename T>
isg_status launch(hipStream_t st, const void *o_p, const float *lse_p, const int32_t *perm, int B, int H, int N,
                  int d, void *o, Strides os, float *lse)
{
    const int64_t total = (int64_t)B * H * N * (d * (int64_t)sizeof(T) / 16);
    const int grid = (int)std::min<int64_t>((total + 255) / 256, 1 << 20);
    switch (d) {
    case 16:
        unpermute_kernel<T, 16><<<grid, 256, 0, st>>>((const T *)o_p, lse_p, perm, H, N, (T *)o, os, lse, total);
        break;
    case 64:
        unpermute_kernel<T, 64><<<grid, 256, 0, st>>>((const T *)o_p, lse_p, perm, H, N, (T *)o, os, lse, total);
        break;
    case 128:
        unpermute_kernel<T, 128><<<grid, 256, 0, st>>>((const T *)o_p, lse_p, perm, H, N, (T *)o, os, lse, total);
        break;
    default:
        return isg_fail(ISG_E_UNSUPPORTED, "isg_unpermute: d=%d not built (16, 64, 128)", d);
    }
    return isg_check_launch("isg_unpermute");
}

}  // namespace

extern "C" isg_status isg_unpermute(void *stream, const void *o_p, const float *lse_p, const int32_t *perm_q,
                                    isg_dtype dt, int B, int H, int N, int d, void *o, const int64_t o_strides[3],
                                    float *lse)
{
    ISG_REQUIRE(o_p && perm_q && o && o_strides, ISG_E_ARG, "isg_unpermute: null pointer argument");
    ISG_REQUIRE((lse_p == nullptr) == (lse == nullptr), ISG_E_ARG,
                "isg_unpermute: lse_p and lse must both be given or both be NULL");
    ISG_REQUIRE(B >= 1 && H >= 1 && N >= 1, ISG_E_ARG, "isg_unpermute: B, H, N must be >= 1");
    ISG_REQUIRE(dt == ISG_F32 || dt == ISG_BF16, ISG_E_DTYPE, "isg_unpermute: dtype %d", (int)dt);
    ISG_REQUIRE(d == 16 || d == 64 || d == 128, ISG_E_UNSUPPORTED, "isg_unpermute: d=%d not built", d);
    const int64_t align = dt == ISG_BF16 ? 8 : 4;
    for (int k = 0; k < 3; ++k)
        ISG_REQUIRE(o_strides[k] >= 0 && o_strides[k] % align == 0, ISG_E_ARG,
                    "isg_unpermute: o_strides must be non-negative multiples of %lld elements", (long long)align);
    ISG_REQUIRE(o_strides[2] >= d, ISG_E_ARG, "isg_unpermute: token stride < d");
    ISG_REQUIRE(((uintptr_t)o_p & 15) == 0 && ((uintptr_t)o & 15) == 0, ISG_E_ARG,
                "isg_unpermute: o_p and o must be 16-byte aligned");
    Strides os{o_strides[0], o_strides[1], o_strides[2]};
    hipStream_t st = (hipStream_t)stream;
    if (dt == ISG_F32) return launch<float>(st, o_p, lse_p, perm_q, B, H, N, d, o, os, lse);
    return launch<uint16_t>(st, o_p, lse_p, perm_q, B, H, N, d, o, os, lse);
}
