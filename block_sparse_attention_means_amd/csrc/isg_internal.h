// Internal helpers shared by the libisg translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "isg.h"

// ---------------------------------------------------------------- host side
isg_status isg_fail(isg_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
isg_status isg_check_launch(const char *what);

#define ISG_REQUIRE(cond, status, ...)                     \
    do {                                                   \
        if (!(cond)) return isg_fail((status), __VA_ARGS__); \
    } while (0)

static inline size_t isg_align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------- device side
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Native vector types for 16/8-byte moves: HIP's uint4/uint2 are union-based
// structs whose copies can stay in private (scratch) memory.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 <-> fp32 (bit-level, round to nearest even; inputs are finite).
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b)
{
    return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float *p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float *p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ float load(const uint16_t *p, int64_t i) { return bf16_bits_to_f32(p[i]); }
    static __device__ __forceinline__ void store(uint16_t *p, int64_t i, float v) { p[i] = f32_to_bf16_bits(v); }
};

// Map a launch-order block id to a logical tile id so that consecutive logical
// tiles run on the same XCD (work-groups are dealt to the 8 XCDs round robin).
// nblocks must be a multiple of 8.
__device__ __forceinline__ int xcd_logical_block(int p, int nblocks)
{
    return (p & 7) * (nblocks >> 3) + (p >> 3);
}

// Inclusive prefix sum across the 64 lanes of a wave.
template <typename V>
__device__ __forceinline__ V wave_inclusive_scan(V x)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const V y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

// Exclusive block scan over `n` values held in shared memory `a` (in place).
// Thread t takes a contiguous run of ceil(n / blockDim.x) values; the runs' sums
// are scanned within each wave by shuffles and across waves through `tmp`
// (>= blockDim.x / 64 entries).  blockDim.x must be a multiple of 64.  Returns
// the total.  All threads call it.
template <typename V>
__device__ __forceinline__ V block_exclusive_scan(V *a, int n, V *tmp)
{
    const int T = blockDim.x, tid = threadIdx.x, wave = tid >> 6, nw = T >> 6;
    const int per = (n + T - 1) / T;
    const int lo = min(n, tid * per), hi = min(n, lo + per);
    V s = 0;
    for (int k = lo; k < hi; ++k) s += a[k];
    const V incl = wave_inclusive_scan(s);
    if ((tid & 63) == 63) tmp[wave] = incl;
    __syncthreads();
    V base = 0, total = 0;
    for (int w = 0; w < nw; ++w) {
        const V t = tmp[w];
        if (w < wave) base += t;
        total += t;
    }
    V run = base + incl - s;
    for (int k = lo; k < hi; ++k) {
        const V v = a[k];
        a[k] = run;
        run += v;
    }
    __syncthreads();
    return total;
}

__device__ __forceinline__ int block_exclusive_scan_int(int *a, int n, int *tmp)
{
    return block_exclusive_scan<int>(a, n, tmp);
}

__device__ __forceinline__ uint64_t block_exclusive_scan_u64(uint64_t *a, int n, uint64_t *tmp)
{
    return block_exclusive_scan<uint64_t>(a, n, tmp);
}
