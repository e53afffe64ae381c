// Shared device helpers for the MoE grouped-GEMM kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moegg {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxExperts = 1024;
constexpr int kXcds = 8;  // MI355X: 8 XCDs; workgroup b is dispatched to XCD b % 8

// Device error bits (mirrors MOEGG_DERR_* in moegg.h).
constexpr int kErrExpertId = 1;
constexpr int kErrMSizes = 2;
constexpr int kErrGather = 4;

__device__ __forceinline__ void raise_error(int32_t *err, int bits)
{
    if (err)
        atomicOr(err, bits);  // vector-memory atomic; sticky, never cleared here
}

// Two fp32 -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32), packed low/high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    f32x2_t f = {lo, hi};
    bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
    return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ uint16_t to_bf16(float f)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Workgroup id -> logical slot so that logical slots [x*G/8, (x+1)*G/8) all run
// on XCD x: consecutive tiles (which share operand panels) then share one L2.
__device__ __forceinline__ int xcd_logical_block(int bid, int grid)
{
    if (grid % kXcds != 0)
        return bid;
    return (bid % kXcds) * (grid / kXcds) + bid / kXcds;
}

// Exclusive scan of n <= 64 * 16 ints held in LDS, done by wave 0 alone.
// All threads of the block must call it (it contains barriers).  Writes the
// total to *total.
__device__ inline void wave0_exclusive_scan(int *vals, int n, int *total)
{
    __syncthreads();
    if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        const int per = (n + kWave - 1) / kWave;
        const int lo = lane * per;
        const int hi = min(n, lo + per);
        int sum = 0;
        for (int i = lo; i < hi; ++i)
            sum += vals[i];
        int incl = sum;
        for (int d = 1; d < kWave; d <<= 1) {
            int v = __shfl_up(incl, d, kWave);
            if (lane >= d)
                incl += v;
        }
        int run = incl - sum;
        for (int i = lo; i < hi; ++i) {
            int v = vals[i];
            vals[i] = run;
            run += v;
        }
        if (lane == kWave - 1)
            *total = incl;
    }
    __syncthreads();
}

// Largest e in [0, n) with starts[e] <= t (starts non-decreasing, starts[0] = 0).
__device__ __forceinline__ int upper_index(const int *starts, int n, int t)
{
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (starts[mid] <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// s_roff[0..E]: expert row starts clipped to [0, S] (s_roff[E] = end);
// s_tstart[0..E]: first tile of each expert for tiles_of(rows).  Flags
// negative m_sizes and sums past S.
template <class TilesOf>
__device__ __forceinline__ int build_expert_tables(const int32_t *m_sizes, int E, int64_t S,
                                                   int *s_roff, int *s_tstart, int *s_scratch,
                                                   int32_t *err, TilesOf tiles_of)
{
    bool bad = false;
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int m = m_sizes[e];
        bad |= m < 0;
        s_roff[e] = m < 0 ? 0 : m;
    }
    wave0_exclusive_scan(s_roff, E, &s_scratch[0]);
    const int total = s_scratch[0];
    if (threadIdx.x == 0) {
        bad |= total > S || total < 0;
        s_roff[E] = (int)min((int64_t)total, S);
    }
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        s_roff[e] = (int)min((int64_t)s_roff[e], S);
    if (bad)
        raise_error(err, kErrMSizes);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        s_tstart[e] = tiles_of(s_roff[e + 1] - s_roff[e]);
    wave0_exclusive_scan(s_tstart, E, &s_scratch[1]);
    if (threadIdx.x == 0)
        s_tstart[E] = s_scratch[1];
    __syncthreads();
    return s_tstart[E];
}

}  // namespace moegg
