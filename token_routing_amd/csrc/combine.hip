// Top-k combine (unpermute with routing weights) and its backward, gfx950.
//
// The combine is the unpermute of the pages (wall_x fusions backend:
// expert outputs back to token order, the top-k copies of a token weighted by
// their routing probabilities and summed; the n_expts_act reduction at the
// end of triton_kernels matmul_ogs):
//   out[t, :] = sum_j w[t*k + j] * Y[row(t*k + j), :]     (fp32, j ascending)
// row(s) = scatter[s] when Y is in expert-sorted order, else s.  Its
// backward (unpermute_bwd):
//   dY[row(s), :] = w[s] * dOut[t, :],   dw[s] = <dOut[t, :], Y[row(s), :]>.
//
// Both are streaming kernels bound by HBM: no LDS and no MFMA.  A wave moves
// 16 bytes per lane (8 bf16), so one wave covers a 512-column chunk of a row;
// row indices and weights are uniform per wave and come in as scalar loads.
// Outputs are stored with the nontemporal (streaming) hint, so that the
// written lines do not take cache space from the rows still to be read:
// the combine on 8192 tokens x top-8 x 2048 columns went from 0.085 to
// 0.062 ms (3.5 -> 4.8 TB/s), its backward from 0.107 to 0.106 ms.
#include "common.h"

#include "gemm_params.h"

namespace moegg {

constexpr int kChunk = kWave * 8;  // columns per wave and row pass

typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef unsigned u32x4v_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x8_t widen8(const u32x4v_t &v)
{
    f32x8_t f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __builtin_bit_cast(float, v[i] << 16);
        f[2 * i + 1] = __builtin_bit_cast(float, v[i] & 0xffff0000u);
    }
    return f;
}

__device__ __forceinline__ u32x4v_t narrow8(const f32x8_t &f)
{
    u32x4v_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return v;
}

// Row of Y for slot s (-1: dropped or invalid; invalid entries are reported).
__device__ __forceinline__ int64_t combine_row(const CombineParams &a, int64_t s)
{
    if (!a.scatter)
        return s;
    const int r = a.scatter[s];
    if (r >= a.y_rows) {
        raise_error(a.err, kErrGather);
        return -1;
    }
    return r;
}

// One wave per token: it walks the token's k rows chunk by chunk (512
// columns per chunk, 16 bytes per lane), loading all k rows of CPI chunks
// before summing.  Each of the token's rows is thus read front to back by one
// wave, in 1 KiB pieces close together in time, which HBM serves better than
// the same pieces spread over several waves.
constexpr int kCombineCpi = 4;

__global__ __launch_bounds__(256) void combine_fwd_kernel(CombineParams a)
{
    const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) +
                      __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (t >= a.T)
        return;
    const int lane = threadIdx.x & (kWave - 1);
    for (int c0 = 0; c0 < a.N; c0 += kChunk * kCombineCpi) {
        f32x8_t acc[kCombineCpi];
#pragma unroll
        for (int c = 0; c < kCombineCpi; ++c)
            acc[c] = f32x8_t{};
        for (int j0 = 0; j0 < a.topk; j0 += 8) {
            u32x4v_t v[8][kCombineCpi];
            float w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t s = t * a.topk + j0 + j;
                const int64_t row = (j0 + j < a.topk) ? combine_row(a, s) : -1;
                w[j] = row < 0 ? 0.0f : (a.weights ? a.weights[s] : 1.0f);
#pragma unroll
                for (int c = 0; c < kCombineCpi; ++c) {
                    const int col = c0 + c * kChunk + lane * 8;
                    v[j][c] = (row >= 0 && col < a.N)
                                  ? *reinterpret_cast<const u32x4v_t *>(a.Y + (row * a.N + col) * 2)
                                  : u32x4v_t{0, 0, 0, 0};
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int c = 0; c < kCombineCpi; ++c)
                    acc[c] += w[j] * widen8(v[j][c]);
        }
#pragma unroll
        for (int c = 0; c < kCombineCpi; ++c) {
            const int col = c0 + c * kChunk + lane * 8;
            if (col >= a.N)
                continue;
            if (a.f32_out)
                __builtin_nontemporal_store(
                    acc[c], reinterpret_cast<f32x8_t *>(reinterpret_cast<float *>(a.out) + t * a.N + col));
            else
                __builtin_nontemporal_store(narrow8(acc[c]),
                                            reinterpret_cast<u32x4v_t *>(a.out + (t * a.N + col) * 2));
        }
    }
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1)
        v += __shfl_xor(v, d, kWave);
    return v;
}

// One wave per slot s = t*k + j: dY[row(s)] = w[s] * dOut[t] and, when dw is
// requested, dw[s] = <dOut[t], Y[row(s)]> (per-lane fp32 partial sums over
// the row's chunks, then a wave sum).  The k slots of a token are adjacent
// waves, so dOut[t] is read from HBM once and then from L2.
__global__ __launch_bounds__(256) void combine_bwd_kernel(CombineBwdParams a)
{
    const int64_t s = (int64_t)blockIdx.x * (blockDim.x / kWave) +
                      __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (s >= a.T * a.topk)
        return;
    const int64_t t = s / a.topk;
    int64_t row = s;
    if (a.scatter) {
        row = a.scatter[s];
        if (row >= a.y_rows) {
            raise_error(a.err, kErrGather);
            row = -1;
        }
    }
    const float w = a.weights ? a.weights[s] : 1.0f;
    const int lane = threadIdx.x & (kWave - 1);
    float dot = 0.0f;
    if (row >= 0) {
#pragma unroll 4
        for (int c0 = 0; c0 < a.N; c0 += kChunk) {
            const int col = c0 + lane * 8;
            if (col >= a.N)
                continue;
            const f32x8_t g =
                widen8(*reinterpret_cast<const u32x4v_t *>(a.dOut + (t * a.N + col) * 2));
            if (a.dw) {
                const f32x8_t y =
                    widen8(*reinterpret_cast<const u32x4v_t *>(a.Y + (row * a.N + col) * 2));
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    dot += g[i] * y[i];
            }
            __builtin_nontemporal_store(narrow8(w * g),
                                        reinterpret_cast<u32x4v_t *>(a.dY + (row * a.N + col) * 2));
        }
    }
    if (a.dw) {
        dot = wave_sum(dot);
        if (lane == 0)
            a.dw[s] = dot;
    }
}

// Any N and 2-byte-aligned rows (rows that are not whole 16-byte chunks):
// the same sums, one column per lane and step, loaded and stored as 2-byte
// elements.  Not tuned: the tiled kernels above take every N that is a
// multiple of 8 with 16-byte aligned operands.
__device__ __forceinline__ float bf16_at(const char *base, int64_t elem)
{
    const uint32_t h = *reinterpret_cast<const uint16_t *>(base + elem * 2);
    return __builtin_bit_cast(float, h << 16);
}

__global__ __launch_bounds__(256) void combine_fwd_any_kernel(CombineParams a)
{
    const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) +
                      __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (t >= a.T)
        return;
    const int lane = threadIdx.x & (kWave - 1);
    for (int c0 = 0; c0 < a.N; c0 += kWave) {
        const int col = c0 + lane;
        float acc = 0.0f;
        for (int j = 0; j < a.topk; ++j) {
            const int64_t s = t * a.topk + j;
            const int64_t row = combine_row(a, s);
            if (row >= 0 && col < a.N)
                acc += (a.weights ? a.weights[s] : 1.0f) * bf16_at(a.Y, row * a.N + col);
        }
        if (col >= a.N)
            continue;
        if (a.f32_out)
            reinterpret_cast<float *>(a.out)[t * a.N + col] = acc;
        else
            *reinterpret_cast<uint16_t *>(a.out + (t * a.N + col) * 2) = to_bf16(acc);
    }
}

__global__ __launch_bounds__(256) void combine_bwd_any_kernel(CombineBwdParams a)
{
    const int64_t s = (int64_t)blockIdx.x * (blockDim.x / kWave) +
                      __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (s >= a.T * a.topk)
        return;
    const int64_t t = s / a.topk;
    int64_t row = s;
    if (a.scatter) {
        row = a.scatter[s];
        if (row >= a.y_rows) {
            raise_error(a.err, kErrGather);
            row = -1;
        }
    }
    const float w = a.weights ? a.weights[s] : 1.0f;
    const int lane = threadIdx.x & (kWave - 1);
    float dot = 0.0f;
    if (row >= 0) {
        for (int col = lane; col < a.N; col += kWave) {
            const float g = bf16_at(a.dOut, t * a.N + col);
            if (a.dw)
                dot += g * bf16_at(a.Y, row * a.N + col);
            *reinterpret_cast<uint16_t *>(a.dY + (row * a.N + col) * 2) = to_bf16(w * g);
        }
    }
    if (a.dw) {
        dot = wave_sum(dot);
        if (lane == 0)
            a.dw[s] = dot;
    }
}

hipError_t combine_any_launch(const CombineParams &p, hipStream_t stream)
{
    if (p.T == 0)
        return hipSuccess;
    hipLaunchKernelGGL(combine_fwd_any_kernel, dim3((unsigned)((p.T + 3) / 4)), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

hipError_t combine_bwd_any_launch(const CombineBwdParams &p, hipStream_t stream)
{
    const int64_t items = p.T * p.topk;
    if (items == 0)
        return hipSuccess;
    hipLaunchKernelGGL(combine_bwd_any_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

hipError_t combine_launch(const CombineParams &p, hipStream_t stream)
{
    if (p.T == 0)
        return hipSuccess;
    hipLaunchKernelGGL(combine_fwd_kernel, dim3((unsigned)((p.T + 3) / 4)), dim3(256), 0, stream,
                       p);
    return hipGetLastError();
}

hipError_t combine_bwd_launch(const CombineBwdParams &p, hipStream_t stream)
{
    const int64_t items = p.T * p.topk;
    if (items == 0)
        return hipSuccess;
    hipLaunchKernelGGL(combine_bwd_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, stream,
                       p);
    return hipGetLastError();
}

}  // namespace moegg
