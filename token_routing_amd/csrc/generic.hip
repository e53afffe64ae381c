// Grouped GEMMs of any shape, gfx950: the path taken when a row cannot be
// moved as whole 16-byte chunks, i.e. K or N (or a group's n, k or leading
// dimension) is not a multiple of 8, or an operand is not 16-byte aligned.
// The pages put no such condition on their sizes.
//
// The definitions are those of the tiled kernels: the forward of
// grouped_gemm_forward (unsloth grouped_gemm/interface.py) with permute_x,
// permute_y, fuse_mul_post and the gated activation (FusedActivation with
// reduction_n = 2 in triton_kernels/matmul_ogs.py), grouped_gemm_dX and
// grouped_gemm_dW, and the explicit groups of asym_dual_gmm_separated
// (wall_x/fusions/backend.py).
//
// Design: a wave owns one 32 x 32 output block at a time and, once the
// workgroup has built the expert table, works alone (no more barriers).  The
// reduction runs 16 deep per v_mfma_f32_32x32x16_bf16.  Lane l loads the 8
// reduction elements of its fragment row or column with 2-byte buffer loads:
// an offset past the operand reads zero, which masks rows past an expert,
// bad gather entries and the reduction tail.  Lane l holds outputs of rows
// 8 (r / 4) + 4 (l / 32) + r % 4 of column l % 32 and stores them one
// element at a time.  Correct for every shape, not tuned: aligned shapes
// never come here.
#include "common.h"

#include "gemm_params.h"

namespace moegg {

namespace {

constexpr int kAnyWaves = 4;
constexpr int kAnyThreads = kAnyWaves * kWave;
// Operands are below 2 GiB (checked on the host), so a masked element is the
// offset kAnyOOB, which reads zero.
constexpr uint32_t kAnyOOB = 0x80000000u;

typedef unsigned short u16x8a_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t any_rsrc(const void *base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ bf16x8_t load8(__amdgpu_buffer_rsrc_t r, const uint32_t (&off)[8])
{
    u16x8a_t v;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b16(r, off[i], 0, 0);
    return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ void zero16(f32x16_t &acc)
{
#pragma unroll
    for (int r = 0; r < 16; ++r)
        acc[r] = 0.0f;
}

// Output row (within the 32 x 32 block) of accumulator element r of this lane.
__device__ __forceinline__ int out_row(int r)
{
    return 8 * (r >> 2) + 4 * ((threadIdx.x & (kWave - 1)) >> 5) + (r & 3);
}

__device__ __forceinline__ void store_bf16(char *base, int64_t elem, float v)
{
    *reinterpret_cast<uint16_t *>(base + elem * 2) = to_bf16(v);
}

}  // namespace

// Forward: rows are an expert's sorted positions, columns the N outputs
// (pre-activation), reduction over K.
template <bool GATED>
__global__ __launch_bounds__(kAnyThreads) void fwd_any_kernel(FwdParams a)
{
    __shared__ int s_roff[kMaxExperts + 1];
    __shared__ int s_tstart[kMaxExperts + 1];
    __shared__ int s_scratch[2];
    const int ct = (a.N + 31) / 32;
    const int total = build_expert_tables(a.m_sizes, a.E, a.S, s_roff, s_tstart, s_scratch, a.err,
                                          [&](int rows) { return (rows + 31) / 32 * ct; });
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int col = lane & 31, half = lane >> 5;
    const bool px = a.flags & MOEGG_PERMUTE_X, py = a.flags & MOEGG_PERMUTE_Y;
    const bool fm = a.flags & MOEGG_FUSE_MUL_POST;
    const int64_t x_rows = px ? a.S / a.topk : a.S;
    const __amdgpu_buffer_rsrc_t xr = any_rsrc(a.X, x_rows * a.K * 2);
    const int64_t wbytes = (int64_t)a.N * a.K * 2;
    const int ncols = GATED ? a.N / 2 : a.N;
    bool bad = false;
    for (int t = blockIdx.x * kAnyWaves + wave; t < total; t += gridDim.x * kAnyWaves) {
        const int e = upper_index(s_tstart, a.E, t);
        const int u = t - s_tstart[e];
        const int i0 = (u / ct) * 32, n0 = (u % ct) * 32;
        const int pb = s_roff[e], pe = s_roff[e + 1];
        const __amdgpu_buffer_rsrc_t wr = any_rsrc(a.W + e * wbytes, wbytes);
        // A: this lane's row, position pb + i0 + col; B: W row n0 + col.
        const int p = pb + i0 + col;
        int g = p;
        if (px || py)
            g = a.gather[min(p, pe - 1)];
        const bool gok = !(px || py) || (uint32_t)g < (uint32_t)a.S;
        const bool aok = p < pe && gok;
        bad |= p < pe && !gok;
        const uint32_t arow = aok ? (uint32_t)((px ? g / a.topk : p) * (int64_t)a.K * 2) : 0;
        const bool bok = n0 + col < a.N;
        const uint32_t brow = bok ? (uint32_t)((n0 + col) * (int64_t)a.K * 2) : 0;
        f32x16_t acc;
        zero16(acc);
        for (int k0 = 0; k0 < a.K; k0 += 16) {
            uint32_t ao[8], bo[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int k = k0 + 8 * half + i;
                ao[i] = aok && k < a.K ? arow + k * 2 : kAnyOOB;
                bo[i] = bok && k < a.K ? brow + k * 2 : kAnyOOB;
            }
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load8(xr, ao), load8(wr, bo), acc, 0, 0,
                                                          0);
        }
        const int n = n0 + col;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int q = pb + i0 + out_row(r);
            float v = acc[r];
            float partner = 0.0f;
            if constexpr (GATED)
                partner = __shfl_xor(v, 1, kWave);  // column n ^ 1 of the same row
            if (q >= pe)
                continue;
            int gq = q;
            if (px || py) {
                gq = a.gather[q];
                if ((uint32_t)gq >= (uint32_t)a.S)
                    continue;  // reported by the lane that loaded this row
            }
            const int64_t dst = py ? gq : q;
            if constexpr (GATED) {
                if ((n & 1) == 0 && n + 1 < a.N)
                    store_bf16(a.Y, dst * ncols + n / 2, v / (1.0f + __expf(-v)) * partner);
            } else if (n < a.N) {
                if (fm)
                    v *= a.topk_w[gq];
                store_bf16(a.Y, dst * ncols + n, v);
            }
        }
    }
    if (bad)
        raise_error(a.err, kErrGather);
}

// dX: rows are an expert's sorted positions, columns the K outputs,
// reduction over N (W read down its columns).
__global__ __launch_bounds__(kAnyThreads) void dx_any_kernel(DxParams a)
{
    __shared__ int s_roff[kMaxExperts + 1];
    __shared__ int s_tstart[kMaxExperts + 1];
    __shared__ int s_scratch[2];
    const int ct = (a.K + 31) / 32;
    const int total = build_expert_tables(a.m_sizes, a.E, a.S, s_roff, s_tstart, s_scratch, a.err,
                                          [&](int rows) { return (rows + 31) / 32 * ct; });
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int col = lane & 31, half = lane >> 5;
    const bool px = a.flags & MOEGG_PERMUTE_X, py = a.flags & MOEGG_PERMUTE_Y;
    const __amdgpu_buffer_rsrc_t yr = any_rsrc(a.dY, a.S * a.N * 2);
    const int64_t wbytes = (int64_t)a.N * a.K * 2;
    bool bad = false;
    for (int t = blockIdx.x * kAnyWaves + wave; t < total; t += gridDim.x * kAnyWaves) {
        const int e = upper_index(s_tstart, a.E, t);
        const int u = t - s_tstart[e];
        const int i0 = (u / ct) * 32, k0 = (u % ct) * 32;
        const int pb = s_roff[e], pe = s_roff[e + 1];
        const __amdgpu_buffer_rsrc_t wr = any_rsrc(a.W + e * wbytes, wbytes);
        const int p = pb + i0 + col;
        int g = p;
        if (px || py)
            g = a.gather[min(p, pe - 1)];
        const bool gok = !(px || py) || (uint32_t)g < (uint32_t)a.S;
        const bool aok = p < pe && gok;
        bad |= p < pe && !gok;
        const uint32_t arow = aok ? (uint32_t)((py ? g : p) * (int64_t)a.N * 2) : 0;
        const bool bok = k0 + col < a.K;
        const uint32_t bcol = (uint32_t)(k0 + col) * 2;
        f32x16_t acc;
        zero16(acc);
        for (int r0 = 0; r0 < a.N; r0 += 16) {
            uint32_t ao[8], bo[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int n = r0 + 8 * half + i;
                ao[i] = aok && n < a.N ? arow + n * 2 : kAnyOOB;
                bo[i] = bok && n < a.N ? (uint32_t)(n * (int64_t)a.K * 2) + bcol : kAnyOOB;
            }
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load8(yr, ao), load8(wr, bo), acc, 0, 0,
                                                          0);
        }
        const int k = k0 + col;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int q = pb + i0 + out_row(r);
            if (q >= pe || k >= a.K)
                continue;
            int64_t dst = q;
            if (px) {
                const int gq = a.gather[q];
                if ((uint32_t)gq >= (uint32_t)a.S)
                    continue;
                dst = gq;
            } else if (py && (uint32_t)a.gather[q] >= (uint32_t)a.S) {
                continue;
            }
            store_bf16(a.dX, dst * a.K + k, acc[r]);
        }
    }
    if (bad)
        raise_error(a.err, kErrGather);
}

// dW: for every expert (an empty one gets zeros), rows are the N outputs and
// columns the K outputs; the reduction runs over the expert's sorted
// positions, whose HBM rows each lane looks up 8 at a time.
__global__ __launch_bounds__(kAnyThreads) void dw_any_kernel(DwParams a)
{
    __shared__ int s_roff[kMaxExperts + 1];
    __shared__ int s_tstart[kMaxExperts + 1];
    __shared__ int s_scratch[2];
    build_expert_tables(a.m_sizes, a.E, a.S, s_roff, s_tstart, s_scratch, a.err,
                        [](int) { return 0; });
    const int rt = (a.N + 31) / 32, ct = (a.K + 31) / 32;
    const int64_t total = (int64_t)a.E * rt * ct;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int col = lane & 31, half = lane >> 5;
    const bool px = a.flags & MOEGG_PERMUTE_X, py = a.flags & MOEGG_PERMUTE_Y;
    const bool f32out = a.flags & MOEGG_DW_FP32_OUT;
    const int64_t x_rows = px ? a.S / a.topk : a.S;
    const __amdgpu_buffer_rsrc_t xr = any_rsrc(a.X, x_rows * a.K * 2);
    const __amdgpu_buffer_rsrc_t yr = any_rsrc(a.dY, a.S * a.N * 2);
    bool bad = false;
    for (int64_t t = (int64_t)blockIdx.x * kAnyWaves + wave; t < total;
         t += (int64_t)gridDim.x * kAnyWaves) {
        const int e = (int)(t / (rt * ct));
        const int u = (int)(t % (rt * ct));
        const int n0 = (u / ct) * 32, k0 = (u % ct) * 32;
        const int pb = s_roff[e], pe = s_roff[e + 1];
        const bool nok = n0 + col < a.N, kok = k0 + col < a.K;
        f32x16_t acc;
        zero16(acc);
        for (int c0 = pb; c0 < pe; c0 += 16) {
            uint32_t ao[8], bo[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int p = c0 + 8 * half + i;
                const bool in = p < pe;
                int g = p;
                if (px || py)
                    g = a.gather[min(p, pe - 1)];
                const bool gok = !(px || py) || (uint32_t)g < (uint32_t)a.S;
                bad |= in && !gok;
                const bool ok = in && gok;
                const int64_t ry = py ? g : p, rx = px ? g / a.topk : p;
                ao[i] = ok && nok ? (uint32_t)(ry * a.N * 2) + (uint32_t)(n0 + col) * 2 : kAnyOOB;
                bo[i] = ok && kok ? (uint32_t)(rx * a.K * 2) + (uint32_t)(k0 + col) * 2 : kAnyOOB;
            }
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load8(yr, ao), load8(xr, bo), acc, 0, 0,
                                                          0);
        }
        const int k = k0 + col;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int n = n0 + out_row(r);
            if (n >= a.N || k >= a.K)
                continue;
            const int64_t o = ((int64_t)e * a.N + n) * a.K + k;
            if (f32out)
                reinterpret_cast<float *>(a.dW)[o] = acc[r];
            else
                store_bf16(a.dW, o, acc[r]);
        }
    }
    if (bad)
        raise_error(a.err, kErrGather);
}

// Explicit groups: y = x @ w with w [k, n] (trans_b 0) or [n, k] (1).
__global__ __launch_bounds__(kAnyThreads) void groups_any_kernel(GroupsParams a, int trans_b)
{
    __shared__ int s_tstart[MOEGG_MAX_GROUPS + 1];
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int i = 0; i < a.num; ++i) {
            s_tstart[i] = acc;
            acc += ((a.g[i].m + 31) / 32) * ((a.g[i].n + 31) / 32);
        }
        s_tstart[a.num] = acc;
    }
    __syncthreads();
    const int total = s_tstart[a.num];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int col = lane & 31, half = lane >> 5;
    for (int t = blockIdx.x * kAnyWaves + wave; t < total; t += gridDim.x * kAnyWaves) {
        const int gi = upper_index(s_tstart, a.num, t);
        const moegg_group &g = a.g[gi];
        const int ct = (g.n + 31) / 32;
        const int u = t - s_tstart[gi];
        const int i0 = (u / ct) * 32, j0 = (u % ct) * 32;
        const __amdgpu_buffer_rsrc_t xr =
            any_rsrc(g.x, ((int64_t)(g.m - 1) * g.ldx + g.k) * 2);
        const int64_t wrows = trans_b ? g.n : g.k, wcols = trans_b ? g.k : g.n;
        const __amdgpu_buffer_rsrc_t wr = any_rsrc(g.w, ((wrows - 1) * g.ldw + wcols) * 2);
        const bool aok = i0 + col < g.m, bok = j0 + col < g.n;
        const uint32_t arow = (uint32_t)((int64_t)(i0 + col) * g.ldx * 2);
        f32x16_t acc;
        zero16(acc);
        for (int r0 = 0; r0 < g.k; r0 += 16) {
            uint32_t ao[8], bo[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = r0 + 8 * half + i;
                ao[i] = aok && r < g.k ? arow + r * 2 : kAnyOOB;
                const int64_t woff = trans_b ? (int64_t)(j0 + col) * g.ldw + r
                                             : (int64_t)r * g.ldw + j0 + col;
                bo[i] = bok && r < g.k ? (uint32_t)(woff * 2) : kAnyOOB;
            }
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load8(xr, ao), load8(wr, bo), acc, 0, 0,
                                                          0);
        }
        const int j = j0 + col;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = i0 + out_row(r);
            if (i < g.m && j < g.n)
                store_bf16(static_cast<char *>(g.y), (int64_t)i * g.ldy + j, acc[r]);
        }
    }
}

namespace {

// Waves for `items` output blocks, at most 8 workgroups per CU.
unsigned any_grid(int64_t items, int cus)
{
    const int64_t wg = (items + kAnyWaves - 1) / kAnyWaves;
    const int64_t cap = (int64_t)cus * 8;
    return (unsigned)(wg < 1 ? 1 : wg < cap ? wg : cap);
}

}  // namespace

hipError_t fwd_any_launch(const FwdParams &p, int cus, hipStream_t stream)
{
    // Blocks: at most S / 32 + E row blocks times the column blocks.
    const int64_t items = (p.S / 32 + p.E) * (((int64_t)p.N + 31) / 32);
    if (p.flags & MOEGG_GATED_SILU)
        hipLaunchKernelGGL(fwd_any_kernel<true>, dim3(any_grid(items, cus)), dim3(kAnyThreads), 0,
                           stream, p);
    else
        hipLaunchKernelGGL(fwd_any_kernel<false>, dim3(any_grid(items, cus)), dim3(kAnyThreads), 0,
                           stream, p);
    return hipGetLastError();
}

hipError_t dx_any_launch(const DxParams &p, int cus, hipStream_t stream)
{
    const int64_t items = (p.S / 32 + p.E) * (((int64_t)p.K + 31) / 32);
    hipLaunchKernelGGL(dx_any_kernel, dim3(any_grid(items, cus)), dim3(kAnyThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t dw_any_launch(const DwParams &p, int cus, hipStream_t stream)
{
    const int64_t items = (int64_t)p.E * (((int64_t)p.N + 31) / 32) * (((int64_t)p.K + 31) / 32);
    hipLaunchKernelGGL(dw_any_kernel, dim3(any_grid(items, cus)), dim3(kAnyThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t groups_any_launch(const GroupsParams &p, int trans_b, int cus, hipStream_t stream)
{
    int64_t items = 0;
    for (int i = 0; i < p.num; ++i)
        items += (int64_t)((p.g[i].m + 31) / 32) * ((p.g[i].n + 31) / 32);
    hipLaunchKernelGGL(groups_any_kernel, dim3(any_grid(items, cus)), dim3(kAnyThreads), 0, stream,
                       p, trans_b);
    return hipGetLastError();
}

}  // namespace moegg
