// Kernel parameter blocks and host launchers of the grouped-GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moegg.h"

namespace moegg {

// Forward: Y = grouped X W_e^T with permute_x / permute_y / fuse_mul_post.
struct FwdParams {
    const char *X;
    const char *W;
    const int32_t *m_sizes;
    const int32_t *gather;
    const float *topk_w;
    char *Y;
    int32_t *err;
    int64_t S;
    int topk, E, N, K;
    uint32_t flags;
};

// dX = grouped dY_e W_e.  ws: workspace for the tail split, or null.
struct DxParams {
    const char *dY;
    const char *W;
    const int32_t *m_sizes;
    const int32_t *gather;
    char *dX;
    int32_t *err;
    char *ws;
    int64_t S;
    int topk, E, N, K;
    uint32_t flags;
};

// Tail split (stream-K for the last round of a persistent grid): when the
// tiles do not fill whole rounds of the G workgroups, each of the R tiles of
// the last round has its reduction cut into P = G / R parts, one per
// otherwise idle workgroup.  A part writes its fp32 [BM, BN] partial into the
// workspace; a second launch sums the parts of each tile in part order and
// stores the tile.  The workspace holds a header (int32: R, P, then p0, rows,
// column 0 and expert of each tail tile; kTailMaxTiles entries) and then the
// partials, tail tile r part q at index r * P + q.
constexpr int kTailMaxTiles = 4096;
__host__ __device__ inline int64_t tail_header_bytes()
{
    return ((2 + 4 * (int64_t)kTailMaxTiles) * 4 + 255) / 256 * 256;
}

// The finishing launch: out[dst(p0 + i), c0 + j] = sum_q partial[r * P +
// q][i, j] as bf16, dst(p) = gather[p] when scatter_out, else p.
struct TailReduceParams {
    const char *ws;
    char *out;
    const int32_t *gather;
    int64_t S;
    int ldo, ncols;
    bool scatter_out;
};

// n / d for 0 <= n < 2^31 as (umulhi(n, mul) + n) >> shift, d >= 1.
struct FastDiv {
    uint32_t mul, shift;
};

inline FastDiv make_fastdiv(uint32_t d)
{
    uint32_t l = 0;
    while ((1ull << l) < d)
        ++l;
    FastDiv f;
    f.mul = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
    f.shift = l;
    return f;
}

// dW_e = dY_e^T X_e.
//
// Split reduction: with split_rows > 0, an expert with more than split_rows
// rows has its reduction cut into chunks of about equal length (a multiple of
// the reduction step); each chunk's tile writes an fp32 partial [N, K] into
// the workspace and dw_reduce_launch sums the chunks in chunk order.  The
// workspace starts with a header (int32: number of split experts, then
// (expert, chunks, first partial) per split expert) of dw_header_bytes(E).
struct DwParams {
    const char *X;
    const char *dY;
    const int32_t *m_sizes;
    const int32_t *gather;
    char *dW;
    int32_t *err;
    char *ws;          // workspace (header + partials), or null
    char *xg;          // X rows gathered into expert order (permute_x), or null
    int64_t S;
    int topk, E, N, K;
    int split_rows;    // 0: never split
    uint32_t flags;
    FastDiv topk_div;
};

// Explicit groups (passed by value in the kernel arguments).
struct GroupsParams {
    moegg_group g[MOEGG_MAX_GROUPS];
    int num;
};

// Top-k combine: out[t] = sum_j w[t*k+j] * Y[row(t*k+j)].
struct CombineParams {
    const char *Y;           // bf16 [y_rows, N]
    const int32_t *scatter;  // slot -> row of Y, or null (Y in slot order)
    const float *weights;    // [T*k] or null (1)
    char *out;               // bf16 or fp32 [T, N]
    int32_t *err;
    int64_t T, y_rows;
    int topk, N;
    bool f32_out;
};

// Its backward: dY[row(s)] = w[s] * dOut[t], dw[s] = <dOut[t], Y[row(s)]>.
struct CombineBwdParams {
    const char *dOut;        // bf16 [T, N]
    const char *Y;           // bf16 [y_rows, N] (read only when dw is requested)
    const int32_t *scatter;
    const float *weights;
    char *dY;                // bf16 [y_rows, N]
    float *dw;               // [T*k] or null
    int32_t *err;
    int64_t T, y_rows;
    int topk, N;
};

hipError_t fwd_launch(const FwdParams &p, int cus, hipStream_t stream);
hipError_t dx_launch(const DxParams &p, int cus, hipStream_t stream);
int64_t dx_workspace_bytes(int64_t S, int E, int N, int K, int cus);
hipError_t dw_launch(const DwParams &p, int cus, hipStream_t stream);
// True when dw_launch takes the short-reduction kernel for S slots (X with
// x_rows rows): no split and no gather copy, so no workspace is used.
bool dw_short_launch(int64_t S, int64_t x_rows, int E, int N, int K);

// Split plan sizes: rows per chunk for a launch of S rows (0: no expert can
// split), the header size and the whole workspace (0 when no split is possible).
int dw_split_rows(int64_t S, int N, int K);
int64_t dw_workspace_bytes(int64_t S, int E, int N, int K);
int64_t dw_gather_offset(int64_t S, int E, int N, int K);

__host__ __device__ inline int64_t dw_header_bytes(int E)
{
    return (4 + 12 * (int64_t)E + 255) / 256 * 256;
}
hipError_t groups_launch(const GroupsParams &p, int trans_b, int cus, hipStream_t stream);

// Any-shape path (any K, N, leading dimensions; operands 2-byte aligned):
// the same results as the launches above, for sizes whose rows cannot be
// moved as 16-byte chunks.  No workspace.
hipError_t fwd_any_launch(const FwdParams &p, int cus, hipStream_t stream);
hipError_t dx_any_launch(const DxParams &p, int cus, hipStream_t stream);
hipError_t dw_any_launch(const DwParams &p, int cus, hipStream_t stream);
hipError_t groups_any_launch(const GroupsParams &p, int trans_b, int cus, hipStream_t stream);

hipError_t combine_launch(const CombineParams &p, hipStream_t stream);
hipError_t combine_bwd_launch(const CombineBwdParams &p, hipStream_t stream);
// Any N, rows 2-byte aligned (not whole 16-byte chunks).
hipError_t combine_any_launch(const CombineParams &p, hipStream_t stream);
hipError_t combine_bwd_any_launch(const CombineBwdParams &p, hipStream_t stream);

int64_t route_chunks(int64_t S);
hipError_t route_scratch(int32_t **out);
hipError_t route_launch(const int32_t *ids, int64_t S, int E, int block_m, int32_t *m_sizes,
                        int32_t *offsets, int32_t *padded_offsets, int32_t *tile_offsets,
                        int32_t *gather, int32_t *scatter, int32_t *counts, int32_t *err,
                        hipStream_t stream);

}  // namespace moegg
