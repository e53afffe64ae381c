// extern "C" entry points of libmoegg.so: argument checks, then launches.
//
// The checks are the preconditions the pages' launchers assert
// (grouped_gemm_forward, grouped_gemm_dX, grouped_gemm_dW and
// check_valid_config_* in unsloth grouped_gemm/interface.py;
// _allocate_asymmetric_dual_outputs in wall_x/fusions/backend.py), turned into
// status codes.  Every check runs on the host before anything is enqueued, so
// a rejected call touches neither the device nor the stream.
#include "common.h"

#include "../../include/moegg.h"

#include "gemm_params.h"

namespace {

constexpr int kMaxDevices = 64;
int g_cus[kMaxDevices];

// Compute units of the current device (queried once per device).
int device_cus(int *cus)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return -1;
    if (g_cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n < 1)
            return -1;
        g_cus[dev] = n;
    }
    *cus = g_cus[dev];
    return 0;
}

bool aligned16(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// bf16 (fp32) elements need 2- (4-) byte alignment on every path.
bool aligned2(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 1u) == 0;
}
bool aligned4(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 3u) == 0;
}

// The tiled kernels move rows as 16-byte chunks: row lengths that are
// multiples of 8 elements and 16-byte aligned operands.  Other shapes take
// the any-shape launches.
bool tiled_rows(int64_t n, int64_t k)
{
    return n % 8 == 0 && k % 8 == 0;
}

moegg_status check_gemm_common(int32_t num_tokens, int32_t topk, int32_t E, int32_t N, int32_t K)
{
    if (num_tokens < 0 || topk < 1 || E < 1 || E > MOEGG_MAX_EXPERTS || N < 1 || K < 1)
        return MOEGG_ESHAPE;
    if ((int64_t)num_tokens * topk > INT32_MAX)
        return MOEGG_ESHAPE;
    return MOEGG_OK;
}

// Gather indices are required with a permute flag whenever there are rows.
moegg_status check_permute_flags(uint32_t flags, const int32_t *gather_idx, int64_t S)
{
    const bool px = flags & MOEGG_PERMUTE_X, py = flags & MOEGG_PERMUTE_Y;
    if (px && py)
        return MOEGG_EINVAL;  // the pages' launcher rejects both permutes at once
    if ((px || py) && S > 0 && gather_idx == nullptr)
        return MOEGG_EINVAL;  // gather_indices required with a permute flag
    return MOEGG_OK;
}

// Operands are addressed through buffer resources with 32-bit offsets and an
// out-of-range sentinel at 2^31: every operand must stay below 2 GiB.
constexpr int64_t kMaxOperandBytes = (int64_t)1 << 31;

bool fits(int64_t rows, int64_t row_elems, int64_t elem_bytes = 2)
{
    return rows * row_elems * elem_bytes < kMaxOperandBytes;
}

moegg_status from_hip(hipError_t e)
{
    return e == hipSuccess ? MOEGG_OK : MOEGG_EHIP;
}

}  // namespace

extern "C" {

const char *moegg_status_string(moegg_status s)
{
    switch (s) {
    case MOEGG_OK: return "ok";
    case MOEGG_EINVAL: return "invalid argument or flag combination";
    case MOEGG_ESHAPE: return "invalid or inconsistent sizes";
    case MOEGG_EUNSUPPORTED: return "unsupported option";
    case MOEGG_EWORKSPACE: return "workspace missing or too small";
    case MOEGG_EHIP: return "HIP error";
    }
    return "unknown status";
}

int32_t moegg_version(void)
{
    return 100;
}

size_t moegg_route_workspace_bytes(int64_t num_slots, int32_t num_experts)
{
    if (num_slots <= 0 || num_experts < 1)
        return 0;
    return (size_t)moegg::route_chunks(num_slots) * (size_t)num_experts * sizeof(int32_t);
}

moegg_status moegg_route(const int32_t *topk_ids, int32_t num_tokens, int32_t topk,
                         int32_t num_experts, int32_t block_m, int32_t *m_sizes,
                         int32_t *offsets, int32_t *padded_offsets, int32_t *tile_offsets,
                         int32_t *gather_idx, int32_t *scatter_idx, void *workspace,
                         size_t workspace_bytes, int32_t *error_flags, void *stream)
{
    if (num_tokens < 0 || topk < 1 || num_experts < 1 || num_experts > MOEGG_MAX_EXPERTS ||
        block_m < 1)
        return MOEGG_ESHAPE;
    const int64_t S = (int64_t)num_tokens * topk;
    if (S > INT32_MAX)
        return MOEGG_ESHAPE;
    if (m_sizes == nullptr || offsets == nullptr)
        return MOEGG_EINVAL;
    if (S > 0 && (topk_ids == nullptr || gather_idx == nullptr))
        return MOEGG_EINVAL;
    const size_t need = moegg_route_workspace_bytes(S, num_experts);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return MOEGG_EWORKSPACE;
    return from_hip(moegg::route_launch(topk_ids, S, num_experts, block_m, m_sizes, offsets,
                                        padded_offsets, tile_offsets, gather_idx, scatter_idx,
                                        static_cast<int32_t *>(workspace), error_flags,
                                        static_cast<hipStream_t>(stream)));
}

moegg_status moegg_route_noalloc(const int32_t *topk_ids, int32_t num_tokens, int32_t topk,
                                 int32_t num_experts, int32_t block_m, int32_t *m_sizes,
                                 int32_t *offsets, int32_t *padded_offsets, int32_t *tile_offsets,
                                 int32_t *gather_idx, int32_t *scatter_idx, int32_t *error_flags,
                                 void *stream)
{
    if (num_tokens < 0 || topk < 1 || num_experts < 1 || num_experts > MOEGG_MAX_EXPERTS ||
        block_m < 1)
        return MOEGG_ESHAPE;
    const int64_t S = (int64_t)num_tokens * topk;
    if (S > INT32_MAX)
        return MOEGG_ESHAPE;
    if (m_sizes == nullptr || offsets == nullptr)
        return MOEGG_EINVAL;
    if (S > 0 && (topk_ids == nullptr || gather_idx == nullptr))
        return MOEGG_EINVAL;
    if (moegg_route_workspace_bytes(S, num_experts) > MOEGG_ROUTE_NOALLOC_MAX_BYTES)
        return MOEGG_EWORKSPACE;  // more per-chunk counts than the static array holds
    int32_t *counts = nullptr;
    hipError_t e = moegg::route_scratch(&counts);
    if (e != hipSuccess)
        return MOEGG_EHIP;
    return from_hip(moegg::route_launch(topk_ids, S, num_experts, block_m, m_sizes, offsets,
                                        padded_offsets, tile_offsets, gather_idx, scatter_idx,
                                        counts, error_flags, static_cast<hipStream_t>(stream)));
}

moegg_status moegg_grouped_gemm_fwd(const void *X, const void *W, const int32_t *m_sizes,
                                    const int32_t *gather_idx, const float *topk_weights,
                                    int32_t num_tokens, int32_t topk, int32_t num_experts,
                                    int32_t N, int32_t K, uint32_t flags, void *Y,
                                    int32_t *error_flags, void *stream)
{
    moegg_status st = check_gemm_common(num_tokens, topk, num_experts, N, K);
    if (st != MOEGG_OK)
        return st;
    if (flags & ~(MOEGG_PERMUTE_X | MOEGG_PERMUTE_Y | MOEGG_FUSE_MUL_POST | MOEGG_GATED_SILU))
        return MOEGG_EINVAL;
    if ((st = check_permute_flags(flags, gather_idx, (int64_t)num_tokens * topk)) != MOEGG_OK)
        return st;
    if ((flags & MOEGG_FUSE_MUL_POST) && !(flags & MOEGG_PERMUTE_Y))
        return MOEGG_EINVAL;  // the gate multiply is fused only with permute_y
    if ((flags & MOEGG_GATED_SILU) && (flags & (MOEGG_PERMUTE_Y | MOEGG_FUSE_MUL_POST)))
        return MOEGG_EINVAL;  // the activation belongs to the first GEMM
    if ((flags & MOEGG_GATED_SILU) && N % 2 != 0)
        return MOEGG_ESHAPE;  // W rows come in (gate, linear) pairs
    if ((flags & MOEGG_FUSE_MUL_POST) && num_tokens > 0 && topk_weights == nullptr)
        return MOEGG_EINVAL;
    if (num_tokens == 0)
        return MOEGG_OK;
    if (X == nullptr || W == nullptr || m_sizes == nullptr || Y == nullptr)
        return MOEGG_EINVAL;
    if (!aligned2(X) || !aligned2(W) || !aligned2(Y))
        return MOEGG_ESHAPE;
    const bool tiled = tiled_rows(N, K) && (!(flags & MOEGG_GATED_SILU) || N % 16 == 0) &&
                       aligned16(X) && aligned16(W) && aligned16(Y);
    {
        const int64_t S = (int64_t)num_tokens * topk;
        const int64_t x_rows = (flags & MOEGG_PERMUTE_X) ? num_tokens : S;
        if (!fits(x_rows, K) || !fits(N, K))
            return MOEGG_ESHAPE;
    }
    int cus = 0;
    if (device_cus(&cus) != 0)
        return MOEGG_EHIP;
    moegg::FwdParams p;
    p.X = static_cast<const char *>(X);
    p.W = static_cast<const char *>(W);
    p.m_sizes = m_sizes;
    p.gather = gather_idx;
    p.topk_w = topk_weights;
    p.Y = static_cast<char *>(Y);
    p.err = error_flags;
    p.S = (int64_t)num_tokens * topk;
    p.topk = topk;
    p.E = num_experts;
    p.N = N;
    p.K = K;
    p.flags = flags;
    return from_hip(tiled ? moegg::fwd_launch(p, cus, static_cast<hipStream_t>(stream))
                          : moegg::fwd_any_launch(p, cus, static_cast<hipStream_t>(stream)));
}

moegg_status moegg_grouped_gemm_dX(const void *dY, const void *W, const int32_t *m_sizes,
                                   const int32_t *gather_idx, int32_t num_tokens, int32_t topk,
                                   int32_t num_experts, int32_t N, int32_t K, uint32_t flags,
                                   void *dX, void *workspace, size_t workspace_bytes,
                                   int32_t *error_flags, void *stream)
{
    moegg_status st = check_gemm_common(num_tokens, topk, num_experts, N, K);
    if (st != MOEGG_OK)
        return st;
    if (flags & MOEGG_FUSE_MUL_POST)
        return MOEGG_EUNSUPPORTED;  // fuse_mul is for inference only
    if (flags & ~(MOEGG_PERMUTE_X | MOEGG_PERMUTE_Y))
        return MOEGG_EINVAL;
    if ((st = check_permute_flags(flags, gather_idx, (int64_t)num_tokens * topk)) != MOEGG_OK)
        return st;
    if (num_tokens == 0)
        return MOEGG_OK;
    if (dY == nullptr || W == nullptr || m_sizes == nullptr || dX == nullptr)
        return MOEGG_EINVAL;
    if (!aligned2(dY) || !aligned2(W) || !aligned2(dX) || !aligned16(workspace))
        return MOEGG_ESHAPE;
    if (!fits((int64_t)num_tokens * topk, N) || !fits(N, K))
        return MOEGG_ESHAPE;
    const bool tiled = tiled_rows(N, K) && aligned16(dY) && aligned16(W) && aligned16(dX);
    int cus = 0;
    if (device_cus(&cus) != 0)
        return MOEGG_EHIP;
    const int64_t ws_need =
        tiled ? moegg::dx_workspace_bytes((int64_t)num_tokens * topk, num_experts, N, K, cus) : 0;
    if (workspace != nullptr && (int64_t)workspace_bytes < ws_need)
        return MOEGG_EWORKSPACE;
    moegg::DxParams p;
    p.ws = workspace != nullptr && ws_need > 0 ? static_cast<char *>(workspace) : nullptr;
    p.dY = static_cast<const char *>(dY);
    p.W = static_cast<const char *>(W);
    p.m_sizes = m_sizes;
    p.gather = gather_idx;
    p.dX = static_cast<char *>(dX);
    p.err = error_flags;
    p.S = (int64_t)num_tokens * topk;
    p.topk = topk;
    p.E = num_experts;
    p.N = N;
    p.K = K;
    p.flags = flags;
    return from_hip(tiled ? moegg::dx_launch(p, cus, static_cast<hipStream_t>(stream))
                          : moegg::dx_any_launch(p, cus, static_cast<hipStream_t>(stream)));
}

moegg_status moegg_grouped_gemm_dW(const void *X, const void *dY, const int32_t *m_sizes,
                                   const int32_t *gather_idx, int32_t num_tokens, int32_t topk,
                                   int32_t num_experts, int32_t N, int32_t K, uint32_t flags,
                                   void *dW, void *workspace, size_t workspace_bytes,
                                   int32_t *error_flags, void *stream)
{
    moegg_status st = check_gemm_common(num_tokens, topk, num_experts, N, K);
    if (st != MOEGG_OK)
        return st;
    if (flags & MOEGG_FUSE_MUL_POST)
        return MOEGG_EUNSUPPORTED;
    if (flags & ~(MOEGG_PERMUTE_X | MOEGG_PERMUTE_Y | MOEGG_DW_FP32_OUT))
        return MOEGG_EINVAL;
    if ((st = check_permute_flags(flags, gather_idx, (int64_t)num_tokens * topk)) != MOEGG_OK)
        return st;
    if (dW == nullptr || m_sizes == nullptr)
        return MOEGG_EINVAL;
    if (num_tokens > 0 && (X == nullptr || dY == nullptr))
        return MOEGG_EINVAL;
    if (!aligned2(X) || !aligned2(dY) || !aligned2(dW) || !aligned16(workspace))
        return MOEGG_ESHAPE;
    if ((flags & MOEGG_DW_FP32_OUT) && !aligned4(dW))
        return MOEGG_ESHAPE;
    {
        const int64_t S = (int64_t)num_tokens * topk;
        const int64_t x_rows = (flags & MOEGG_PERMUTE_X) ? num_tokens : S;
        if (!fits(x_rows, K) || !fits(S, N))
            return MOEGG_ESHAPE;
    }
    const bool tiled = tiled_rows(N, K) && aligned16(X) && aligned16(dY) && aligned16(dW);
    const int64_t ws_need =
        tiled ? moegg::dw_workspace_bytes((int64_t)num_tokens * topk, num_experts, N, K) : 0;
    const bool use_ws = workspace != nullptr && ws_need > 0;
    if (workspace != nullptr && (int64_t)workspace_bytes < ws_need)
        return MOEGG_EWORKSPACE;
    // Room for X's rows in expert order after the partials: gather them first.
    // The copy is an operand of the reduction like X itself, so it must stay
    // below 2 GiB too; a larger one keeps the gather inside the reduction.
    const int64_t xg_off = moegg::dw_gather_offset((int64_t)num_tokens * topk, num_experts, N, K);
    const int64_t xg_bytes = (int64_t)num_tokens * topk * K * 2;
    const bool use_xg = tiled && workspace != nullptr && (flags & MOEGG_PERMUTE_X) && xg_bytes > 0 &&
                        fits((int64_t)num_tokens * topk, K) &&
                        (int64_t)workspace_bytes >= xg_off + xg_bytes;
    int cus = 0;
    if (device_cus(&cus) != 0)
        return MOEGG_EHIP;
    // T = 0 still writes dW: every expert is empty, so dW is all zeros.
    moegg::DwParams p;
    p.X = static_cast<const char *>(X);
    p.dY = static_cast<const char *>(dY);
    p.m_sizes = m_sizes;
    p.gather = gather_idx;
    p.dW = static_cast<char *>(dW);
    p.err = error_flags;
    p.S = (int64_t)num_tokens * topk;
    p.topk = topk;
    p.E = num_experts;
    p.N = N;
    p.K = K;
    p.flags = flags;
    p.topk_div = moegg::make_fastdiv((uint32_t)topk);
    p.ws = use_ws ? static_cast<char *>(workspace) : nullptr;
    p.xg = use_xg ? static_cast<char *>(workspace) + xg_off : nullptr;
    p.split_rows = use_ws ? moegg::dw_split_rows(p.S, N, K) : 0;
    return from_hip(tiled ? moegg::dw_launch(p, cus, static_cast<hipStream_t>(stream))
                          : moegg::dw_any_launch(p, cus, static_cast<hipStream_t>(stream)));
}

size_t moegg_grouped_gemm_dX_workspace_bytes(int32_t num_tokens, int32_t topk,
                                             int32_t num_experts, int32_t N, int32_t K)
{
    if (check_gemm_common(num_tokens, topk, num_experts, N, K) != MOEGG_OK || !tiled_rows(N, K))
        return 0;
    int cus = 0;
    if (device_cus(&cus) != 0)
        return 0;
    return (size_t)moegg::dx_workspace_bytes((int64_t)num_tokens * topk, num_experts, N, K, cus);
}

size_t moegg_grouped_gemm_dW_workspace_bytes(int32_t num_tokens, int32_t topk,
                                             int32_t num_experts, int32_t N, int32_t K)
{
    if (check_gemm_common(num_tokens, topk, num_experts, N, K) != MOEGG_OK || !tiled_rows(N, K))
        return 0;
    return (size_t)moegg::dw_workspace_bytes((int64_t)num_tokens * topk, num_experts, N, K);
}

size_t moegg_grouped_gemm_dW_gather_workspace_bytes(int32_t num_tokens, int32_t topk,
                                                    int32_t num_experts, int32_t N, int32_t K)
{
    if (check_gemm_common(num_tokens, topk, num_experts, N, K) != MOEGG_OK || !tiled_rows(N, K))
        return 0;
    const int64_t S = (int64_t)num_tokens * topk;
    // No copy: the rows are gathered inside the reduction.
    if (!fits(S, K) || moegg::dw_short_launch(S, num_tokens, num_experts, N, K))
        return (size_t)moegg::dw_workspace_bytes(S, num_experts, N, K);
    return (size_t)(moegg::dw_gather_offset(S, num_experts, N, K) + S * K * 2);
}

moegg_status moegg_grouped_gemm_groups(const moegg_group *groups, int32_t num_groups,
                                       int32_t trans_b, void *stream)
{
    if (groups == nullptr || (trans_b != 0 && trans_b != 1))
        return MOEGG_EINVAL;
    if (num_groups < 1 || num_groups > MOEGG_MAX_GROUPS)
        return MOEGG_ESHAPE;
    moegg::GroupsParams p;
    p.num = num_groups;
    bool any = false, tiled = true;
    for (int i = 0; i < num_groups; ++i) {
        const moegg_group &g = groups[i];
        if (g.m < 0 || g.n < 1 || g.k < 1)
            return MOEGG_ESHAPE;
        if (g.ldx < g.k || g.ldy < g.n || g.ldw < (trans_b ? g.k : g.n))
            return MOEGG_ESHAPE;
        if (g.m > 0 && (g.x == nullptr || g.w == nullptr || g.y == nullptr))
            return MOEGG_EINVAL;
        if (!aligned2(g.x) || !aligned2(g.w) || !aligned2(g.y))
            return MOEGG_ESHAPE;
        tiled &= !(g.n % 8 || g.k % 8 || g.ldx % 8 || g.ldw % 8 || g.ldy % 8) &&
                 aligned16(g.x) && aligned16(g.w) && aligned16(g.y);
        if (!fits(g.m, g.ldx) || !fits(trans_b ? g.n : g.k, g.ldw))
            return MOEGG_ESHAPE;
        any |= g.m > 0;
        p.g[i] = g;
    }
    if (!any)
        return MOEGG_OK;
    int cus = 0;
    if (device_cus(&cus) != 0)
        return MOEGG_EHIP;
    return from_hip(tiled ? moegg::groups_launch(p, trans_b, cus, static_cast<hipStream_t>(stream))
                          : moegg::groups_any_launch(p, trans_b, cus,
                                                     static_cast<hipStream_t>(stream)));
}

// Shared checks of the combine entry points.
static moegg_status check_combine(int64_t num_tokens, int32_t topk, int32_t N, int64_t y_rows,
                                  const int32_t *scatter)
{
    if (num_tokens < 0 || topk < 1 || N < 1 || y_rows < 0)
        return MOEGG_ESHAPE;
    if (num_tokens * topk > INT32_MAX)
        return MOEGG_ESHAPE;
    if (scatter == nullptr && y_rows < num_tokens * topk)
        return MOEGG_ESHAPE;  // slot-order Y has one row per slot
    if (y_rows * (int64_t)N * 2 >= ((int64_t)1 << 40) || num_tokens * (int64_t)N * 4 >= ((int64_t)1 << 40))
        return MOEGG_ESHAPE;
    return MOEGG_OK;
}

moegg_status moegg_combine(const void *Y, const int32_t *scatter_idx, const float *topk_weights,
                           int64_t num_tokens, int32_t topk, int32_t N, int64_t y_rows,
                           uint32_t flags, void *out, int32_t *error_flags, void *stream)
{
    moegg_status st = check_combine(num_tokens, topk, N, y_rows, scatter_idx);
    if (st != MOEGG_OK)
        return st;
    if (flags & ~(uint32_t)MOEGG_COMBINE_FP32_OUT)
        return MOEGG_EINVAL;
    if (num_tokens == 0)
        return MOEGG_OK;
    if (!Y || !out || !aligned2(Y) || !aligned2(out))
        return MOEGG_EINVAL;
    if ((flags & MOEGG_COMBINE_FP32_OUT) && !aligned4(out))
        return MOEGG_EINVAL;
    const bool tiled = N % 8 == 0 && aligned16(Y) && aligned16(out);
    moegg::CombineParams p;
    p.Y = static_cast<const char *>(Y);
    p.scatter = scatter_idx;
    p.weights = topk_weights;
    p.out = static_cast<char *>(out);
    p.err = error_flags;
    p.T = num_tokens;
    p.y_rows = y_rows;
    p.topk = topk;
    p.N = N;
    p.f32_out = flags & MOEGG_COMBINE_FP32_OUT;
    return from_hip(tiled ? moegg::combine_launch(p, static_cast<hipStream_t>(stream))
                          : moegg::combine_any_launch(p, static_cast<hipStream_t>(stream)));
}

moegg_status moegg_combine_bwd(const void *dOut, const void *Y, const int32_t *scatter_idx,
                               const float *topk_weights, int64_t num_tokens, int32_t topk,
                               int32_t N, int64_t y_rows, void *dY, float *dw,
                               int32_t *error_flags, void *stream)
{
    moegg_status st = check_combine(num_tokens, topk, N, y_rows, scatter_idx);
    if (st != MOEGG_OK)
        return st;
    if (num_tokens == 0)
        return MOEGG_OK;
    if (!dOut || !dY || !aligned2(dOut) || !aligned2(dY))
        return MOEGG_EINVAL;
    if (dw && (!Y || !aligned2(Y)))
        return MOEGG_EINVAL;  // the weight gradient reads the forward input
    const bool tiled = N % 8 == 0 && aligned16(dOut) && aligned16(dY) && (!dw || aligned16(Y));
    moegg::CombineBwdParams p;
    p.dOut = static_cast<const char *>(dOut);
    p.Y = static_cast<const char *>(Y);
    p.scatter = scatter_idx;
    p.weights = topk_weights;
    p.dY = static_cast<char *>(dY);
    p.dw = dw;
    p.err = error_flags;
    p.T = num_tokens;
    p.y_rows = y_rows;
    p.topk = topk;
    p.N = N;
    return from_hip(tiled ? moegg::combine_bwd_launch(p, static_cast<hipStream_t>(stream))
                          : moegg::combine_bwd_any_launch(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
