/*
 * moegg.h -- MoE grouped GEMM for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libmoegg.so: expert routing metadata, the forward grouped GEMM
 * with its gather / scatter / gate-multiply fusions, its two backward
 * GEMMs, and a launch of explicit GEMM groups of different shapes.
 *
 * Conventions shared by every entry point
 *   T = num_tokens, k = topk, S = T * k routed slots; slot s = t * k + j is
 *   the j-th expert choice of token t (row-major [T, k] order).
 *   E = num_experts.  W is [E, N, K] row-major (K contiguous), the layout of
 *   grouped_gemm_forward in unsloth grouped_gemm/interface.py.
 *   bf16 tensors are row-major, 2 bytes per element; base pointers must be
 *   2-byte aligned (fp32 outputs 4-byte).  Any K and N are accepted: when
 *   every row of a call is whole 16-byte chunks (K and N multiples of 8 and
 *   operands 16-byte aligned) the tiled kernels run, otherwise slower
 *   any-shape kernels that compute the same definitions (no workspace;
 *   workspace arguments are then ignored and the workspace size queries
 *   return 0 for such K and N).
 *   Each input operand (X, dY, one expert's W, a group's x or w) must be
 *   smaller than 2 GiB: the kernels address them with 32-bit offsets.
 *   Index tensors are int32.  "sorted position" p indexes the expert-grouped
 *   order: expert e owns positions [off[e], off[e] + m_sizes[e]).
 *
 * Ownership and ordering
 *   Every pointer is a device pointer owned by the caller (unless stated as
 *   a host pointer).  The library never allocates, frees or synchronises;
 *   each call enqueues its kernels on `stream` (a hipStream_t; NULL is the
 *   default stream) and returns.  Calls on one stream run in order.
 *   Every element of every output is written by the call (the caller need
 *   not clear outputs), except rows that belong to dropped slots.
 *
 * Errors
 *   Host-checkable preconditions (the asserts of the pages' launchers)
 *   return a status before anything is enqueued.  Data-dependent problems
 *   found on the device (an expert id outside [0, E), m_sizes that are
 *   negative or sum past S, a gather index outside [0, S)) are ORed as
 *   MOEGG_DERR_* bits into *error_flags when that pointer is non-NULL; the
 *   kernels skip the offending rows instead of faulting.  *error_flags is
 *   sticky: the library never clears it.
 */
#ifndef MOEGG_H
#define MOEGG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOEGG_OK = 0,
    MOEGG_EINVAL = 1,       /* illegal flag combination or missing pointer       */
    MOEGG_ESHAPE = 2,       /* non-positive, misaligned or inconsistent sizes     */
    MOEGG_EUNSUPPORTED = 3, /* legal on the pages but not offered here            */
    MOEGG_EWORKSPACE = 4,   /* workspace missing or smaller than required         */
    MOEGG_EHIP = 5          /* a HIP launch or query failed                       */
} moegg_status;

/* Flags: the pages' fusion switches (grouped_gemm_forward arguments). */
#define MOEGG_PERMUTE_X 1u     /* gather X rows from token order on load          */
#define MOEGG_PERMUTE_Y 2u     /* scatter output rows back to slot order on store */
#define MOEGG_FUSE_MUL_POST 4u /* multiply each output row by its gate weight     */
#define MOEGG_DW_FP32_OUT 8u   /* dW only: write fp32 instead of bf16             */
#define MOEGG_GATED_SILU 32u   /* forward only: gated SiLU on (gate, linear) pairs */

/* Device error bits ORed into *error_flags. */
#define MOEGG_DERR_EXPERT_ID 1 /* a top-k expert id outside [0, E): slot dropped  */
#define MOEGG_DERR_M_SIZES 2   /* m_sizes negative or summing past S: clipped     */
#define MOEGG_DERR_GATHER 4    /* a gather index outside [0, S): row skipped      */

#define MOEGG_MAX_EXPERTS 1024
#define MOEGG_MAX_GROUPS 16

/* Human-readable name of a status code (static string). */
const char *moegg_status_string(moegg_status status);

/* Library ABI version (major * 100 + minor). */
int32_t moegg_version(void);

/*
 * Bytes of device workspace moegg_route needs for num_slots = T * k slots
 * and num_experts experts (per-chunk expert counts).  0 for num_slots = 0.
 */
size_t moegg_route_workspace_bytes(int64_t num_slots, int32_t num_experts);

/*
 * moegg_route -- expert histogram, offsets and stable gather/scatter indices.
 *
 * Follows the routing metadata the pages consume: m_sizes (the per-expert
 * slot counts of the grouped_gemm_forward docstring,
 * grouped_gemm/interface.py), expt_hist and its cumsum offsets, the
 * block-padded layout of the ragged dw comment block, and GatherIndx /
 * ScatterIndx in triton_kernels/matmul_ogs.py, where the scatter index is
 * the inverse permutation of the gather index.
 *
 *   topk_ids       [S] int32, slot order (the router's [T, k] ids).
 *   m_sizes        out [E]   number of slots routed to each expert.
 *   offsets        out [E+1] exclusive prefix sum of m_sizes.
 *   padded_offsets out [E+1] the same with each count rounded up to a
 *                  multiple of block_m; may be NULL.
 *   tile_offsets   out [E+1] exclusive prefix sum of ceil(m_sizes/block_m);
 *                  may be NULL.
 *   gather_idx     out [S] slot held at sorted position p.  Within an expert,
 *                  slots appear in ascending order (a stable sort).
 *   scatter_idx    out [S] sorted position of slot s (the inverse of
 *                  gather_idx); may be NULL.
 *   workspace      device scratch of moegg_route_workspace_bytes(S, E) bytes,
 *                  contents need no initialisation.
 *
 * A slot whose id is outside [0, E) is dropped: scatter_idx = -1, the
 * positions it would have used stay at the end with gather_idx = -1, and
 * MOEGG_DERR_EXPERT_ID is raised.  Results are bit-for-bit deterministic.
 * Errors: ESHAPE if T < 0, k < 1, E < 1, E > MOEGG_MAX_EXPERTS or
 * block_m < 1; EINVAL for a NULL required pointer; EWORKSPACE if
 * workspace_bytes is too small.  T = 0 writes zero histograms and offsets.
 */
moegg_status moegg_route(const int32_t *topk_ids, int32_t num_tokens, int32_t topk,
                         int32_t num_experts, int32_t block_m, int32_t *m_sizes,
                         int32_t *offsets, int32_t *padded_offsets, int32_t *tile_offsets,
                         int32_t *gather_idx, int32_t *scatter_idx, void *workspace,
                         size_t workspace_bytes, int32_t *error_flags, void *stream);

/* Size of the device array moegg_route_noalloc keeps its counts in. */
#define MOEGG_ROUTE_NOALLOC_MAX_BYTES (1u << 20)

/*
 * moegg_route_noalloc -- moegg_route without a workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It calls no allocating routine.
 *
 * The per-chunk counts go to a static device array of
 * MOEGG_ROUTE_NOALLOC_MAX_BYTES bytes that the library holds on every device
 * it runs on until the process ends (its address is looked up on the first
 * call on each device).  A call with moegg_route_workspace_bytes(T * topk, E)
 * larger than that (e.g. more than 65,536 slots with E = 1024, or more than
 * 2^21 slots with E = 32) returns MOEGG_EWORKSPACE before anything is
 * enqueued.  All calls on one device share the array: calls that may run at
 * the same time on that GPU (streams without ordering between them) race and
 * give wrong results; calls ordered on one stream do not, since each call
 * writes every count it reads.  Otherwise the same arguments, results and
 * errors as moegg_route.
 */
moegg_status moegg_route_noalloc(const int32_t *topk_ids, int32_t num_tokens, int32_t topk,
                                 int32_t num_experts, int32_t block_m, int32_t *m_sizes,
                                 int32_t *offsets, int32_t *padded_offsets, int32_t *tile_offsets,
                                 int32_t *gather_idx, int32_t *scatter_idx, int32_t *error_flags,
                                 void *stream);

/*
 * moegg_grouped_gemm_fwd -- Y_e = X_e W_e^T for every expert, one launch.
 *
 * grouped_gemm_forward (grouped_gemm/interface.py) and the per-expert loop
 * of matmul_ogs_torch (triton_kernels/matmul_ogs.py).  For sorted position p
 * of expert e, with fp32 accumulation:
 *   y[n] = sum_k X[src(p), k] * W[e, n, k]
 *   src(p) = gather_idx[p] / topk with MOEGG_PERMUTE_X (X is [T, K], token
 *            order), else p (X is [S, K], already in expert order);
 *   MOEGG_FUSE_MUL_POST: y *= topk_weights[gather_idx[p]] (fp32 gate of the
 *            slot, topk_weights is [S] in slot order);
 *   stored as bf16 (round to nearest even) to row gather_idx[p] of Y with
 *   MOEGG_PERMUTE_Y, else to row p.  Y is [S, N].
 *   MOEGG_GATED_SILU: the gate_up GEMM with its activation fused (the
 *            FusedActivation of triton_kernels/matmul_ogs.py with
 *            reduction_n = 2, output width N/2).  W rows come in adjacent
 *            (gate, linear) pairs and
 *              out[c] = silu(y[2c]) * y[2c + 1],  silu(x) = x / (1 + e^-x),
 *            from the fp32 accumulators, rounded once to bf16.  Y is
 *            [S, N/2].  Not with PERMUTE_Y or FUSE_MUL_POST (the activation
 *            belongs to the first GEMM); N must be even.
 *
 *   m_sizes     [E] device int32 rows per expert (moegg_route output); read
 *               on the device, no host synchronisation.
 *   gather_idx  [S] device int32; required with either permute flag.
 *   error_flags optional device int32 (see Errors above).
 *
 * Errors: EINVAL if both permute flags are set, FUSE_MUL_POST without
 * PERMUTE_Y, GATED_SILU with PERMUTE_Y or FUSE_MUL_POST, an unknown flag, or
 * a required pointer is NULL (gather_idx with a permute flag, topk_weights
 * with FUSE_MUL_POST); ESHAPE for non-positive sizes, odd N with
 * GATED_SILU, E > MOEGG_MAX_EXPERTS, a pointer that is not 2-byte aligned.
 * T = 0 is a no-op.
 */
moegg_status moegg_grouped_gemm_fwd(const void *X, const void *W, const int32_t *m_sizes,
                                    const int32_t *gather_idx, const float *topk_weights,
                                    int32_t num_tokens, int32_t topk, int32_t num_experts,
                                    int32_t N, int32_t K, uint32_t flags, void *Y,
                                    int32_t *error_flags, void *stream);

/*
 * moegg_grouped_gemm_dX -- dX_e = dY_e W_e (reduction over N), one launch.
 *
 * grouped_gemm_dX (grouped_gemm/interface.py).  `flags` are the permute
 * flags the forward used:
 *   dY row     q(p) = gather_idx[p] if the forward used PERMUTE_Y (dY is in
 *              slot order and is gathered on load), else p;
 *   dX[., k]   = sum_n dY[q(p), n] * W[e, n, k]   (fp32 accumulation)
 *   stored bf16 to row gather_idx[p] if the forward used PERMUTE_X (scatter
 *   back to slot order), else row p.  dY is [S, N], dX is [S, K]; summing a
 *   token's top-k rows is left to the caller.
 *
 * Tail balancing (optional): a persistent launch runs its tiles in rounds
 * of one tile per workgroup.  With a workspace, the tiles of a last, partial
 * round have their reductions over N cut into parts spread over the
 * otherwise idle workgroups (the split-k of triton_kernels/matmul_ogs.py,
 * fp32 partials summed by a separate launch), summed in part order:
 * deterministic, and equal to the unsplit result up to fp32 rounding order.
 *   workspace       device, 16-byte aligned, at least
 *                   moegg_grouped_gemm_dX_workspace_bytes(...) bytes (no
 *                   initialisation needed), or NULL: no split.
 *   workspace_bytes its size; 0 with NULL.
 * Errors: EINVAL for both permute flags or a missing gather_idx;
 * EUNSUPPORTED for FUSE_MUL_POST (the pages forbid it in training);
 * ESHAPE as for the forward; EWORKSPACE for a workspace smaller than needed.
 */
moegg_status moegg_grouped_gemm_dX(const void *dY, const void *W, const int32_t *m_sizes,
                                   const int32_t *gather_idx, int32_t num_tokens, int32_t topk,
                                   int32_t num_experts, int32_t N, int32_t K, uint32_t flags,
                                   void *dX, void *workspace, size_t workspace_bytes,
                                   int32_t *error_flags, void *stream);

/*
 * Bytes of workspace moegg_grouped_gemm_dX can use to balance its last
 * round of tiles, for these sizes on the current device (it depends on the
 * device's compute units): a small header plus fp32 partials of at most one
 * tile per workgroup of the launch.  0 if the sizes are invalid or the
 * device cannot be queried.
 */
size_t moegg_grouped_gemm_dX_workspace_bytes(int32_t num_tokens, int32_t topk,
                                             int32_t num_experts, int32_t N, int32_t K);

/*
 * moegg_grouped_gemm_dW -- dW_e = dY_e^T X_e, a reduction over each expert's
 * own (ragged) number of rows, one launch.
 *
 * grouped_gemm_dW (grouped_gemm/interface.py) and the ragged-K formulation of
 * triton_kernels/matmul_ogs.py, which computes dw as a grouped matmul of x
 * transposed with dy:
 *   dW[e, n, k] = sum_{p in e} dY[q(p), n] * X[r(p), k]  (fp32 accumulation)
 *   r(p) = gather_idx[p] / topk with PERMUTE_X (X is [T, K]), else p
 *   (X is [S, K]); q(p) = gather_idx[p] with PERMUTE_Y, else p.
 * dW is [E, N, K], bf16, or fp32 with MOEGG_DW_FP32_OUT.  Experts with no
 * rows get exact zeros.
 *
 * Short launches (S <= 1024 and S <= 16 * num_experts, each operand below
 * 1 GiB, e.g. a decode step) run a kernel whose cost is its output stores:
 * no split and no gather copy, so any workspace is left unused.
 *
 * Split reduction (the split-k of triton_kernels/matmul_ogs.py, whose fp32
 * partials a separate reduce sums, applied to the rows of hot experts):
 * with a workspace, an expert holding many more rows than the average is
 * cut into chunks of rows whose fp32 partial products go to the workspace;
 * a second launch on the same stream sums each expert's partials in chunk
 * order and writes its dW.  The result is deterministic (the same for every
 * run with the same inputs and workspace size), and differs from the
 * unsplit sum only by fp32 rounding order.
 *   workspace       device, 16-byte aligned, of at least
 *                   moegg_grouped_gemm_dW_workspace_bytes(...) bytes
 *                   (contents need no initialisation), or NULL: no split.
 *   workspace_bytes its size; 0 with NULL.
 * Errors: as for dX; EWORKSPACE if a workspace is given but smaller than
 * needed.
 */
moegg_status moegg_grouped_gemm_dW(const void *X, const void *dY, const int32_t *m_sizes,
                                   const int32_t *gather_idx, int32_t num_tokens, int32_t topk,
                                   int32_t num_experts, int32_t N, int32_t K, uint32_t flags,
                                   void *dW, void *workspace, size_t workspace_bytes,
                                   int32_t *error_flags, void *stream);

/*
 * Bytes of workspace moegg_grouped_gemm_dW can use to split hot experts'
 * reductions, for these sizes: a small header plus fp32 [N, K] partials for
 * fewer than 2 S / split_rows chunks, where split_rows is about
 * S * ceil(N/256) * ceil(K/256) / 768 rows (at least 256).  0 when no
 * expert can hold more than split_rows rows, or when S <= 1024 (reductions
 * that short are never split); the workspace is then unused.
 */
size_t moegg_grouped_gemm_dW_workspace_bytes(int32_t num_tokens, int32_t topk,
                                             int32_t num_experts, int32_t N, int32_t K);

/*
 * Bytes of workspace with which moegg_grouped_gemm_dW under MOEGG_PERMUTE_X
 * also copies X's rows into expert order before the reduction: the split
 * area above rounded up to 256 bytes, plus S * K * 2 for the copy.  The copy
 * (X[gather_idx[p] / topk, :] for every sorted position p below the sum of
 * m_sizes) is a separate launch on the same stream; the reduction then
 * reads it in sorted order.  The result is the same as with the gather
 * inside the reduction, including zeros and MOEGG_DERR_GATHER for entries
 * outside [0, S); positions past the sum of m_sizes, where routing leaves
 * its dropped slots, are read by neither.  On MI355X the copy plus the
 * reduction take less time.  The copy is an operand like X and must stay
 * below 2 GiB: when S * K * 2 >= 2^31, or for a short launch (see
 * moegg_grouped_gemm_dW), this returns moegg_grouped_gemm_dW_workspace_bytes(...)
 * and moegg_grouped_gemm_dW gathers inside the reduction whatever the
 * workspace size.  A workspace of
 * at least moegg_grouped_gemm_dW_workspace_bytes(...) bytes but less than
 * this keeps the gather inside the reduction.  Without MOEGG_PERMUTE_X the
 * extra bytes are unused.
 */
size_t moegg_grouped_gemm_dW_gather_workspace_bytes(int32_t num_tokens, int32_t topk,
                                                    int32_t num_experts, int32_t N, int32_t K);

/*
 * One GEMM group: y[m, n] = x[m, k] @ w, bf16 in, fp32 accumulation, bf16 out.
 * w is [k, n] row-major (ldw >= n) when the call's trans_b is 0, as in
 * asym_dual_gmm_separated (wall_x/fusions/backend.py), or [n, k] row-major
 * (ldw >= k) when trans_b is 1.  Leading dimensions are in elements.
 */
typedef struct {
    const void *x;
    const void *w;
    void *y;
    int32_t m, n, k;
    int32_t ldx, ldw, ldy;
} moegg_group;

/*
 * moegg_grouped_gemm_groups -- several independent GEMMs of different shapes
 * in one launch: the asymmetric dual-expert GEMM of asym_dual_gmm_separated
 * (wall_x/fusions/backend.py), which multiplies each expert's own input by
 * its own weight and computes both products in one fused call.
 *
 *   groups      HOST array of num_groups descriptors (copied at launch; it
 *               may be freed when the call returns).  1 <= num_groups <=
 *               MOEGG_MAX_GROUPS.  A group with m = 0 is skipped.
 *   trans_b     0: w is [k, n]; 1: w is [n, k].  trans_a is not offered
 *               (inputs are [m, k]).
 * Errors: EINVAL for a NULL pointer or bad trans_b; ESHAPE for negative
 * sizes, a pointer that is not 2-byte aligned, or a leading dimension
 * smaller than its row.
 */
moegg_status moegg_grouped_gemm_groups(const moegg_group *groups, int32_t num_groups,
                                       int32_t trans_b, void *stream);

/* Combine flag: write the combine's output in fp32 instead of bf16. */
#define MOEGG_COMBINE_FP32_OUT 16u

/*
 * moegg_combine -- the top-k combine after the second grouped GEMM: each
 * token's k expert outputs, weighted by their routing probabilities and
 * summed.  This is the unpermute of wall_x/fusions/backend.py (expert outputs
 * back to token order, combined with the routing probabilities) and the
 * n_expts_act reduction at the end of matmul_ogs in
 * triton_kernels/matmul_ogs.py (matmul_ogs_torch accumulates it in fp32):
 *
 *   out[t, n] = sum_{j<k} w[t*k + j] * Y[row(t*k + j), n]   (fp32, j ascending)
 *
 *   Y              [y_rows, N] bf16 device, row-major.
 *   scatter_idx    [T*k] int32 device: row of Y holding slot s (moegg_route's
 *                  scatter_idx when Y is in expert-sorted order); a negative
 *                  entry is a dropped slot and adds nothing.  NULL: Y is in
 *                  slot order (the PERMUTE_Y output), row(s) = s, and
 *                  y_rows >= T*k.
 *   topk_weights   [T*k] fp32 device, slot order, or NULL for weight 1 (the
 *                  rows already carry the gates, as after FUSE_MUL_POST).
 *   flags          0 or MOEGG_COMBINE_FP32_OUT.
 *   out            [T, N] device, bf16 (rounded once from the fp32 sum) or
 *                  fp32.  Every element is written.
 *   error_flags    optional device int32; an entry of scatter_idx at or above
 *                  y_rows sets MOEGG_DERR_GATHER and the slot is skipped.
 * Any N; Y and out 2-byte aligned (out 4-byte for fp32).  T = 0 is a no-op.
 * Errors: ESHAPE for bad sizes, EINVAL for unknown flags, NULL or misaligned
 * pointers.
 */
moegg_status moegg_combine(const void *Y, const int32_t *scatter_idx, const float *topk_weights,
                           int64_t num_tokens, int32_t topk, int32_t N, int64_t y_rows,
                           uint32_t flags, void *out, int32_t *error_flags, void *stream);

/*
 * moegg_combine_bwd -- backward of moegg_combine (unpermute_bwd,
 * wall_x/fusions/backend.py, which takes the forward input so that the
 * routing probabilities get a gradient as well):
 *
 *   dY[row(s), n] = w[s] * dOut[t, n]                    (rounded to bf16)
 *   dw[s]         = sum_n dOut[t, n] * Y[row(s), n]      (fp32)
 *
 * for s = t*k + j, with row() and w as in moegg_combine (w = 1 when
 * topk_weights is NULL).
 *   dOut   [T, N] bf16 device.
 *   Y      the forward's input [y_rows, N] bf16; read only when dw != NULL.
 *   dY     [y_rows, N] bf16 device; only rows some slot maps to are written
 *          (all of them when scatter_idx is a permutation or NULL).
 *   dw     [T*k] fp32 device, or NULL to skip the weight gradient.  A dropped
 *          slot gets dw = 0 and writes no dY row.
 * Alignment, sizes and errors as moegg_combine.
 */
moegg_status moegg_combine_bwd(const void *dOut, const void *Y, const int32_t *scatter_idx,
                               const float *topk_weights, int64_t num_tokens, int32_t topk,
                               int32_t N, int64_t y_rows, void *dY, float *dw,
                               int32_t *error_flags, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEGG_H */
