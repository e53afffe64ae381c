/*
 * moe_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU statement of what the MoE grouped-GEMM
 * path computes.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this file's library; the product (the HIP
 * library under token_routing_amd/) never includes, links or calls it, and
 * it includes nothing from the product.
 *
 * Conventions (the same as the pages' interfaces):
 *   T   = num_tokens, k = topk, S = T*k slots, slot s = t*k + j.
 *   E   = experts, W is [E, N, K] (K contiguous), X is [rows, K].
 *   bf16 values arrive as their raw 16-bit patterns (uint16_t) and are
 *   widened exactly to fp32 (a bf16 is the top half of an fp32).
 *   Every product is accumulated in fp32, in ascending order of the
 *   reduction index, as the torch reference of
 *   triton_kernels/matmul_ogs.py (matmul_ogs_torch) does with .float()
 *   matmuls.  Outputs are fp32; the GPU's bf16 results are compared
 *   against them with a tolerance.
 *
 * Nothing here is blocked, fused or reordered: each function is the loop
 * nest its definition states.  Built with gcc -O2 and no -ffast-math, so the
 * compiler may not reassociate the fp32 sums.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_PERMUTE_X 1u
#define OR_PERMUTE_Y 2u
#define OR_FUSE_MUL_POST 4u

static float widen_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * Upper bound on the number of block_m-row tiles that any split of n_rows
 * rows over E experts can need -- RoutingData.n_blocks in
 * triton_kernels/matmul_ogs.py: n_rows itself when n_rows <= E, otherwise
 * ceil((n_rows - E + 1) / block_m) + E - 1.
 */
int64_t oracle_n_blocks(int64_t n_rows, int32_t n_experts, int32_t block_m)
{
    if (n_rows <= n_experts)
        return n_rows;
    int64_t r = n_rows - n_experts + 1;
    if (r < 0)
        r = 0;
    return (r + block_m - 1) / block_m + n_experts - 1;
}

/*
 * Routing metadata from the flat top-k expert ids (slot order).
 *
 * hist[e]  : number of slots routed to expert e -- m_sizes in
 *            grouped_gemm/interface.py (grouped_gemm_forward docstring),
 *            expt_hist in triton_kernels/matmul_ogs.py (RoutingData).
 * off[e]   : exclusive prefix sum of hist, off[E] = total; the torch
 *            reference builds it as off[1:] = cumsum(expt_hist).
 * poff[e]  : the same with every expert's count rounded up to a multiple of
 *            block_m -- the padded layout of the ragged-dw comment block in
 *            triton_kernels/matmul_ogs.py (worked example with
 *            expt_hist = [60, 33, 0, 32, 25], block 32).
 * toff[e]  : exclusive prefix sum of ceil(hist[e] / block_m): the first
 *            tile of each expert.
 * gather[p]: slot id held at sorted position p.  Positions are assigned by
 *            walking slots in ascending order and handing each one the next
 *            free position of its expert (a stable counting sort).  Cutting
 *            gather at the cumulative m_sizes then yields each expert's slots
 *            (the grouped_gemm_forward docstring relies on this), here in
 *            ascending slot order inside each expert.
 * scatter[s]: the inverse, sorted position of slot s (the inverse
 *            permutation that GatherIndx/ScatterIndx in
 *            triton_kernels/matmul_ogs.py describe); -1 marks a slot whose id is
 *            outside [0, E) and was therefore dropped.  gather[p] = -1 for
 *            the positions such dropped slots leave unused at the end.
 *
 * Returns the number of dropped slots.
 */
int64_t oracle_route(const int32_t *ids, int64_t S, int32_t E, int32_t block_m,
                     int32_t *hist, int32_t *off, int32_t *poff, int32_t *toff,
                     int32_t *gather, int32_t *scatter)
{
    int64_t dropped = 0;
    for (int32_t e = 0; e < E; ++e)
        hist[e] = 0;
    for (int64_t s = 0; s < S; ++s) {
        int32_t e = ids[s];
        if (e >= 0 && e < E)
            hist[e] += 1;
        else
            dropped += 1;
    }

    off[0] = 0;
    poff[0] = 0;
    toff[0] = 0;
    for (int32_t e = 0; e < E; ++e) {
        int32_t tiles = (hist[e] + block_m - 1) / block_m;
        off[e + 1] = off[e] + hist[e];
        poff[e + 1] = poff[e] + tiles * block_m;
        toff[e + 1] = toff[e] + tiles;
    }

    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int32_t e = 0; e < E; ++e)
        cursor[e] = off[e];
    for (int64_t p = 0; p < S; ++p)
        gather[p] = -1;
    for (int64_t s = 0; s < S; ++s) {
        int32_t e = ids[s];
        if (e >= 0 && e < E) {
            int32_t p = cursor[e];
            cursor[e] += 1;
            gather[p] = (int32_t)s;
            scatter[s] = p;
        } else {
            scatter[s] = -1;
        }
    }
    free(cursor);
    return dropped;
}

/* Output selection helper: sel == NULL selects every row r as row r. */
static int64_t selected(const int64_t *sel, int64_t r)
{
    return sel ? sel[r] : r;
}

static int32_t column(const int32_t *cols, int32_t c)
{
    return cols ? cols[c] : c;
}

/*
 * Forward grouped GEMM with the pages' fusions -- grouped_gemm_forward
 * (grouped_gemm/interface.py) and the per-expert loop of matmul_ogs_torch
 * (triton_kernels/matmul_ogs.py):
 *
 *   for every expert e and every sorted position p of e's group:
 *     source row   r = gather[p] / topk  with permute_x (X is [T, K] in
 *                                         token order), else p (X is [S, K]
 *                                         already in expert order);
 *     y[n]         = sum_k X[r, k] * W[e, n, k]            (fp32, k ascending)
 *     fuse_mul_post: y[n] *= topk_w[gather[p]]   (the router weight of the
 *                                         slot, topk_w in slot order [T*k])
 *     destination  row gather[p] with permute_y (slot order), else p.
 *
 * Selection, to compute a sample of a large output: out_sel[row] (length S,
 * indexed by destination row) gives the row of Yc to write, or -1 to skip;
 * NULL writes every row.  cols (ncols entries) picks output columns n; NULL
 * means all N.  Yc is [rows selected, ncols] fp32, row-major.
 *
 * m_sizes is used as given (groups are consecutive from position 0); the
 * caller guarantees sum(m_sizes) <= S and valid gather entries.
 */
void oracle_grouped_gemm_fwd(const uint16_t *X, const uint16_t *W, const int32_t *m_sizes,
                             const int32_t *gather, const float *topk_w, int64_t T,
                             int32_t topk, int32_t E, int32_t N, int32_t K, uint32_t flags,
                             const int64_t *out_sel, const int32_t *cols, int32_t ncols,
                             float *Yc)
{
    (void)T;
    int32_t nc = cols ? ncols : N;
    int64_t p0 = 0;
    for (int32_t e = 0; e < E; ++e) {
        const uint16_t *We = W + (int64_t)e * N * K;
        for (int64_t p = p0; p < p0 + m_sizes[e]; ++p) {
            int64_t src = (flags & OR_PERMUTE_X) ? gather[p] / topk : p;
            int64_t dst = (flags & OR_PERMUTE_Y) ? gather[p] : p;
            int64_t out = selected(out_sel, dst);
            if (out < 0)
                continue;
            const uint16_t *xr = X + src * K;
            for (int32_t c = 0; c < nc; ++c) {
                int32_t n = column(cols, c);
                const uint16_t *wr = We + (int64_t)n * K;
                float acc = 0.0f;
                for (int32_t k = 0; k < K; ++k)
                    acc += widen_bf16(xr[k]) * widen_bf16(wr[k]);
                if (flags & OR_FUSE_MUL_POST)
                    acc *= topk_w[gather[p]];
                Yc[out * nc + c] = acc;
            }
        }
        p0 += m_sizes[e];
    }
}

/*
 * dX of the grouped GEMM -- grouped_gemm_dX (grouped_gemm/interface.py):
 * dX_e = dY_e * W_e, a reduction over N.
 *   dY row   q = gather[p] if the forward used permute_y (dY then arrives in
 *              token/slot order and is gathered on load), else p;
 *   dX[row, k] = sum_n dY[q, n] * W[e, n, k]            (fp32, n ascending)
 *   stored at row gather[p] if the forward used permute_x (the forward
 *   gathered X, so the gradient is scattered back to slot order), else p.
 * The output is [S, K] in both cases; summing the top-k copies of a token
 * is a separate step (GroupedGemm.backward).
 * Selection as in oracle_grouped_gemm_fwd, with cols picking k columns.
 */
void oracle_grouped_gemm_dX(const uint16_t *dY, const uint16_t *W, const int32_t *m_sizes,
                            const int32_t *gather, int64_t T, int32_t topk, int32_t E,
                            int32_t N, int32_t K, uint32_t flags, const int64_t *out_sel,
                            const int32_t *cols, int32_t ncols, float *dXc)
{
    (void)T;
    (void)topk;
    int32_t nc = cols ? ncols : K;
    int64_t p0 = 0;
    for (int32_t e = 0; e < E; ++e) {
        const uint16_t *We = W + (int64_t)e * N * K;
        for (int64_t p = p0; p < p0 + m_sizes[e]; ++p) {
            int64_t q = (flags & OR_PERMUTE_Y) ? gather[p] : p;
            int64_t dst = (flags & OR_PERMUTE_X) ? gather[p] : p;
            int64_t out = selected(out_sel, dst);
            if (out < 0)
                continue;
            const uint16_t *dyr = dY + q * N;
            for (int32_t c = 0; c < nc; ++c) {
                int32_t k = column(cols, c);
                float acc = 0.0f;
                for (int32_t n = 0; n < N; ++n)
                    acc += widen_bf16(dyr[n]) * widen_bf16(We[(int64_t)n * K + k]);
                dXc[out * nc + c] = acc;
            }
        }
        p0 += m_sizes[e];
    }
}

/*
 * dW of the grouped GEMM -- grouped_gemm_dW (grouped_gemm/interface.py):
 * dW_e = dY_e^T * X_e, a reduction over the m_sizes[e] rows of expert e
 * (a ragged reduction length; triton_kernels/matmul_ogs.py computes dw the
 * same way, as a grouped matmul of x transposed with dy):
 *   dW[e, n, k] = sum_{p in e} dY[q(p), n] * X[r(p), k]   (fp32, p ascending)
 *   r(p) = gather[p] / topk with permute_x, else p;
 *   q(p) = gather[p] with permute_y, else p.
 * An expert with no rows gets an all-zero dW[e] (the torch reference starts
 * from zeros and only fills experts whose count is positive).
 * Selection: out_sel has E*N entries indexed by e*N + n (NULL: all), cols
 * picks k columns.  dWc is [rows selected, ncols] fp32.
 */
void oracle_grouped_gemm_dW(const uint16_t *X, const uint16_t *dY, const int32_t *m_sizes,
                            const int32_t *gather, int64_t T, int32_t topk, int32_t E,
                            int32_t N, int32_t K, uint32_t flags, const int64_t *out_sel,
                            const int32_t *cols, int32_t ncols, float *dWc)
{
    (void)T;
    int32_t nc = cols ? ncols : K;
    int64_t p0 = 0;
    for (int32_t e = 0; e < E; ++e) {
        for (int32_t n = 0; n < N; ++n) {
            int64_t out = selected(out_sel, (int64_t)e * N + n);
            if (out < 0)
                continue;
            for (int32_t c = 0; c < nc; ++c) {
                int32_t k = column(cols, c);
                float acc = 0.0f;
                for (int64_t p = p0; p < p0 + m_sizes[e]; ++p) {
                    int64_t r = (flags & OR_PERMUTE_X) ? gather[p] / topk : p;
                    int64_t q = (flags & OR_PERMUTE_Y) ? gather[p] : p;
                    acc += widen_bf16(dY[q * N + n]) * widen_bf16(X[r * K + k]);
                }
                dWc[out * nc + c] = acc;
            }
        }
        p0 += m_sizes[e];
    }
}

/*
 * One dense GEMM group as the asymmetric dual-expert interface states it
 * (asym_dual_gmm_separated, wall_x/fusions/backend.py):
 * output = input @ weight, input [m, k] row-major, weight [k, n] row-major
 * (trans_a = trans_b = false), fp32 accumulation over k ascending.
 * Y is [m, n] fp32.
 */
void oracle_dense_gemm_kn(const uint16_t *X, const uint16_t *W, int32_t m, int32_t n, int32_t k,
                          float *Y)
{
    for (int32_t i = 0; i < m; ++i)
        for (int32_t j = 0; j < n; ++j) {
            float acc = 0.0f;
            for (int32_t kk = 0; kk < k; ++kk)
                acc += widen_bf16(X[(int64_t)i * k + kk]) * widen_bf16(W[(int64_t)kk * n + j]);
            Y[(int64_t)i * n + j] = acc;
        }
}

/*
 * Top-k combine: the unpermute of the pages (unpermute in
 * wall_x/fusions/backend.py: expert outputs back to token order, the top-k
 * copies of a token weighted by their routing probabilities and summed),
 * which is also the n_expts_act reduction at the end of matmul_ogs_torch
 * (triton_kernels/matmul_ogs.py):
 *   out[t, n] = sum_{j < k} w[t*k + j] * Y[row(t*k + j), n]   (fp32, j ascending)
 *   row(s) = scatter[s] when Y is in expert-sorted order (scatter != NULL;
 *            a negative entry is a dropped slot and adds nothing), else s
 *            (Y already in slot order, the permute_y output);
 *   w = 1 when NULL (matmul_ogs's form, whose rows already carry the gates).
 * out is [T, N] fp32.
 */
void oracle_combine(const uint16_t *Y, const int32_t *scatter, const float *w, int64_t T,
                    int32_t topk, int32_t N, float *out)
{
    for (int64_t t = 0; t < T; ++t)
        for (int32_t n = 0; n < N; ++n) {
            float acc = 0.0f;
            for (int32_t j = 0; j < topk; ++j) {
                int64_t s = t * topk + j;
                int64_t row = scatter ? scatter[s] : s;
                if (row < 0)
                    continue;
                float ws = w ? w[s] : 1.0f;
                acc += ws * widen_bf16(Y[row * N + n]);
            }
            out[t * N + n] = acc;
        }
}

/*
 * Backward of the combine (unpermute_bwd, wall_x/fusions/backend.py, which
 * takes the forward's input so that the probabilities get a gradient too):
 *   dY[row(s), n] = w[s] * dOut[t, n]                     (fp32)
 *   dw[s]         = sum_n dOut[t, n] * Y[row(s), n]       (fp32, n ascending)
 * for s = t*k + j, with row() and w as in oracle_combine.  A dropped slot
 * (row < 0) writes no dY row and has dw = 0.  dY is [rows of Y, N] fp32 and
 * only the rows some slot maps to are written; dw is [T*k] (may be NULL).
 */
void oracle_combine_bwd(const uint16_t *dOut, const uint16_t *Y, const int32_t *scatter,
                        const float *w, int64_t T, int32_t topk, int32_t N, float *dY, float *dw)
{
    for (int64_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < topk; ++j) {
            int64_t s = t * topk + j;
            int64_t row = scatter ? scatter[s] : s;
            float ws = w ? w[s] : 1.0f;
            float acc = 0.0f;
            if (row >= 0) {
                for (int32_t n = 0; n < N; ++n) {
                    float g = widen_bf16(dOut[t * N + n]);
                    dY[row * N + n] = ws * g;
                    acc += g * widen_bf16(Y[row * N + n]);
                }
            }
            if (dw)
                dw[s] = acc;
        }
}

/*
 * Gated activation on the output of the first (gate_up) GEMM: the
 * FusedActivation of triton_kernels/matmul_ogs.py with reduction_n = 2,
 * whose output keeps N / 2 columns.  The pages leave the function open; it
 * is taken as the SiLU-gated unit of Mixtral-shaped experts, with the two
 * columns that reduce into one output column adjacent, gate first:
 *   out[r, c] = silu(A[r, 2c]) * A[r, 2c + 1],   silu(x) = x / (1 + exp(-x)),
 * evaluated in double from the fp32 inputs and rounded once to fp32.
 * A is [rows, N] fp32 with N even; out is [rows, N / 2].
 */
void oracle_gated_silu(const float *A, int64_t rows, int32_t N, float *out)
{
    int32_t H = N / 2;
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t c = 0; c < H; ++c) {
            double g = A[r * N + 2 * c];
            double u = A[r * N + 2 * c + 1];
            out[r * H + c] = (float)(g / (1.0 + exp(-g)) * u);
        }
}
