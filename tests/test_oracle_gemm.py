"""Pins of the oracle's grouped GEMMs (forward, dX, dW, dense K x N groups).

The oracle accumulates exact bf16 x bf16 products in fp32, so its result
must sit within the recursive-summation bound gamma(K) * sum|x w| of the
exact (float64, library matmul) value.  On tiny inputs a pure-Python float32
emulation in the stated order must agree bit for bit.  The fusions are pinned
by identities that a dropped term, a wrong index or a transposed operand
breaks: permute_y equals the unfused output moved by the gather index,
permute_x equals the unfused GEMM on pre-gathered rows, fuse_mul_post with
unit weights is the identity and scales each row by its slot's weight.
dX and dW are pinned by torch autograd of a float64 forward, by exact zeros
for empty experts and by the trace identities <dW, W> = <dY, Y> = <dX, X>.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._util import fwd_reference_f64, gamma, widen, within_fp32_bound

PX, PY, FM = oracle.PERMUTE_X, oracle.PERMUTE_Y, oracle.FUSE_MUL_POST


def _case(T, K, N, E, topk, flags, seed, empty=(), with_dy=False):
    wl = synth.random_case(T, K, N, E, topk, flags, seed, empty=empty, with_dy=with_dy)
    ids = wl.ids.numpy().reshape(-1)
    r = oracle.route(ids, E, 16)
    return wl, ids, r


def _fwd(wl, r, flags, **kw):
    return oracle.grouped_gemm_fwd(synth.bits(wl.X), synth.bits(wl.W), r["m_sizes"], r["gather"],
                                   wl.weights.numpy().reshape(-1), wl.topk, flags, **kw)


@pytest.mark.parametrize("flags", [0, PX, PY, PY | FM])
@pytest.mark.parametrize("T,K,N,E,topk,seed,empty", [
    (40, 48, 24, 5, 2, 1, (3,)),       # N != K, one empty expert
    (33, 64, 80, 8, 3, 2, ()),
    (7, 16, 8, 12, 4, 3, (0, 5, 11)),  # several empty experts, most experts tiny
])
def test_fwd_within_fp32_bound_of_float64_matmul(flags, T, K, N, E, topk, seed, empty):
    wl, ids, r = _case(T, K, N, E, topk, flags, seed, empty)
    got = _fwd(wl, r, flags)
    ref, absprod = fwd_reference_f64(synth.bits(wl.X), synth.bits(wl.W), ids,
                                     wl.weights.numpy(), topk, flags)
    ok, excess = within_fp32_bound(got, ref, absprod, K + 1)
    assert ok, excess


def _f32_dot(xs, ws):
    acc = np.float32(0.0)
    for x, w in zip(xs, ws):
        acc = np.float32(acc + np.float32(np.float32(x) * np.float32(w)))
    return acc


def test_fwd_brute_force_bit_exact():
    T, K, N, E, topk = 6, 8, 5, 3, 2
    flags = PY | FM
    wl, ids, r = _case(T, K, N, E, topk, flags, 11)
    X = widen(synth.bits(wl.X)).astype(np.float32)
    W = widen(synth.bits(wl.W)).astype(np.float32)
    wts = wl.weights.numpy().reshape(-1)
    got = _fwd(wl, r, flags)
    S = T * topk
    order = [s for e in range(E) for s in range(S) if ids[s] == e]   # stable by construction
    p = 0
    for e in range(E):
        for s in [s for s in order if ids[s] == e]:
            for n in range(N):
                want = np.float32(_f32_dot(X[p], W[e, n]) * np.float32(wts[s]))
                assert got[s, n] == want, (s, n)
            p += 1


def test_fwd_permute_identities_exact():
    T, K, N, E, topk = 50, 32, 40, 6, 2
    wl, ids, r = _case(T, K, N, E, topk, 0, 5, empty=(2,))
    g = r["gather"]
    plain = _fwd(wl, r, 0)
    # permute_y: the same rows, moved from sorted position p to slot g[p].
    y_perm = _fwd(wl, r, PY)
    assert np.array_equal(y_perm[g], plain)
    # fuse_mul_post with unit weights changes nothing; otherwise scales row g[p] by w[g[p]].
    ones = np.ones(T * topk, np.float32)
    y_one = oracle.grouped_gemm_fwd(synth.bits(wl.X), synth.bits(wl.W), r["m_sizes"], g, ones,
                                    topk, PY | FM)
    assert np.array_equal(y_one, y_perm)
    wts = wl.weights.numpy().reshape(-1)
    y_w = _fwd(wl, r, PY | FM)
    assert np.array_equal(y_w, (y_perm * wts[:, None]).astype(np.float32))
    # permute_x: gathering token rows on load == unfused GEMM on rows pre-gathered by g // topk.
    wlx, idsx, rx = _case(T, K, N, E, topk, PX, 6, empty=(1,))
    gx = rx["gather"]
    y_px = _fwd(wlx, rx, PX)
    Xpre = wlx.X[torch.from_numpy(gx // topk).long()]
    y_pre = oracle.grouped_gemm_fwd(synth.bits(Xpre), synth.bits(wlx.W), rx["m_sizes"], gx,
                                    None, topk, 0)
    assert np.array_equal(y_px, y_pre)


def test_fwd_selection_matches_full():
    wl, ids, r = _case(30, 24, 40, 4, 2, PY | FM, 9)
    full = _fwd(wl, r, PY | FM)
    rows = np.array([0, 17, 59, 3])
    cols = np.array([39, 0, 5], np.int32)
    part = _fwd(wl, r, PY | FM, rows=rows, cols=cols)
    assert np.array_equal(part, full[rows][:, cols])


def _autograd_bwd(wl, r, flags):
    """float64 torch autograd of the grouped forward; returns (dX per output row, dW, Y)."""
    ids = wl.ids.numpy().reshape(-1)
    g = r["gather"]
    topk = wl.topk
    S = ids.size
    E, N, K = wl.W.shape
    src = (g // topk) if (flags & PX) else np.arange(S)
    Xs = torch.from_numpy(widen(synth.bits(wl.X)))[torch.from_numpy(src)].clone().requires_grad_(True)
    W = torch.from_numpy(widen(synth.bits(wl.W))).requires_grad_(True)
    dY = torch.from_numpy(widen(synth.bits(wl.dY)))
    off = r["offsets"]
    outs = []
    for e in range(E):
        outs.append(Xs[off[e]:off[e + 1]] @ W[e].T)
    Ys = torch.cat(outs, 0)                         # sorted order
    dYs = dY[torch.from_numpy(g)] if (flags & PY) else dY
    (Ys * dYs).sum().backward()
    dX_sorted = Xs.grad.numpy()
    if flags & PX:
        dX = np.zeros_like(dX_sorted)
        dX[g] = dX_sorted
    else:
        dX = dX_sorted
    return dX, W.grad.numpy(), Ys.detach().numpy(), Xs.detach().numpy(), dYs.numpy()


@pytest.mark.parametrize("flags", [0, PX, PY])
@pytest.mark.parametrize("T,K,N,E,topk,seed,empty", [
    (40, 24, 48, 5, 2, 21, (3,)),
    (17, 40, 16, 9, 3, 22, (0, 8)),
])
def test_bwd_against_autograd(flags, T, K, N, E, topk, seed, empty):
    wl, ids, r = _case(T, K, N, E, topk, flags, seed, empty, with_dy=True)
    dX_ref, dW_ref, Ys, Xs, dYs = _autograd_bwd(wl, r, flags)
    dY, W, X = synth.bits(wl.dY), synth.bits(wl.W), synth.bits(wl.X)
    dX = oracle.grouped_gemm_dX(dY, W, r["m_sizes"], r["gather"], topk, flags)
    dW = oracle.grouped_gemm_dW(X, dY, r["m_sizes"], r["gather"], topk, flags, E).reshape(E, N, K)
    # bounds: sums over N terms (dX) and over m_e rows (dW)
    Wa = np.abs(widen(W))
    off = r["offsets"]
    g = r["gather"]
    absdX = np.zeros_like(dX_ref)
    absdW = np.zeros_like(dW_ref)
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        rows_out = g[lo:hi] if (flags & PX) else np.arange(lo, hi)
        absdX[rows_out] = np.abs(dYs[lo:hi]) @ Wa[e]
        absdW[e] = np.abs(dYs[lo:hi]).T @ np.abs(Xs[lo:hi])
    ok, ex = within_fp32_bound(dX, dX_ref, absdX, N + 1)
    assert ok, ex
    ok, ex = within_fp32_bound(dW, dW_ref, absdW, int(r["m_sizes"].max()) + 1)
    assert ok, ex
    for e in empty:
        assert np.all(dW[e] == 0.0)
    # Trace identities in float64: <dW, W> = <dY, Y> = <dX, X_sorted>.
    tw = float(np.sum(dW.astype(np.float64) * widen(W).reshape(E, N, K)))
    ty = float(np.sum(dYs * Ys))
    dX_sorted = dX[g] if (flags & PX) else dX
    tx = float(np.sum(dX_sorted.astype(np.float64) * Xs))
    # Each side differs from the exact value only by the oracle's fp32 sums
    # (ty is float64 of exact products), so the gap is bounded by those sums' bounds.
    m_max = int(r["m_sizes"].max()) + 1
    tol_w = 2 * gamma(m_max) * float(np.sum(absdW * Wa)) + 1e-12
    tol_x = 2 * gamma(N + 1) * float(np.sum(absdX[g] * np.abs(Xs) if (flags & PX)
                                             else absdX * np.abs(Xs))) + 1e-12
    assert abs(tw - ty) <= tol_w, (tw, ty, tol_w)
    assert abs(tx - ty) <= tol_x, (tx, ty, tol_x)


def test_bwd_brute_force_bit_exact():
    T, K, N, E, topk = 5, 6, 7, 3, 2
    flags = PY
    wl, ids, r = _case(T, K, N, E, topk, flags, 31, with_dy=True)
    X = widen(synth.bits(wl.X)).astype(np.float32)
    W = widen(synth.bits(wl.W)).astype(np.float32)
    dY = widen(synth.bits(wl.dY)).astype(np.float32)
    g, off = r["gather"], r["offsets"]
    dX = oracle.grouped_gemm_dX(synth.bits(wl.dY), synth.bits(wl.W), r["m_sizes"], g, topk, flags)
    dW = oracle.grouped_gemm_dW(synth.bits(wl.X), synth.bits(wl.dY), r["m_sizes"], g, topk, flags,
                                E).reshape(E, N, K)
    for e in range(E):
        for p in range(off[e], off[e + 1]):
            for k in range(K):
                assert dX[p, k] == _f32_dot(dY[g[p]], W[e, :, k])
        for n in range(N):
            for k in range(K):
                ps = range(off[e], off[e + 1])
                assert dW[e, n, k] == _f32_dot([dY[g[p], n] for p in ps], [X[p, k] for p in ps])


def test_bwd_selection_matches_full():
    wl, ids, r = _case(30, 24, 40, 4, 2, PY, 19, with_dy=True)
    E, N, K = wl.W.shape
    dY, W, X = synth.bits(wl.dY), synth.bits(wl.W), synth.bits(wl.X)
    full_dx = oracle.grouped_gemm_dX(dY, W, r["m_sizes"], r["gather"], 2, PY)
    rows, cols = np.array([5, 0, 33]), np.array([23, 1], np.int32)
    assert np.array_equal(oracle.grouped_gemm_dX(dY, W, r["m_sizes"], r["gather"], 2, PY,
                                                 rows=rows, cols=cols), full_dx[rows][:, cols])
    full_dw = oracle.grouped_gemm_dW(X, dY, r["m_sizes"], r["gather"], 2, PY, E)
    rows = np.array([0, 3 * N + 7, 2 * N])
    assert np.array_equal(oracle.grouped_gemm_dW(X, dY, r["m_sizes"], r["gather"], 2, PY, E,
                                                 rows=rows, cols=cols), full_dw[rows][:, cols])


def test_dense_kn_groups_against_matmul_and_brute_force():
    wl = synth.dual(shapes=((12, 40, 24), (5, 40, 56)))
    for Xt, Wt in wl.groups:
        Xb, Wb = synth.bits(Xt), synth.bits(Wt)
        got = oracle.dense_gemm_kn(Xb, Wb)
        X, W = widen(Xb), widen(Wb)
        ok, ex = within_fp32_bound(got, X @ W, np.abs(X) @ np.abs(W), X.shape[1] + 1)
        assert ok, ex
        Xf, Wf = X.astype(np.float32), W.astype(np.float32)
        for i in range(0, Xf.shape[0], 3):
            for j in range(0, Wf.shape[1], 5):
                assert got[i, j] == _f32_dot(Xf[i], Wf[:, j])
    with pytest.raises(ValueError):
        oracle.dense_gemm_kn(synth.bits(wl.groups[0][0]), synth.bits(wl.groups[1][0]))


def test_gamma_bound_is_meaningful():
    # The summation bound must be tight enough to catch a single dropped term.
    assert gamma(4096) < 3e-4
