"""Pins of the oracle's top-k combine (unpermute with weights) and its backward.

The combine is the step after the second grouped GEMM: the k expert outputs
of a token, weighted by their routing probabilities and summed (the
unpermute of the wall_x interface; the n_expts_act reduction of
matmul_ogs_torch).  Pins, each from outside the oracle:

* Unpermute of a permute is the identity: with Y[p] = X[gather[p] // k] (the
  permute, from a library stable argsort) and weights 1/k, the combine
  returns X exactly for k = 1, 2, 4 (the sums are exact in fp32).
* The combine is the sparse product M Y with M[t, row(s)] = w[s]; a library
  sparse matmul in float64 must agree within the fp32 summation bound.
* The whole down projection: routed grouped GEMM (permute_y, fuse_mul_post)
  rounded to bf16, then the unweighted combine, equals per token the float64
  sum over its k slots of w_s X[p(s)] W_{e(s)}^T from torch.matmul (p(s):
  the slot's sorted position), within the bf16 rounding of the GEMM outputs.
* Backward: the adjoint identity <combine(Y), G> = <Y, dY(G)>; dw[s] equals
  <combine with w = e_s, G>, which is the exact dot product of Y[row(s)] and
  G[t]; and torch autograd of a float64 combine built from index_add.
* Dropped slots (scatter = -1) add nothing, write no dY row and get dw = 0.
"""

import numpy as np
import pytest
import scipy.sparse as sp
import torch

import oracle
import synth
from tests._util import fwd_reference_f64, gamma, widen


def _routed(T, K, N, E, topk, seed, flags=0, empty=()):
    wl = synth.random_case(T, K, N, E, topk, flags, seed, empty=empty)
    ids = wl.ids.numpy().reshape(-1)
    r = oracle.route(ids, E, 16)
    return wl, ids, r


def _bf16_rows(rng, rows, N, std=1.0):
    return synth.bits(torch.from_numpy(rng.normal(0, std, (rows, N)).astype(np.float32))
                      .to(torch.bfloat16))


@pytest.mark.parametrize("topk", [1, 2, 4])
def test_unpermute_of_permute_is_identity(topk):
    wl, ids, r = _routed(37, 24, 8, 5, topk, 31)
    X = synth.bits(synth.normal_bf16((37, 40), 1.0, synth.generator(7)))
    order = np.argsort(ids, kind="stable")          # library stable sort = the permute
    Y_sorted = X[order // topk]
    w = np.full(37 * topk, 1.0 / topk, np.float32)
    out = oracle.combine(Y_sorted, topk, scatter=r["scatter"], weights=w)
    assert np.array_equal(out, widen(X).astype(np.float32))


@pytest.mark.parametrize("sorted_input", [False, True])
def test_combine_is_a_sparse_product(sorted_input):
    rng = np.random.default_rng(5)
    T, topk, N, E = 53, 3, 72, 6
    wl, ids, r = _routed(T, 8, 8, E, topk, 32)
    S = T * topk
    Y = _bf16_rows(rng, S, N)
    w = rng.normal(0, 1, S).astype(np.float32)
    scatter = r["scatter"] if sorted_input else None
    out = oracle.combine(Y, topk, scatter=scatter, weights=w)
    rows = r["scatter"] if sorted_input else np.arange(S)
    M = sp.coo_matrix((w.astype(np.float64), (np.arange(S) // topk, rows)), shape=(T, S)).tocsr()
    ref = M @ widen(Y)
    absref = abs(M) @ np.abs(widen(Y))
    assert np.all(np.abs(out - ref) <= 2 * gamma(topk) * absref + 1e-30)


def test_layer_equals_per_token_dense():
    # down projection: X arrives in expert-sorted order (row scatter[s] for
    # slot s); Y = grouped(X) with permute_y + fuse_mul_post, rounded to
    # bf16, then summed over k -> per token sum_j w_j X[scatter[s]] W_{e_j}^T
    T, K, N, E, topk = 29, 40, 24, 5, 2
    flags = oracle.PERMUTE_Y | oracle.FUSE_MUL_POST
    wl, ids, r = _routed(T, K, N, E, topk, 33, flags=flags, empty=(2,))
    w = wl.weights.numpy().reshape(-1)
    Yf = oracle.grouped_gemm_fwd(synth.bits(wl.X), synth.bits(wl.W), r["m_sizes"], r["gather"],
                                 w, topk, flags)
    Yb = synth.bits(torch.from_numpy(Yf).to(torch.bfloat16))
    out = oracle.combine(Yb, topk)
    Xd = torch.from_numpy(widen(synth.bits(wl.X)))
    Wd = torch.from_numpy(widen(synth.bits(wl.W)))
    ref = np.zeros((T, N))
    bound = np.zeros((T, N))
    for s in range(T * topk):
        t, e = s // topk, int(ids[s])
        term = (Xd[int(r["scatter"][s])] @ Wd[e].T).numpy() * float(w[s])
        ref[t] += term
        bound[t] += np.abs(term)
    # bf16 rounding of each GEMM output (2^-9 relative) plus fp32 sums
    assert np.all(np.abs(out - ref) <= bound * (2.0 ** -8) + 1e-6)


def test_backward_adjoint_and_dw():
    rng = np.random.default_rng(9)
    T, topk, N, E = 41, 4, 56, 7
    wl, ids, r = _routed(T, 8, 8, E, topk, 34)
    S = T * topk
    Y = _bf16_rows(rng, S, N)
    G = _bf16_rows(rng, T, N, 0.1)
    w = rng.normal(0, 1, S).astype(np.float32)
    out = oracle.combine(Y, topk, scatter=r["scatter"], weights=w)
    dY, dw = oracle.combine_bwd(G, Y, topk, scatter=r["scatter"], weights=w)
    lhs = float(np.sum(out.astype(np.float64) * widen(G)))
    rhs = float(np.sum(widen(Y) * dY.astype(np.float64)))
    assert abs(lhs - rhs) <= 1e-5 * (np.sum(np.abs(out) * np.abs(widen(G))) + 1e-30)
    for s in (0, 5, S // 2, S - 1):
        e_s = np.zeros(S, np.float32)
        e_s[s] = 1.0
        one = oracle.combine(Y, topk, scatter=r["scatter"], weights=e_s)   # exactly Y[row(s)]
        exact = float(np.sum(one.astype(np.float64) * widen(G)))
        t = s // topk
        absdot = float(np.sum(np.abs(widen(Y)[r["scatter"][s]]) * np.abs(widen(G)[t])))
        assert abs(dw[s] - exact) <= 2 * gamma(N) * absdot + 1e-30


def test_backward_matches_autograd():
    rng = np.random.default_rng(11)
    T, topk, N, E = 23, 3, 40, 5
    wl, ids, r = _routed(T, 8, 8, E, topk, 35)
    S = T * topk
    Y = _bf16_rows(rng, S, N)
    G = _bf16_rows(rng, T, N, 0.1)
    w = rng.normal(0, 1, S).astype(np.float32)
    Yt = torch.from_numpy(widen(Y)).requires_grad_(True)
    wt = torch.from_numpy(w.astype(np.float64)).requires_grad_(True)
    rows = torch.from_numpy(r["scatter"].astype(np.int64))
    tok = torch.arange(S) // topk
    out = torch.zeros(T, N, dtype=torch.float64).index_add(0, tok, Yt[rows] * wt[:, None])
    (out * torch.from_numpy(widen(G))).sum().backward()
    dY, dw = oracle.combine_bwd(G, Y, topk, scatter=r["scatter"], weights=w)
    assert np.allclose(dY, Yt.grad.numpy(), rtol=1e-6, atol=1e-30)
    assert np.allclose(dw, wt.grad.numpy(), rtol=1e-4, atol=1e-6)


def test_dropped_slots_and_unit_weights():
    rng = np.random.default_rng(13)
    T, topk, N = 10, 2, 16
    S = T * topk
    Y = _bf16_rows(rng, S, N)
    scatter = np.arange(S, dtype=np.int32)[::-1].copy()
    scatter[[3, 8]] = -1
    G = _bf16_rows(rng, T, N)
    out = oracle.combine(Y, topk, scatter=scatter)
    for t in range(T):
        want = np.zeros(N, np.float32)
        for j in range(topk):
            s = t * topk + j
            if scatter[s] >= 0:
                want = want + widen(Y[scatter[s]]).astype(np.float32)
        assert np.array_equal(out[t], want)
    dY, dw = oracle.combine_bwd(G, Y, topk, scatter=scatter)
    assert dw[3] == 0.0 and dw[8] == 0.0
    unmapped = sorted(set(range(S)) - set(scatter[scatter >= 0].tolist()))
    assert np.all(dY[unmapped] == 0.0)      # rows no slot maps to stay untouched
    s = 4
    assert np.array_equal(dY[scatter[s]], widen(G[s // topk]).astype(np.float32))
