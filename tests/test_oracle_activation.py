"""Pins of the oracle's gated activation on the gate_up output.

The fused activation of triton_kernels/matmul_ogs.py (FusedActivation with
reduction_n = 2) halves the output width.  The oracle takes it as the
SiLU-gated unit, gate and linear columns adjacent (gate first):
out[:, c] = silu(A[:, 2c]) * A[:, 2c + 1].  Pins, each from outside the oracle:

* Closed forms of silu: sigmoid(ln 3) = 3/4, so silu(+-ln 3) = +-ln 3 * 3/4
  and +-ln 3 * 1/4 resp.; silu(1) = e / (1 + e); silu(0) = 0; silu(x) -> x as
  x -> +inf and -> 0 as x -> -inf; a zero linear column gives 0.
* The identity silu(x) - silu(-x) = x for any x (a sign error in the
  exponent, or a dropped factor, breaks it).
* Pairing and function against a library routine: torch.nn.functional.silu
  in float64 on the even columns times the odd columns (a swapped pair or
  halves instead of adjacent pairs fails).
* The whole gated gate_up layer with permute_x against float64 torch.matmul
  per expert followed by the library silu, within the fp32 summation bound
  carried through the activation.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._util import fwd_reference_f64, gamma


def _act(pairs):
    A = np.asarray(pairs, np.float32).reshape(1, -1)
    return oracle.gated_silu(A)[0].astype(np.float64)


def test_closed_forms():
    l3 = math.log(3.0)
    got = _act([l3, 1.0, -l3, 1.0, 1.0, 1.0, 0.0, 5.0, 3.0, 0.0, 40.0, 2.0, -40.0, 2.0])
    # The inputs are fp32: ln 3 rounds, so compare against the rounded argument.
    l3f = float(np.float32(l3))
    want = [0.75 * l3f, -0.25 * l3f, math.e / (1.0 + math.e), 0.0, 0.0, 80.0, 0.0]
    s3 = 1.0 / (1.0 + math.exp(-l3f))  # |3/4 - s3| <= fp32 rounding of ln 3
    assert abs(s3 - 0.75) < 1e-7
    np.testing.assert_allclose(got[:3], want[:3], rtol=3e-7, atol=0)
    assert got[3] == 0.0 and got[4] == 0.0
    assert abs(got[5] - 80.0) <= 80.0 * 2.0 ** -23
    assert abs(got[6]) < 1e-15


def test_odd_part_identity():
    rng = np.random.default_rng(11)
    x = rng.normal(0, 3, 257).astype(np.float32)
    pos = oracle.gated_silu(np.stack([x, np.ones_like(x)], 1).reshape(1, -1))[0]
    neg = oracle.gated_silu(np.stack([-x, np.ones_like(x)], 1).reshape(1, -1))[0]
    # Each side is rounded once to fp32; the difference is x within that.
    err = np.abs(pos.astype(np.float64) - neg.astype(np.float64) - x.astype(np.float64))
    assert np.all(err <= 2.0 ** -23 * (np.abs(pos) + np.abs(neg)) + 1e-30)


def test_pairing_against_library_silu():
    rng = np.random.default_rng(12)
    A = rng.normal(0, 2, (9, 40)).astype(np.float32)
    got = oracle.gated_silu(A).astype(np.float64)
    t = torch.from_numpy(A.astype(np.float64))
    ref = (torch.nn.functional.silu(t[:, 0::2]) * t[:, 1::2]).numpy()
    np.testing.assert_allclose(got, ref, rtol=2.0 ** -23, atol=1e-30)
    # Neither the swapped pair nor the halves layout would agree.
    swapped = (torch.nn.functional.silu(t[:, 1::2]) * t[:, 0::2]).numpy()
    halves = (torch.nn.functional.silu(t[:, :20]) * t[:, 20:]).numpy()
    assert not np.allclose(got, swapped) and not np.allclose(got, halves)


@pytest.mark.parametrize("flags", [oracle.PERMUTE_X, 0])
def test_gated_layer_matches_library(flags):
    T, K, N, E, topk = 29, 48, 40, 5, 2
    wl = synth.random_case(T, K, N, E, topk, flags, 41, empty=(3,))
    ids = wl.ids.numpy().reshape(-1)
    r = oracle.route(ids, E, 16)
    X, W = synth.bits(wl.X), synth.bits(wl.W)
    got = oracle.grouped_gemm_fwd_gated(X, W, r["m_sizes"], r["gather"], topk, flags)
    A, absprod = fwd_reference_f64(X, W, ids, None, topk, flags)
    t = torch.from_numpy(A)
    ref = (torch.nn.functional.silu(t[:, 0::2]) * t[:, 1::2]).numpy()
    # Error of the fp32 GEMM outputs, carried through silu(g) u:
    # |d/dg| = |silu'(g) u| <= 1.1 |u|, |d/du| = |silu(g)|.
    eg = 2.0 * gamma(K) * absprod[:, 0::2]
    eu = 2.0 * gamma(K) * absprod[:, 1::2]
    sg = np.abs(torch.nn.functional.silu(t[:, 0::2]).numpy())
    bound = 1.1 * np.abs(A[:, 1::2]) * eg + sg * eu + eg * eu + 2.0 ** -23 * np.abs(ref) + 1e-30
    assert got.shape == (T * topk, N // 2)
    assert np.all(np.abs(got - ref) <= bound)


def test_gated_column_sample_matches_full():
    T, K, N, E, topk = 21, 32, 24, 4, 2
    wl = synth.random_case(T, K, N, E, topk, oracle.PERMUTE_X, 43)
    r = oracle.route(wl.ids.numpy().reshape(-1), E, 16)
    X, W = synth.bits(wl.X), synth.bits(wl.W)
    full = oracle.grouped_gemm_fwd_gated(X, W, r["m_sizes"], r["gather"], topk, oracle.PERMUTE_X)
    rows, cols = np.array([0, 5, 17, 41]), np.array([11, 0, 7])
    part = oracle.grouped_gemm_fwd_gated(X, W, r["m_sizes"], r["gather"], topk, oracle.PERMUTE_X,
                                         rows=rows, cols=cols)
    assert np.array_equal(part, full[np.ix_(rows, cols)])
