"""Helpers shared by the tests: library reference computations and error bounds.

Nothing here is used by the product; the float64 references below are built
from library routines (torch matmul / autograd) so that they pin the oracle
from outside it.
"""

from __future__ import annotations

import numpy as np
import torch

U32 = 2.0 ** -24  # unit roundoff of fp32


def widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def gamma(n: int) -> float:
    """Bound factor for recursive fp32 summation of n exact terms (n u / (1 - n u))."""
    nu = n * U32
    return nu / (1.0 - nu)


def sorted_rows(ids: np.ndarray, topk: int, flags: int, X: np.ndarray):
    """Per sorted position: source row of X, via a library stable argsort."""
    order = np.argsort(ids.reshape(-1), kind="stable")
    return order // topk if (flags & 1) else np.arange(order.size)


def fwd_reference_f64(Xb, Wb, ids, w, topk, flags):
    """Grouped forward in float64 from torch.matmul per expert.

    Returns (Y [S, N] in the output's own row order, absprod [S, N] =
    sum_k |x_k w_k| for the error bound).
    """
    ids = ids.reshape(-1)
    order = np.argsort(ids, kind="stable")
    E, N, K = Wb.shape
    X = torch.from_numpy(widen(Xb))
    W = torch.from_numpy(widen(Wb))
    S = ids.size
    Y = torch.zeros(S, N, dtype=torch.float64)
    A = torch.zeros(S, N, dtype=torch.float64)
    for e in range(E):
        pos = np.nonzero(ids[order] == e)[0]
        if pos.size == 0:
            continue
        slots = order[pos]
        src = slots // topk if (flags & 1) else pos
        xe = X[torch.from_numpy(src)]
        ye = xe @ W[e].T
        ae = xe.abs() @ W[e].abs().T
        if flags & 4:
            ye = ye * torch.from_numpy(w.reshape(-1)[slots].astype(np.float64))[:, None]
            ae = ae * torch.from_numpy(np.abs(w.reshape(-1)[slots]).astype(np.float64))[:, None]
        dst = torch.from_numpy(slots if (flags & 2) else pos)
        Y[dst] = ye
        A[dst] = ae
    return Y.numpy(), A.numpy()


def within_fp32_bound(got, ref, absprod, n_terms, slack=2.0):
    """|got - ref| <= slack * gamma(n) * sum|terms| + tiny, elementwise."""
    bound = slack * gamma(max(n_terms, 1)) * absprod + 1e-30
    err = np.abs(got.astype(np.float64) - ref)
    return bool(np.all(err <= bound)), float(np.max(err - bound)) if err.size else 0.0


def rel_fro(got, ref) -> float:
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def bf16_tolerance_ok(got, ref, rel_fro_max=5e-3, max_elem=3e-2):
    """The bf16-output tolerance: relative Frobenius error and an elementwise
    bound of max_elem * max(1, |ref|) (absolute below 1, relative above)."""
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    rf = rel_fro(got, ref)
    lim = max_elem * np.maximum(1.0, np.abs(ref))
    worst = float(np.max(np.abs(got - ref) - lim)) if ref.size else -1.0
    ok = (rf <= rel_fro_max) and (worst <= 0.0)
    return ok, {"rel_fro": rf, "max_abs": float(np.max(np.abs(got - ref))) if ref.size else 0.0,
                "worst_excess": worst}
