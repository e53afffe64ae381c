"""CPU oracle for the MoE grouped-GEMM path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library
(``token_routing_amd``) neither imports nor links it, and this package
imports nothing from the product.

The arithmetic lives in ``moe_oracle.c`` (plain loops, fp32 accumulation in
ascending reduction order, the loop nests of the torch reference
``matmul_ogs_torch`` in triton_kernels/matmul_ogs.py and of the docstrings
of grouped_gemm/interface.py).  This module only builds that file with the
host compiler and marshals numpy arrays to it.

Arrays are numpy: integer inputs int32, bf16 inputs as uint16 bit patterns
(``torch_tensor.view(torch.int16).numpy().view(np.uint16)``), gate weights
float32.  Results are float32.

Every function is pinned by ``tests/test_oracle_*.py`` against values the
pages print, library routines (numpy.bincount, stable argsort, float64
matmul, torch autograd), brute force on tiny inputs and exact identities.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

PERMUTE_X = 1
PERMUTE_Y = 2
FUSE_MUL_POST = 4

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc (-O2, no fast-math) into libmoe_oracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fPIC", "-shared", _SRC, "-o", tmp,
             "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        stale = (not os.path.exists(_LIB)
                 or os.path.getmtime(_LIB) < os.path.getmtime(_SRC))
        build(force=stale)
        lib = ctypes.CDLL(_LIB)
        vp = ctypes.c_void_p
        i32, i64, u32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32
        lib.oracle_n_blocks.argtypes = [i64, i32, i32]
        lib.oracle_n_blocks.restype = i64
        lib.oracle_route.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp, vp, vp]
        lib.oracle_route.restype = i64
        gemm_args = [vp, vp, vp, vp, i64, i32, i32, i32, i32, u32, vp, vp, i32, vp]
        lib.oracle_grouped_gemm_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, i32,
                                                u32, vp, vp, i32, vp]
        lib.oracle_grouped_gemm_fwd.restype = None
        lib.oracle_grouped_gemm_dX.argtypes = gemm_args
        lib.oracle_grouped_gemm_dX.restype = None
        lib.oracle_grouped_gemm_dW.argtypes = gemm_args
        lib.oracle_grouped_gemm_dW.restype = None
        lib.oracle_dense_gemm_kn.argtypes = [vp, vp, i32, i32, i32, vp]
        lib.oracle_dense_gemm_kn.restype = None
        lib.oracle_combine.argtypes = [vp, vp, vp, i64, i32, i32, vp]
        lib.oracle_combine.restype = None
        lib.oracle_combine_bwd.argtypes = [vp, vp, vp, vp, i64, i32, i32, vp, vp]
        lib.oracle_combine_bwd.restype = None
        lib.oracle_gated_silu.argtypes = [vp, i64, i32, vp]
        lib.oracle_gated_silu.restype = None
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def _bf16_bits(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 operands are passed as uint16 bit patterns")
    return a


def n_blocks(n_rows: int, n_experts: int, block_m: int) -> int:
    return int(_load().oracle_n_blocks(n_rows, n_experts, block_m))


def route(ids, num_experts: int, block_m: int):
    """Histogram, offsets (plain, padded, tile) and stable gather/scatter indices.

    Returns a dict with int32 arrays ``m_sizes[E]``, ``offsets[E+1]``,
    ``padded_offsets[E+1]``, ``tile_offsets[E+1]``, ``gather[S]``,
    ``scatter[S]`` and the number of ``dropped`` slots.
    """
    ids = _c(ids, np.int32).reshape(-1)
    S, E = ids.size, int(num_experts)
    out = {
        "m_sizes": np.zeros(E, np.int32),
        "offsets": np.zeros(E + 1, np.int32),
        "padded_offsets": np.zeros(E + 1, np.int32),
        "tile_offsets": np.zeros(E + 1, np.int32),
        "gather": np.zeros(S, np.int32),
        "scatter": np.zeros(S, np.int32),
    }
    out["dropped"] = int(_load().oracle_route(
        _ptr(ids), S, E, int(block_m), _ptr(out["m_sizes"]), _ptr(out["offsets"]),
        _ptr(out["padded_offsets"]), _ptr(out["tile_offsets"]), _ptr(out["gather"]),
        _ptr(out["scatter"])))
    return out


def _selection(n_out_rows: int, rows):
    """rows=None -> every row; else an int64 map out_row -> compact row (-1 skip)."""
    if rows is None:
        return None, n_out_rows
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    sel = np.full(n_out_rows, -1, dtype=np.int64)
    sel[rows] = np.arange(rows.size, dtype=np.int64)
    return sel, rows.size


def grouped_gemm_fwd(X, W, m_sizes, gather, topk_weights, topk: int, flags: int,
                     rows=None, cols=None):
    """Y = grouped X W_e^T with permute_x / permute_y / fuse_mul_post.

    X: uint16 [T, K] (permute_x) or [S, K]; W: uint16 [E, N, K].
    rows: destination rows of Y to compute (default all S, in Y's own order);
    cols: output columns (default all N).  Returns float32 [len(rows), len(cols)].
    """
    X, W = _bf16_bits(X), _bf16_bits(W)
    E, N, K = W.shape
    m_sizes = _c(m_sizes, np.int32)
    gather = _c(gather, np.int32)
    S = int(gather.size) if gather is not None else int(X.shape[0])
    T = S // topk
    topk_weights = _c(topk_weights, np.float32)
    sel, nrows = _selection(S, rows)
    cols = _c(cols, np.int32)
    nc = N if cols is None else cols.size
    Y = np.zeros((nrows, nc), np.float32)
    _load().oracle_grouped_gemm_fwd(_ptr(X), _ptr(W), _ptr(m_sizes), _ptr(gather),
                                    _ptr(topk_weights), T, topk, E, N, K, flags, _ptr(sel),
                                    _ptr(cols), nc, _ptr(Y))
    return Y


def grouped_gemm_dX(dY, W, m_sizes, gather, topk: int, flags: int, rows=None, cols=None):
    """dX = grouped dY_e W_e; dY uint16 [S, N]; returns float32 [len(rows), len(cols)]."""
    dY, W = _bf16_bits(dY), _bf16_bits(W)
    E, N, K = W.shape
    S = int(dY.shape[0])
    m_sizes = _c(m_sizes, np.int32)
    gather = _c(gather, np.int32)
    sel, nrows = _selection(S, rows)
    cols = _c(cols, np.int32)
    nc = K if cols is None else cols.size
    dX = np.zeros((nrows, nc), np.float32)
    _load().oracle_grouped_gemm_dX(_ptr(dY), _ptr(W), _ptr(m_sizes), _ptr(gather), S // topk,
                                   topk, E, N, K, flags, _ptr(sel), _ptr(cols), nc, _ptr(dX))
    return dX


def grouped_gemm_dW(X, dY, m_sizes, gather, topk: int, flags: int, num_experts: int,
                    rows=None, cols=None):
    """dW[e] = dY_e^T X_e (ragged); rows index e*N + n; returns float32 [len(rows), len(cols)]."""
    X, dY = _bf16_bits(X), _bf16_bits(dY)
    S, N = dY.shape
    K = int(X.shape[1])
    E = int(num_experts)
    m_sizes = _c(m_sizes, np.int32)
    gather = _c(gather, np.int32)
    sel, nrows = _selection(E * N, rows)
    cols = _c(cols, np.int32)
    nc = K if cols is None else cols.size
    dW = np.zeros((nrows, nc), np.float32)
    _load().oracle_grouped_gemm_dW(_ptr(X), _ptr(dY), _ptr(m_sizes), _ptr(gather), S // topk,
                                   topk, E, N, K, flags, _ptr(sel), _ptr(cols), nc, _ptr(dW))
    return dW


def dense_gemm_kn(X, W):
    """One group of the dual-expert GEMM: X uint16 [m, k] @ W uint16 [k, n] -> float32 [m, n]."""
    X, W = _bf16_bits(X), _bf16_bits(W)
    m, k = X.shape
    k2, n = W.shape
    if k != k2:
        raise ValueError("inner dimensions differ")
    Y = np.zeros((m, n), np.float32)
    _load().oracle_dense_gemm_kn(_ptr(X), _ptr(W), m, n, k, _ptr(Y))
    return Y


def combine(Y, topk: int, scatter=None, weights=None, num_tokens=None):
    """Top-k combine: out[t] = sum_j w[t*k+j] * Y[row(t*k+j)] (fp32).

    Y: uint16 [rows, N]; scatter: int32 [T*k] (Y in expert-sorted order) or
    None (Y in slot order, rows = T*k); weights: float32 [T*k] or None (1).
    Returns float32 [T, N].
    """
    Y = _bf16_bits(Y)
    N = int(Y.shape[1])
    scatter = _c(scatter, np.int32)
    weights = _c(weights, np.float32)
    S = int(scatter.size) if scatter is not None else int(Y.shape[0])
    T = S // topk if num_tokens is None else int(num_tokens)
    out = np.zeros((T, N), np.float32)
    _load().oracle_combine(_ptr(Y), _ptr(scatter), _ptr(weights), T, topk, N, _ptr(out))
    return out


def combine_bwd(dOut, Y, topk: int, scatter=None, weights=None):
    """Backward of combine: (dY float32 [rows of Y, N] (unmapped rows 0), dw float32 [T*k])."""
    dOut, Y = _bf16_bits(dOut), _bf16_bits(Y)
    T, N = dOut.shape
    scatter = _c(scatter, np.int32)
    weights = _c(weights, np.float32)
    dY = np.zeros(Y.shape, np.float32)
    dw = np.zeros(T * topk, np.float32)
    _load().oracle_combine_bwd(_ptr(dOut), _ptr(Y), _ptr(scatter), _ptr(weights), T, topk, N,
                               _ptr(dY), _ptr(dw))
    return dY, dw


def gated_silu(A):
    """Gated activation: out[:, c] = silu(A[:, 2c]) * A[:, 2c + 1] (double, rounded to fp32).

    A: float32 [rows, N] with N even.  Returns float32 [rows, N // 2].
    """
    A = np.ascontiguousarray(A, dtype=np.float32)
    rows, N = A.shape
    if N % 2:
        raise ValueError("the gated activation needs an even number of columns")
    out = np.zeros((rows, N // 2), np.float32)
    _load().oracle_gated_silu(_ptr(A), rows, N, _ptr(out))
    return out


def grouped_gemm_fwd_gated(X, W, m_sizes, gather, topk: int, flags: int, rows=None, cols=None):
    """The gate_up forward followed by the gated activation.

    Output column c of the [S, N/2] result takes W rows 2c (gate) and 2c + 1
    (linear) of its expert.  rows as in grouped_gemm_fwd; cols: output
    columns in [0, N/2) (default all).  Returns float32 [len(rows), len(cols)].
    """
    N = int(W.shape[1])
    oc = np.arange(N // 2, dtype=np.int64) if cols is None else np.asarray(cols, np.int64)
    wc = np.stack([2 * oc, 2 * oc + 1], axis=1).reshape(-1)
    A = grouped_gemm_fwd(X, W, m_sizes, gather, None, topk, flags, rows=rows, cols=wc)
    return gated_silu(A)
