"""token_routing_amd -- MoE grouped GEMM on AMD MI355X (gfx950).

A thin ctypes binding over libmoegg.so (``include/moegg.h``).  The functions
here have the C entry points' names and only marshal arguments: every step
of routing and every GEMM runs in the library's HIP kernels.  PyTorch is used
for device memory and the current stream; outputs that the caller does not
pass are allocated with torch.

There is no fallback: if libmoegg.so is missing or fails to load, the first
call raises OSError, and every call raises MoeggError on a non-OK status.
"""

from __future__ import annotations

import ctypes
import os

import torch

PERMUTE_X = 1
PERMUTE_Y = 2
FUSE_MUL_POST = 4
DW_FP32_OUT = 8
GATED_SILU = 32

DERR_EXPERT_ID = 1
DERR_M_SIZES = 2
DERR_GATHER = 4

MAX_EXPERTS = 1024
MAX_GROUPS = 16

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoegg.so")

STATUS = {0: "OK", 1: "EINVAL", 2: "ESHAPE", 3: "EUNSUPPORTED", 4: "EWORKSPACE", 5: "EHIP"}


class MoeggError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_status_string(status)})")


class MoeggGroup(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("w", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("m", ctypes.c_int32), ("n", ctypes.c_int32), ("k", ctypes.c_int32),
                ("ldx", ctypes.c_int32), ("ldw", ctypes.c_int32), ("ldy", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoegg.so (raises OSError if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError(f"{path} is not built; run `python -m token_routing_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, u32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                             ctypes.c_size_t)
    lib.moegg_status_string.argtypes = [ctypes.c_int]
    lib.moegg_status_string.restype = ctypes.c_char_p
    lib.moegg_version.argtypes = []
    lib.moegg_version.restype = i32
    lib.moegg_route_workspace_bytes.argtypes = [i64, i32]
    lib.moegg_route_workspace_bytes.restype = sz
    lib.moegg_route.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
    lib.moegg_route.restype = ctypes.c_int
    lib.moegg_route_noalloc.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.moegg_route_noalloc.restype = ctypes.c_int
    lib.moegg_grouped_gemm_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, u32, vp,
                                           vp, vp]
    lib.moegg_grouped_gemm_fwd.restype = ctypes.c_int
    lib.moegg_grouped_gemm_dX.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, u32, vp, vp,
                                          sz, vp, vp]
    lib.moegg_grouped_gemm_dX.restype = ctypes.c_int
    lib.moegg_grouped_gemm_dX_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.moegg_grouped_gemm_dX_workspace_bytes.restype = sz
    lib.moegg_grouped_gemm_dW.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, u32, vp, vp,
                                          sz, vp, vp]
    lib.moegg_grouped_gemm_dW.restype = ctypes.c_int
    lib.moegg_grouped_gemm_dW_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.moegg_grouped_gemm_dW_workspace_bytes.restype = sz
    lib.moegg_grouped_gemm_dW_gather_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.moegg_grouped_gemm_dW_gather_workspace_bytes.restype = sz
    lib.moegg_grouped_gemm_groups.argtypes = [ctypes.POINTER(MoeggGroup), i32, i32, vp]
    lib.moegg_grouped_gemm_groups.restype = ctypes.c_int
    lib.moegg_combine.argtypes = [vp, vp, vp, i64, i32, i32, i64, u32, vp, vp, vp]
    lib.moegg_combine.restype = ctypes.c_int
    lib.moegg_combine_bwd.argtypes = [vp, vp, vp, vp, i64, i32, i32, i64, vp, vp, vp, vp]
    lib.moegg_combine_bwd.restype = ctypes.c_int
    _lib = lib
    return lib


def _status_string(status: int) -> str:
    try:
        return load_library().moegg_status_string(status).decode()
    except OSError:
        return "library not loaded"


def _check(status: int, what: str) -> None:
    if status != 0:
        raise MoeggError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _device_tensor(t, dtype, name):
    if t is None:
        return None
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")
    return t


def route_workspace_bytes(num_slots: int, num_experts: int) -> int:
    return int(load_library().moegg_route_workspace_bytes(num_slots, num_experts))


def moe_route(topk_ids: torch.Tensor, num_experts: int, block_m: int = 128, *, out=None,
              workspace=None, error_flags=None, stream=None):
    """Expert histogram, offsets and stable gather/scatter indices (moegg_route).

    topk_ids: int32 CUDA tensor [T, topk] (or [S]).  Returns a dict of int32
    CUDA tensors m_sizes [E], offsets / padded_offsets / tile_offsets [E+1],
    gather [S], scatter [S].
    """
    lib = load_library()
    ids = _device_tensor(topk_ids, torch.int32, "topk_ids")
    topk = ids.shape[-1] if ids.dim() == 2 else 1
    T = ids.numel() // topk
    S, E = T * topk, int(num_experts)
    dev = ids.device
    if out is None:
        out = {"m_sizes": torch.empty(E, dtype=torch.int32, device=dev),
               "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
               "padded_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
               "tile_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
               "gather": torch.empty(S, dtype=torch.int32, device=dev),
               "scatter": torch.empty(S, dtype=torch.int32, device=dev)}
    need = route_workspace_bytes(S, E)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(lib.moegg_route(
        _ptr(ids), T, topk, E, int(block_m), _ptr(out["m_sizes"]), _ptr(out["offsets"]),
        _ptr(out.get("padded_offsets")), _ptr(out.get("tile_offsets")), _ptr(out["gather"]),
        _ptr(out.get("scatter")), _ptr(workspace), workspace.numel(), _ptr(error_flags),
        _stream(stream)), "moegg_route")
    return out


ROUTE_NOALLOC_MAX_BYTES = 1 << 20


def moe_route_noalloc(topk_ids: torch.Tensor, num_experts: int, block_m: int = 128, *, out,
                      error_flags=None, stream=None):
    """moe_route without a workspace (moegg_route_noalloc): the library keeps
    the per-chunk counts in its own static device array, so the call
    allocates nothing.  `out` holds the output tensors, as moe_route returns
    them (m_sizes and offsets required; padded_offsets, tile_offsets and
    scatter optional); calls that overlap on one GPU race."""
    lib = load_library()
    ids = _device_tensor(topk_ids, torch.int32, "topk_ids")
    topk = ids.shape[-1] if ids.dim() == 2 else 1
    T = ids.numel() // topk
    _check(lib.moegg_route_noalloc(
        _ptr(ids), T, topk, int(num_experts), int(block_m), _ptr(out["m_sizes"]),
        _ptr(out["offsets"]), _ptr(out.get("padded_offsets")), _ptr(out.get("tile_offsets")),
        _ptr(out["gather"]), _ptr(out.get("scatter")), _ptr(error_flags), _stream(stream)),
        "moegg_route_noalloc")
    return out


def grouped_gemm_fwd(X, W, m_sizes, gather_idx, topk_weights, topk: int, flags: int, *,
                     Y=None, error_flags=None, stream=None):
    """Y = grouped X W_e^T with the permute_x / permute_y / fuse_mul_post fusions.

    X: bf16 [T, K] (PERMUTE_X) or [T*topk, K]; W: bf16 [E, N, K]; m_sizes int32
    [E]; gather_idx int32 [T*topk]; topk_weights fp32 [T*topk] (slot order).
    Returns Y bf16 [T*topk, N], or [T*topk, N/2] with GATED_SILU (W rows in
    (gate, linear) pairs).
    """
    lib = load_library()
    E, N, K = W.shape
    S = gather_idx.numel() if gather_idx is not None else X.shape[0]
    T = S // topk
    if Y is None:
        Y = torch.empty(S, N // 2 if (flags & GATED_SILU) else N, dtype=torch.bfloat16,
                        device=X.device)
    _check(lib.moegg_grouped_gemm_fwd(
        _ptr(_device_tensor(X, torch.bfloat16, "X")), _ptr(_device_tensor(W, torch.bfloat16, "W")),
        _ptr(_device_tensor(m_sizes, torch.int32, "m_sizes")),
        _ptr(_device_tensor(gather_idx, torch.int32, "gather_idx")),
        _ptr(_device_tensor(topk_weights, torch.float32, "topk_weights")), T, topk, E, N, K,
        int(flags), _ptr(_device_tensor(Y, torch.bfloat16, "Y")), _ptr(error_flags),
        _stream(stream)), "moegg_grouped_gemm_fwd")
    return Y

def dx_workspace_bytes(num_tokens: int, topk: int, num_experts: int, N: int, K: int) -> int:
    """Workspace bytes that let grouped_gemm_dX balance its last round (current device)."""
    return int(load_library().moegg_grouped_gemm_dX_workspace_bytes(num_tokens, topk,
                                                                       num_experts, N, K))


def _workspace(need: int, workspace, device):
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace is None:
        return None, 0
    workspace = _device_tensor(workspace, torch.uint8, "workspace")
    return workspace, workspace.numel()


def grouped_gemm_dX(dY, W, m_sizes, gather_idx, topk: int, flags: int, *, dX=None,
                    workspace=None, split: bool = True, error_flags=None, stream=None):
    """dX = grouped dY_e W_e; flags are the forward's permute flags. Returns bf16 [S, K].

    split: let the library balance the last round of tiles (fp32 partials in
    `workspace`, a uint8 CUDA tensor of dx_workspace_bytes(...) bytes,
    allocated here when not given).  split=False passes no workspace.
    """
    lib = load_library()
    E, N, K = W.shape
    S = dY.shape[0]
    if dX is None:
        dX = torch.empty(S, K, dtype=torch.bfloat16, device=dY.device)
    need = dx_workspace_bytes(S // topk, topk, E, N, K) if split else 0
    ws, ws_bytes = _workspace(need, workspace if split else None, dY.device)
    _check(lib.moegg_grouped_gemm_dX(
        _ptr(_device_tensor(dY, torch.bfloat16, "dY")), _ptr(_device_tensor(W, torch.bfloat16, "W")),
        _ptr(_device_tensor(m_sizes, torch.int32, "m_sizes")),
        _ptr(_device_tensor(gather_idx, torch.int32, "gather_idx")), S // topk, topk, E, N, K,
        int(flags), _ptr(_device_tensor(dX, torch.bfloat16, "dX")), _ptr(ws), ws_bytes,
        _ptr(error_flags), _stream(stream)), "moegg_grouped_gemm_dX")
    return dX

def dw_workspace_bytes(num_tokens: int, topk: int, num_experts: int, N: int, K: int) -> int:
    """Workspace bytes that let grouped_gemm_dW split hot experts' reductions (0: none)."""
    return int(load_library().moegg_grouped_gemm_dW_workspace_bytes(num_tokens, topk,
                                                                       num_experts, N, K))


def dw_gather_workspace_bytes(num_tokens: int, topk: int, num_experts: int, N: int,
                              K: int) -> int:
    """Workspace bytes with which grouped_gemm_dW under PERMUTE_X also copies X's rows
    into expert order before the reduction (the split area plus S * K * 2)."""
    return int(load_library().moegg_grouped_gemm_dW_gather_workspace_bytes(
        num_tokens, topk, num_experts, N, K))


def grouped_gemm_dW(X, dY, m_sizes, gather_idx, topk: int, flags: int, *, dW=None,
                    workspace=None, split: bool = True, error_flags=None, stream=None):
    """dW[e] = dY_e^T X_e (ragged per expert). Returns [E, N, K] bf16 (fp32 with DW_FP32_OUT).

    split: pass the library a workspace (`workspace`, a uint8 CUDA tensor,
    allocated here when not given: dw_gather_workspace_bytes(...) bytes under
    PERMUTE_X, else dw_workspace_bytes(...)).  It cuts hot experts'
    reductions into chunks with fp32 partials there and, under PERMUTE_X
    with room for them, copies X's rows into expert order first.
    split=False passes no workspace: one launch, rows gathered inside it.
    """
    lib = load_library()
    S, N = dY.shape
    K = X.shape[1]
    E = m_sizes.numel()
    if dW is None:
        dt = torch.float32 if (flags & DW_FP32_OUT) else torch.bfloat16
        dW = torch.empty(E, N, K, dtype=dt, device=dY.device)
    ws_bytes = 0
    if not split:
        workspace = None
    elif workspace is None:
        if flags & PERMUTE_X:
            need = dw_gather_workspace_bytes(S // topk, topk, E, N, K)
        else:
            need = dw_workspace_bytes(S // topk, topk, E, N, K)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dY.device)
    if workspace is not None:
        workspace = _device_tensor(workspace, torch.uint8, "workspace")
        ws_bytes = workspace.numel()
    _check(lib.moegg_grouped_gemm_dW(
        _ptr(_device_tensor(X, torch.bfloat16, "X")), _ptr(_device_tensor(dY, torch.bfloat16, "dY")),
        _ptr(_device_tensor(m_sizes, torch.int32, "m_sizes")),
        _ptr(_device_tensor(gather_idx, torch.int32, "gather_idx")), S // topk, topk, E, N, K,
        int(flags), _ptr(dW), _ptr(workspace), ws_bytes, _ptr(error_flags), _stream(stream)),
        "moegg_grouped_gemm_dW")
    return dW


def grouped_gemm_groups(groups, trans_b: int = 0, *, outputs=None, stream=None):
    """Independent GEMMs y_g = x_g @ w_g in one launch.

    groups: list of (x [m, k], w [k, n] (trans_b=0) or [n, k] (trans_b=1)) bf16
    CUDA tensors.  Returns the list of y [m, n] bf16.
    """
    lib = load_library()
    if not 1 <= len(groups) <= MAX_GROUPS:
        raise ValueError("1..16 groups")
    arr = (MoeggGroup * len(groups))()
    ys = []
    for i, (x, w) in enumerate(groups):
        for t, name in ((x, "x"), (w, "w")):
            if not t.is_cuda or t.dtype != torch.bfloat16 or t.dim() != 2 or t.stride(1) != 1:
                raise ValueError(f"group {i}: {name} must be a row-major bf16 CUDA matrix")
        m, k = x.shape
        n = w.shape[0] if trans_b else w.shape[1]
        y = outputs[i] if outputs is not None else torch.empty(m, n, dtype=torch.bfloat16,
                                                               device=x.device)
        ys.append(y)
        arr[i] = MoeggGroup(x.data_ptr(), w.data_ptr(), y.data_ptr(), m, n, k, x.stride(0),
                            w.stride(0), y.stride(0))
    _check(lib.moegg_grouped_gemm_groups(arr, len(groups), int(trans_b), _stream(stream)),
           "moegg_grouped_gemm_groups")
    return ys


COMBINE_FP32_OUT = 16


def combine(Y, topk: int, scatter_idx=None, topk_weights=None, *, num_tokens=None,
            fp32_out: bool = False, out=None, error_flags=None, stream=None):
    """Top-k combine (moegg_combine): out[t] = sum_j w[t*k+j] * Y[row(t*k+j)].

    Y: bf16 [rows, N]; scatter_idx: int32 [T*k] (Y in expert-sorted order) or
    None (Y in slot order); topk_weights: float32 [T*k] or None (weight 1).
    Returns out [T, N], bf16 (fp32 with fp32_out).
    """
    lib = load_library()
    Y = _device_tensor(Y, torch.bfloat16, "Y")
    scatter_idx = _device_tensor(scatter_idx, torch.int32, "scatter_idx")
    topk_weights = _device_tensor(topk_weights, torch.float32, "topk_weights")
    S = scatter_idx.numel() if scatter_idx is not None else Y.shape[0]
    T = S // topk if num_tokens is None else int(num_tokens)
    N = Y.shape[1]
    if out is None:
        out = torch.empty(T, N, dtype=torch.float32 if fp32_out else torch.bfloat16,
                          device=Y.device)
    _check(lib.moegg_combine(_ptr(Y), _ptr(scatter_idx), _ptr(topk_weights), T, topk, N,
                             Y.shape[0], COMBINE_FP32_OUT if fp32_out else 0, _ptr(out),
                             _ptr(error_flags), _stream(stream)), "moegg_combine")
    return out


def combine_bwd(dOut, Y, topk: int, scatter_idx=None, topk_weights=None, *, want_dw=True,
                dY=None, dw=None, error_flags=None, stream=None):
    """Backward of combine (moegg_combine_bwd): returns (dY bf16 [rows, N], dw float32 [T*k]
    or None).  Y (the forward input) is read only for dw."""
    lib = load_library()
    dOut = _device_tensor(dOut, torch.bfloat16, "dOut")
    Y = _device_tensor(Y, torch.bfloat16, "Y")
    scatter_idx = _device_tensor(scatter_idx, torch.int32, "scatter_idx")
    topk_weights = _device_tensor(topk_weights, torch.float32, "topk_weights")
    T, N = dOut.shape
    rows = Y.shape[0] if Y is not None else T * topk
    if dY is None:
        dY = torch.empty(rows, N, dtype=torch.bfloat16, device=dOut.device)
    if want_dw and dw is None:
        dw = torch.empty(T * topk, dtype=torch.float32, device=dOut.device)
    _check(lib.moegg_combine_bwd(_ptr(dOut), _ptr(Y), _ptr(scatter_idx), _ptr(topk_weights), T,
                                 topk, N, rows, _ptr(dY), _ptr(dw if want_dw else None),
                                 _ptr(error_flags), _stream(stream)), "moegg_combine_bwd")
    return dY, (dw if want_dw else None)
