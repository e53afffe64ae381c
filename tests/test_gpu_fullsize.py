"""Every output element of the Mixtral-shaped step (forward with permute_x,
dX scattered to slot order, dW), at full size and in the launch
configuration bench.py times, against per-expert fp32 products computed by
torch on the GPU.

This complements the oracle parity tests, which check these workloads on
sampled rows and columns: here no tile of the 256 x 256 grid is left out.
The routing comes from the CPU oracle.  The reference is X_e W_e^T, dY_e W_e
and dY_e^T X_e for each expert's rows, in fp32 (torch.matmul on 2-D
contiguous operands).  The bar is the bf16-output tolerance of the parity
tests, computed in float64 on the GPU: relative Frobenius error <= 5e-3 and
|y - ref| <= 3e-2 * max(1, |ref|) elementwise.
"""

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_routing_amd as m
    m.load_library()
    return m


class _Tol:
    """Accumulates the tolerance terms over blocks of one output."""

    def __init__(self):
        self.err2 = 0.0
        self.ref2 = 0.0
        self.worst = -1.0

    def add(self, got, ref):
        got, ref = got.double(), ref.double()
        d = got - ref
        self.err2 += float((d * d).sum())
        self.ref2 += float((ref * ref).sum())
        lim = 3e-2 * torch.clamp(ref.abs(), min=1.0)
        self.worst = max(self.worst, float((d.abs() - lim).max()))

    def check(self, what):
        rf = (self.err2 / self.ref2) ** 0.5
        assert rf <= 5e-3 and self.worst <= 0.0, f"{what}: rel_fro {rf:.3e}, worst {self.worst:.3e}"


def test_mixtral_step_every_element(mg):
    wl = synth.mixtral()
    E, N, K = wl.W.shape
    S, topk = wl.S, wl.topk
    dY = synth.normal_bf16((S, N), 0.01, synth.generator(synth.SEEDS["mixtral_bwd_dy"])).cuda()
    X, W = wl.X.cuda(), wl.W.cuda()
    route = oracle.route(wl.ids.numpy().reshape(-1), E, 128)
    gather = torch.from_numpy(route["gather"]).cuda()
    m_sizes = torch.from_numpy(route["m_sizes"]).cuda()
    off = route["offsets"]

    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    Y = mg.grouped_gemm_fwd(X, W, m_sizes, gather, None, topk, synth.PERMUTE_X, error_flags=err)
    dX = mg.grouped_gemm_dX(dY, W, m_sizes, gather, topk, synth.PERMUTE_X, error_flags=err)
    dW = mg.grouped_gemm_dW(X, dY, m_sizes, gather, topk, synth.PERMUTE_X, error_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0

    ty, tdx, tdw = _Tol(), _Tol(), _Tol()
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        assert hi > lo
        slots = gather[lo:hi].long()
        Xe = X[slots // topk].float().contiguous()      # the expert's token rows
        We = W[e].float().contiguous()                  # [N, K]
        dYe = dY[lo:hi].float().contiguous()            # sorted order (no permute_y)
        ty.add(Y[lo:hi], Xe @ We.t().contiguous())
        tdx.add(dX[slots], dYe @ We)
        tdw.add(dW[e], dYe.t().contiguous() @ Xe)
        del Xe, We, dYe
    ty.check("forward")
    tdx.check("dX")
    tdw.check("dW")
    assert np.sum(route["m_sizes"]) == S


def test_fine_step_every_element(mg):
    """The fine-grained down projection in a training step (128 experts, Zipf
    routing with empty and hot experts): forward with permute_y, then dX and
    dW with dY gathered on load (hot experts split through the workspace).
    The gate multiply is not part of a training forward; the forward with
    fuse_mul_post is checked on the same routing as well."""
    wl = synth.fine_bwd()
    E, N, K = wl.W.shape
    S, topk = wl.S, wl.topk
    flags = wl.flags
    bflags = flags & (synth.PERMUTE_X | synth.PERMUTE_Y)
    assert flags & synth.PERMUTE_Y and not flags & synth.PERMUTE_X
    dY = synth.normal_bf16((S, N), 0.01, synth.generator(synth.SEEDS["fine_bwd_dy"])).cuda()
    X, W = wl.X.cuda(), wl.W.cuda()
    w = wl.weights.reshape(-1).cuda()
    route = oracle.route(wl.ids.numpy().reshape(-1), E, 128)
    gather = torch.from_numpy(route["gather"]).cuda()
    m_sizes = torch.from_numpy(route["m_sizes"]).cuda()
    off = route["offsets"]

    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    Y = mg.grouped_gemm_fwd(X, W, m_sizes, gather, w, topk, flags, error_flags=err)
    Yg = mg.grouped_gemm_fwd(X, W, m_sizes, gather, w, topk, flags | synth.FUSE_MUL_POST,
                             error_flags=err)
    dX = mg.grouped_gemm_dX(dY, W, m_sizes, gather, topk, bflags, error_flags=err)
    dW = mg.grouped_gemm_dW(X, dY, m_sizes, gather, topk, bflags, error_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0

    ty, tyg, tdx, tdw = _Tol(), _Tol(), _Tol(), _Tol()
    empty = 0
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            assert torch.count_nonzero(dW[e]).item() == 0
            empty += 1
            continue
        slots = gather[lo:hi].long()
        Xe = X[lo:hi].float().contiguous()              # already in sorted order
        We = W[e].float().contiguous()
        dYe = dY[slots].float().contiguous()            # gathered on load
        ye = Xe @ We.t().contiguous()
        ty.add(Y[slots], ye)
        tyg.add(Yg[slots], ye * w[slots].float()[:, None])
        del ye
        tdx.add(dX[lo:hi], dYe @ We)
        tdw.add(dW[e], dYe.t().contiguous() @ Xe)
        del Xe, We, dYe
    assert empty > 0
    ty.check("forward")
    tyg.check("forward with fuse_mul_post")
    tdx.check("dX")
    tdw.check("dW")
