"""GPU parity of the any-shape path: sizes whose rows are not whole 16-byte
chunks (K, N, a group's n, k or leading dimension not a multiple of 8) and
operands that are only 2-byte aligned.  The pages put no condition on these
sizes; the library sends such calls to its any-shape kernels.

Each case is compared with the oracle to the same bar as the tiled kernels
(bf16: relative Frobenius <= 5e-3 and |y - ref| <= 3e-2 * max(1, |ref|);
fp32 dW: 1e-5 relative Frobenius), including ragged experts, empty experts,
every permute flag, the gate multiply, the gated activation, the explicit
groups (with the (m, n, k) = (1000, 700, 2) shape) and the top-k combine.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._util import bf16_tolerance_ok, gamma, widen

pytestmark = pytest.mark.gpu

PX, PY, FM = synth.PERMUTE_X, synth.PERMUTE_Y, synth.FUSE_MUL_POST
GS = 32  # MOEGG_GATED_SILU


@pytest.fixture(scope="module")
def mg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_routing_amd as m
    m.load_library()
    return m


def _dev(t):
    return t.to("cuda").contiguous()


def _shifted(t):
    """A contiguous CUDA copy of t whose data starts 2 bytes past a 16-byte
    boundary (a view into a larger buffer)."""
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device="cuda")
    v = flat[1:1 + t.numel()].view(t.shape)
    v.copy_(t.to("cuda"))
    assert v.is_contiguous() and v.data_ptr() % 16 == 2
    return v


def _check(got, ref, what, **kw):
    got = got.float().cpu().numpy() if isinstance(got, torch.Tensor) else got
    ok, info = bf16_tolerance_ok(got, ref, **kw)
    print(f"{what}: {info}", flush=True)
    assert ok, (what, info)


def _routes(mg, wl):
    r = mg.moe_route(_dev(wl.ids), wl.E, 128)
    ref = oracle.route(wl.ids.numpy().reshape(-1), wl.E, 128)
    assert np.array_equal(r["gather"].cpu().numpy(), ref["gather"])
    return r, ref


ODD = [
    # T, K, N, E, topk, seed, empty  -- K and N not multiples of 8
    (50, 70, 45, 5, 2, 51, (3,)),         # ragged experts, N and K tails inside a 32-block
    (33, 2, 700, 40, 8, 52, (1, 5, 39)),  # K = 2, many empty experts
    (130, 137, 33, 3, 3, 53, ()),         # more than one 32-row block per expert
]
IDS = [f"T{c[0]}K{c[1]}N{c[2]}E{c[3]}k{c[4]}" for c in ODD]


@pytest.mark.parametrize("flags", [0, PX, PY, PY | FM], ids=["plain", "px", "py", "py_fm"])
@pytest.mark.parametrize("case", ODD, ids=IDS)
def test_fwd_any_shape(mg, flags, case):
    T, K, N, E, topk, seed, empty = case
    wl = synth.random_case(T, K, N, E, topk, flags, seed, empty=empty)
    r, ref_route = _routes(mg, wl)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    Y = mg.grouped_gemm_fwd(_dev(wl.X), _dev(wl.W), r["m_sizes"], r["gather"],
                            _dev(wl.weights.reshape(-1)), wl.topk, flags, error_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref = oracle.grouped_gemm_fwd(synth.bits(wl.X), synth.bits(wl.W), ref_route["m_sizes"],
                                  ref_route["gather"], wl.weights.numpy().reshape(-1), wl.topk,
                                  flags)
    _check(Y, ref, f"fwd {case} flags={flags}")


GATED = [(50, 70, 46, 5, 2, 54, (3,)), (40, 64, 40, 4, 4, 55, ())]  # N/2 odd; N = 40


@pytest.mark.parametrize("flags", [0, PX], ids=["plain", "px"])
@pytest.mark.parametrize("case", GATED, ids=[f"T{c[0]}K{c[1]}N{c[2]}" for c in GATED])
def test_gated_any_shape(mg, flags, case):
    T, K, N, E, topk, seed, empty = case
    wl = synth.random_case(T, K, N, E, topk, flags, seed, empty=empty)
    r, ref_route = _routes(mg, wl)
    Y = mg.grouped_gemm_fwd(_dev(wl.X), _dev(wl.W), r["m_sizes"], r["gather"], None, wl.topk,
                            flags | GS)
    torch.cuda.synchronize()
    assert tuple(Y.shape) == (wl.S, N // 2)
    ref = oracle.grouped_gemm_fwd_gated(synth.bits(wl.X), synth.bits(wl.W), ref_route["m_sizes"],
                                        ref_route["gather"], wl.topk, flags)
    _check(Y, ref, f"gated {case} flags={flags}")


@pytest.mark.parametrize("flags", [0, PX, PY], ids=["plain", "px", "py"])
@pytest.mark.parametrize("case", ODD, ids=IDS)
def test_bwd_any_shape(mg, flags, case):
    T, K, N, E, topk, seed, empty = case
    wl = synth.random_case(T, K, N, E, topk, flags, seed, empty=empty, with_dy=True)
    r, ref_route = _routes(mg, wl)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dX = mg.grouped_gemm_dX(_dev(wl.dY), _dev(wl.W), r["m_sizes"], r["gather"], wl.topk, flags,
                            error_flags=err)
    dW = mg.grouped_gemm_dW(_dev(wl.X), _dev(wl.dY), r["m_sizes"], r["gather"], wl.topk, flags,
                            error_flags=err)
    dW32 = mg.grouped_gemm_dW(_dev(wl.X), _dev(wl.dY), r["m_sizes"], r["gather"], wl.topk,
                              flags | mg.DW_FP32_OUT, error_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref_dx = oracle.grouped_gemm_dX(synth.bits(wl.dY), synth.bits(wl.W), ref_route["m_sizes"],
                                    ref_route["gather"], wl.topk, flags)
    ref_dw = oracle.grouped_gemm_dW(synth.bits(wl.X), synth.bits(wl.dY), ref_route["m_sizes"],
                                    ref_route["gather"], wl.topk, flags, E)
    _check(dX, ref_dx, f"dX {case} flags={flags}")
    _check(dW.reshape(E * N, K), ref_dw, f"dW {case} flags={flags}")
    _check(dW32.reshape(E * N, K), ref_dw, f"dW fp32 {case} flags={flags}", rel_fro_max=1e-5,
           max_elem=1e-4)
    for e in np.nonzero(ref_route["m_sizes"] == 0)[0]:
        assert torch.count_nonzero(dW[int(e)]).item() == 0


def test_aligned_sizes_with_unaligned_operands(mg):
    """K and N multiples of 8 but operands 2 bytes past a 16-byte boundary:
    the any-shape path, same results as the tiled one within the bar."""
    wl = synth.random_case(60, 72, 136, 4, 2, PX, 56, empty=(1,), with_dy=True)
    r, ref_route = _routes(mg, wl)
    E, N, K = wl.W.shape
    Y = mg.grouped_gemm_fwd(_shifted(wl.X), _dev(wl.W), r["m_sizes"], r["gather"], None, wl.topk,
                            PX)
    dX = mg.grouped_gemm_dX(_shifted(wl.dY), _dev(wl.W), r["m_sizes"], r["gather"], wl.topk, PX)
    dW = mg.grouped_gemm_dW(_dev(wl.X), _shifted(wl.dY), r["m_sizes"], r["gather"], wl.topk, PX)
    torch.cuda.synchronize()
    rr, rg = ref_route["m_sizes"], ref_route["gather"]
    _check(Y, oracle.grouped_gemm_fwd(synth.bits(wl.X), synth.bits(wl.W), rr, rg, None, wl.topk,
                                      PX), "fwd shifted")
    _check(dX, oracle.grouped_gemm_dX(synth.bits(wl.dY), synth.bits(wl.W), rr, rg, wl.topk, PX),
           "dX shifted")
    _check(dW.reshape(E * N, K), oracle.grouped_gemm_dW(synth.bits(wl.X), synth.bits(wl.dY), rr,
                                                        rg, wl.topk, PX, E), "dW shifted")


def test_any_shape_bad_gather_is_flagged(mg):
    wl = synth.random_case(20, 70, 45, 3, 2, PX, 57, with_dy=True)
    r, _ = _routes(mg, wl)
    bad = r["gather"].clone()
    bad[3] = 10 ** 6
    for call in ("fwd", "dX", "dW"):
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        if call == "fwd":
            mg.grouped_gemm_fwd(_dev(wl.X), _dev(wl.W), r["m_sizes"], bad, None, 2, PX,
                                error_flags=err)
        elif call == "dX":
            mg.grouped_gemm_dX(_dev(wl.dY), _dev(wl.W), r["m_sizes"], bad, 2, PX, error_flags=err)
        else:
            mg.grouped_gemm_dW(_dev(wl.X), _dev(wl.dY), r["m_sizes"], bad, 2, PX, error_flags=err)
        torch.cuda.synchronize()
        assert int(err.item()) & mg.DERR_GATHER, call


@pytest.mark.parametrize("trans_b", [0, 1])
def test_groups_any_shape(mg, trans_b):
    """Groups with odd sizes, including (m, n, k) = (1000, 700, 2), beside an
    aligned group (one launch takes one path for all of its groups)."""
    g = synth.generator(58)
    shapes = [(1000, 2, 700), (37, 45, 13), (0, 8, 8), (64, 64, 64)]  # (m, k, n)
    xs = [synth.normal_bf16((m, k), 0.5, g) for m, k, n in shapes]
    ws = [synth.normal_bf16((k, n), 0.5, g) for m, k, n in shapes]
    pairs = [(_dev(x), _dev(w if trans_b == 0 else w.t().contiguous())) for x, w in zip(xs, ws)]
    ys = mg.grouped_gemm_groups(pairs, trans_b=trans_b)
    torch.cuda.synchronize()
    for (m, k, n), x, w, y in zip(shapes, xs, ws, ys):
        if m == 0:
            continue
        _check(y, oracle.dense_gemm_kn(synth.bits(x), synth.bits(w)), f"group {m}x{k}x{n}")


COMBINE = [(37, 2, 45, 5, 61), (64, 8, 700, 16, 62), (5, 1, 3, 3, 63)]


@pytest.mark.parametrize("case", COMBINE, ids=[f"T{c[0]}k{c[1]}N{c[2]}" for c in COMBINE])
def test_combine_any_n(mg, case):
    T, topk, N, E, seed = case
    g = synth.generator(seed)
    ids, w = synth.random_routing(T, E, topk, g, ())
    w = w.reshape(-1).contiguous()
    Y = synth.normal_bf16((T * topk, N), 1.0, g)
    dOut = synth.normal_bf16((T, N), 0.1, g)
    sc = oracle.route(ids.numpy().reshape(-1), E, 16)["scatter"]
    ref = oracle.combine(synth.bits(Y), topk, scatter=sc, weights=w.numpy())
    out = mg.combine(Y.cuda(), topk, torch.from_numpy(sc).cuda(), w.cuda())
    out32 = mg.combine(Y.cuda(), topk, torch.from_numpy(sc).cuda(), w.cuda(), fp32_out=True)
    dY_ref, dw_ref = oracle.combine_bwd(synth.bits(dOut), synth.bits(Y), topk, scatter=sc,
                                        weights=w.numpy())
    dY, dw = mg.combine_bwd(dOut.cuda(), Y.cuda(), topk, torch.from_numpy(sc).cuda(), w.cuda())
    torch.cuda.synchronize()
    _check(out, ref, f"combine {case}")
    Yw, Gw = widen(synth.bits(Y)), widen(synth.bits(dOut))
    absref = np.zeros((T, N))
    for s in range(T * topk):
        absref[s // topk] += abs(float(w[s])) * np.abs(Yw[sc[s]])
    err = np.abs(out32.cpu().numpy().astype(np.float64) - ref)
    assert np.all(err <= 2 * gamma(topk) * (absref + np.abs(ref)) + 1e-30)
    _check(dY, dY_ref, f"combine dY {case}")
    absdot = np.array([np.sum(np.abs(Gw[s // topk]) * np.abs(Yw[sc[s]])) for s in range(T * topk)])
    err = np.abs(dw.cpu().numpy().astype(np.float64) - dw_ref)
    assert np.all(err <= 2 * gamma(N) * (absdot + np.abs(dw_ref)) + 1e-30)


def test_any_shape_many_blocks(mg):
    """A mid-size odd shape (many 32 x 32 blocks per expert and many waves
    per workgroup loop): T 1024, top-2 over 8 experts, K 1000, N 1001, on
    sampled rows against the oracle."""
    wl = synth.random_case(1024, 1000, 1001, 8, 2, PX, 59, empty=(5,), with_dy=True)
    r, ref_route = _routes(mg, wl)
    E, N, K = wl.W.shape
    rows = np.unique(np.concatenate([np.arange(0, wl.S, 97), [wl.S - 1]]))
    Y = mg.grouped_gemm_fwd(_dev(wl.X), _dev(wl.W), r["m_sizes"], r["gather"], None, wl.topk, PX)
    dX = mg.grouped_gemm_dX(_dev(wl.dY), _dev(wl.W), r["m_sizes"], r["gather"], wl.topk, PX)
    dW = mg.grouped_gemm_dW(_dev(wl.X), _dev(wl.dY), r["m_sizes"], r["gather"], wl.topk, PX)
    torch.cuda.synchronize()
    rr, rg = ref_route["m_sizes"], ref_route["gather"]
    sel = torch.as_tensor(rows, dtype=torch.long, device="cuda")
    _check(Y[sel], oracle.grouped_gemm_fwd(synth.bits(wl.X), synth.bits(wl.W), rr, rg, None,
                                          wl.topk, PX, rows=rows), "fwd 1024x1000x1001")
    _check(dX[sel], oracle.grouped_gemm_dX(synth.bits(wl.dY), synth.bits(wl.W), rr, rg, wl.topk,
                                          PX, rows=rows), "dX 1024x1000x1001")
    wrows = np.unique(np.concatenate([np.arange(0, E * N, 131), [E * N - 1]]))
    wsel = torch.as_tensor(wrows, dtype=torch.long, device="cuda")
    _check(dW.reshape(E * N, K)[wsel], oracle.grouped_gemm_dW(
        synth.bits(wl.X), synth.bits(wl.dY), rr, rg, wl.topk, PX, E, rows=wrows),
        "dW 1024x1000x1001")
    assert torch.count_nonzero(dW[5]).item() == 0
