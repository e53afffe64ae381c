"""GPU parity of the top-k combine and its backward (moegg_combine,
moegg_combine_bwd) against the oracle, through the C ABI.

bf16 outputs meet the GEMMs' bar (relative Frobenius <= 5e-3, elementwise
<= 3e-2 * max(1, |ref|)); fp32 outputs and the weight gradient are held to
the fp32 summation bound of their own sums (the GPU adds in another order).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._util import bf16_tolerance_ok, gamma, widen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_routing_amd as m
    m.load_library()
    return m


def _inputs(T, topk, N, E, seed, rows_extra=0):
    g = synth.generator(seed)
    ids, w = synth.random_routing(T, E, topk, g, ())
    S = T * topk
    Y = synth.normal_bf16((S + rows_extra, N), 1.0, g)
    dOut = synth.normal_bf16((T, N), 0.1, g)
    r = oracle.route(ids.numpy().reshape(-1), E, 16)
    return ids, w.reshape(-1).contiguous(), Y, dOut, r


def _ok(got, ref, what):
    ok, info = bf16_tolerance_ok(got, ref)
    assert ok, f"{what}: {info}"


def _within_sum_bound(got, ref, absref, n, what):
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    bound = 2 * gamma(n) * absref + 1e-30
    assert np.all(err <= bound + 2 * gamma(n) * np.abs(ref)), f"{what}: max excess {np.max(err - bound)}"


CASES = [(37, 2, 136, 5, 41), (64, 8, 520, 16, 42), (5, 1, 8, 3, 43), (200, 4, 1032, 9, 44)]


@pytest.mark.parametrize("sorted_input", [True, False], ids=["sorted", "slot_order"])
@pytest.mark.parametrize("weighted", [True, False], ids=["w", "now"])
@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}k{c[1]}N{c[2]}" for c in CASES])
def test_combine_fwd(mg, case, sorted_input, weighted):
    T, topk, N, E, seed = case
    ids, w, Y, dOut, r = _inputs(T, topk, N, E, seed)
    sc = r["scatter"] if sorted_input else None
    ww = w.numpy() if weighted else None
    ref = oracle.combine(synth.bits(Y), topk, scatter=sc, weights=ww)
    out = mg.combine(Y.cuda(), topk, None if sc is None else torch.from_numpy(sc).cuda(),
                     w.cuda() if weighted else None)
    out32 = mg.combine(Y.cuda(), topk, None if sc is None else torch.from_numpy(sc).cuda(),
                       w.cuda() if weighted else None, fp32_out=True)
    torch.cuda.synchronize()
    _ok(out.float().cpu().numpy(), ref, f"combine {case}")
    # fp32 output: within the fp32 bound of the k-term sum
    rows = sc if sc is not None else np.arange(T * topk)
    absref = np.zeros((T, N))
    for s in range(T * topk):
        absref[s // topk] += abs(float(ww[s]) if weighted else 1.0) * np.abs(widen(synth.bits(Y)[rows[s]]))
    _within_sum_bound(out32.cpu().numpy(), ref, absref, topk, f"combine fp32 {case}")


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}k{c[1]}N{c[2]}" for c in CASES])
def test_combine_bwd(mg, case):
    T, topk, N, E, seed = case
    ids, w, Y, dOut, r = _inputs(T, topk, N, E, seed)
    sc = r["scatter"]
    dY_ref, dw_ref = oracle.combine_bwd(synth.bits(dOut), synth.bits(Y), topk, scatter=sc,
                                        weights=w.numpy())
    dY, dw = mg.combine_bwd(dOut.cuda(), Y.cuda(), topk, torch.from_numpy(sc).cuda(), w.cuda())
    dY_now, none = mg.combine_bwd(dOut.cuda(), Y.cuda(), topk, torch.from_numpy(sc).cuda(),
                                  w.cuda(), want_dw=False)
    torch.cuda.synchronize()
    assert none is None
    _ok(dY.float().cpu().numpy(), dY_ref, f"dY {case}")
    assert torch.equal(dY, dY_now)
    # dw[s] = <dOut[t], Y[row(s)]>: fp32 bound of an N-term dot product
    Yw, Gw = widen(synth.bits(Y)), widen(synth.bits(dOut))
    absdot = np.array([np.sum(np.abs(Gw[s // topk]) * np.abs(Yw[sc[s]])) for s in range(T * topk)])
    _within_sum_bound(dw.cpu().numpy(), dw_ref, absdot, N, f"dw {case}")


def test_combine_dropped_and_bad_rows(mg):
    T, topk, N, E = 20, 2, 64, 4
    ids, w, Y, dOut, r = _inputs(T, topk, N, E, 45, rows_extra=3)
    sc = r["scatter"].copy()
    sc[[1, 7]] = -1                      # dropped slots
    sc[12] = T * topk + 3 + 5            # past y_rows: flagged and skipped
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = mg.combine(Y.cuda(), topk, torch.from_numpy(sc).cuda(), w.cuda(), fp32_out=True,
                     num_tokens=T, error_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == mg.DERR_GATHER
    sc_ref = sc.copy()
    sc_ref[12] = -1
    ref = oracle.combine(synth.bits(Y), topk, scatter=sc_ref, weights=w.numpy())
    _within_sum_bound(out.cpu().numpy(), ref, np.abs(ref) + 1.0, topk, "dropped")
    err.zero_()
    dY = torch.full((Y.shape[0], N), 7.0, dtype=torch.bfloat16, device="cuda")
    dYo, dw = mg.combine_bwd(dOut.cuda(), Y.cuda(), topk, torch.from_numpy(sc).cuda(), w.cuda(),
                             dY=dY, error_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == mg.DERR_GATHER
    dwc = dw.cpu().numpy()
    assert dwc[1] == 0 and dwc[7] == 0 and dwc[12] == 0
    untouched = sorted(set(range(Y.shape[0])) - set(int(x) for x in sc_ref if x >= 0))
    assert torch.all(dYo[untouched] == 7.0)


def test_combine_zero_tokens(mg):
    Y = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    out = mg.combine(Y, 2, None, None, num_tokens=0)
    assert out.shape == (0, 64)


def test_combine_fine_shape(mg):
    # the fine-grained down projection's combine: T 8192, top-8, N 2048, sorted input
    wl = synth.fine_down()
    r = oracle.route(wl.ids.numpy().reshape(-1), wl.E, 128)
    g = synth.generator(46)
    Y = synth.normal_bf16((wl.S, wl.N), 1.0, g)
    dOut = synth.normal_bf16((wl.T, wl.N), 0.1, g)
    w = wl.weights.reshape(-1).contiguous()
    sc = torch.from_numpy(r["scatter"]).cuda()
    out = mg.combine(Y.cuda(), wl.topk, sc, w.cuda())
    dY, dw = mg.combine_bwd(dOut.cuda(), Y.cuda(), wl.topk, sc, w.cuda())
    torch.cuda.synchronize()
    ref = oracle.combine(synth.bits(Y), wl.topk, scatter=r["scatter"], weights=w.numpy())
    _ok(out.float().cpu().numpy(), ref, "combine fine")
    dY_ref, dw_ref = oracle.combine_bwd(synth.bits(dOut), synth.bits(Y), wl.topk,
                                        scatter=r["scatter"], weights=w.numpy())
    _ok(dY.float().cpu().numpy(), dY_ref, "dY fine")
    ok, info = bf16_tolerance_ok(dw.cpu().numpy(), dw_ref, rel_fro_max=1e-5, max_elem=1e-3)
    assert ok, info


@pytest.mark.parametrize("case", [(300, 136, 264, 5, 2, 51), (96, 520, 136, 8, 4, 52)],
                         ids=["T300K136N264k2", "T96K520N136k4"])
def test_first_gemm_backward_token_gradient(mg, case):
    """Backward of the first MoE GEMM (forward with permute_x): dX scattered to
    slot order by moegg_grouped_gemm_dX, then summed over each token's k
    slots by the unweighted combine, gives the gradient of the token rows X."""
    T, K, N, E, topk, seed = case
    wl = synth.random_case(T, K, N, E, topk, synth.PERMUTE_X, seed, with_dy=True)
    r = oracle.route(wl.ids.numpy().reshape(-1), E, 128)
    g = mg.moe_route(wl.ids.cuda(), E, 128)
    dX = mg.grouped_gemm_dX(wl.dY.cuda(), wl.W.cuda(), g["m_sizes"], g["gather"], topk,
                            synth.PERMUTE_X)
    dXt = mg.combine(dX, topk)
    torch.cuda.synchronize()
    assert dXt.shape == (T, K)
    ref_slots = oracle.grouped_gemm_dX(synth.bits(wl.dY), synth.bits(wl.W), r["m_sizes"],
                                       r["gather"], topk, synth.PERMUTE_X)
    ref = ref_slots.astype(np.float64).reshape(T, topk, K).sum(axis=1)
    _ok(dXt.float().cpu().numpy(), ref.astype(np.float32), f"token gradient {case}")
