"""GPU parity of the gate_up forward with the gated SiLU activation fused.

The HIP forward with MOEGG_GATED_SILU (W rows in adjacent (gate, linear)
pairs, output [S, N/2]) against the oracle's grouped forward followed by its
gated activation, to the bf16 tolerance: relative Frobenius error <= 5e-3
and |y - ref| <= 3e-2 * max(1, |ref|).  Small cases cover both tile paths,
ragged tails in every dimension and empty experts; the Mixtral-shaped
gate_up layer is checked on sampled rows and columns.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._util import bf16_tolerance_ok

pytestmark = pytest.mark.gpu

PX = synth.PERMUTE_X
GS = 32  # MOEGG_GATED_SILU


@pytest.fixture(scope="module")
def mg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_routing_amd as mg
    mg.load_library()
    assert mg.GATED_SILU == GS
    return mg


def _dev(t):
    return t.to("cuda").contiguous()


def _gated_case(mg, wl, flags, rows=None, cols=None):
    r = mg.moe_route(_dev(wl.ids), wl.E, 128)
    ref_route = oracle.route(wl.ids.numpy().reshape(-1), wl.E, 128)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    Y = mg.grouped_gemm_fwd(_dev(wl.X), _dev(wl.W), r["m_sizes"], r["gather"], None, wl.topk,
                            flags | GS, error_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert tuple(Y.shape) == (wl.S, wl.N // 2)
    ref = oracle.grouped_gemm_fwd_gated(synth.bits(wl.X), synth.bits(wl.W), ref_route["m_sizes"],
                                        ref_route["gather"], wl.topk, flags, rows=rows, cols=cols)
    got = Y
    if rows is not None:
        got = got[torch.as_tensor(rows, dtype=torch.long, device="cuda")]
    if cols is not None:
        got = got[:, torch.as_tensor(cols, dtype=torch.long, device="cuda")]
    return got.float().cpu().numpy(), ref


def _check(got, ref, what):
    ok, info = bf16_tolerance_ok(got, ref)
    print(f"{what}: {info}", flush=True)
    assert ok, (what, info)


GATED_SMALL = [
    # T, K, N (= 2 x output columns), E, topk, seed, empty
    (300, 320, 528, 5, 2, 21, (3,)),       # avg 120 rows/expert -> large tiles, N tail
    (700, 136, 1040, 6, 3, 22, (0,)),      # K not a multiple of 64
    (64, 256, 512, 16, 4, 23, (2, 9)),     # avg 16 rows -> small tiles
    (33, 64, 272, 40, 8, 24, (1, 5, 39)),  # tiny groups, many empty experts, N tail
]


@pytest.mark.parametrize("flags", [PX, 0], ids=["px", "plain"])
@pytest.mark.parametrize("case", GATED_SMALL,
                         ids=[f"T{c[0]}K{c[1]}N{c[2]}E{c[3]}k{c[4]}" for c in GATED_SMALL])
def test_gated_small(mg, flags, case):
    T, K, N, E, topk, seed, empty = case
    wl = synth.random_case(T, K, N, E, topk, flags, seed, empty=empty)
    got, ref = _gated_case(mg, wl, flags)
    _check(got, ref, f"gated {case} flags={flags}")


def test_gated_pairs_are_adjacent_rows(mg):
    # With every linear (odd) W row zero the output is exactly zero, and with
    # every gate (even) row zero it is silu(0) * u = 0 as well; a layout that
    # paired other rows would leave nonzero outputs.
    wl = synth.random_case(200, 128, 512, 4, 2, PX, 25)
    for parity in (0, 1):
        W = wl.W.clone()
        W[:, parity::2, :] = 0
        r = mg.moe_route(_dev(wl.ids), wl.E, 128)
        Y = mg.grouped_gemm_fwd(_dev(wl.X), _dev(W), r["m_sizes"], r["gather"], None, wl.topk,
                                PX | GS)
        torch.cuda.synchronize()
        assert torch.count_nonzero(Y).item() == 0


def test_gated_zero_tokens(mg):
    wl = synth.random_case(8, 64, 256, 4, 2, PX, 26)
    m_sizes = torch.zeros(4, dtype=torch.int32, device="cuda")
    Y = mg.grouped_gemm_fwd(_dev(wl.X[:0]), _dev(wl.W), m_sizes,
                            torch.zeros(0, dtype=torch.int32, device="cuda"), None, 2, PX | GS)
    torch.cuda.synchronize()
    assert tuple(Y.shape) == (0, 128)


def _sample(offsets, S, H, rng):
    rows = set()
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            rows.update([lo, hi - 1, (lo + hi) // 2])
            for b in range(lo + 255, hi, 256):
                rows.update([b, min(b + 1, hi - 1)])
    rows.update(rng.integers(0, S, size=16).tolist())
    cols = {0, H - 1}
    for b in range(127, H, 128 * 7):
        cols.update([b, min(b + 1, H - 1)])
    cols.update(rng.integers(0, H, size=48).tolist())
    return np.array(sorted(rows)), np.array(sorted(cols), dtype=np.int64)


def test_gated_mixtral_sampled(mg):
    wl = synth.mixtral()
    rng = np.random.default_rng(7)
    ref_route = oracle.route(wl.ids.numpy().reshape(-1), wl.E, 128)
    rows, cols = _sample(ref_route["offsets"], wl.S, wl.N // 2, rng)
    got, ref = _gated_case(mg, wl, wl.flags, rows=rows, cols=cols)
    _check(got, ref, "gated mixtral sampled")
