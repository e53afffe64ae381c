"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Routing outputs must match bit for bit.  bf16 GEMM outputs are compared with
the oracle's fp32 results: relative Frobenius error <= 5e-3 and
|y - ref| <= 3e-2 * max(1, |ref|) elementwise.  Small cases span several
tiles with ragged tails, empty experts and every flag combination; the
full-size workloads are checked on sampled rows and columns (all experts,
tile boundaries, first and last rows) that the oracle computes one by one.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._util import bf16_tolerance_ok

pytestmark = pytest.mark.gpu

PX, PY, FM = synth.PERMUTE_X, synth.PERMUTE_Y, synth.FUSE_MUL_POST


@pytest.fixture(scope="module")
def mg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_routing_amd as mg
    mg.load_library()
    return mg


def _dev(t):
    return t.to("cuda").contiguous()


def _np(t):
    return t.cpu().numpy()


def _assert_close(got_bf16, ref_f32, what):
    got = got_bf16.float().cpu().numpy() if isinstance(got_bf16, torch.Tensor) else got_bf16
    ok, info = bf16_tolerance_ok(got, ref_f32)
    print(f"{what}: {info}", flush=True)
    assert ok, (what, info)


# ---------------------------------------------------------------------------
# Routing
# ---------------------------------------------------------------------------

def _route_both(mg, ids_cpu, E, block_m):
    ref = oracle.route(ids_cpu.numpy().reshape(-1), E, block_m)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = mg.moe_route(_dev(ids_cpu), E, block_m, error_flags=err)
    torch.cuda.synchronize()
    return ref, {k: _np(v) for k, v in out.items()}, int(err.item())


ROUTE_CASES = [
    ("tiny", lambda: synth.tiny().ids, 8, 32),
    ("mixtral", lambda: synth.route_softmax_topk(4096, 8, 2, synth.generator(1003))[0], 8, 256),
    ("fine_down", lambda: synth.fine_down().ids, 128, 256),
    ("fine_decode", lambda: synth.fine_decode().ids, 128, 32),
    ("E1024", lambda: torch.randint(0, 1024, (3001, 5), generator=synth.generator(9),
                                    dtype=torch.int32), 1024, 64),
    ("E1_odd", lambda: torch.zeros(777, 1, dtype=torch.int32), 1, 7),
    ("E3_ragged", lambda: torch.randint(0, 3, (1000, 1), generator=synth.generator(3),
                                        dtype=torch.int32), 3, 128),
]


@pytest.mark.parametrize("name,make,E,B", ROUTE_CASES, ids=[c[0] for c in ROUTE_CASES])
def test_route_bit_exact(mg, name, make, E, B):
    ids = make()
    ref, got, err = _route_both(mg, ids, E, B)
    assert err == 0
    for k in ("m_sizes", "offsets", "padded_offsets", "tile_offsets", "gather", "scatter"):
        assert np.array_equal(got[k], ref[k]), k


def test_route_deterministic(mg):
    ids = _dev(synth.fine_down().ids)
    first = {k: v.clone() for k, v in mg.moe_route(ids, 128, 256).items()}
    for _ in range(10):
        again = mg.moe_route(ids, 128, 256)
        for k in first:
            assert torch.equal(first[k], again[k]), k


def test_route_drops_bad_ids(mg):
    ids = torch.randint(0, 16, (513, 3), generator=synth.generator(5), dtype=torch.int32)
    ids[7, 1] = -3
    ids[400, 0] = 16
    ids[512, 2] = 1 << 30
    ref, got, err = _route_both(mg, ids, 16, 32)
    assert err & 1
    assert ref["dropped"] == 3
    for k in ("m_sizes", "offsets", "gather", "scatter"):
        assert np.array_equal(got[k], ref[k]), k


def test_route_pages_worked_example(mg):
    """The ragged dw comment block's example (expt_hist [60, 33, 0, 32, 25],
    block 32) fed to the GPU routing: its padded ranges and tile counts, read
    from the golden file, come out of padded_offsets and tile_offsets."""
    import json
    import os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                       "ragged_padded_example.json")))
    hist, B = gold["expt_hist"], gold["block"]
    ids = np.concatenate([np.full(h, e, np.int32) for e, h in enumerate(hist)])
    ids = ids[np.random.default_rng(60).permutation(ids.size)]
    ref, got, err = _route_both(mg, torch.from_numpy(ids).reshape(-1, 1), len(hist), B)
    assert err == 0
    assert got["m_sizes"].tolist() == hist
    starts = got["padded_offsets"].tolist()
    for e, (lo, hi) in gold["padded_ranges"].items():
        assert starts[int(e)] == lo and starts[int(e)] + hist[int(e)] == hi
    assert starts[-1] == gold["padded_end"]
    assert got["offsets"].tolist()[-1] == gold["unpadded_end"]
    tiles = np.diff(got["tile_offsets"]).tolist()
    assert tiles == [(h + B - 1) // B for h in hist] == [2, 2, 0, 1, 1]
    for k in ("m_sizes", "offsets", "padded_offsets", "tile_offsets", "gather", "scatter"):
        assert np.array_equal(got[k], ref[k]), k


def test_route_empty(mg):
    out = mg.moe_route(torch.zeros(0, 2, dtype=torch.int32, device="cuda"), 8, 32)
    torch.cuda.synchronize()
    assert _np(out["m_sizes"]).tolist() == [0] * 8
    assert _np(out["offsets"]).tolist() == [0] * 9


# ---------------------------------------------------------------------------
# Forward
# ---------------------------------------------------------------------------

def _gpu_route(mg, wl, block_m=128):
    return mg.moe_route(_dev(wl.ids), wl.E, block_m)


def _fwd_case(mg, wl, flags, rows=None, cols=None):
    r = _gpu_route(mg, wl)
    ref_route = oracle.route(wl.ids.numpy().reshape(-1), wl.E, 128)
    assert np.array_equal(_np(r["gather"]), ref_route["gather"])
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    Y = mg.grouped_gemm_fwd(_dev(wl.X), _dev(wl.W), r["m_sizes"], r["gather"],
                            _dev(wl.weights.reshape(-1)), wl.topk, flags, error_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref = oracle.grouped_gemm_fwd(synth.bits(wl.X), synth.bits(wl.W), ref_route["m_sizes"],
                                  ref_route["gather"], wl.weights.numpy().reshape(-1), wl.topk,
                                  flags, rows=rows, cols=cols)
    got = Y.float().cpu().numpy()
    if rows is not None:
        got = got[np.asarray(rows)]
    if cols is not None:
        got = got[:, np.asarray(cols)]
    return got, ref, Y


FWD_SMALL = [
    # T, K, N, E, topk, seed, empty  -- ragged groups, tails in every dimension
    (300, 320, 264, 5, 2, 1, (3,)),       # avg 120 rows/expert -> large-tile path
    (700, 136, 520, 6, 3, 2, (0,)),       # K not a multiple of 64, N not of 256
    (64, 256, 512, 16, 4, 3, (2, 9)),     # avg 16 rows -> small-tile path
    (33, 64, 136, 40, 8, 4, (1, 5, 39)),  # tiny groups, many empty experts
    (40, 136, 264, 4, 4, 5, ()),          # avg 40 rows: two 32-row blocks per expert,
                                          # K = 8.5 steps of 16, a ragged 32-column block
]


@pytest.mark.parametrize("flags", [0, PX, PY, PY | FM], ids=["plain", "px", "py", "py_fm"])
@pytest.mark.parametrize("case", FWD_SMALL, ids=[f"T{c[0]}K{c[1]}N{c[2]}E{c[3]}k{c[4]}" for c in FWD_SMALL])
def test_fwd_small(mg, flags, case):
    T, K, N, E, topk, seed, empty = case
    wl = synth.random_case(T, K, N, E, topk, flags, seed, empty=empty)
    got, ref, _ = _fwd_case(mg, wl, flags)
    _assert_close(got, ref, f"fwd {case} flags={flags}")


def test_fwd_tiny_config(mg):
    wl = synth.tiny()
    got, ref, _ = _fwd_case(mg, wl, wl.flags)
    _assert_close(got, ref, "fwd tiny")


def test_fwd_decode_config(mg):
    wl = synth.fine_decode()
    got, ref, _ = _fwd_case(mg, wl, wl.flags)
    _assert_close(got, ref, "fwd fine_decode")


def _sample_rows(offsets, BM, extra, rng, S):
    rows = set()
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        rows.update([lo, hi - 1, (lo + hi) // 2])
        for b in range(lo + BM - 1, hi, BM):
            rows.update([b, min(b + 1, hi - 1)])
    rows.update(rng.integers(0, S, size=extra).tolist())
    return np.array(sorted(rows))


def _sample_cols(N, BN, extra, rng):
    cols = {0, N - 1}
    for b in range(BN - 1, N, BN * 7):
        cols.update([b, min(b + 1, N - 1)])
    cols.update(rng.integers(0, N, size=extra).tolist())
    return np.array(sorted(cols), dtype=np.int32)


def test_fwd_mixtral_sampled(mg):
    wl = synth.mixtral()
    rng = np.random.default_rng(0)
    ref_route = oracle.route(wl.ids.numpy().reshape(-1), wl.E, 128)
    rows_sorted = _sample_rows(ref_route["offsets"], 256, 16, rng, wl.S)
    cols = _sample_cols(wl.N, 256, 48, rng)
    got, ref, _ = _fwd_case(mg, wl, wl.flags, rows=rows_sorted, cols=cols)
    _assert_close(got, ref, "fwd mixtral sampled")


def test_fwd_fine_down_sampled(mg):
    wl = synth.fine_down()
    rng = np.random.default_rng(1)
    ref_route = oracle.route(wl.ids.numpy().reshape(-1), wl.E, 128)
    sorted_rows = _sample_rows(ref_route["offsets"], 256, 64, rng, wl.S)
    out_rows = ref_route["gather"][sorted_rows]      # permute_y: output row = slot
    cols = _sample_cols(wl.N, 256, 64, rng)
    got, ref, _ = _fwd_case(mg, wl, wl.flags, rows=out_rows, cols=cols)
    _assert_close(got, ref, "fwd fine_down sampled")


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------

def _bwd_case(mg, wl, flags, dw_flags_extra=0, rows_dx=None, rows_dw=None, cols_dx=None,
              cols_dw=None):
    r = _gpu_route(mg, wl)
    ref_route = oracle.route(wl.ids.numpy().reshape(-1), wl.E, 128)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dY, W, X = _dev(wl.dY), _dev(wl.W), _dev(wl.X)
    dX = mg.grouped_gemm_dX(dY, W, r["m_sizes"], r["gather"], wl.topk, flags, error_flags=err)
    dW = mg.grouped_gemm_dW(X, dY, r["m_sizes"], r["gather"], wl.topk, flags | dw_flags_extra,
                            error_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    E, N, K = wl.W.shape
    ref_dx = oracle.grouped_gemm_dX(synth.bits(wl.dY), synth.bits(wl.W), ref_route["m_sizes"],
                                    ref_route["gather"], wl.topk, flags, rows=rows_dx, cols=cols_dx)
    ref_dw = oracle.grouped_gemm_dW(synth.bits(wl.X), synth.bits(wl.dY), ref_route["m_sizes"],
                                    ref_route["gather"], wl.topk, flags, E, rows=rows_dw,
                                    cols=cols_dw)
    def pick(t, rows, cols):
        # select on the device: a full-size dW is 1.9 GB
        if rows is not None:
            t = t[torch.as_tensor(rows, dtype=torch.long, device=t.device)]
        if cols is not None:
            t = t[:, torch.as_tensor(cols, dtype=torch.long, device=t.device)]
        return t.float().cpu().numpy()

    got_dx = pick(dX, rows_dx, cols_dx)
    got_dw = pick(dW.reshape(E * N, K), rows_dw, cols_dw)
    return got_dx, ref_dx, got_dw, ref_dw, dW, ref_route


BWD_SMALL = [
    (300, 320, 264, 5, 2, 11, (3,)),
    (700, 136, 520, 6, 3, 12, (0,)),
    (33, 64, 136, 40, 8, 13, (1, 5, 39)),   # avg 6 rows/expert -> small-M dX tiles
    (100, 200, 264, 24, 4, 15, (3,)),        # small-M dX tiles with K and N tails
    (520, 200, 264, 5, 2, 16, (1,)),         # 1040 slots: dW on the tile engine, with tails
]


@pytest.mark.parametrize("flags", [0, PX, PY], ids=["plain", "px", "py"])
@pytest.mark.parametrize("case", BWD_SMALL, ids=[f"T{c[0]}K{c[1]}N{c[2]}E{c[3]}k{c[4]}" for c in BWD_SMALL])
def test_bwd_small(mg, flags, case):
    T, K, N, E, topk, seed, empty = case
    wl = synth.random_case(T, K, N, E, topk, flags, seed, empty=empty, with_dy=True)
    gdx, rdx, gdw, rdw, dW, _ = _bwd_case(mg, wl, flags)
    _assert_close(gdx, rdx, f"dX {case} flags={flags}")
    _assert_close(gdw, rdw, f"dW {case} flags={flags}")
    for e in empty:
        assert torch.count_nonzero(dW[e]).item() == 0


# dX over a long reduction (N >= 8192) runs the four-wave engine: N = 8200
# leaves a ragged last 32-row slot, K = 520 a ragged last column tile.
BWD_LONG_N = [(150, 520, 8200, 5, 2, 14, (2,))]


@pytest.mark.parametrize("flags", [0, PX, PY], ids=["plain", "px", "py"])
@pytest.mark.parametrize("case", BWD_LONG_N, ids=[f"T{c[0]}K{c[1]}N{c[2]}E{c[3]}k{c[4]}" for c in BWD_LONG_N])
def test_bwd_long_reduction(mg, flags, case):
    T, K, N, E, topk, seed, empty = case
    wl = synth.random_case(T, K, N, E, topk, flags, seed, empty=empty, with_dy=True)
    gdx, rdx, gdw, rdw, dW, _ = _bwd_case(mg, wl, flags)
    _assert_close(gdx, rdx, f"dX {case} flags={flags}")
    _assert_close(gdw, rdw, f"dW {case} flags={flags}")
    for e in empty:
        assert torch.count_nonzero(dW[e]).item() == 0


# dW over long experts without the split workspace: the reduction crosses
# the 1024-row segments in which gather entries are staged (two segments for
# 1100 and 1500 rows, three for 2200) and ends in a ragged 32-row slot.
# K = 72 and N = 264 leave ragged output tiles.
DW_LONG_ROWS = [(1100, 72, 264, 2, 2, 16, ()), (1500, 136, 136, 3, 2, 17, (1,)),
                (2200, 72, 264, 2, 2, 19, ())]


@pytest.mark.parametrize("flags", [0, PX, PY], ids=["plain", "px", "py"])
@pytest.mark.parametrize("case", DW_LONG_ROWS,
                         ids=[f"T{c[0]}K{c[1]}N{c[2]}E{c[3]}k{c[4]}" for c in DW_LONG_ROWS])
def test_dw_long_rows_unsplit(mg, flags, case):
    T, K, N, E, topk, seed, empty = case
    wl = synth.random_case(T, K, N, E, topk, flags, seed, empty=empty, with_dy=True)
    r = _gpu_route(mg, wl)
    ref_route = oracle.route(wl.ids.numpy().reshape(-1), wl.E, 128)
    assert ref_route["m_sizes"].max() > 1024
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dW = mg.grouped_gemm_dW(_dev(wl.X), _dev(wl.dY), r["m_sizes"], r["gather"], wl.topk, flags,
                            split=False, error_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref = oracle.grouped_gemm_dW(synth.bits(wl.X), synth.bits(wl.dY), ref_route["m_sizes"],
                                 ref_route["gather"], wl.topk, flags, E)
    _assert_close(dW.reshape(E * N, K).float().cpu().numpy(), ref, f"dW {case} flags={flags}")
    for e in empty:
        assert torch.count_nonzero(dW[e]).item() == 0


# Experts of more than 8 row tiles of 256 are rastered in bands of 8 row tiles
# (forward over N tiles, dX over K tiles): 2 experts of 2200 rows give a full
# band of 8 and a ragged band of 1, with ragged column tiles on both sides.
BANDED = [(2200, 520, 264, 2, 2, 18, ())]


@pytest.mark.parametrize("flags", [0, PX, PY], ids=["plain", "px", "py"])
@pytest.mark.parametrize("case", BANDED, ids=[f"T{c[0]}K{c[1]}N{c[2]}E{c[3]}k{c[4]}" for c in BANDED])
def test_banded_raster_long_experts(mg, flags, case):
    T, K, N, E, topk, seed, empty = case
    wl = synth.random_case(T, K, N, E, topk, flags, seed, empty=empty, with_dy=True)
    got, ref, _ = _fwd_case(mg, wl, flags)
    _assert_close(got, ref, f"fwd {case} flags={flags}")
    r = _gpu_route(mg, wl)
    ref_route = oracle.route(wl.ids.numpy().reshape(-1), wl.E, 128)
    assert ref_route["m_sizes"].min() > 8 * 256
    for split in (False, True):
        dX = mg.grouped_gemm_dX(_dev(wl.dY), _dev(wl.W), r["m_sizes"], r["gather"], wl.topk,
                                flags, split=split)
        ref_dx = oracle.grouped_gemm_dX(synth.bits(wl.dY), synth.bits(wl.W),
                                        ref_route["m_sizes"], ref_route["gather"], wl.topk, flags)
        _assert_close(dX.float().cpu().numpy(), ref_dx, f"dX {case} flags={flags} split={split}")


def test_bwd_mixtral_sampled(mg):
    wl = synth.mixtral()
    wl.dY = synth.normal_bf16((wl.S, wl.N), 0.01, synth.generator(synth.SEEDS["mixtral_bwd_dy"]))
    rng = np.random.default_rng(3)
    ref_route = oracle.route(wl.ids.numpy().reshape(-1), wl.E, 128)
    rows_dx = _sample_rows(ref_route["offsets"], 256, 16, rng, wl.S)
    cols_dx = _sample_cols(wl.K, 256, 24, rng)
    E, N, K = wl.W.shape
    rows_dw = np.array(sorted({e * N + n for e in range(E) for n in [0, 255, 256, N - 1]
                               + rng.integers(0, N, 3).tolist()}))
    cols_dw = _sample_cols(K, 256, 16, rng)
    gdx, rdx, gdw, rdw, _, _ = _bwd_case(mg, wl, wl.flags, rows_dx=rows_dx, rows_dw=rows_dw,
                                         cols_dx=cols_dx, cols_dw=cols_dw)
    _assert_close(gdx, rdx, "dX mixtral sampled")
    _assert_close(gdw, rdw, "dW mixtral sampled")


def test_bwd_decode_full(mg):
    # the decode-shaped backward (T = 64 of the fine-grained layer), every output
    wl = synth.fine_decode_bwd()
    gdx, rdx, gdw, rdw, dW, ref_route = _bwd_case(mg, wl, wl.flags)
    _assert_close(gdx, rdx, "dX decode")
    _assert_close(gdw, rdw, "dW decode")
    for e in np.nonzero(ref_route["m_sizes"] == 0)[0]:
        assert torch.count_nonzero(dW[int(e)]).item() == 0


EDGE_SHAPES = [
    # T, K, N, E, topk, seed, empty -- the expert-table capacity (E = 1024, about
    # one row per expert, most experts empty) and the smallest legal K and N
    (700, 64, 64, 1024, 2, 16, ()),
    (50, 8, 8, 3, 2, 17, ()),
    (1, 8, 16, 4, 1, 18, ()),
]


@pytest.mark.parametrize("flags", [PX, PY], ids=["px", "py"])
@pytest.mark.parametrize("case", EDGE_SHAPES, ids=[f"T{c[0]}K{c[1]}N{c[2]}E{c[3]}k{c[4]}" for c in EDGE_SHAPES])
def test_edge_shapes(mg, flags, case):
    T, K, N, E, topk, seed, empty = case
    wl = synth.random_case(T, K, N, E, topk, flags, seed, empty=empty, with_dy=True)
    got, ref, _ = _fwd_case(mg, wl, flags)
    _assert_close(got, ref, f"fwd {case} flags={flags}")
    gdx, rdx, gdw, rdw, dW, ref_route = _bwd_case(mg, wl, flags)
    _assert_close(gdx, rdx, f"dX {case} flags={flags}")
    _assert_close(gdw, rdw, f"dW {case} flags={flags}")
    for e in np.nonzero(ref_route["m_sizes"] == 0)[0][:64]:
        assert torch.count_nonzero(dW[int(e)]).item() == 0


# dW of launches with at most 1024 slots and 16 rows per expert on average
# runs the short-reduction kernel (64 x 64 tiles per wave, fragments loaded
# straight from global memory): N and K tails inside a 64-wide tile and past
# a 32-wide fragment, empty experts, and the 1024-slot boundary.
DW_SHORT = [
    # T, K, N, E, topk, seed, empty
    (128, 200, 136, 64, 8, 31, (1, 5, 60)),   # 1024 slots, avg 16 rows/expert
    (33, 72, 264, 40, 8, 32, (0, 7)),         # 264 slots, K = 64 + 8, N = 4 x 64 + 8
    (3, 64, 64, 9, 3, 34, (4,)),              # 9 slots over 9 experts
]


@pytest.mark.parametrize("flags", [0, PX, PY], ids=["plain", "px", "py"])
@pytest.mark.parametrize("case", DW_SHORT, ids=[f"T{c[0]}K{c[1]}N{c[2]}E{c[3]}k{c[4]}" for c in DW_SHORT])
def test_dw_short_reduction(mg, flags, case):
    T, K, N, E, topk, seed, empty = case
    assert T * topk <= 1024
    wl = synth.random_case(T, K, N, E, topk, flags, seed, empty=empty, with_dy=True)
    _, _, gdw, rdw, dW, ref_route = _bwd_case(mg, wl, flags)
    _assert_close(gdw, rdw, f"dW {case} flags={flags}")
    for e in np.nonzero(ref_route["m_sizes"] == 0)[0]:
        assert torch.count_nonzero(dW[int(e)]).item() == 0


@pytest.mark.parametrize("flags", [PX, PY], ids=["px", "py"])
def test_dw_short_reduction_zipf(mg, flags):
    """Zipf(1.2) routing of 128 tokens over 64 experts, top-8: a hot expert
    of 126 rows (eight sixteen-row steps, the last one partial) beside
    experts of one or two rows and empty ones, all in one short launch."""
    wl = synth._fine("zipf_short", 128, 200, 136, 64, 8, 1.2, 36, 36, True)
    wl.flags = flags
    _, _, gdw, rdw, dW, ref_route = _bwd_case(mg, wl, flags)
    assert ref_route["m_sizes"].max() == 126
    _assert_close(gdw, rdw, f"dW zipf flags={flags}")
    for e in np.nonzero(ref_route["m_sizes"] == 0)[0]:
        assert torch.count_nonzero(dW[int(e)]).item() == 0


@pytest.mark.parametrize("flags", [PX, PY], ids=["px", "py"])
def test_dw_short_reduction_bad_gather(mg, flags):
    """A gather entry outside [0, S) drops its slot's term from dW and sets
    the gather error bit.  Expected: the oracle with that slot's other
    operand row (dY under permute_x, X under permute_y) zeroed instead."""
    wl = synth.random_case(16, 72, 136, 16, 8, flags, 37, with_dy=True)
    S, E = wl.S, wl.E
    route = oracle.route(wl.ids.numpy().reshape(-1), E, 128)
    bad_p = 5
    gather = torch.from_numpy(route["gather"].copy())
    gather[bad_p] = S + 7
    X, dY = wl.X.clone(), wl.dY.clone()
    if flags & PX:
        dY[bad_p] = 0
    else:
        X[bad_p] = 0
    ref = oracle.grouped_gemm_dW(synth.bits(X), synth.bits(dY), route["m_sizes"],
                                 route["gather"], wl.topk, flags, E)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dW = mg.grouped_gemm_dW(_dev(wl.X), _dev(wl.dY), _dev(torch.from_numpy(route["m_sizes"])),
                            _dev(gather), wl.topk, flags, error_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) & mg.DERR_GATHER
    _assert_close(dW.reshape(E * wl.N, wl.K).float().cpu().numpy(), ref, "dW bad gather")


def test_dw_short_reduction_fp32_out(mg):
    wl = synth.random_case(100, 200, 136, 32, 4, PY, 35, empty=(3,), with_dy=True)
    _, _, gdw, rdw, dW, _ = _bwd_case(mg, wl, PY, dw_flags_extra=mg.DW_FP32_OUT)
    assert dW.dtype == torch.float32
    ok, info = bf16_tolerance_ok(gdw, rdw, rel_fro_max=1e-5, max_elem=1e-4)
    assert ok, info
    assert torch.count_nonzero(dW[3]).item() == 0


def test_dw_fp32_out(mg):
    wl = synth.random_case(300, 136, 264, 5, 2, PY, 21, empty=(2,), with_dy=True)
    _, _, gdw, rdw, dW, _ = _bwd_case(mg, wl, PY, dw_flags_extra=mg.DW_FP32_OUT)
    assert dW.dtype == torch.float32
    ok, info = bf16_tolerance_ok(gdw, rdw, rel_fro_max=1e-5, max_elem=1e-4)
    assert ok, info


def test_bwd_fine_sampled(mg):
    wl = synth.fine_bwd()
    rng = np.random.default_rng(2)
    ref_route = oracle.route(wl.ids.numpy().reshape(-1), wl.E, 128)
    rows_dx = _sample_rows(ref_route["offsets"], 256, 32, rng, wl.S)
    cols_dx = _sample_cols(wl.K, 256, 32, rng)
    E, N, K = wl.W.shape
    h = ref_route["m_sizes"]
    experts = sorted(set([int(np.argmax(h)), int(np.argmin(np.where(h > 0, h, 10 ** 9)))]
                         + rng.integers(0, E, 6).tolist() + np.nonzero(h == 0)[0][:2].tolist()))
    rows_dw = np.array(sorted({e * N + n for e in experts for n in [0, 255, 256, N - 1]
                               + rng.integers(0, N, 4).tolist()}))
    cols_dw = _sample_cols(K, 256, 16, rng)
    gdx, rdx, gdw, rdw, dW, _ = _bwd_case(mg, wl, wl.flags, rows_dx=rows_dx, rows_dw=rows_dw,
                                           cols_dx=cols_dx, cols_dw=cols_dw)
    _assert_close(gdx, rdx, "dX fine sampled")
    _assert_close(gdw, rdw, "dW fine sampled")
    for e in np.nonzero(h == 0)[0]:
        assert torch.count_nonzero(dW[int(e)]).item() == 0


# ---------------------------------------------------------------------------
# Explicit groups
# ---------------------------------------------------------------------------

def test_groups_dual_config(mg):
    wl = synth.dual()
    ys = mg.grouped_gemm_groups([(_dev(x), _dev(w)) for x, w in wl.groups], trans_b=0)
    torch.cuda.synchronize()
    for i, ((x, w), y) in enumerate(zip(wl.groups, ys)):
        ref = oracle.dense_gemm_kn(synth.bits(x), synth.bits(w))
        _assert_close(y, ref, f"dual group {i}")


def test_groups_ragged_and_trans_b(mg):
    g = synth.generator(77)
    shapes = [(1, 64, 8), (130, 200, 264), (0, 64, 64), (257, 72, 136)]
    xs = [synth.normal_bf16((m, k), 0.5, g) for m, k, n in shapes]
    ws = [synth.normal_bf16((k, n), 0.5, g) for m, k, n in shapes]
    ys = mg.grouped_gemm_groups([(_dev(x), _dev(w)) for x, w in zip(xs, ws)], trans_b=0)
    ysT = mg.grouped_gemm_groups([(_dev(x), _dev(w.t().contiguous())) for x, w in zip(xs, ws)],
                                 trans_b=1)
    torch.cuda.synchronize()
    for (m, k, n), x, w, y, yT in zip(shapes, xs, ws, ys, ysT):
        if m == 0:
            continue
        ref = oracle.dense_gemm_kn(synth.bits(x), synth.bits(w))
        _assert_close(y, ref, f"group {m}x{k}x{n}")
        _assert_close(yT, ref, f"group trans_b {m}x{k}x{n}")


# ---------------------------------------------------------------------------
# Degenerate inputs and device-side error reporting
# ---------------------------------------------------------------------------

def test_zero_tokens_is_noop(mg):
    W = torch.zeros(4, 64, 64, dtype=torch.bfloat16, device="cuda")
    X = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda")
    m = torch.zeros(4, dtype=torch.int32, device="cuda")
    g = torch.zeros(0, dtype=torch.int32, device="cuda")
    Y = mg.grouped_gemm_fwd(X, W, m, g, None, 2, PX)
    assert Y.shape == (0, 64)
    dW = mg.grouped_gemm_dW(X, torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda"), m, g, 2, 0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dW).item() == 0


def test_bad_m_sizes_and_gather_are_flagged(mg):
    wl = synth.random_case(64, 64, 64, 4, 2, PX, 31)
    r = _gpu_route(mg, wl)
    X, W = _dev(wl.X), _dev(wl.W)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    bad_m = r["m_sizes"].clone()
    bad_m[0] += 1000                      # sums past S: clipped, flagged
    mg.grouped_gemm_fwd(X, W, bad_m, r["gather"], None, 2, PX, error_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 2
    err.zero_()
    bad_g = r["gather"].clone()
    bad_g[5] = 10 ** 6                    # outside [0, S): row skipped, flagged
    mg.grouped_gemm_fwd(X, W, r["m_sizes"], bad_g, None, 2, PX, error_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 4


def test_host_validation_statuses(mg):
    X = torch.zeros(8, 64, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros(2, 64, 64, dtype=torch.bfloat16, device="cuda")
    m = torch.tensor([4, 4], dtype=torch.int32, device="cuda")
    g = torch.arange(8, dtype=torch.int32, device="cuda")
    with pytest.raises(mg.MoeggError) as e:
        mg.grouped_gemm_fwd(X, W, m, g, None, 1, PX | PY)
    assert e.value.status == 1
    with pytest.raises(mg.MoeggError) as e:
        mg.grouped_gemm_dX(X, W, m, g, 1, FM)
    assert e.value.status == 3


# dW under permute_x with a workspace large enough for X's rows in expert
# order: a separate copy launch, then the reduction on the copy.  Against
# the gather inside the reduction with the same split (a workspace of just
# the split area, so hot experts are cut into the same chunks) the sums are
# the same in the same order, so the two agree bit for bit; the copy path is
# also checked against the oracle.
DW_GATHERED = [(300, 72, 264, 4, 2, 21), (1100, 136, 136, 3, 2, 22), (37, 264, 72, 4, 3, 23)]


@pytest.mark.parametrize("T,N,K,E,topk,seed", DW_GATHERED)
def test_dw_permute_x_gathered_copy(mg, T, N, K, E, topk, seed):
    g = torch.Generator().manual_seed(seed)
    S = T * topk
    ids = torch.randint(0, E, (T, topk), generator=g, dtype=torch.int32)
    X = (torch.randn(T, K, generator=g) * 0.5).to(torch.bfloat16)
    dY = (torch.randn(S, N, generator=g) * 0.5).to(torch.bfloat16)
    route = oracle.route(ids.numpy().reshape(-1), E, 128)
    gather = torch.from_numpy(route["gather"]).cuda()
    m_sizes = torch.from_numpy(route["m_sizes"]).cuda()
    Xd, dYd = X.cuda(), dY.cuda()
    need = mg.dw_gather_workspace_bytes(T, topk, E, N, K)
    assert need >= S * K * 2 + mg.dw_workspace_bytes(T, topk, E, N, K)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dW_copy = mg.grouped_gemm_dW(Xd, dYd, m_sizes, gather, topk, mg.PERMUTE_X, workspace=ws,
                                 error_flags=err)
    split_ws = torch.empty(max(mg.dw_workspace_bytes(T, topk, E, N, K), 16), dtype=torch.uint8,
                           device="cuda")
    dW_fused = mg.grouped_gemm_dW(Xd, dYd, m_sizes, gather, topk, mg.PERMUTE_X,
                                  workspace=split_ws, error_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(dW_copy, dW_fused)
    ref = oracle.grouped_gemm_dW(synth.bits(X), synth.bits(dY), route["m_sizes"],
                                 route["gather"], topk, mg.PERMUTE_X, E)
    _assert_close(dW_copy.reshape(E * N, K), ref, f"dW gathered copy T={T} N={N} K={K}")


def test_dw_gathered_copy_flags_bad_gather(mg):
    """An entry outside [0, S) gives a zero row and the gather error bit, as
    the gather inside the reduction does."""
    T, N, K, E, topk = 64, 72, 136, 2, 2
    S = T * topk
    g = torch.Generator().manual_seed(24)
    X = (torch.randn(T, K, generator=g) * 0.5).to(torch.bfloat16).cuda()
    dY = (torch.randn(S, N, generator=g) * 0.5).to(torch.bfloat16).cuda()
    m_sizes = torch.tensor([S // 2, S // 2], dtype=torch.int32, device="cuda")
    gather = torch.arange(S, dtype=torch.int32, device="cuda")
    gather[5] = S + 7
    ws = torch.empty(mg.dw_gather_workspace_bytes(T, topk, E, N, K), dtype=torch.uint8,
                     device="cuda")
    e1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    e2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    a = mg.grouped_gemm_dW(X, dY, m_sizes, gather, topk, mg.PERMUTE_X, workspace=ws,
                           error_flags=e1)
    b = mg.grouped_gemm_dW(X, dY, m_sizes, gather, topk, mg.PERMUTE_X, split=False,
                           error_flags=e2)
    torch.cuda.synchronize()
    assert int(e1.item()) & mg.DERR_GATHER and int(e2.item()) & mg.DERR_GATHER
    assert torch.equal(a, b)


def test_dw_gathered_copy_with_dropped_ids(mg):
    """Routing that dropped slots leaves -1 gather entries past sum(m_sizes).
    Neither dW path reads them: the copy path (X rows copied into expert
    order first) and the gather inside the reduction give the same bits and
    the same (clear) error flags, and both match the oracle."""
    T, N, K, E, topk = 400, 72, 136, 5, 3
    S = T * topk
    g = torch.Generator().manual_seed(31)
    ids = torch.randint(0, E, (T, topk), generator=g, dtype=torch.int32)
    ids[3, 0] = -1
    ids[150, 2] = E
    ids[399, 1] = 1 << 20
    X = (torch.randn(T, K, generator=g) * 0.5).to(torch.bfloat16)
    dY = (torch.randn(S, N, generator=g) * 0.5).to(torch.bfloat16)
    ref_route = oracle.route(ids.numpy().reshape(-1), E, 128)
    assert ref_route["dropped"] == 3
    r = mg.moe_route(_dev(ids), E, 128)
    torch.cuda.synchronize()
    assert np.array_equal(_np(r["gather"]), ref_route["gather"])
    assert (_np(r["gather"])[S - 3:] == -1).all()
    Xd, dYd = _dev(X), _dev(dY)
    ws_copy = torch.empty(mg.dw_gather_workspace_bytes(T, topk, E, N, K), dtype=torch.uint8,
                          device="cuda")
    ws_split = torch.empty(max(mg.dw_workspace_bytes(T, topk, E, N, K), 16), dtype=torch.uint8,
                           device="cuda")
    e1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    e2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    a = mg.grouped_gemm_dW(Xd, dYd, r["m_sizes"], r["gather"], topk, PX, workspace=ws_copy,
                           error_flags=e1)
    b = mg.grouped_gemm_dW(Xd, dYd, r["m_sizes"], r["gather"], topk, PX, workspace=ws_split,
                           error_flags=e2)
    torch.cuda.synchronize()
    assert int(e1.item()) == int(e2.item()) == 0
    assert torch.equal(a, b)
    ref = oracle.grouped_gemm_dW(synth.bits(X), synth.bits(dY), ref_route["m_sizes"],
                                 ref_route["gather"], topk, PX, E)
    _assert_close(a.reshape(E * N, K), ref, "dW copy path, dropped ids")


def test_dw_permute_x_copy_would_exceed_2gib(mg):
    """S*K*2 >= 2 GiB > T*K*2 under permute_x: the X copy would not fit the
    32-bit operand offsets, so dW gathers inside the reduction, with the
    binding's default workspace and with one that has room for the copy.
    Sampled dW rows (every expert; first, last and 32-row block boundary
    columns of N) x column blocks against the oracle."""
    T, N, K, E, topk = 20000, 64, 8192, 4, 8
    S = T * topk
    assert T * K * 2 < 2 ** 31 <= S * K * 2
    g = torch.Generator().manual_seed(41)
    ids = torch.randint(0, E, (T, topk), generator=g, dtype=torch.int32)
    X = (torch.randn(T, K, generator=g)).to(torch.bfloat16)
    dY = (torch.randn(S, N, generator=g) * 0.1).to(torch.bfloat16)
    print(f"dW over 2 GiB copy area: T={T} topk={topk} K={K} N={N} E={E}", flush=True)
    ref_route = oracle.route(ids.numpy().reshape(-1), E, 128)
    r = mg.moe_route(_dev(ids), E, 128)
    Xd, dYd = _dev(X), _dev(dY)
    assert mg.dw_gather_workspace_bytes(T, topk, E, N, K) == mg.dw_workspace_bytes(T, topk, E, N,
                                                                                    K)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dW = mg.grouped_gemm_dW(Xd, dYd, r["m_sizes"], r["gather"], topk, PX, error_flags=err)
    big = torch.empty(mg.dw_workspace_bytes(T, topk, E, N, K) + S * K * 2 + 4096,
                      dtype=torch.uint8, device="cuda")
    dW_big = mg.grouped_gemm_dW(Xd, dYd, r["m_sizes"], r["gather"], topk, PX, workspace=big,
                                error_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(dW, dW_big)
    del big
    ns = [0, 1, 31, 32, 62, 63]
    rows = np.array([e * N + n for e in range(E) for n in ns])
    cols = np.concatenate([np.arange(0, 32), np.arange(4096 - 16, 4096 + 16),
                           np.arange(K - 32, K)]).astype(np.int32)
    ref = oracle.grouped_gemm_dW(synth.bits(X), synth.bits(dY), ref_route["m_sizes"],
                                 ref_route["gather"], topk, PX, E, rows=rows, cols=cols)
    got = dW.reshape(E * N, K)[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).long().cuda()]
    _assert_close(got, ref, "dW, copy area over 2 GiB")
