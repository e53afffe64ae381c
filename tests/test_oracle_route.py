"""Pins of the oracle's routing step (histogram, offsets, gather/scatter indices).

Each check comes from outside the oracle: the worked example printed in
triton_kernels/matmul_ogs.py (ragged dw layout comment), brute force over all
histograms for the n_blocks bound, numpy.bincount and numpy's stable argsort,
and the permutation identities.
"""

import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ragged_padded_example.json")


def _ids_with_hist(hist, seed=0):
    rng = np.random.default_rng(seed)
    ids = np.concatenate([np.full(h, e, np.int32) for e, h in enumerate(hist)])
    rng.shuffle(ids)
    return ids


def test_worked_example_offsets():
    g = json.load(open(GOLDEN))
    hist, B = g["expt_hist"], g["block"]
    E = len(hist)
    r = oracle.route(_ids_with_hist(hist), E, B)
    assert r["m_sizes"].tolist() == hist
    # Unpadded offsets: expert e starts where the page's unpadded range starts;
    # the empty expert starts where the next one does.
    starts = [g["unpadded_ranges"].get(str(e), [None])[0] for e in range(E)]
    for e in range(E - 1, -1, -1):
        if starts[e] is None:
            starts[e] = starts[e + 1]
    assert r["offsets"].tolist() == starts + [g["unpadded_end"]]
    pstarts = [g["padded_ranges"].get(str(e), [None])[0] for e in range(E)]
    for e in range(E - 1, -1, -1):
        if pstarts[e] is None:
            pstarts[e] = pstarts[e + 1]
    assert r["padded_offsets"].tolist() == pstarts + [g["padded_end"]]
    # Tiles per expert = padded width / block, read off the page's table.
    widths = np.diff(np.array(pstarts + [g["padded_end"]]))
    assert widths.tolist() == [64, 64, 0, 32, 32]
    assert r["tile_offsets"].tolist() == [0] + np.cumsum(widths // B).tolist()
    # The unpadded/padded ranges themselves (end = start + count).
    for e_str, (lo, hi) in g["padded_ranges"].items():
        e = int(e_str)
        assert r["padded_offsets"][e] == lo and lo + hist[e] == hi
    # The page's padding gaps are exactly the space between an expert's end and the next start.
    gaps = [[int(r["padded_offsets"][e] + hist[e]), int(r["padded_offsets"][e + 1])]
            for e in range(E) if r["padded_offsets"][e] + hist[e] < r["padded_offsets"][e + 1]]
    assert gaps == g["padding"]
    # The example's tile count sits under the n_blocks bound of RoutingData.
    assert r["tile_offsets"][-1] == 6 <= oracle.n_blocks(150, 5, 32) == 9


def _compositions(total, parts):
    for cuts in itertools.combinations(range(total + parts - 1), parts - 1):
        prev, out = -1, []
        for c in cuts:
            out.append(c - prev - 1)
            prev = c
        out.append(total + parts - 1 - prev - 1)
        yield out


@pytest.mark.parametrize("E", [1, 2, 3, 4])
@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_n_blocks_is_tight_bound_brute_force(E, B):
    for M in range(0, 13):
        worst = 0
        for hist in _compositions(M, E):
            tiles = sum(-(-h // B) for h in hist)
            worst = max(worst, tiles)
            r = oracle.route(_ids_with_hist(hist, seed=M), E, B)
            assert r["tile_offsets"][-1] == tiles
        assert worst == oracle.n_blocks(M, E, B), (M, E, B)


@pytest.mark.parametrize("S,E,B,seed", [(1, 1, 32, 0), (257, 8, 32, 1), (4096, 128, 64, 2),
                                        (65536, 128, 128, 3), (1000, 5, 7, 4), (64, 1024, 16, 5)])
def test_route_against_library(S, E, B, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=S).astype(np.int32)
    r = oracle.route(ids, E, B)
    assert r["dropped"] == 0
    assert np.array_equal(r["m_sizes"], np.bincount(ids, minlength=E))
    assert r["m_sizes"].sum() == S
    assert np.array_equal(r["offsets"], np.concatenate([[0], np.cumsum(np.bincount(ids, minlength=E))]))
    h = np.bincount(ids, minlength=E)
    assert np.array_equal(r["padded_offsets"], np.concatenate([[0], np.cumsum(-(-h // B) * B)]))
    assert np.array_equal(r["tile_offsets"], np.concatenate([[0], np.cumsum(-(-h // B))]))
    assert r["tile_offsets"][-1] <= oracle.n_blocks(S, E, B)
    g, sc = r["gather"], r["scatter"]
    assert np.array_equal(g, np.argsort(ids, kind="stable"))
    assert np.array_equal(np.sort(g), np.arange(S))
    assert np.array_equal(sc[g], np.arange(S))
    assert np.all(np.diff(ids[g]) >= 0)
    for e in range(E):
        grp = g[r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(ids[grp] == e)
        assert np.all(np.diff(grp) > 0)


def test_permute_then_unpermute_is_identity():
    rng = np.random.default_rng(7)
    T, k, E, K = 300, 4, 16, 5
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    r = oracle.route(ids, E, 32)
    rows = rng.standard_normal((T * k, K))
    permuted = rows[r["gather"]]            # token order -> expert order
    back = permuted[r["scatter"]]           # expert order -> token order
    assert np.array_equal(back, rows)
    back2 = np.empty_like(rows)
    back2[r["gather"]] = permuted           # scatter form of the same inverse
    assert np.array_equal(back2, rows)
    # Gathering token rows (permute_x form: row = slot // topk) per expert.
    tok = rng.standard_normal((T, K))
    px = tok[r["gather"] // k]
    for p in range(T * k):
        assert np.array_equal(px[p], tok[r["gather"][p] // k])
        assert ids.reshape(-1)[r["gather"][p]] == np.searchsorted(r["offsets"], p, side="right") - 1


def test_out_of_range_ids_are_dropped():
    ids = np.array([3, -1, 0, 5, 3, 2, 7, 0], np.int32)
    E = 5
    r = oracle.route(ids, E, 2)
    valid = (ids >= 0) & (ids < E)
    assert r["dropped"] == int((~valid).sum()) == 3
    assert np.array_equal(r["m_sizes"], np.bincount(ids[valid], minlength=E))
    nv = int(valid.sum())
    assert np.array_equal(r["gather"][:nv], np.nonzero(valid)[0][np.argsort(ids[valid], kind="stable")])
    assert np.all(r["gather"][nv:] == -1)
    assert np.all(r["scatter"][~valid] == -1)
    assert np.array_equal(r["scatter"][r["gather"][:nv]], np.arange(nv))


def test_degenerate_routing():
    r = oracle.route(np.zeros(0, np.int32), 4, 8)
    assert r["m_sizes"].tolist() == [0, 0, 0, 0]
    assert r["offsets"].tolist() == [0] * 5
    ids = np.zeros(10, np.int32)
    r = oracle.route(ids, 1, 4)
    assert r["m_sizes"].tolist() == [10]
    assert r["gather"].tolist() == list(range(10))
    assert r["tile_offsets"].tolist() == [0, 3]
    assert oracle.n_blocks(0, 4, 8) == 0
