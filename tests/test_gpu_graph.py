"""The whole step captured in a HIP graph: routing, forward, dX, dW and the
top-k combine, with every output and workspace allocated before capture
(the library itself never allocates, frees, synchronises or clears memory
with a memset).

Each case is run eagerly once, then captured and replayed three times with
eager work and synchronisations between the replays; every replay must give
the eager results bit for bit (every kernel here is deterministic).  One
case takes the one-launch routing and the short-reduction dW (a decode-like
step), the other the three-launch routing, the tail-balanced dX and dW with
its X copy.
"""

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

PX = synth.PERMUTE_X


@pytest.fixture(scope="module")
def mg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_routing_amd as m
    m.load_library()
    return m


CASES = [
    # T, K, N, E, topk, seed: a short step (512 slots over 64 experts) and a longer one
    (64, 136, 264, 64, 8, 71),
    (2600, 264, 520, 6, 2, 72),
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}E{c[3]}k{c[4]}" for c in CASES])
def test_step_in_a_graph_replays_bit_exactly(mg, case):
    T, K, N, E, topk, seed = case
    wl = synth.random_case(T, K, N, E, topk, PX, seed, with_dy=True)
    dev = torch.device("cuda")
    S = T * topk
    ids, X, W, dY = wl.ids.to(dev), wl.X.to(dev), wl.W.to(dev), wl.dY.to(dev)
    w = wl.weights.reshape(-1).contiguous().to(dev)
    # Everything the step writes, allocated up front.
    r = {"m_sizes": torch.empty(E, dtype=torch.int32, device=dev),
         "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
         "padded_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
         "tile_offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
         "gather": torch.empty(S, dtype=torch.int32, device=dev),
         "scatter": torch.empty(S, dtype=torch.int32, device=dev)}
    rws = torch.empty(max(mg.route_workspace_bytes(S, E), 16), dtype=torch.uint8, device=dev)
    Y = torch.empty(S, N, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(S, K, dtype=torch.bfloat16, device=dev)
    dW = torch.empty(E, N, K, dtype=torch.bfloat16, device=dev)
    out = torch.empty(T, K, dtype=torch.bfloat16, device=dev)  # the combine of dX
    xws = torch.empty(max(mg.dx_workspace_bytes(T, topk, E, N, K), 16), dtype=torch.uint8,
                      device=dev)
    wws = torch.empty(max(mg.dw_gather_workspace_bytes(T, topk, E, N, K), 16),
                      dtype=torch.uint8, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    outs = (r["m_sizes"], r["offsets"], r["gather"], r["scatter"], Y, dX, dW, out)

    def step():
        mg.moe_route(ids, E, 128, out=r, workspace=rws, error_flags=err)
        mg.grouped_gemm_fwd(X, W, r["m_sizes"], r["gather"], None, topk, PX, Y=Y,
                            error_flags=err)
        mg.grouped_gemm_dX(dY, W, r["m_sizes"], r["gather"], topk, PX, dX=dX, workspace=xws,
                           error_flags=err)
        mg.grouped_gemm_dW(X, dY, r["m_sizes"], r["gather"], topk, PX, dW=dW, workspace=wws,
                           error_flags=err)
        mg.combine(dX, topk, None, w, num_tokens=T, out=out, error_flags=err)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # eager, on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    eager = [t.clone() for t in outs]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in outs:
            t.fill_(7)  # eager work between replays, which the replay must overwrite
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b), f"replay {rep}"
    assert int(err.item()) == 0
