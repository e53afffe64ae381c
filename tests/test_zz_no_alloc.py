"""moegg_route_noalloc (routing with the counts in the library's static device
array, for callers that cannot allocate) against moegg_route with a caller
workspace: bit-identical outputs on two calls in a row, the second smaller,
both large enough to take the multi-launch path that uses the counts."""

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
    import token_routing_amd as mg
    mg.load_library()
    return mg


def _outputs(S, E, dev="cuda"):
    return {"m_sizes": torch.full((E,), -7, dtype=torch.int32, device=dev),
            "offsets": torch.full((E + 1,), -7, dtype=torch.int32, device=dev),
            "padded_offsets": torch.full((E + 1,), -7, dtype=torch.int32, device=dev),
            "tile_offsets": torch.full((E + 1,), -7, dtype=torch.int32, device=dev),
            "gather": torch.full((S,), -7, dtype=torch.int32, device=dev),
            "scatter": torch.full((S,), -7, dtype=torch.int32, device=dev)}


def test_route_noalloc_matches_route_twice(mg):
    big = synth.fine_down().ids                       # 65,536 slots, 128 experts (Zipf)
    small = torch.randint(0, 64, (2500, 8), generator=synth.generator(77), dtype=torch.int32)
    small[17, 3] = 64                                 # one dropped slot
    for ids, E, B in ((big, 128, 256), (small, 64, 128)):
        S = ids.numel()
        assert S > 4096 and mg.route_workspace_bytes(S, E) <= mg.ROUTE_NOALLOC_MAX_BYTES
        print(f"route_noalloc S={S} E={E} block_m={B}", flush=True)
        d = ids.cuda()
        e1 = torch.zeros(1, dtype=torch.int32, device="cuda")
        e2 = torch.zeros(1, dtype=torch.int32, device="cuda")
        ref = mg.moe_route(d, E, B, error_flags=e1)
        got = mg.moe_route_noalloc(d, E, B, out=_outputs(S, E), error_flags=e2)
        torch.cuda.synchronize()
        assert int(e1.item()) == int(e2.item())
        for k in ref:
            assert torch.equal(ref[k], got[k]), k
        o = oracle.route(ids.numpy().reshape(-1), E, B)
        for k in ("m_sizes", "offsets", "padded_offsets", "tile_offsets", "gather", "scatter"):
            assert np.array_equal(got[k].cpu().numpy(), o[k]), k


def test_route_noalloc_rejects_sizes_past_its_array(mg):
    E = 1024
    S = 65536 + 256                                   # 257 chunks x 1024 experts x 4 B > 1 MiB
    assert mg.route_workspace_bytes(S, E) > mg.ROUTE_NOALLOC_MAX_BYTES
    ids = torch.zeros(S, 1, dtype=torch.int32, device="cuda")
    with pytest.raises(mg.MoeggError) as e:
        mg.moe_route_noalloc(ids, E, 128, out=_outputs(S, E))
    assert e.value.status == 4
