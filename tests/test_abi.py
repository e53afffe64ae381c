"""CPU checks of the C ABI: libmoegg.so loads, exports every function that
include/moegg.h declares, and rejects bad arguments on the host with the
documented status codes before any GPU call is made."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moegg.h")


@pytest.fixture(scope="module")
def lib():
    import token_routing_amd as mg
    if not os.path.exists(mg.LIB_PATH):
        from token_routing_amd import build
        build.build()
    return mg.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moegg_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert lib.moegg_version() >= 100
    for code in range(6):
        assert lib.moegg_status_string(code)


def test_route_workspace_size(lib):
    # one int32 count per (expert, 256-slot chunk)
    assert lib.moegg_route_workspace_bytes(65536, 128) == 256 * 128 * 4
    assert lib.moegg_route_workspace_bytes(1, 8) == 8 * 4
    assert lib.moegg_route_workspace_bytes(0, 8) == 0


EINVAL, ESHAPE, EUNSUP, EWS = 1, 2, 3, 4
PX, PY, FM, F32, GS = 1, 2, 4, 8, 32
FAKE = ctypes.c_void_p(1 << 20)  # never dereferenced: every case fails on the host


@pytest.mark.parametrize("flags,want", [
    (PX | PY, EINVAL),        # cannot permute both X and Y
    (FM, EINVAL),             # fuse_mul_post requires permute_y
    (PX | FM, EINVAL),
    (16, EINVAL),             # unknown flag
    (64, EINVAL),
    (GS | PY, EINVAL),        # the gated activation belongs to the first GEMM
    (GS | PY | FM, EINVAL),
])
def test_fwd_flag_checks(lib, flags, want):
    st = lib.moegg_grouped_gemm_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 10, 2, 8, 64, 64, flags, FAKE,
                                    None, None)
    assert st == want


def test_fwd_missing_pointers(lib):
    # permute flag without gather indices; fuse_mul_post without weights
    assert lib.moegg_grouped_gemm_fwd(FAKE, FAKE, FAKE, None, None, 10, 2, 8, 64, 64, PX, FAKE,
                                      None, None) == EINVAL
    assert lib.moegg_grouped_gemm_fwd(FAKE, FAKE, FAKE, FAKE, None, 10, 2, 8, 64, 64, PY | FM,
                                      FAKE, None, None) == EINVAL


@pytest.mark.parametrize("T,k,E,N,K", [(-1, 2, 8, 64, 64), (10, 0, 8, 64, 64), (10, 2, 0, 64, 64),
                                       (10, 2, 1025, 64, 64), (10, 2, 8, 0, 64),
                                       (10, 2, 8, 64, 0)])
def test_fwd_shape_checks(lib, T, k, E, N, K):
    assert lib.moegg_grouped_gemm_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, T, k, E, N, K, 0, FAKE, None,
                                      None) == ESHAPE


ODD = ctypes.c_void_p((1 << 20) + 1)  # not even 2-byte aligned: never valid for bf16


def test_misaligned_element_pointers(lib):
    # any K and N are accepted (rows that are not whole 16-byte chunks take
    # the any-shape kernels), but a bf16 operand must be 2-byte aligned
    assert lib.moegg_grouped_gemm_fwd(ODD, FAKE, FAKE, FAKE, FAKE, 10, 2, 8, 60, 70, 0, FAKE,
                                      None, None) == ESHAPE
    assert lib.moegg_grouped_gemm_dX(FAKE, FAKE, FAKE, FAKE, 10, 2, 8, 60, 70, 0, ODD, None, 0,
                                     None, None) == ESHAPE
    assert lib.moegg_grouped_gemm_dW(FAKE, ODD, FAKE, FAKE, 10, 2, 8, 60, 70, 0, FAKE, None, 0,
                                     None, None) == ESHAPE
    # fp32 dW needs 4-byte alignment
    two = ctypes.c_void_p((1 << 20) + 2)
    assert lib.moegg_grouped_gemm_dW(FAKE, FAKE, FAKE, FAKE, 10, 2, 8, 60, 70, F32, two, None, 0,
                                     None, None) == ESHAPE


def test_gated_shape_and_backward_checks(lib):
    # W rows come in (gate, linear) pairs: N must be even
    assert lib.moegg_grouped_gemm_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 10, 2, 8, 41, 64, GS | PX,
                                      FAKE, None, None) == ESHAPE
    # the backward kernels take no activation flag
    assert lib.moegg_grouped_gemm_dX(FAKE, FAKE, FAKE, FAKE, 10, 2, 8, 64, 64, GS, FAKE, None, 0,
                                     None, None) == EINVAL
    assert lib.moegg_grouped_gemm_dW(FAKE, FAKE, FAKE, FAKE, 10, 2, 8, 64, 64, GS, FAKE, None,
                                     0, None, None) == EINVAL


def test_dx_workspace_checks(lib):
    # invalid sizes answer 0 before the device is queried
    assert lib.moegg_grouped_gemm_dX_workspace_bytes(-1, 2, 8, 64, 64) == 0
    assert lib.moegg_grouped_gemm_dX_workspace_bytes(10, 2, 8, 60, 64) == 0


def test_dw_workspace(lib):
    # fine-grained layer: 65536 slots, 2048 x 768 per expert -> chunks of 2048 rows,
    # fewer than 64 partials of 2048 x 768 fp32 after a 256-byte-aligned header
    hdr = (4 + 12 * 128 + 255) // 256 * 256
    assert lib.moegg_grouped_gemm_dW_workspace_bytes(8192, 8, 128, 2048, 768) == \
        hdr + 64 * 2048 * 768 * 4
    # Mixtral-shaped layer: an expert can never exceed the chunk length
    assert lib.moegg_grouped_gemm_dW_workspace_bytes(4096, 2, 8, 28672, 4096) == 0
    assert lib.moegg_grouped_gemm_dW_workspace_bytes(-1, 2, 8, 64, 64) == 0
    # a decode step (64 tokens, top-8: 512 slots) is never split
    assert lib.moegg_grouped_gemm_dW_workspace_bytes(64, 8, 128, 2048, 768) == 0
    assert lib.moegg_grouped_gemm_dW_workspace_bytes(129, 8, 128, 2048, 768) > 0
    # a workspace smaller than needed is rejected before anything runs
    assert lib.moegg_grouped_gemm_dW(FAKE, FAKE, FAKE, FAKE, 8192, 8, 128, 2048, 768, PY, FAKE,
                                     FAKE, 1024, None, None) == EWS


def test_dw_gather_copy_size_rule(lib):
    """The X copy of dW under permute_x is an operand like X: only below 2 GiB.

    With room for it the gather workspace is the split area (256-byte aligned)
    plus S*K*2; at S*K*2 >= 2^31 it is the split area alone (the rows are then
    gathered inside the reduction), even where T*K*2 is far below 2 GiB."""
    def both(T, k, E, N, K):
        return (lib.moegg_grouped_gemm_dW_gather_workspace_bytes(T, k, E, N, K),
                lib.moegg_grouped_gemm_dW_workspace_bytes(T, k, E, N, K))

    g, w = both(300, 2, 4, 72, 264)
    assert g == (w + 255) // 256 * 256 + 300 * 2 * 264 * 2
    # S*K*2 one row below 2 GiB: the copy is still offered
    g, w = both(16383, 8, 4, 64, 8192)
    assert g == (w + 255) // 256 * 256 + 16383 * 8 * 8192 * 2
    # exactly 2 GiB, and above it with T*K*2 = 328 MB: no copy
    for T in (16384, 20000):
        g, w = both(T, 8, 4, 64, 8192)
        assert T * 8192 * 2 < 2 ** 31 <= T * 8 * 8192 * 2
        assert g == w and w > 0
    # a short launch (S <= 1024 and S <= 16 E) never copies
    assert both(64, 8, 128, 2048, 768) == (0, 0)
    assert both(64, 8, 32, 2048, 768) == (0, 0)
    g, w = both(64, 8, 31, 2048, 768)          # 512 slots > 16 x 31
    assert w == 0 and g == 512 * 768 * 2


def test_operand_size_limit(lib):
    # one expert's W of 2 GiB does not fit 32-bit buffer offsets
    assert lib.moegg_grouped_gemm_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 10, 2, 8, 32768, 32768, 0,
                                      FAKE, None, None) == ESHAPE


def test_backward_rejects_fuse_mul(lib):
    assert lib.moegg_grouped_gemm_dX(FAKE, FAKE, FAKE, FAKE, 10, 2, 8, 64, 64, FM, FAKE, None, 0,
                                     None, None) == EUNSUP
    assert lib.moegg_grouped_gemm_dW(FAKE, FAKE, FAKE, FAKE, 10, 2, 8, 64, 64, FM, FAKE, None,
                                     0, None, None) == EUNSUP
    assert lib.moegg_grouped_gemm_dX(FAKE, FAKE, FAKE, FAKE, 10, 2, 8, 64, 64, PX | PY, FAKE,
                                     None, 0, None, None) == EINVAL
    assert lib.moegg_grouped_gemm_dW(FAKE, FAKE, FAKE, None, 10, 2, 8, 64, 64, PY, FAKE, None,
                                     0, None, None) == EINVAL
    assert lib.moegg_grouped_gemm_dX(FAKE, FAKE, FAKE, FAKE, 10, 2, 8, 64, 64, F32, FAKE, None, 0,
                                     None, None) == EINVAL


def test_route_checks(lib):
    assert lib.moegg_route(FAKE, 10, 2, 8, 0, FAKE, FAKE, None, None, FAKE, None, FAKE, 1 << 20,
                           None, None) == ESHAPE
    assert lib.moegg_route(FAKE, 10, 2, 2000, 32, FAKE, FAKE, None, None, FAKE, None, FAKE,
                           1 << 20, None, None) == ESHAPE
    assert lib.moegg_route(FAKE, 10, 2, 8, 32, FAKE, FAKE, None, None, FAKE, None, FAKE, 4, None,
                           None) == EWS
    assert lib.moegg_route(FAKE, 10, 2, 8, 32, None, FAKE, None, None, FAKE, None, FAKE, 1 << 20,
                           None, None) == EINVAL


def test_groups_checks(lib):
    import token_routing_amd as mg
    g = (mg.MoeggGroup * 2)()
    g[0] = mg.MoeggGroup(1 << 20, 1 << 20, 1 << 20, 16, 64, 64, 64, 64, 64)
    g[1] = mg.MoeggGroup(1 << 20, (1 << 20) + 1, 1 << 20, 16, 60, 64, 64, 64, 64)  # odd address
    assert lib.moegg_grouped_gemm_groups(g, 2, 0, None) == ESHAPE
    assert lib.moegg_grouped_gemm_groups(g, 1, 2, None) == EINVAL       # bad trans_b
    assert lib.moegg_grouped_gemm_groups(g, 0, 0, None) == ESHAPE       # no groups
    assert lib.moegg_grouped_gemm_groups(g, 17, 0, None) == ESHAPE
    g[1] = mg.MoeggGroup(1 << 20, 1 << 20, 1 << 20, 16, 64, 64, 32, 64, 64)  # ldx < k
    assert lib.moegg_grouped_gemm_groups(g, 2, 0, None) == ESHAPE


def test_combine_checks(lib):
    CF32 = 16
    # an odd address (any N is accepted); negative tokens; slot-order Y with too few rows
    assert lib.moegg_combine(ODD, None, None, 10, 2, 60, 20, 0, FAKE, None, None) == EINVAL
    assert lib.moegg_combine(FAKE, None, None, -1, 2, 64, 20, 0, FAKE, None, None) == ESHAPE
    assert lib.moegg_combine(FAKE, None, None, 10, 2, 64, 19, 0, FAKE, None, None) == ESHAPE
    assert lib.moegg_combine(FAKE, None, None, 10, 0, 64, 20, 0, FAKE, None, None) == ESHAPE
    # unknown flag, NULL output
    assert lib.moegg_combine(FAKE, None, None, 10, 2, 64, 20, 32, FAKE, None, None) == EINVAL
    assert lib.moegg_combine(FAKE, None, None, 10, 2, 64, 20, CF32, None, None, None) == EINVAL
    # zero tokens: no-op even with NULL pointers
    assert lib.moegg_combine(None, None, None, 0, 2, 64, 0, 0, None, None, None) == 0
    # backward: dw needs the forward input
    assert lib.moegg_combine_bwd(FAKE, None, None, None, 10, 2, 64, 20, FAKE, FAKE, None,
                                 None) == EINVAL
    assert lib.moegg_combine_bwd(FAKE, FAKE, None, None, 10, 2, 60, -1, FAKE, None, None,
                                 None) == ESHAPE
    assert lib.moegg_combine_bwd(None, None, None, None, 0, 2, 64, 0, None, None, None,
                                 None) == 0
