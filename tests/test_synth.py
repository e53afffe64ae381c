"""The seeded generators: determinism, shapes and the routing properties the
workloads ask for (distinct experts per token, renormalised gates, Zipf skew
with empty experts)."""

import numpy as np
import torch

import synth


def test_deterministic_and_shaped():
    a, b = synth.tiny(), synth.tiny()
    assert torch.equal(a.ids, b.ids) and torch.equal(a.X.view(torch.int16), b.X.view(torch.int16))
    assert a.ids.shape == (128, 2) and a.ids.dtype == torch.int32
    assert a.X.shape == (128, 256) and a.W.shape == (8, 512, 256)
    assert a.X.dtype == torch.bfloat16
    # N(0, 0.02): sample std within a few percent
    assert abs(float(a.W.float().std()) - 0.02) < 0.002
    # distinct experts per token, weights are the chosen softmax probabilities (descending)
    ids = a.ids.numpy()
    assert all(len(set(r)) == 2 for r in ids)
    assert np.all(np.diff(a.weights.numpy(), axis=1) <= 0)


def test_zipf_routing_skew_and_gates():
    rank = synth.zipf_rank(128, synth.generator(1))
    ids, w = synth.route_zipf(2048, 128, 8, 1.2, rank, synth.generator(2))
    ids = ids.numpy()
    assert all(len(set(r)) == 8 for r in ids)
    assert np.allclose(w.sum(-1).numpy(), 1.0, atol=1e-6)
    h = np.bincount(ids.reshape(-1), minlength=128)
    never = (rank.numpy() > 120)
    assert np.all(h[never] == 0)
    # the most popular expert (rank 1) is the hottest
    assert h[int(np.argmin(rank.numpy()))] == h.max()


def test_dual_shapes():
    wl = synth.dual()
    (x0, w0), (x1, w1) = wl.groups
    assert x0.shape == (512, 1024) and w0.shape == (1024, 2048)
    assert x1.shape == (256, 1024) and w1.shape == (1024, 4096)
    assert abs(float(w1.float().std()) - 1 / 32) < 1e-3
