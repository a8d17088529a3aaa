"""Captured decoder forwards (HIP graphs) against the same forwards launched
one by one.

A forward at the stored weights is captured on the second evaluation of a
(tokens, batch, seq) key and replayed from then on; with timing enabled the
library launches eagerly.  Every replay must give the eager loss bit for
bit, with eager work (in-place perturbations) and synchronisations between
the replays, for several keys, and a whole in-place step must leave the same
losses, g and weights.
"""
import numpy as np
import pytest
import torch

from test_gpu_decoder import decoder_setup
from zeroth_order_backprop_amd import zo

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _loss(model, batch, eager):
    zo.timing_enable(eager)
    try:
        out = torch.zeros(1, dtype=torch.float64, device=DEV)
        model.forward_loss(batch, out)
        torch.cuda.synchronize()
        return out.cpu().numpy()[0]
    finally:
        zo.timing_enable(False)
        zo.timing_reset()


def test_replayed_forward_equals_eager():
    model, b, tok, arena, obatch = decoder_setup()
    seen = []
    for k in range(6):
        model.perturb(11, k, 1e-2)  # eager work between the replays
        torch.cuda.synchronize()
        want = _loss(model, b, eager=True)
        got = _loss(model, b, eager=False)  # k = 0: first sight, 1: capture, then replays
        assert got == want, (k, got, want)
        seen.append(got)
    assert len(set(seen)) == len(seen)  # the weights changed between evaluations


def test_replayed_forward_per_batch():
    model, b1, tok1, arena, obatch = decoder_setup(seq=64)
    tok2 = torch.flip(tok1, dims=[1]).contiguous()
    b2 = zo.make_batch(tokens=tok2, batch=2, seq=64)
    for k in range(4):
        for b in (b1, b2):
            want = _loss(model, b, eager=True)
            assert _loss(model, b, eager=False) == want
        model.perturb(5, k, -1e-2)
        torch.cuda.synchronize()
    assert _loss(model, b1, eager=False) != _loss(model, b2, eager=False)


@pytest.mark.parametrize("n", [1, 4])
def test_inplace_step_with_graphs_equals_eager(n):
    model, b, tok, arena, obatch = decoder_setup()
    w0 = model.arena.clone()
    res = []
    for eager in (True, False, False):
        model.arena.copy_(w0)
        losses = torch.zeros(2 * n, dtype=torch.float64, device=DEV)
        g = torch.zeros(n, dtype=torch.float64, device=DEV)
        zo.timing_enable(eager)
        try:
            model.step(b, 21, n, 1e-3, 1e-2, zo.ZO_MODE_INPLACE, losses, g)
            torch.cuda.synchronize()
        finally:
            zo.timing_enable(False)
            zo.timing_reset()
        res.append((losses.cpu().numpy(), g.cpu().numpy(), model.arena.clone()))
    for losses, g, w in res[1:]:
        assert np.array_equal(losses, res[0][0])
        assert np.array_equal(g, res[0][1])
        assert torch.equal(w, res[0][2])
    assert not torch.equal(res[0][2], w0)


def test_timing_subfamilies_cover_the_layer_gemms():
    """The layer GEMMs are timed as gemm_bf16.{qkv,o,up,down}; the family name
    covers them (query and selection), one launch of each per layer."""
    layers = 2
    model, b, tok, arena, obatch = decoder_setup(layers=layers)
    zo.timing_reset()
    zo.timing_enable(True)
    try:
        out = torch.zeros(1, dtype=torch.float64, device=DEV)
        model.forward_loss(b, out)
        torch.cuda.synchronize()
        total = zo.timing_query("gemm_bf16")
        parts = {p: zo.timing_query(f"gemm_bf16.{p}") for p in ("qkv", "o", "up", "down")}
        assert all(n == layers for _, n in parts.values()), parts
        assert total[1] == 4 * layers
        assert abs(total[0] - sum(ms for ms, _ in parts.values())) <= 1e-6 * max(1.0, total[0])
        assert zo.timing_query("gemm_bf")[1] == 0  # a prefix that is not a family name covers nothing
        # selecting the family brackets its sub-families and nothing else
        zo.timing_reset()
        zo.timing_select("gemm_bf16")
        model.forward_loss(b, out)
        torch.cuda.synchronize()
        assert zo.timing_query("gemm_bf16")[1] == 4 * layers
        assert zo.timing_query("attention")[1] == 0
    finally:
        zo.timing_select(None)
        zo.timing_enable(False)
        zo.timing_reset()
