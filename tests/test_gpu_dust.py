"""GPU parity of the Dust step of the MLP (activation noise with per-token
rewards) against the CPU oracle, through the C ABI: the clean, hidden-draw
and head-draw per-token losses, and both weight blocks after the step, on the
configured MLP and on ragged shapes (hidden units past the 128-wide tiles,
tokens past the 64-row tiles, 3 and 16 classes); refusals and non-finite
losses."""
import numpy as np
import pytest
import torch

from oracle import oracle
from zeroth_order_backprop_amd import zo

from test_gpu_fp32_models import DEV, LOSS_RTOL, W_ATOL, mlp_setup

pytestmark = pytest.mark.gpu


def _run(kw, k1, k2, s1=0.1, s2=0.1, lr=1e-3, steps=1, seed0=50):
    model, batch, keep, arena, obatch = mlp_setup(**kw)
    M = kw.get("batch", 256)
    losses = torch.zeros((1 + k1 + k2) * M, dtype=torch.float64, device=DEV)
    for t in range(steps):
        model.step_dust(batch, seed0 + t, k1, k2, s1, s2, lr, losses)
        l1, l2, l0, _, _ = oracle.dust_step(arena, obatch, seed=seed0 + t, k1=k1, sigma1=s1, k2=k2, sigma2=s2, lr=lr)
        torch.cuda.synchronize()
        got = losses.cpu().numpy()
        np.testing.assert_allclose(got[:M], l0, rtol=LOSS_RTOL)
        np.testing.assert_allclose(got[M:(1 + k1) * M].reshape(k1, M), l1, rtol=LOSS_RTOL)
        np.testing.assert_allclose(got[(1 + k1) * M:].reshape(k2, M), l2, rtol=LOSS_RTOL)
        w = model.arena.cpu().numpy().astype(np.float64)
        assert np.abs(w - arena.values()).max() <= W_ATOL, t
    return model, arena


@pytest.mark.parametrize("kw,k1,k2", [
    (dict(batch=64, d_in=64, hidden=256), 8, 16),
    (dict(batch=96, d_in=160, hidden=100, classes=3), 5, 7),
    (dict(batch=64, d_in=96, hidden=388, classes=16), 3, 4),
])
def test_dust_step_parity(kw, k1, k2):
    _run(kw, k1, k2, steps=2)


def test_dust_step_full_mlp():
    """The 1024 -> 4096 -> 10 MLP, batch 256: k1 = 64 hidden draws, k2 = 256 head draws."""
    _run({}, 64, 256, s1=0.05, s2=0.05, lr=1e-4)


def test_dust_refusals_and_nonfinite():
    model, batch, (x, lab), arena, obatch = mlp_setup(batch=64, d_in=64, hidden=256)
    losses = torch.zeros(64 * 200, dtype=torch.float64, device=DEV)
    before = model.arena.clone()
    for k1, k2, s in ((0, 1, 0.1), (129, 1, 0.1), (2, 0, 0.1), (2, 2, 0.0)):
        with pytest.raises(zo.ZoError):
            model.step_dust(batch, 0, k1, k2, s, s, 1e-3, losses)
    m2, b2, *_ = mlp_setup(batch=37, d_in=64, hidden=100, classes=3)  # batch % 32 != 0
    with pytest.raises(zo.ZoError) as e:
        m2.step_dust(b2, 0, 2, 2, 0.1, 0.1, 1e-3, losses)
    assert e.value.status == zo.ZO_ERR_UNSUPPORTED
    x[3, 5] = float("nan")
    model.step_dust(batch, 0, 2, 2, 0.1, 0.1, 1e-3, losses)
    torch.cuda.synchronize()
    assert not np.isfinite(losses.cpu().numpy()[:64 * 5]).all()
    assert torch.equal(model.arena, before)
