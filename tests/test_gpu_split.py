"""GPU parity of the split-perturbation (FedSPZO) step of the MLP against the
CPU oracle, through the C ABI: all 4 p1 ps losses, g1 and g2 as the stated
formulas of the GPU's own losses, and the weights after the step (both
blocks), on the configured MLP, ragged shapes, the largest ps, and a p1 that
needs more than one launch."""
import numpy as np
import pytest
import torch

from oracle import oracle
from zeroth_order_backprop_amd import zo

from test_gpu_fp32_models import DEV, LOSS_RTOL, W_ATOL, mlp_setup

pytestmark = pytest.mark.gpu


def _host_g(L, p1, ps, sig):
    g2 = (L[0::2] - L[1::2]) / (2.0 * sig)
    g1 = np.zeros(p1)
    for d in range(p1):
        sp = sm = 0.0
        for j in range(2 * ps):
            sp += L[2 * d * 2 * ps + j]
            sm += L[(2 * d + 1) * 2 * ps + j]
        g1[d] = (sp / (2 * ps) - sm / (2 * ps)) / (2.0 * sig)
    return g1, g2


def _run(setup_kw, p1, ps, eps=1e-2, lr=1e-2, steps=1, seed0=30):
    model, batch, keep, arena, obatch = mlp_setup(**setup_kw)
    sig = float(np.float32(eps))
    losses = torch.zeros(4 * p1 * ps, dtype=torch.float64, device=DEV)
    g1 = torch.zeros(p1, dtype=torch.float64, device=DEV)
    g2 = torch.zeros(2 * p1 * ps, dtype=torch.float64, device=DEV)
    for t in range(steps):
        model.step_split(batch, seed0 + t, p1, ps, eps, lr, losses, g1, g2)
        ol, og1, og2 = oracle.fedspzo_step(arena, obatch, seed=seed0 + t, p1=p1, ps=ps, eps=eps, lr=lr)
        torch.cuda.synchronize()
        gl = losses.cpu().numpy()
        np.testing.assert_allclose(gl, ol, rtol=LOSS_RTOL)
        h1, h2 = _host_g(gl, p1, ps, sig)
        np.testing.assert_allclose(g1.cpu().numpy(), h1, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g2.cpu().numpy(), h2, rtol=1e-12, atol=1e-12)
        w = model.arena.cpu().numpy().astype(np.float64)
        assert np.abs(w - arena.values()).max() <= W_ATOL, t
    return model, arena


@pytest.mark.parametrize("kw,p1,ps", [
    (dict(batch=64, d_in=64, hidden=256), 3, 2),
    (dict(batch=37, d_in=96, hidden=100, classes=3), 2, 3),
    (dict(batch=300, d_in=160, hidden=388, classes=16), 2, 2),
    (dict(batch=64, d_in=64, hidden=256), 1, 4),
])
def test_split_step_parity(kw, p1, ps):
    _run(kw, p1, ps, steps=2)


def test_split_step_many_launches():
    """p1 = 25 with ps = 2 on a 256-unit hidden layer needs two launches."""
    _run(dict(batch=64, d_in=64, hidden=256), 25, 2)


def test_split_step_full_mlp():
    """The 1024 -> 4096 -> 10 MLP, batch 256: p1 = 8, ps = 4 (p2 = 64)."""
    _run({}, 8, 4, eps=1e-3, lr=1e-3)


def test_split_step_refusals():
    model, batch, keep, arena, obatch = mlp_setup(batch=64, d_in=64, hidden=256)
    losses = torch.zeros(64, dtype=torch.float64, device=DEV)
    g1 = torch.zeros(8, dtype=torch.float64, device=DEV)
    g2 = torch.zeros(64, dtype=torch.float64, device=DEV)
    before = model.arena.clone()
    for p1, ps in ((0, 1), (2, 0), (2, 5)):
        with pytest.raises(zo.ZoError):
            model.step_split(batch, 0, p1, ps, 1e-3, 1e-3, losses, g1, g2)
    with pytest.raises(zo.ZoError):
        model.step_split(batch, 0, 2, 2, 0.0, 1e-3, losses, g1, g2)
    m2, b2, *_ = mlp_setup(batch=37, d_in=12, hidden=100, classes=3)  # d_in % 32 != 0
    with pytest.raises(zo.ZoError) as e:
        m2.step_split(b2, 0, 2, 2, 1e-3, 1e-3, losses, g1, g2)
    assert e.value.status == zo.ZO_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.equal(model.arena, before)


def test_split_step_nonfinite_skips_update():
    model, batch, (x, lab), arena, obatch = mlp_setup(batch=64, d_in=64, hidden=256)
    x[5, 3] = float("nan")
    before = model.arena.clone()
    losses = torch.zeros(16, dtype=torch.float64, device=DEV)
    g1 = torch.zeros(2, dtype=torch.float64, device=DEV)
    g2 = torch.zeros(8, dtype=torch.float64, device=DEV)
    model.step_split(batch, 0, 2, 2, 1e-3, 1e-2, losses, g1, g2)
    torch.cuda.synchronize()
    assert not np.isfinite(losses.cpu().numpy()).all()
    assert torch.equal(model.arena, before)
