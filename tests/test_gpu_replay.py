"""Seed replay on the GPU, through the C ABI: a model trained for a few steps
is rebuilt bit for bit from its initial weights and the recorded (seed, g_i)
of each step, with the log written to and read back from disk.  Fused and
in-place steps, plain and 1.5-SPSA, fp32 (MLP) and bf16 (decoder) arenas."""
import numpy as np
import pytest
import torch

from zeroth_order_backprop_amd import checkpoint, zo

from test_gpu_decoder import decoder_setup
from test_gpu_fp32_models import DEV, mlp_setup

pytestmark = pytest.mark.gpu


def _train_and_replay(setup, tmp_path, schedule, n=4, eps=1e-2, lr=1e-3):
    model, batch, keep, arena, obatch = setup()
    w0 = model.arena.clone()
    log = checkpoint.StepLog()
    losses = torch.zeros(2 * n + 1, dtype=torch.float64, device=DEV)
    g = torch.zeros(n, dtype=torch.float64, device=DEV)
    for t, (mode, pc) in enumerate(schedule):
        model.step(batch, 100 + t, n, eps, lr, mode, losses, g, precond=pc, curv_floor=1.0)
        torch.cuda.synchronize()
        log.record(100 + t, n, eps, lr, mode, g)
    path = tmp_path / "steps.npz"
    log.save(path)
    trained = model.arena.clone()
    assert not torch.equal(trained, w0)
    model.arena.copy_(w0)
    checkpoint.replay(model, checkpoint.StepLog.load(path))
    torch.cuda.synchronize()
    assert torch.equal(model.arena, trained)


@pytest.mark.parametrize("mode", [zo.ZO_MODE_FUSED, zo.ZO_MODE_INPLACE])
def test_mlp_replay_is_bitwise(mode, tmp_path):
    _train_and_replay(lambda: mlp_setup(batch=64, d_in=64, hidden=256), tmp_path,
                      [(mode, 0), (mode, 1), (mode, 0), (mode, 1)])


def test_mlp_replay_mixed_modes(tmp_path):
    f, i = zo.ZO_MODE_FUSED, zo.ZO_MODE_INPLACE
    _train_and_replay(lambda: mlp_setup(batch=64, d_in=64, hidden=256), tmp_path,
                      [(f, 0), (i, 0), (i, 1), (f, 1), (f, 0)])


@pytest.mark.parametrize("mode", [zo.ZO_MODE_FUSED, zo.ZO_MODE_INPLACE])
def test_decoder_replay_is_bitwise(mode, tmp_path):
    _train_and_replay(lambda: decoder_setup(), tmp_path, [(mode, 0), (mode, 1), (mode, 0)], eps=1e-3, lr=1e-2)


def test_replay_rejects_bad_arguments():
    model, batch, keep, arena, obatch = mlp_setup(batch=64, d_in=64, hidden=256)
    before = model.arena.clone()
    g = torch.zeros(4, dtype=torch.float64, device=DEV)
    with pytest.raises(zo.ZoError):
        model.replay_step(0, 0, 1e-3, 1e-3, zo.ZO_MODE_FUSED, g)
    with pytest.raises(zo.ZoError):
        model.replay_step(0, 4, 0.0, 1e-3, zo.ZO_MODE_INPLACE, g)
    with pytest.raises(zo.ZoError):
        model.replay_step(0, 4, 1e-3, 1e-3, 7, g)
    with pytest.raises(ValueError):
        model.replay_step(0, 5, 1e-3, 1e-3, zo.ZO_MODE_FUSED, g)
    torch.cuda.synchronize()
    assert torch.equal(model.arena, before)
