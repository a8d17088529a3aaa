"""Seed replay on the GPU, through the C ABI: a model trained for a few steps
is rebuilt bit for bit from its initial weights and the recorded (seed, g_i)
of each step, with the log written to and read back from disk.  Fused and
in-place steps, plain and 1.5-SPSA, fp32 (MLP) and bf16 (decoder) arenas.

The same log is also replayed by the CPU oracle from the same initial weights
(FedSPZO summary, "통신 프로토콜": the server rebuilds the client's model from
the seeds and the scalar gradients alone): in place the step's 3N perturb /
restore passes in order, then the update with c_i = -lr g_i / N.  The oracle's
weights must match the GPU-trained ones to 1e-5 absolute (fp32) or, for bf16,
bit for bit except at rounding boundaries (GPU directions are within 1e-6 of
the oracle's, which can move a value that sits at a boundary by one ulp)."""
import numpy as np
import pytest
import torch

from oracle import oracle
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
    # the oracle rebuilds the same weights from the log alone
    log = checkpoint.StepLog.load(path)
    rebuilt, peak = oracle_replay(arena.copy(), log)
    if rebuilt.dtype == "f32":
        got = trained.cpu().numpy().astype(np.float64)
        assert np.abs(got - rebuilt.values()).max() <= 1e-5
    else:
        got = oracle.bf16_bits_to_f64(trained.cpu().numpy().view(np.uint16))
        want = rebuilt.values()
        # GPU directions are within 1e-6 of the oracle's and the GPU rounds
        # through fp32: a value at a rounding boundary can land one ulp away,
        # an ulp of the magnitude the value had then (the largest along the
        # trajectory), which its final magnitude's ulp does not bound
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(peak, 2.0**-126))) - 7)
        r = np.abs(got - want) / ulp
        bad = r > 3.0001
        print(f"bf16 replay: {np.mean(got != want):.2e} of elements differ, max {r.max():.2f} ulp of the peak")
        assert not bad.any(), (np.nonzero(bad)[0][:8], got[bad][:8], want[bad][:8], peak[bad][:8])
        assert np.mean(got == want) >= 0.999


def oracle_replay(arena, log):
    """The oracle's own replay of a step log: for each step, in place its
    perturb / restore passes (+eps, -2 eps, +eps per probe, in probe order),
    then W <- D(W + sum_i c_i z_i) with c_i = -lr g_i / N.  Returns the arena
    and each element's largest magnitude along the way."""
    peak = np.abs(arena.values())
    for st in log.steps:
        n, eps = st["n_probes"], st["eps"]
        if st["mode"] == zo.ZO_MODE_INPLACE:
            for i in range(n):
                for sg in (eps, -2.0 * eps, eps):
                    arena.perturb(st["seed"], i, sg)
                    peak = np.maximum(peak, np.abs(arena.values()))
        arena.update(st["seed"], -st["lr"] * np.asarray(st["g"], np.float64) / n)
        peak = np.maximum(peak, np.abs(arena.values()))
    return arena, peak


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
