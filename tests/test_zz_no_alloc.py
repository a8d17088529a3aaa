"""zo_step_noalloc (the step for callers that cannot allocate) against zo_step,
through the C ABI: the same kernels on the library's static scratch instead of
a caller workspace, so losses, scalars and weights must be bit-identical.
Two calls in a row on one GPU, the second with a smaller input, for the
least-squares model and the MLP in both modes; a model whose workspace
exceeds the scratch is refused before anything runs."""
import numpy as np
import pytest
import torch

from oracle import oracle
from zeroth_order_backprop_amd import inputs, zo

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _mlp(batch, d_in, hidden, classes, seed):
    inp = inputs.mlp_inputs(seed, batch=batch, d_in=d_in, hidden=hidden, classes=classes)
    odesc = {"kind": "mlp", "batch": batch, "d_in": d_in, "hidden": hidden, "classes": classes}
    desc = zo.make_desc(zo.ZO_MODEL_MLP, batch=batch, d_in=d_in, hidden=hidden, classes=classes)
    layout, total = oracle.param_layout(odesc)
    arena = np.zeros(total, np.float32)
    for name, off, shape in layout:
        arena[off:off + int(np.prod(shape))] = inp[name].ravel()
    x = torch.from_numpy(inp["X"]).to(DEV)
    lab = torch.from_numpy(inp["labels"]).to(DEV)
    return desc, arena, zo.make_batch(x=x, labels=lab, batch=batch)


def _lsq(n, d_in, d_out, seed):
    inp = inputs.lsq_inputs(seed, n=n, d_in=d_in, d_out=d_out)
    desc = zo.make_desc(zo.ZO_MODEL_LSQ, batch=n, d_in=d_in, d_out=d_out)
    x = torch.from_numpy(inp["X"]).to(DEV)
    y = torch.from_numpy(inp["Y"]).to(DEV)
    return desc, inp["W"].ravel().copy(), zo.make_batch(x=x, y=y, batch=n)


def _both(desc, arena, batch, seed, n, eps, lr, mode, precond=0):
    """(losses, g, weights) of zo_step and of zo_step_noalloc from the same start."""
    out = []
    for which in ("step", "noalloc"):
        w = torch.from_numpy(arena.copy()).to(DEV)
        losses = torch.full((2 * n + 1,), -1.0, dtype=torch.float64, device=DEV)
        g = torch.full((n,), -1.0, dtype=torch.float64, device=DEV)
        if which == "step":
            m = zo.Model(desc, w)
            m.step(batch, seed, n, eps, lr, mode, losses, g, precond=precond, curv_floor=1.0)
        else:
            zo.step_noalloc(desc, w, batch, seed, n, eps, lr, mode, losses, g, precond=precond, curv_floor=1.0)
        torch.cuda.synchronize()
        out.append((losses.cpu().numpy(), g.cpu().numpy(), w.cpu().numpy()))
    return out


def _same(a, b):
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


@pytest.mark.parametrize("mode", [zo.ZO_MODE_FUSED, zo.ZO_MODE_INPLACE])
def test_noalloc_mlp_two_calls(mode):
    # the MLP workload's full size (its workspace is about 46 MiB of the 64 MiB)
    desc, arena, batch = _mlp(256, 1024, 4096, 10, seed=0)
    a, b = _both(desc, arena, batch, 5, 16, 1e-3, 1e-3, mode)
    _same(a, b)
    assert np.isfinite(a[0][:32]).all() and not np.array_equal(a[2], arena)
    # then a smaller model and batch on the same scratch (it keeps the last call's contents)
    desc2, arena2, batch2 = _mlp(100, 64, 256, 7, seed=1)
    a, b = _both(desc2, arena2, batch2, 6, 3, 1e-3, 1e-2, mode, precond=1)
    _same(a, b)


def test_noalloc_lsq_two_calls():
    desc, arena, batch = _lsq(512, 256, 256, seed=0)
    a, b = _both(desc, arena, batch, 3, 4, 1e-3, 1e-2, zo.ZO_MODE_FUSED)
    _same(a, b)
    desc2, arena2, batch2 = _lsq(200, 64, 48, seed=2)
    a, b = _both(desc2, arena2, batch2, 4, 2, 1e-3, 1e-3, zo.ZO_MODE_INPLACE)
    _same(a, b)


def test_noalloc_refuses_large_workspace():
    """The GPT-small-shaped decoder at 8 x 512 tokens needs about 68 MiB of
    workspace: refused, nothing launched."""
    desc = zo.make_desc(zo.ZO_MODEL_DECODER, batch=8, seq=512, layers=12, d_model=768, heads=12, ffn=3072,
                        vocab=32000, max_seq=512)
    assert zo.workspace_bytes(desc) > 64 << 20
    _, total = zo.param_layout(desc)
    w = torch.zeros(total, dtype=torch.int16, device=DEV)
    tok = torch.zeros(8, 512, dtype=torch.int32, device=DEV)
    batch = zo.make_batch(tokens=tok, batch=8, seq=512)
    losses = torch.zeros(2, dtype=torch.float64, device=DEV)
    g = torch.zeros(1, dtype=torch.float64, device=DEV)
    with pytest.raises(zo.ZoError) as e:
        zo.step_noalloc(desc, w, batch, 0, 1, 1e-3, 1e-3, zo.ZO_MODE_INPLACE, losses, g)
    assert e.value.status == zo.ZO_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert not w.any()
