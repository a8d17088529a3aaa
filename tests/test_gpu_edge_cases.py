"""GPU edge cases of the step's entry points, through the C ABI: empty
ranges, zero scales (exact no-ops), a batch smaller than the model was sized
for, and single-probe steps in both modes, each against the CPU oracle or an
exact invariant."""
import numpy as np
import pytest
import torch

from oracle import oracle
from zeroth_order_backprop_amd import inputs, zo

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _arena(dtype, n, seed=0):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal(n).astype(np.float32)
    if dtype == zo.ZO_F32:
        return torch.from_numpy(w).to(DEV)
    return torch.from_numpy(inputs.f32_to_bf16_bits(w).view(np.int16)).to(DEV)


@pytest.mark.parametrize("dtype", [zo.ZO_F32, zo.ZO_BF16])
def test_empty_ranges_are_noops(dtype):
    w = _arena(dtype, 4096)
    before = w.clone()
    g = torch.ones(2, dtype=torch.float64, device=DEV)
    zo.perturb_buffer(w, 0, 0, 7, 0, 1.0, dtype)
    zo.update_buffer(w, 0, 0, 7, 2, g, 1.0, dtype)
    z = torch.full((8,), 3.0, dtype=torch.float32, device=DEV)
    zo.debug_rng(7, 0, 0, 0, z=z)
    torch.cuda.synchronize()
    assert torch.equal(w, before)
    assert (z.cpu() == 3.0).all()


@pytest.mark.parametrize("dtype", [zo.ZO_F32, zo.ZO_BF16])
def test_zero_scale_is_exact_noop(dtype):
    """sigma = 0 perturbs nothing and g = 0 updates nothing, bit for bit: every
    direction value is finite, so fma(0, z, w) = w."""
    n = (1 << 16) + 37
    w = _arena(dtype, n, seed=1)
    before = w.clone()
    zo.perturb_buffer(w, n, 0, 3, 5, 0.0, dtype)
    g = torch.zeros(4, dtype=torch.float64, device=DEV)
    zo.update_buffer(w, n, 0, 3, 4, g, 1e-3, dtype)
    torch.cuda.synchronize()
    assert torch.equal(w, before)


def _mlp(batch_model, d_in=1024, hidden=4096, classes=10):
    inp = inputs.mlp_inputs(0, batch=batch_model, d_in=d_in, hidden=hidden, classes=classes)
    odesc = {"kind": "mlp", "batch": batch_model, "d_in": d_in, "hidden": hidden, "classes": classes}
    desc = zo.make_desc(zo.ZO_MODEL_MLP, batch=batch_model, d_in=d_in, hidden=hidden, classes=classes)
    layout, total = oracle.param_layout(odesc)
    arena = np.zeros(total, np.float32)
    for name, off, shape in layout:
        arena[off:off + int(np.prod(shape))] = inp[name].ravel()
    model = zo.Model(desc, torch.from_numpy(arena.copy()).to(DEV))
    return model, inp, oracle.Arena(odesc, arena)


def test_mlp_batch_smaller_than_model():
    """A model sized for 256 rows evaluated on the first 100 (ragged against
    the 256-row tiles); stored and paired perturbed evaluations."""
    model, inp, arena = _mlp(256)
    rows = 100
    x = torch.from_numpy(inp["X"]).to(DEV)
    lab = torch.from_numpy(inp["labels"]).to(DEV)
    b = zo.make_batch(x=x, labels=lab, batch=rows)
    obatch = {"X": inp["X"][:rows], "labels": inp["labels"][:rows]}
    eps = float(np.float32(1e-3))
    perts = [(9, 0, eps), (9, 0, -eps), (9, 1, eps), (9, 1, -eps)]
    out = torch.zeros(1 + len(perts), dtype=torch.float64, device=DEV)
    model.forward_loss(b, out[:1])
    model.forward_loss(b, out[1:], perts=perts)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = [oracle.model_loss(arena, obatch)]
    for s, i, sg in perts:
        a = arena.copy()
        a.perturb(s, i, sg)
        want.append(oracle.model_loss(a, obatch))
    np.testing.assert_allclose(got, want, rtol=1e-5)


@pytest.mark.parametrize("mode", [zo.ZO_MODE_FUSED, zo.ZO_MODE_INPLACE])
def test_single_probe_step(mode):
    """N = 1: one direction, two evaluations, one update."""
    model, inp, arena = _mlp(64, d_in=64, hidden=256)
    x = torch.from_numpy(inp["X"]).to(DEV)
    lab = torch.from_numpy(inp["labels"]).to(DEV)
    b = zo.make_batch(x=x, labels=lab, batch=64)
    obatch = {"X": inp["X"], "labels": inp["labels"]}
    losses = torch.zeros(2, dtype=torch.float64, device=DEV)
    g = torch.zeros(1, dtype=torch.float64, device=DEV)
    model.step(b, 11, 1, 1e-3, 1e-3, mode, losses, g)
    torch.cuda.synchronize()
    ol, og = oracle.spsa_step(arena, obatch, seed=11, n_probes=1, eps=1e-3, lr=1e-3,
                              mode="fused" if mode == zo.ZO_MODE_FUSED else "inplace")
    np.testing.assert_allclose(losses.cpu().numpy(), ol, rtol=1e-5)
    assert g.item() == pytest.approx(og[0], rel=1e-2, abs=1e-3)
    w = model.arena.cpu().numpy().astype(np.float64)
    assert np.abs(w - arena.values()).max() <= 1e-5


@pytest.mark.parametrize("pos,val", [(0, -1), (17, 500), (63, 1 << 30), (64 + 5, 999)])
@pytest.mark.parametrize("fused", [False, True])
def test_decoder_token_out_of_range_gives_nan(pos, val, fused):
    """A token id outside [0, vocab) reads nothing out of bounds; the loss of
    every evaluation that sees it is NaN (first, middle and last position of
    a sequence; negative and too-large ids), and a step then leaves the
    weights unchanged."""
    from test_gpu_decoder import decoder_setup
    model, b, tok, arena, obatch = decoder_setup()
    bad = tok.clone()
    bad.view(-1)[pos] = val
    bb = zo.make_batch(tokens=bad, batch=2, seq=64)
    eps = float(np.float32(1e-3))
    out = torch.zeros(2, dtype=torch.float64, device=DEV)
    model.forward_loss(bb, out, perts=[(3, 0, eps), (3, 0, -eps)] if fused else None)
    torch.cuda.synchronize()
    vals = out.cpu().numpy()[:2 if fused else 1]
    assert np.isnan(vals).all(), vals
    before = model.arena.clone()
    losses = torch.zeros(2, dtype=torch.float64, device=DEV)
    g = torch.zeros(1, dtype=torch.float64, device=DEV)
    model.step(bb, 5, 1, 1e-3, 1e-3, zo.ZO_MODE_FUSED if fused else zo.ZO_MODE_INPLACE, losses, g)
    torch.cuda.synchronize()
    assert not np.isfinite(g.cpu().numpy()).any()
    if fused:
        assert torch.equal(model.arena, before)
    else:
        # in place the perturb / restore passes ran and no update followed:
        # the same three passes on a copy give the same bits
        ref = before.clone()
        for sg in (eps, -2 * eps, eps):
            zo.perturb_buffer(ref, ref.numel(), 0, 5, 0, sg, zo.ZO_BF16)
        torch.cuda.synchronize()
        assert torch.equal(model.arena, ref)
    # the good batch still evaluates to the oracle's loss afterwards
    good = torch.zeros(1, dtype=torch.float64, device=DEV)
    model2, b2, _, arena2, obatch2 = decoder_setup()
    model2.forward_loss(b2, good)
    torch.cuda.synchronize()
    assert good.item() == pytest.approx(oracle.model_loss(arena2, obatch2), rel=2e-3)


@pytest.mark.parametrize("val", [-1, 10, 77])
def test_mlp_label_out_of_range_gives_nan(val):
    """A label outside [0, classes) makes the loss NaN in the stored and the
    fused evaluations (and so the step skips its update)."""
    model, inp, arena = _mlp(64, d_in=64, hidden=256)
    x = torch.from_numpy(inp["X"]).to(DEV)
    lab = torch.from_numpy(inp["labels"]).to(DEV)
    lab[13] = val
    b = zo.make_batch(x=x, labels=lab, batch=64)
    out = torch.zeros(3, dtype=torch.float64, device=DEV)
    eps = float(np.float32(1e-3))
    model.forward_loss(b, out[:1])
    model.forward_loss(b, out[1:], perts=[(2, 0, eps), (2, 0, -eps)])
    before = model.arena.clone()
    losses = torch.zeros(4, dtype=torch.float64, device=DEV)
    g = torch.zeros(2, dtype=torch.float64, device=DEV)
    model.step(b, 3, 2, 1e-3, 1e-3, zo.ZO_MODE_FUSED, losses, g)
    torch.cuda.synchronize()
    assert np.isnan(out.cpu().numpy()).all()
    assert torch.equal(model.arena, before)


def test_make_batch_rejects_wrong_tensors():
    x = torch.zeros(8, 4, dtype=torch.float64, device=DEV)
    with pytest.raises(ValueError):
        zo.make_batch(x=x, batch=8)
    tok = torch.zeros(2, 8, dtype=torch.int64, device=DEV)
    with pytest.raises(ValueError):
        zo.make_batch(tokens=tok, batch=2, seq=8)
    tok32 = torch.zeros(8, 2, dtype=torch.int32, device=DEV).t()
    with pytest.raises(ValueError):
        zo.make_batch(tokens=tok32, batch=2, seq=8)
