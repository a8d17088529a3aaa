"""The copies step mode (ZO_MODE_COPIES) against the oracle and the fused mode.

The step is the multi-probe SPSA step of the ZOO blog ("backprop의 메모리
세금"): for each probe i the losses at W + eps z_i and W - eps z_i, then
g_i = (L+_i - L-_i) / (2 eps) and the update W <- D(W - (lr / N) sum g_i z_i).
In the copies mode the evaluated weights D(W +- eps z_i) are written to
their own copies of the arena (one pass per group of P probes) and the 2P
copies are evaluated side by side in one forward; W itself changes only in the
update.  Those are the weights the fused reading evaluates, so the oracle's
fused step is the reference: losses within the bf16 loss bar (2e-3 relative),
weights within the bound that the loss noise in g allows.
"""
import os

import numpy as np
import pytest
import torch

from helpers import oracle_par
from oracle import oracle
from test_gpu_decoder import LOSS_RTOL, decoder_setup, from_bf16_dev, ulp_bf16
from zeroth_order_backprop_amd import inputs, zo

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _step(model, b, seed, n, eps, lr, mode, precond=0):
    losses = torch.zeros(2 * n + precond, dtype=torch.float64, device=DEV)
    g = torch.zeros(n, dtype=torch.float64, device=DEV)
    model.step(b, seed, n, eps, lr, mode, losses, g, precond=precond, curv_floor=1e-3)
    torch.cuda.synchronize()
    return losses.cpu().numpy(), g.cpu().numpy()


def _weights_bound(arena_data_size, seed, n, lr, g_a, g_b):
    Z = np.stack([oracle.gauss(seed, i, 0, arena_data_size).astype(np.float64) for i in range(n)])
    return (lr / n) * (np.abs(g_a - g_b) @ np.abs(Z))


# rows per evaluation: 2 x 128 = 256 (copies side by side in one forward),
# 2 x 64 = 128 (not a multiple of 256: the copies are evaluated one by one)
@pytest.mark.parametrize("kw,n", [(dict(batch=2, seq=128, max_seq=128), 3),
                                  (dict(batch=2, seq=128, max_seq=128, act="relu"), 5),
                                  (dict(batch=2, seq=64), 2),
                                  (dict(batch=1, seq=256, max_seq=256, d=256, heads=2, ffn=512), 4)])
def test_copies_step_vs_oracle(kw, n):
    model, b, keep, arena, obatch = decoder_setup(**kw)
    lr = 1e-3
    gl, gg = _step(model, b, 4, n, 1e-3, lr, zo.ZO_MODE_COPIES)
    ol, og = oracle.spsa_step(arena, obatch, seed=4, n_probes=n, eps=1e-3, lr=lr, mode="fused")
    np.testing.assert_allclose(gl, ol, rtol=LOSS_RTOL)
    bound = _weights_bound(arena.data.size, 4, n, lr, gg, og)
    w = from_bf16_dev(model.arena)
    wo = arena.values()
    assert (np.abs(w - wo) <= bound + 2 * ulp_bf16(np.maximum(np.abs(w), np.abs(wo)))).all()


def test_copies_many_groups_match_fused():
    """N = 40 probes at 256 rows: groups of 16 probes (32 copies side by side),
    16, then a ragged 8; the losses equal the fused mode's, the weights within
    the g-noise bound of the fused step's."""
    kw = dict(batch=4, seq=64, max_seq=64)
    n, lr = 40, 1e-3
    m_c, b_c, keep_c, arena, obatch = decoder_setup(**kw)
    m_f, b_f, keep_f, _, _ = decoder_setup(**kw)
    lc, gc = _step(m_c, b_c, 11, n, 1e-3, lr, zo.ZO_MODE_COPIES)
    lf, gf = _step(m_f, b_f, 11, n, 1e-3, lr, zo.ZO_MODE_FUSED)
    np.testing.assert_allclose(lc, lf, rtol=LOSS_RTOL)
    wc, wf = from_bf16_dev(m_c.arena), from_bf16_dev(m_f.arena)
    bound = _weights_bound(arena.data.size, 11, n, lr, gc, gf)
    assert (np.abs(wc - wf) <= bound + ulp_bf16(np.maximum(np.abs(wc), np.abs(wf)))).all()
    # a second step reuses the model's copies buffer
    lc2, _ = _step(m_c, b_c, 12, 3, 1e-3, lr, zo.ZO_MODE_COPIES)
    lf2, _ = _step(m_f, b_f, 12, 3, 1e-3, lr, zo.ZO_MODE_FUSED)
    np.testing.assert_allclose(lc2, lf2, rtol=LOSS_RTOL)


def test_copies_precond_vs_oracle():
    model, b, keep, arena, obatch = decoder_setup(batch=2, seq=128, max_seq=128)
    gl, gg = _step(model, b, 6, 3, 1e-3, 1e-3, zo.ZO_MODE_COPIES, precond=1)
    ol, og = oracle.spsa_step(arena, obatch, seed=6, n_probes=3, eps=1e-3, lr=1e-3, mode="fused", precond=True,
                              curv_floor=1e-3)
    np.testing.assert_allclose(gl, ol, rtol=LOSS_RTOL)


def test_copies_refusals():
    # not a decoder
    from test_gpu_fp32_models import mlp_setup
    model, batch, keep, arena, obatch = mlp_setup(batch=64, d_in=64, hidden=256)
    losses = torch.zeros(2, dtype=torch.float64, device=DEV)
    g = torch.zeros(1, dtype=torch.float64, device=DEV)
    with pytest.raises(zo.ZoError) as e:
        model.step(batch, 0, 1, 1e-3, 1e-3, zo.ZO_MODE_COPIES, losses, g)
    assert e.value.status == zo.ZO_ERR_UNSUPPORTED
    # (8-bit directions are supported: test_gpu_dirs8.test_copies_step_q8_vs_oracle)
    # the step that cannot allocate
    m8, b8, keep8, _, _ = decoder_setup(batch=2, seq=128, max_seq=128)
    before = m8.arena.clone()
    with pytest.raises(zo.ZoError) as e:
        zo.step_noalloc(m8.desc, m8.arena, b8, 0, 1, 1e-3, 1e-3, zo.ZO_MODE_COPIES, losses, g)
    assert e.value.status == zo.ZO_ERR_UNSUPPORTED
    assert torch.equal(m8.arena, before)


def test_copies_gpt_small_configured_step(tmp_path):
    """The GPT-small-shaped configuration (12 x 768, 12 heads, FFN 3072, vocab
    32000; batch 8 x seq 512 Zipf(1.1) tokens; N = 32, eps = 1e-3) in the
    copies mode: four probes' L+- against the oracle's losses at D(W0 +- eps
    z_i), and the update on 65,536 sampled weights with the GPU's g_i."""
    shape = dict(layers=12, d=768, heads=12, ffn=3072, vocab=32000, max_seq=512, act="gelu")
    B, S, N, EPS, LR, SEED = 8, 512, 32, 1e-3, 1e-5, 7
    odesc = {"kind": "decoder", **shape}
    layout, total = oracle.param_layout(odesc)
    w32 = np.zeros(total, np.float32)
    for k, (name, off, sh) in enumerate(layout):
        w32[off:off + int(np.prod(sh))] = inputs.decoder_tensor_init(name, sh, 0, k).ravel()
    w0 = inputs.f32_to_bf16_bits(w32)
    del w32
    tokens = inputs.zipf_tokens(0, B, S, shape["vocab"])
    desc = zo.make_desc(zo.ZO_MODEL_DECODER, batch=B, seq=S, layers=12, d_model=768, heads=12, ffn=3072,
                        vocab=32000, max_seq=512, act=zo.ZO_ACT_GELU)
    model = zo.Model(desc, torch.from_numpy(w0.view(np.int16).copy()).to(DEV))
    tok = torch.from_numpy(tokens).to(DEV)
    batch = zo.make_batch(tokens=tok, batch=B, seq=S)
    gl, gg = _step(model, batch, SEED, N, EPS, LR, zo.ZO_MODE_COPIES)
    w_gpu = model.arena.cpu().numpy().view(np.uint16)
    del model
    assert np.isfinite(gl).all() and np.isfinite(gg).all()
    sig = float(np.float32(EPS))

    # the oracle: D(W0 +- sig z_i) for the first four probes
    states = []
    with oracle_par.pool() as pool:
        for i in range(4):
            for k, sg in enumerate((sig, -sig)):
                path = str(tmp_path / f"state{i}_{k}.bin")
                mm = np.memmap(path, dtype=np.uint16, mode="w+", shape=(total,))
                mm[:] = w0
                mm.flush()
                del mm
                oracle_par.perturb_file(pool, path, total, SEED, i, sg)
                states.append(path)
    ol = np.array(oracle_par.losses_of_states(odesc, states, total, tokens))
    for p in states:
        os.remove(p)
    np.testing.assert_allclose(gl[:8], ol, rtol=2e-3)

    # the update alone changes W: D(W0 + sum c_i z_i) on sampled elements
    rng = np.random.default_rng(5)
    idx = np.unique(np.concatenate([rng.integers(0, total, 65536 - 2 * len(layout)).astype(np.uint64),
                                    np.array([off for _, off, _ in layout], np.uint64),
                                    np.array([off + int(np.prod(sh)) - 1 for _, off, sh in layout], np.uint64)]))
    idx = np.ascontiguousarray(idx)
    wv = np.ascontiguousarray(w0[idx])
    c = np.ascontiguousarray(-float(np.float32(LR)) * gg / N)
    oracle.lib().oracle_update_bf16_at(oracle._ptr(wv), oracle._ptr(idx), idx.size, SEED, N, oracle._ptr(c))
    got = oracle.bf16_bits_to_f64(w_gpu[idx])
    want = oracle.bf16_bits_to_f64(wv)
    # one rounding: a mismatch is a rounding-boundary case, one ulp apart
    diff = got != want
    assert np.mean(diff) <= 1e-3
    assert (np.abs(got - want)[diff] <= ulp_bf16(np.maximum(np.abs(got), np.abs(want)))[diff] * 1.0001).all()
    assert np.mean(w_gpu[idx] != w0[idx]) > 0.01
