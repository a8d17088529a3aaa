"""The GPT-small-shaped decoder's configured SPSA step against the CPU oracle.

Configuration: 12 layers, d = 768, 12 heads, FFN 3072 (GELU), vocabulary
32000, learned positions, bf16 weights N(0, 0.02^2); batch 8 x seq 512
Zipf(1.1) tokens; N = 32 probes, eps = 1e-3, in place (for each probe +eps,
L+, -2 eps, L-, +eps; then the fused update), the loop of the ZOO blog
("backprop의 메모리 세금").

The GPU runs the whole step through zo_step.  The oracle, from the same
initial weights, repeats the in-place perturb / restore sequence of the first
four probes over the whole arena and evaluates their eight losses (within the
bf16 loss bar, 2e-3 relative); then, on 65,536 sampled elements, it applies
all 96 perturb / restore passes and the update with the GPU's g_i (the bf16
losses carry rounding noise as large as their difference, so g_i itself is
not compared) and must reproduce the GPU's final weights there, bit for bit
except at rounding boundaries.
"""
import os

import numpy as np
import pytest
import torch

from helpers import oracle_par
from oracle import oracle
from zeroth_order_backprop_amd import inputs, zo

pytestmark = pytest.mark.gpu
DEV = "cuda"
SHAPE = dict(layers=12, d=768, heads=12, ffn=3072, vocab=32000, max_seq=512, act="gelu")
B, S, N, EPS, LR, SEED = 8, 512, 32, 1e-3, 1e-5, 7


def test_gpt_small_configured_step(tmp_path):
    odesc = {"kind": "decoder", **SHAPE}
    layout, total = oracle.param_layout(odesc)
    w32 = np.zeros(total, np.float32)
    for k, (name, off, shape) in enumerate(layout):
        w32[off:off + int(np.prod(shape))] = inputs.decoder_tensor_init(name, shape, 0, k).ravel()
    w0 = inputs.f32_to_bf16_bits(w32)
    del w32
    tokens = inputs.zipf_tokens(0, B, S, SHAPE["vocab"])

    # the GPU's configured step
    desc = zo.make_desc(zo.ZO_MODEL_DECODER, batch=B, seq=S, layers=12, d_model=768, heads=12, ffn=3072,
                        vocab=32000, max_seq=512, act=zo.ZO_ACT_GELU)
    model = zo.Model(desc, torch.from_numpy(w0.view(np.int16).copy()).to(DEV))
    tok = torch.from_numpy(tokens).to(DEV)
    batch = zo.make_batch(tokens=tok, batch=B, seq=S)
    losses = torch.zeros(2 * N, dtype=torch.float64, device=DEV)
    g = torch.zeros(N, dtype=torch.float64, device=DEV)
    model.step(batch, SEED, N, EPS, LR, zo.ZO_MODE_INPLACE, losses, g)
    torch.cuda.synchronize()
    gl, gg = losses.cpu().numpy(), g.cpu().numpy()
    w_gpu = model.arena.cpu().numpy().view(np.uint16)
    del model
    assert np.isfinite(gl).all() and np.isfinite(gg).all()
    sig = float(np.float32(EPS))

    # the oracle: the first four probes' in-place sequence over the whole arena
    path = str(tmp_path / "arena.bin")
    mm = np.memmap(path, dtype=np.uint16, mode="w+", shape=(total,))
    mm[:] = w0
    mm.flush()
    del mm
    states = []
    with oracle_par.pool() as pool:
        for i in range(4):
            for k, sg in enumerate((sig, -2.0 * sig)):
                oracle_par.perturb_file(pool, path, total, SEED, i, sg)
                snap = str(tmp_path / f"state{i}_{k}.bin")
                np.array(np.memmap(path, dtype=np.uint16, mode="r", shape=(total,))).tofile(snap)
                states.append(snap)
            oracle_par.perturb_file(pool, path, total, SEED, i, sig)
    ol = np.array(oracle_par.losses_of_states(odesc, states, total, tokens))
    for p in states + [path]:
        os.remove(p)
    np.testing.assert_allclose(gl[:8], ol, rtol=2e-3)
    assert abs(ol[0] - np.log(SHAPE["vocab"])) < 1.5

    # the whole step's weight changes on sampled elements, with the GPU's g
    rng = np.random.default_rng(3)
    idx = np.unique(np.concatenate([rng.integers(0, total, 65536 - 2 * len(layout)).astype(np.uint64),
                                    np.array([off for _, off, _ in layout], np.uint64),
                                    np.array([off + int(np.prod(sh)) - 1 for _, off, sh in layout], np.uint64)]))
    idx = np.ascontiguousarray(idx)
    wv = np.ascontiguousarray(w0[idx])
    peak = np.abs(oracle.bf16_bits_to_f64(wv))
    L = oracle.lib()
    for i in range(N):
        for sg in (sig, -2.0 * sig, sig):
            L.oracle_perturb_bf16_at(oracle._ptr(wv), oracle._ptr(idx), idx.size, SEED, i, float(np.float32(sg)))
            peak = np.maximum(peak, np.abs(oracle.bf16_bits_to_f64(wv)))
    c = np.ascontiguousarray(-float(np.float32(LR)) * gg / N)
    L.oracle_update_bf16_at(oracle._ptr(wv), oracle._ptr(idx), idx.size, SEED, N, oracle._ptr(c))
    got = oracle.bf16_bits_to_f64(w_gpu[idx])
    want = oracle.bf16_bits_to_f64(wv)
    peak = np.maximum(peak, np.abs(want))
    # a value at a rounding boundary (GPU directions within 1e-6 of the
    # oracle's, fp32 intermediate) can land one ulp away in any of the 96
    # passes, an ulp of the magnitude it had then: a few such flips may fall
    # on one element (measured: 4.7e-4 of the elements differ, by at most 4
    # ulps of their largest magnitude along the passes)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(peak, 2.0**-126))) - 7)
    r = np.abs(got - want) / ulp
    bad = r > 8.0001
    print(f"sampled weights: {np.mean(got != want):.2e} differ, max {r.max():.2f} ulp of the peak")
    assert not bad.any(), (idx[bad][:8], got[bad][:8], want[bad][:8], peak[bad][:8])
    assert np.mean(got == want) >= 0.999
    # and the update did change weights
    assert np.mean(w_gpu[idx] != w0[idx]) > 0.01
