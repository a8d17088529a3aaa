"""GPU parity of the bf16 decoder path against the CPU oracle, through the C ABI.

Kernels in isolation (bf16 GEMM with each epilogue, causal attention,
LayerNorm) and whole-model losses (tiny decoder, GPT-small shape at reduced
tokens), stored and perturbed weights, and in-place steps.

Bars: bf16 tensors within one bf16 rounding of the oracle's fp64 value
rounded to bf16 (the GPU accumulates in fp32), attention outputs within a
per-element bound derived from the kernel's arithmetic (the oracle keeps the
softmax exact; the kernel rounds the weights to bf16 before P V); losses
within 2e-3 relative.
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from zeroth_order_backprop_amd import inputs, zo

pytestmark = pytest.mark.gpu
DEV = "cuda"
LOSS_RTOL = 2e-3


def to_bf16_dev(a: np.ndarray) -> torch.Tensor:
    bits = inputs.f32_to_bf16_bits(np.ascontiguousarray(a, np.float32))
    return torch.from_numpy(bits.view(np.int16).copy()).to(DEV)


def from_bf16_dev(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_bits_to_f64(t.cpu().numpy().view(np.uint16))


def ulp_bf16(x):
    a = np.maximum(np.abs(x), 2.0**-126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def assert_bf16_close(got, want, frac_exact=0.9, ulps=1.0, abs_tol=0.0):
    """got within `ulps` bf16 ulps of want, plus `abs_tol` (the fp32 error of
    the terms that cancel into a small result, which no bf16 ulp of the result
    bounds)."""
    err = np.abs(got - want)
    tol = ulps * ulp_bf16(np.maximum(np.abs(got), np.abs(want))) * 1.0001 + abs_tol
    bad = err > tol
    assert not bad.any(), (int(bad.sum()), got[bad][:5], want[bad][:5], np.broadcast_to(tol, err.shape)[bad][:5])
    assert np.mean(got == want) >= frac_exact, np.mean(got == want)


# ------------------------------------------------------------------ GEMM
@pytest.mark.parametrize("M,N,K", [(128, 128, 64), (300, 200, 128), (4096, 2304, 768), (4096, 4096, 256),
                                   (4100, 4200, 192), (8192, 8192, 1024)])
@pytest.mark.parametrize("epi", [0, 1, 2, 3])
def test_gemm_bf16(M, N, K, epi):
    rng = np.random.default_rng(M + N + K + epi)
    A = oracle.bf16_round(rng.standard_normal((M, K)))
    W = oracle.bf16_round(rng.standard_normal((N, K)) * 0.05)
    C0 = oracle.bf16_round(rng.standard_normal((M, N)))
    Ad, Wd = to_bf16_dev(A), to_bf16_dev(W)
    Cd = to_bf16_dev(C0) if epi == 3 else torch.zeros(M * N, dtype=torch.int16, device=DEV)
    zo.debug_gemm_bf16(Ad, Wd, Cd, M, N, K, epi)
    torch.cuda.synchronize()
    got = from_bf16_dev(Cd).reshape(M, N)
    prod = A @ W.T
    if epi == 0:
        want = oracle.bf16_round(prod)
    elif epi == 1:
        want = oracle.bf16_round(oracle.gelu_erf(prod))
    elif epi == 2:
        want = oracle.bf16_round(np.maximum(prod, 0.0))
    else:
        want = oracle.bf16_round(C0 + oracle.bf16_round(prod))
    # fp32 accumulation of K products: |error| <= K 2^-24 sum_k |a_k w_k|; on
    # top of it the result may fall on the other side of a bf16 rounding
    # boundary (twice for the residual sum)
    acc_err = K * 2.0**-24 * (np.abs(A) @ np.abs(W).T)
    if epi == 1:
        acc_err = acc_err * 1.2  # |GELU'| <= 1.13
    if epi == 3:
        # a flip of bf16(product) moves the sum by one ulp of the product
        acc_err = acc_err + ulp_bf16(np.abs(prod) + acc_err) * 1.0001
    assert_bf16_close(got, want, frac_exact=0.95 if epi != 3 else 0.9, abs_tol=acc_err)


# ------------------------------------------------------------- attention
def attention_error_bound(qkv, H):
    """Per-element bound on |kernel - exact| for the causal attention.

    The oracle keeps the softmax exact (fp64).  The kernel computes scores in
    fp32 from bf16 Q, K (error <= dh 2^-24 sum_k |q_k k_k| per score), the
    weights e_j = 2^(s_j c - m) in fp32, rounds each e_j to bf16 before the
    P V product (8 significant bits: relative error <= 2^-8) while the
    normaliser l = sum_j e_j
    keeps the unrounded values, accumulates O and l in fp32 over at most S
    keys, and rounds O / l to bf16.  So

      |err| <= (2^-8 + 2 delta_q + (S + 8) 2^-24) (P |V|) + ulp_bf16(|out|)

    with P the exact softmax, delta_q the largest score error of the query
    scaled by 1/sqrt(dh) (a score error delta moves every normalised weight
    by at most a factor e^(2 delta)), and one bf16 ulp for the output's
    rounding and the side of a rounding boundary it lands on."""
    B, S, three_d = qkv.shape
    d = three_d // 3
    dh = d // H
    Q = qkv[..., :d].reshape(B, S, H, dh).transpose(0, 2, 1, 3)
    K = qkv[..., d:2 * d].reshape(B, S, H, dh).transpose(0, 2, 1, 3)
    V = qkv[..., 2 * d:].reshape(B, S, H, dh).transpose(0, 2, 1, 3)
    mask = np.triu(np.ones((S, S), dtype=bool), k=1)
    s = (Q @ K.transpose(0, 1, 3, 2)) / np.sqrt(dh)
    s[..., mask] = -np.inf
    P = np.exp(s - s.max(axis=-1, keepdims=True))
    P /= P.sum(axis=-1, keepdims=True)
    out = (P @ V).transpose(0, 2, 1, 3).reshape(B, S, d)
    PV = (P @ np.abs(V)).transpose(0, 2, 1, 3).reshape(B, S, d)
    qk = np.abs(Q) @ np.abs(K).transpose(0, 1, 3, 2)
    qk[..., mask] = 0.0
    delta = dh * 2.0**-24 * qk.max(axis=-1) / np.sqrt(dh)               # [B,H,S]
    delta = np.repeat(delta.transpose(0, 2, 1)[..., None], dh, axis=-1).reshape(B, S, d)
    rel = 2.0**-8 + 2 * delta + (S + 8) * 2.0**-24
    return out, rel * PV + ulp_bf16(np.abs(out)) * 1.0001


@pytest.mark.parametrize("B,S,H,dh", [(2, 64, 2, 64), (1, 200, 3, 64), (2, 512, 2, 64), (1, 300, 2, 128),
                                      (1, 128, 1, 128), (1, 1100, 2, 64), (1, 2048, 1, 64), (4, 1024, 32, 64),
                                      (1, 2048, 2, 128),
                                      # sequences shorter than one key tile, a query block or the
                                      # four-tile trip of the d_h 128 loop (its tail of 1-3 tiles)
                                      (1, 1, 1, 128), (2, 1, 2, 64), (3, 5, 2, 128), (2, 33, 1, 64),
                                      (1, 97, 2, 128), (1, 129, 1, 128), (1, 191, 1, 64)])
def test_attention(B, S, H, dh):
    rng = np.random.default_rng(S + dh)
    d = H * dh
    qkv = oracle.bf16_round(rng.standard_normal((B, S, 3 * d)))
    out = torch.zeros(B * S * d, dtype=torch.int16, device=DEV)
    zo.debug_attention(to_bf16_dev(qkv), out, B, S, H, dh)
    torch.cuda.synchronize()
    got = from_bf16_dev(out).reshape(B, S, d)
    want = oracle.causal_attention(qkv, H)
    ref, bound = attention_error_bound(qkv, H)
    assert np.abs(ref - want).max() <= 1e-12  # the bound's softmax is the oracle's
    err = np.abs(got - want)
    bad = err > bound
    assert not bad.any(), (int(bad.sum()), err[bad][:5], bound[bad][:5])
    # the first query attends only to itself: its output is V[0] exactly (bf16)
    assert np.array_equal(got[:, 0, :], qkv[:, 0, 2 * d:])


# ------------------------------------------------------------- LayerNorm
@pytest.mark.parametrize("rows,d", [(64, 64), (33, 768), (8, 7168)])
def test_layernorm(rows, d):
    rng = np.random.default_rng(d)
    h = oracle.bf16_round(rng.standard_normal((rows, d)) * 3 + 0.5)
    g = oracle.bf16_round(1.0 + 0.1 * rng.standard_normal(d))
    b = oracle.bf16_round(0.1 * rng.standard_normal(d))
    x = torch.zeros(rows * d, dtype=torch.int16, device=DEV)
    zo.debug_layernorm(to_bf16_dev(h), to_bf16_dev(g), to_bf16_dev(b), x, rows, d)
    torch.cuda.synchronize()
    got = from_bf16_dev(x).reshape(rows, d)
    want = oracle.bf16_round(oracle.layer_norm(h, g, b))
    # fp32 statistics and fma: a few fp32 ulps of the terms t*g and b that
    # cancel into small outputs
    mu = h.mean(axis=1, keepdims=True)
    t = (h - mu) / np.sqrt(h.var(axis=1, keepdims=True) + 1e-5)
    abs_tol = 16 * 2.0**-24 * (np.abs(t * g) + np.abs(b) + np.abs(mu) * np.abs(g))
    assert_bf16_close(got, want, frac_exact=0.97, abs_tol=abs_tol)


# ------------------------------------------------------------ whole model
def decoder_setup(layers=2, d=128, heads=2, ffn=256, vocab=500, max_seq=64, batch=2, seq=64, act="gelu", seed=0):
    odesc = {"kind": "decoder", "layers": layers, "d": d, "heads": heads, "ffn": ffn, "vocab": vocab,
             "max_seq": max_seq, "act": act}
    desc = zo.make_desc(zo.ZO_MODEL_DECODER, batch=batch, seq=seq, layers=layers, d_model=d, heads=heads, ffn=ffn,
                        vocab=vocab, max_seq=max_seq, act=zo.ZO_ACT_GELU if act == "gelu" else zo.ZO_ACT_RELU)
    layout, total = oracle.param_layout(odesc)
    arena = np.zeros(total, np.float32)
    for k, (name, off, shape) in enumerate(layout):
        arena[off:off + int(np.prod(shape))] = inputs.decoder_tensor_init(name, shape, seed, k).ravel()
    bits = inputs.f32_to_bf16_bits(arena)
    model = zo.Model(desc, torch.from_numpy(bits.view(np.int16).copy()).to(DEV))
    tokens = inputs.zipf_tokens(seed, batch, seq, vocab)
    tok = torch.from_numpy(tokens).to(DEV)
    b = zo.make_batch(tokens=tok, batch=batch, seq=seq)
    return model, b, tok, oracle.Arena(odesc, bits), {"tokens": tokens}


def gpu_losses(model, batch, perts):
    out = torch.zeros(max(1, len(perts)), dtype=torch.float64, device=DEV)
    model.forward_loss(batch, out, perts=perts)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("kw", [dict(), dict(act="relu"), dict(seq=37, vocab=333), dict(d=256, heads=2, ffn=512),
                                dict(d=256, heads=4, seq=200, max_seq=256, batch=1)])
def test_decoder_forward_tiny(kw):
    model, b, keep, arena, obatch = decoder_setup(**kw)
    got = gpu_losses(model, b, [])[0]
    want = oracle.model_loss(arena, obatch)
    assert got == pytest.approx(want, rel=LOSS_RTOL)
    assert abs(want - np.log(kw.get("vocab", 500))) < 1.5  # near-uniform logits at init


def test_decoder_forward_perturbed():
    model, b, keep, arena, obatch = decoder_setup()
    eps = float(np.float32(1e-3))
    perts = [(3, 0, eps), (3, 0, -eps), (9, 5, 0.01)]
    got = gpu_losses(model, b, perts)
    for k, (s, i, sg) in enumerate(perts):
        a = arena.copy()
        a.perturb(s, i, sg)
        assert got[k] == pytest.approx(oracle.model_loss(a, obatch), rel=LOSS_RTOL)
    # fused evaluation leaves the stored weights untouched
    assert np.array_equal(model.arena.cpu().numpy().view(np.uint16), arena.data)


@pytest.mark.parametrize("mode", [zo.ZO_MODE_INPLACE, zo.ZO_MODE_FUSED])
def test_decoder_step(mode):
    model, b, keep, arena, obatch = decoder_setup()
    N = 2
    losses = torch.zeros(2 * N, dtype=torch.float64, device=DEV)
    g = torch.zeros(N, dtype=torch.float64, device=DEV)
    model.step(b, 4, N, 1e-3, 1e-3, mode, losses, g)
    torch.cuda.synchronize()
    ol, og = oracle.spsa_step(arena, obatch, seed=4, n_probes=N, eps=1e-3, lr=1e-3,
                              mode="inplace" if mode == zo.ZO_MODE_INPLACE else "fused")
    np.testing.assert_allclose(losses.cpu().numpy(), ol, rtol=LOSS_RTOL)
    # weights: the GPU's and the oracle's c_i differ only through g (bf16 loss
    # noise), so |w_gpu - w_oracle| <= (lr/N) sum_i |g_i - og_i| |z_i| + 2 ulp,
    # plus in place up to 1.5 ulp of restore drift per probe on each side
    gg = g.cpu().numpy()
    n = arena.data.size
    Z = np.stack([oracle.gauss(4, i, 0, n).astype(np.float64) for i in range(N)])
    bound = (1e-3 / N) * (np.abs(gg - og) @ np.abs(Z))
    w = from_bf16_dev(model.arena)
    wo = arena.values()
    ulps = 2 + (3 * N if mode == zo.ZO_MODE_INPLACE else 0)
    assert (np.abs(w - wo) <= bound + ulps * ulp_bf16(np.maximum(np.abs(w), np.abs(wo)))).all()


def test_decoder_gpt_small_shape_reduced_tokens():
    """GPT-small shape at full width (12 x 768, 12 heads, FFN 3072, vocab
    32000, positions 512), batch 1 x 128 tokens."""
    model, b, keep, arena, obatch = decoder_setup(layers=12, d=768, heads=12, ffn=3072, vocab=32000, max_seq=512,
                                                  batch=1, seq=128)
    got = gpu_losses(model, b, [])[0]
    want = oracle.model_loss(arena, obatch)
    assert got == pytest.approx(want, rel=LOSS_RTOL)
    eps = float(np.float32(1e-3))
    got = gpu_losses(model, b, [(0, 0, eps)])[0]
    a = arena.copy()
    a.perturb(0, 0, eps)
    assert got == pytest.approx(oracle.model_loss(a, obatch), rel=LOSS_RTOL)
