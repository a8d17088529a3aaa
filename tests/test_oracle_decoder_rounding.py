"""Pin of the oracle decoder's bf16 rounding points.

The decoder's readings (pre-LN blocks, learned positions, tied head, causal
LM loss) come from the configs' shapes; the pages fix no precision beyond
bf16 weights.  The declared rounding points are: the embedding sum, every
LayerNorm output, every GEMM output (QKV, the attention output, W_o, the FFN
up product after its activation, W_down), and both residual sums; softmax,
LayerNorm statistics, logits and the cross-entropy stay exact.

Here an independent fp64 forward is built from torch's library layers
(embedding, layer_norm, scaled_dot_product_attention, gelu / relu, linear,
cross_entropy) with the pinned fp64 -> bf16 rounding applied at exactly those
points.  The oracle must agree with it to ~1e-12; and each point is shown to
matter: leaving any one of them out, or adding a rounding at a point that is
not declared (logits, softmax probabilities, the attention scores), moves the
loss by far more than that tolerance, so a dropped or an extra rounding in the
oracle would fail the comparison.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import oracle

POINTS = ["emb", "ln1", "qkv", "attn", "wo", "res1", "ln2", "up", "down", "res2", "lnf"]
EXTRA = ["scores", "probs", "logits"]


def _bf(t: torch.Tensor) -> torch.Tensor:
    return torch.from_numpy(oracle.bf16_round(t.detach().numpy())).reshape(t.shape)


def torch_decoder_loss(desc, p, tokens, rounded=tuple(POINTS)):
    R = lambda name, t: _bf(t) if name in rounded else t
    act = (lambda x: F.gelu(x, approximate="none")) if desc["act"] == "gelu" else F.relu
    T = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    tok = torch.from_numpy(tokens.astype(np.int64))
    B, S = tokens.shape
    d, H = desc["d"], desc["heads"]
    dh = d // H
    h = R("emb", F.embedding(tok, T(p["tok_emb"])) + T(p["pos_emb"])[:S][None])
    causal = torch.ones(S, S, dtype=torch.bool).tril()
    for layer in range(desc["layers"]):
        q = f"l{layer}."
        x = R("ln1", F.layer_norm(h, (d,), T(p[q + "ln1_g"]), T(p[q + "ln1_b"]), eps=1e-5))
        qkv = R("qkv", F.linear(x, T(p[q + "w_qkv"])))
        Q, K, V = (qkv[..., i * d:(i + 1) * d].reshape(B, S, H, dh).transpose(1, 2) for i in range(3))
        if "scores" in rounded or "probs" in rounded:
            s = R("scores", Q @ K.transpose(-1, -2) / np.sqrt(dh)).masked_fill(~causal, float("-inf"))
            o = R("probs", torch.softmax(s, dim=-1)) @ V
        else:
            o = F.scaled_dot_product_attention(Q, K, V, is_causal=True)
        o = R("attn", o.transpose(1, 2).reshape(B, S, d))
        h = R("res1", h + R("wo", F.linear(o, T(p[q + "w_o"]))))
        x = R("ln2", F.layer_norm(h, (d,), T(p[q + "ln2_g"]), T(p[q + "ln2_b"]), eps=1e-5))
        u = R("up", act(F.linear(x, T(p[q + "w_up"]))))
        h = R("res2", h + R("down", F.linear(u, T(p[q + "w_down"]))))
    x = R("lnf", F.layer_norm(h, (d,), T(p["lnf_g"]), T(p["lnf_b"]), eps=1e-5))
    logits = R("logits", F.linear(x[:, :-1], T(p["tok_emb"])))
    return float(F.cross_entropy(logits.reshape(-1, logits.shape[-1]), tok[:, 1:].reshape(-1)))


def _model(act, seed):
    desc = {"kind": "decoder", "layers": 2, "d": 64, "heads": 2, "ffn": 128, "vocab": 300, "max_seq": 24,
            "act": act}
    rng = np.random.default_rng(seed)
    params = {}
    for name, shape in oracle.param_shapes(desc):
        if name.endswith("_g"):
            v = 1.0 + 0.1 * rng.standard_normal(shape)
        elif name.endswith("_b"):
            v = 0.1 * rng.standard_normal(shape)
        else:
            v = 0.2 * rng.standard_normal(shape)  # larger than init, so every rounding shows
        params[name] = oracle.bf16_round(v)
    tokens = rng.integers(0, desc["vocab"], size=(2, 24)).astype(np.int32)
    return desc, params, tokens


@pytest.mark.parametrize("act,seed", [("gelu", 0), ("relu", 1)])
def test_decoder_rounding_points(act, seed):
    desc, params, tokens = _model(act, seed)
    want = torch_decoder_loss(desc, params, tokens)
    got = oracle.decoder_loss(desc, params, tokens, round_bf16=True)
    tol = 1e-12 * abs(want)
    assert abs(got - want) <= tol, (got, want)
    # without rounding the two agree too (the layers themselves match)
    got0 = oracle.decoder_loss(desc, params, tokens, round_bf16=False)
    want0 = torch_decoder_loss(desc, params, tokens, rounded=())
    assert abs(got0 - want0) <= tol
    # every declared point matters, and so would any extra one
    for pt in POINTS:
        moved = torch_decoder_loss(desc, params, tokens, rounded=[q for q in POINTS if q != pt])
        assert abs(moved - want) > 1000 * tol, (pt, moved, want)
    for pt in EXTRA:
        moved = torch_decoder_loss(desc, params, tokens, rounded=POINTS + [pt])
        assert abs(moved - want) > 1000 * tol, (pt, moved, want)
