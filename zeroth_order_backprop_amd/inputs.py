"""Seeded synthetic inputs for the SPSA step: initial weights, batches, labels.

This module holds none of the method's arithmetic (no direction generator, no
perturbation, no loss).  It only draws the fixed inputs that both the HIP path
and the CPU oracle are given, from numpy's own generator, so that both sides
start from identical arrays.  It imports nothing from the rest of the package.

Workload shapes (no dataset is used; these stand in for the pages' public
datasets with synthetic data of the same shape):

* least squares: W 256x256 fp32 init N(0, 0.02^2); X 512x256 ~ N(0,1);
  Y = X W*^T + 0.01 N(0,1), W* ~ N(0, 1/256).
* MLP classifier: 1024 -> 4096 (GELU) -> 10, weights N(0, 1/fan_in), batch 256
  of N(0,1) inputs, labels = argmax of a fixed random 1024x10 projection.
* decoder: token ids i.i.d. Zipf(1.1) over the vocabulary (rank k has
  probability proportional to k^-1.1, id = k-1), weights N(0, 0.02^2),
  LayerNorm gain 1 and bias 0.  Batch 8 x seq 2048 mirrors the memory claim's
  workload in the ZOO blog ("backprop의 메모리 세금": OPT-30B, batch 8,
  sequence length 2048).
"""
from __future__ import annotations

import numpy as np

# Stream tags keep every tensor's draws independent of every other's.
TAG_INIT, TAG_DATA, TAG_TEACHER, TAG_NOISE, TAG_TOKENS = 1, 2, 3, 4, 5


def _rng(seed: int, tag: int, index: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, index])))


# ---------------------------------------------------------------- least squares
def lsq_inputs(seed: int = 0, n: int = 512, d_in: int = 256, d_out: int = 256) -> dict:
    """W0 [d_in][d_out] fp32, X [n][d_in] fp32, Y [n][d_out] fp32."""
    w0 = (_rng(seed, TAG_INIT).standard_normal((d_in, d_out)) * 0.02).astype(np.float32)
    x = _rng(seed, TAG_DATA).standard_normal((n, d_in)).astype(np.float32)
    w_star = _rng(seed, TAG_TEACHER).standard_normal((d_out, d_in)) / np.sqrt(d_in)
    noise = _rng(seed, TAG_NOISE).standard_normal((n, d_out))
    y = (x.astype(np.float64) @ w_star.T + 0.01 * noise).astype(np.float32)
    return {"W": w0, "X": x, "Y": y}


# ------------------------------------------------------------------------ MLP
def mlp_inputs(seed: int = 0, batch: int = 256, d_in: int = 1024, hidden: int = 4096,
               classes: int = 10) -> dict:
    """W1 [hidden][d_in], W2 [classes][hidden] fp32 (nn.Linear layout),
    X [batch][d_in] fp32, labels int32 [batch]."""
    w1 = (_rng(seed, TAG_INIT, 0).standard_normal((hidden, d_in)) / np.sqrt(d_in)).astype(np.float32)
    w2 = (_rng(seed, TAG_INIT, 1).standard_normal((classes, hidden)) / np.sqrt(hidden)).astype(np.float32)
    x = _rng(seed, TAG_DATA).standard_normal((batch, d_in)).astype(np.float32)
    teacher = _rng(seed, TAG_TEACHER).standard_normal((d_in, classes))
    scores = x.astype(np.float64) @ teacher
    labels = np.argmax(scores, axis=1).astype(np.int32)  # ties -> lowest index
    return {"W1": w1, "W2": w2, "X": x, "labels": labels}


# -------------------------------------------------------------------- decoder
def zipf_tokens(seed: int, batch: int, seq: int, vocab: int, s: float = 1.1) -> np.ndarray:
    """int32 [batch][seq], i.i.d. Zipf(s) over ranks 1..vocab by inverse CDF."""
    k = np.arange(1, vocab + 1, dtype=np.float64)
    cdf = np.cumsum(k ** (-s))
    cdf /= cdf[-1]
    u = _rng(seed, TAG_TOKENS).random((batch, seq))
    ids = np.searchsorted(cdf, u, side="left")
    return np.minimum(ids, vocab - 1).astype(np.int32)


def decoder_tensor_init(name: str, shape: tuple, seed: int, index: int) -> np.ndarray:
    """Initial value of one decoder tensor as fp32 (rounded to bf16 by the
    caller's storage).  LayerNorm gains are 1 and biases 0; everything else is
    N(0, 0.02^2)."""
    if name.endswith("_g"):
        return np.ones(shape, np.float32)
    if name.endswith("_b"):
        return np.zeros(shape, np.float32)
    return (_rng(seed, TAG_INIT, index).standard_normal(shape) * 0.02).astype(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (storage conversion of
    the initial weights only; finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
