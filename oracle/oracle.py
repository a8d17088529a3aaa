"""CPU oracle of the multi-probe SPSA step (plain, slow, obviously correct).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with the
HIP path and imports nothing from the product package.

Element-wise parts (direction generator, perturbation, update, bf16 rounding)
are plain C in ``zo_oracle.c``; the model forwards are numpy in fp64, with
numpy's matmul as the only library primitive for a contraction.

What is computed, and where the pages state it:

* The loop (ZOO blog "Backprop 없이 Transformer를 학습시킨다", section
  "backprop의 메모리 세금", flowchart): draw N random directions, perturb
  W +- eps*z_i, evaluate only the loss, form the SPSA estimate, update
  W <- W - eta * g_hat, repeat.
* Two forwards per probe at +1 and -1 times the perturbation (same page,
  section "zero-order optimization이란"), so g_i = (L+_i - L-_i) / (2 eps)
  and g_hat = (1/N) sum_i g_i z_i.
* Gaussian directions (gist.science 2605.15622 summary, P1), regenerated from
  a seed rather than stored (same page P5; FedSPZO summary, section 2
  "통신 프로토콜").
* In-place, inference-mode training: the weights themselves are perturbed and
  restored, nothing else is kept (ZOO blog, "zero-order optimization이란" and
  the OPT-30B in-place paragraph of the 1.5-SPSA section).
* 8-bit packed directions (ZOO blog, 1.5-SPSA section: an 8-bit packing random
  generator with a fused unpack/apply kernel; no format given): read as one
  byte code per element, sixteen per Philox block, each code standing for one
  of 256 equal-probability Gaussian quantiles scaled to unit variance
  (``q8_table``; arena desc key ``"dirs": "q8"``).
* 1.5-SPSA (same section): one clean evaluation per step and a probe-space
  diagonal preconditioner (``spsa_step(precond=True)``).
* Split perturbation with activation reuse (FedSPZO summary, section 2
  "방법론"): ``fedspzo_step`` on the MLP.
* Activation perturbation with per-token rewards (Dust review page):
  ``dust_step`` on the MLP.

Readings where the pages are silent are listed in the repository's design
notes; the ones that fix arithmetic are repeated at each function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile the C part of the oracle (single-threaded, no fp contraction)."""
    src = os.path.join(_HERE, "zo_oracle.c")
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-Wall",
                           "-o", tmp, src, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P, U64, U32, F = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_float
        L.oracle_philox4x32_10.argtypes = [P, P, P]
        L.oracle_rng_words.argtypes = [U64, U32, U64, U64, P]
        L.oracle_box_muller_f64.argtypes = [U32, U32, ctypes.POINTER(ctypes.c_double)]
        L.oracle_box_muller_f64.restype = ctypes.c_double
        L.oracle_gauss.argtypes = [U64, U32, U64, U64, P]
        L.oracle_gauss_at.argtypes = [U64, U32, P, U64, P]
        L.oracle_bf16_from_f32.argtypes = [F]
        L.oracle_bf16_from_f32.restype = ctypes.c_uint16
        L.oracle_bf16_from_f64.argtypes = [ctypes.c_double]
        L.oracle_bf16_from_f64.restype = ctypes.c_uint16
        for name in ("oracle_perturb_f32", "oracle_perturb_bf16"):
            getattr(L, name).argtypes = [P, U64, U64, U64, U32, F]
        for name in ("oracle_perturb_f32_at", "oracle_perturb_bf16_at"):
            getattr(L, name).argtypes = [P, P, U64, U64, U32, F]
        for name in ("oracle_update_f32", "oracle_update_bf16"):
            getattr(L, name).argtypes = [P, U64, U64, U64, U32, P]
        for name in ("oracle_update_f32_at", "oracle_update_bf16_at"):
            getattr(L, name).argtypes = [P, P, U64, U64, U32, P]
        L.oracle_bf16_compare_range.argtypes = [U32, U32, P]
        L.oracle_bf16_compare_range.restype = U64
        L.oracle_round_bf16_array.argtypes = [P, U64]
        L.oracle_round_f32_array.argtypes = [P, U64]
        L.oracle_box_muller_f64_array.argtypes = [P, U64, P]
        L.oracle_gauss_stream.argtypes = [U64, U32, U32, U64, U64, P]
        L.oracle_q8_values.argtypes = [U64, U32, U64, U64, P, P]
        L.oracle_q8_values_at.argtypes = [U64, U32, P, U64, P, P]
        for name in ("oracle_q8_perturb_f32", "oracle_q8_perturb_bf16"):
            getattr(L, name).argtypes = [P, U64, U64, U64, U32, F, P]
        for name in ("oracle_q8_update_f32", "oracle_q8_update_bf16"):
            getattr(L, name).argtypes = [P, U64, U64, U64, U32, P, P]
        for name in ("oracle_q8_perturb_f32_at", "oracle_q8_perturb_bf16_at"):
            getattr(L, name).argtypes = [P, P, U64, U64, U32, F, P]
        for name in ("oracle_q8_update_f32_at", "oracle_q8_update_bf16_at"):
            getattr(L, name).argtypes = [P, P, U64, U64, U32, P, P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.c_void_p)


# ====================================================================== RNG
def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    lib().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def rng_words(seed: int, probe: int, j0: int, n: int) -> np.ndarray:
    out = np.zeros(n, np.uint32)
    lib().oracle_rng_words(seed, probe, j0, n, _ptr(out))
    return out


def box_muller_f64(x_even: int, x_odd: int):
    zo = ctypes.c_double()
    ze = lib().oracle_box_muller_f64(x_even, x_odd, ctypes.byref(zo))
    return ze, zo.value


def box_muller_f64_array(pairs: np.ndarray) -> np.ndarray:
    """pairs uint32 [n][2] -> fp64 [n][2] (z_even, z_odd)."""
    p = np.ascontiguousarray(pairs, dtype=np.uint32)
    out = np.zeros(p.shape, np.float64)
    lib().oracle_box_muller_f64_array(_ptr(p), p.shape[0], _ptr(out))
    return out


def q8_table() -> np.ndarray:
    """The 256 values of the 8-bit directions: x_k = Phi^-1((k + 1/2) / 256),
    divided by r = sqrt(mean_k x_k^2) so the codes (uniform over 0..255) give
    unit variance, rounded once to fp32.  Built from the upper half and
    mirrored (Phi^-1(1 - p) = -Phi^-1(p)), so it is exactly antisymmetric."""
    from scipy.special import ndtri
    up = ndtri((np.arange(128, 256) + 0.5) / 256.0)
    r = np.sqrt(2.0 * np.sum(up * up) / 256.0)
    half = (up / r).astype(np.float32)
    return np.concatenate([-half[::-1], half])


_Q8 = None


def _q8() -> np.ndarray:
    global _Q8
    if _Q8 is None:
        _Q8 = np.ascontiguousarray(q8_table())
    return _Q8


def gauss(seed: int, probe: int, j0: int, n: int) -> np.ndarray:
    """Direction z_probe at elements j0..j0+n-1 (fp32, rounded once from fp64)."""
    return directions("gauss", seed, probe, j0, n)


def directions(kind: str, seed: int, probe: int, j0: int, n: int) -> np.ndarray:
    """Direction values ('gauss' or 'q8') at elements j0..j0+n-1."""
    z = np.zeros(n, np.float32)
    if kind == "gauss":
        lib().oracle_gauss(seed, probe, j0, n, _ptr(z))
    elif kind == "q8":
        lib().oracle_q8_values(seed, probe, j0, n, _ptr(z), _ptr(_q8()))
    else:
        raise ValueError(kind)
    return z


def gauss_stream(seed: int, probe: int, stream: int, j0: int, n: int) -> np.ndarray:
    """Gaussian values of counter stream `stream` (stream 0 = the weight
    directions of ``gauss``)."""
    z = np.zeros(n, np.float32)
    lib().oracle_gauss_stream(seed, probe, stream, j0, n, _ptr(z))
    return z


def gauss_at(seed: int, probe: int, idx: np.ndarray) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.uint64)
    z = np.zeros(idx.size, np.float32)
    lib().oracle_gauss_at(seed, probe, _ptr(idx), idx.size, _ptr(z))
    return z


# ================================================================ bfloat16
def bf16_round(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even) of each fp64 entry, kept as fp64."""
    y = np.array(x, dtype=np.float64, order="C", copy=True)
    lib().oracle_round_bf16_array(_ptr(y), y.size)
    return y


def f32_round(x: np.ndarray) -> np.ndarray:
    y = np.array(x, dtype=np.float64, order="C", copy=True)
    lib().oracle_round_f32_array(_ptr(y), y.size)
    return y


def bf16_bits_to_f64(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ====================================================== parameter arena layout
# Every parameter of a model lives in one flat arena; tensors are placed in
# declaration order, each starting at a multiple of 64 elements.  Element j of
# the arena uses direction element j (the layout is an interface both sides
# state independently; a test checks they agree).
ALIGN = 64


def _align(x: int) -> int:
    return (x + ALIGN - 1) // ALIGN * ALIGN


def param_shapes(desc: dict) -> list:
    kind = desc["kind"]
    if kind == "lsq":
        return [("W", (desc["d_in"], desc["d_out"]))]
    if kind == "mlp":
        return [("W1", (desc["hidden"], desc["d_in"])), ("W2", (desc["classes"], desc["hidden"]))]
    if kind == "decoder":
        d, f, v, s = desc["d"], desc["ffn"], desc["vocab"], desc["max_seq"]
        out = [("tok_emb", (v, d)), ("pos_emb", (s, d))]
        for layer in range(desc["layers"]):
            p = f"l{layer}."
            out += [(p + "ln1_g", (d,)), (p + "ln1_b", (d,)), (p + "w_qkv", (3 * d, d)),
                    (p + "w_o", (d, d)), (p + "ln2_g", (d,)), (p + "ln2_b", (d,)),
                    (p + "w_up", (f, d)), (p + "w_down", (d, f))]
        out += [("lnf_g", (d,)), ("lnf_b", (d,))]
        return out
    raise ValueError(kind)


def param_layout(desc: dict):
    """[(name, offset, shape)], total arena elements."""
    off = 0
    out = []
    for name, shape in param_shapes(desc):
        off = _align(off)
        out.append((name, off, shape))
        off += int(np.prod(shape))
    return out, _align(off)


class LazyParams:
    """Tensor-by-tensor fp64 view of a bf16 arena held elsewhere (e.g. a large
    model in device memory): `fetch(offset, count)` returns the bf16 bit
    patterns of arena[offset:offset+count].  Only `keep` tensors are cached,
    so a forward pass holds one layer's weights at a time."""

    def __init__(self, desc: dict, fetch, keep=("tok_emb",)):
        self.layout = {name: (off, shape) for name, off, shape in param_layout(desc)[0]}
        self.fetch = fetch
        self.keep = set(keep)
        self.cache = {}

    def __getitem__(self, name):
        if name in self.cache:
            return self.cache[name]
        off, shape = self.layout[name]
        bits = self.fetch(off, int(np.prod(shape)))
        v = bf16_bits_to_f64(bits).reshape(shape)
        if name in self.keep:
            self.cache[name] = v
        return v


def unpack(desc: dict, arena_f64: np.ndarray) -> dict:
    layout, _ = param_layout(desc)
    return {name: arena_f64[off:off + int(np.prod(shape))].reshape(shape)
            for name, off, shape in layout}


# ================================================================== models
def gelu_erf(x: np.ndarray) -> np.ndarray:
    from scipy.special import erf
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def logsumexp_rows(a: np.ndarray) -> np.ndarray:
    m = a.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(a - m).sum(axis=-1, keepdims=True)))[..., 0]


def lsq_loss(W: np.ndarray, X: np.ndarray, Y: np.ndarray) -> float:
    """L = ||X W - Y||_F^2 / (2n): the normalisation whose gradient is
    X^T (X W - Y) / n."""
    W, X, Y = (np.asarray(a, np.float64) for a in (W, X, Y))
    r = X @ W - Y
    return float((r * r).sum() / (2.0 * X.shape[0]))


def lsq_grad(W, X, Y) -> np.ndarray:
    W, X, Y = (np.asarray(a, np.float64) for a in (W, X, Y))
    return X.T @ (X @ W - Y) / X.shape[0]


def mean_ce(logits: np.ndarray, labels) -> float:
    lse = logsumexp_rows(logits)
    return float(np.mean(lse - logits[np.arange(logits.shape[0]), labels]))


def mlp_loss(W1, W2, X, labels) -> float:
    """Mean cross-entropy of logits = GELU(X W1^T) W2^T (no biases)."""
    W1, W2, X = (np.asarray(a, np.float64) for a in (W1, W2, X))
    h = gelu_erf(X @ W1.T)
    return mean_ce(h @ W2.T, labels)


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def causal_attention(qkv: np.ndarray, heads: int) -> np.ndarray:
    """softmax(Q K^T / sqrt(dh) + causal mask) V per sequence and head, fp64.
    qkv [B][S][3d] with Q, K, V blocks of d columns, head h at h*dh."""
    B, S, three_d = qkv.shape
    d = three_d // 3
    dh = d // heads
    Q = qkv[..., :d].reshape(B, S, heads, dh).transpose(0, 2, 1, 3)
    K = qkv[..., d:2 * d].reshape(B, S, heads, dh).transpose(0, 2, 1, 3)
    V = qkv[..., 2 * d:].reshape(B, S, heads, dh).transpose(0, 2, 1, 3)
    s = (Q @ K.transpose(0, 1, 3, 2)) / np.sqrt(dh)                       # [B,H,S,S]
    s[..., np.triu(np.ones((S, S), dtype=bool), k=1)] = -np.inf
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    P = e / e.sum(axis=-1, keepdims=True)
    return (P @ V).transpose(0, 2, 1, 3).reshape(B, S, d)


def decoder_loss(desc: dict, params, tokens: np.ndarray, round_bf16: bool = True) -> float:
    """Causal-LM mean cross-entropy of a pre-LN decoder.

    Embedding + learned positions; per block h += W_o Attn(LN1 h),
    h += W_down act(W_up LN2 h); final LN; LM head tied to the token embedding.
    No linear biases, LN eps 1e-5, attention scale 1/sqrt(d_h), causal mask.
    Loss = mean over the B*(S-1) next-token positions.

    bf16 rounding points (when ``round_bf16``): embedding sum, every LN output,
    every GEMM output (QKV, attention output, O, up after the activation, down),
    both residual sums.  Everything else (softmax, LN statistics, logits, CE)
    is exact fp64.  ``params`` maps tensor names to fp64 arrays (any mapping,
    so large models can be fetched tensor by tensor).
    """
    R = bf16_round if round_bf16 else (lambda a: a)
    act = gelu_erf if desc["act"] == "gelu" else (lambda a: np.maximum(a, 0.0))
    B, S = tokens.shape
    p = params
    h = R(p["tok_emb"][tokens] + p["pos_emb"][:S][None, :, :])           # [B,S,d]
    for layer in range(desc["layers"]):
        q = f"l{layer}."
        x = R(layer_norm(h, p[q + "ln1_g"], p[q + "ln1_b"]))
        qkv = R(x @ p[q + "w_qkv"].T)                                      # [B,S,3d]
        o = R(causal_attention(qkv, desc["heads"]))
        h = R(h + R(o @ p[q + "w_o"].T))
        x = R(layer_norm(h, p[q + "ln2_g"], p[q + "ln2_b"]))
        u = R(act(x @ p[q + "w_up"].T))
        h = R(h + R(u @ p[q + "w_down"].T))
    x = R(layer_norm(h, p["lnf_g"], p["lnf_b"]))
    emb = p["tok_emb"]
    tgt = tokens[:, 1:]
    total = 0.0
    for b in range(B):  # one sequence at a time keeps the logits block small
        logits = x[b, :-1, :] @ emb.T                                      # [S-1,V]
        lse = logsumexp_rows(logits)
        total += float(np.sum(lse - logits[np.arange(S - 1), tgt[b]]))
    return total / (B * (S - 1))


# ============================================================ arena helpers
class Arena:
    """A model's flat parameter vector in its storage dtype ('f32' or 'bf16')."""

    def __init__(self, desc: dict, data: np.ndarray):
        self.desc = desc
        self.dtype = "bf16" if data.dtype == np.uint16 else "f32"
        assert data.dtype in (np.uint16, np.float32)
        self.data = np.ascontiguousarray(data)

    def copy(self) -> "Arena":
        return Arena(self.desc, self.data.copy())

    def values(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f64(self.data)
        return self.data.astype(np.float64)

    @property
    def dirs(self) -> str:
        return self.desc.get("dirs", "gauss")

    def perturb(self, seed: int, probe: int, sigma: float) -> None:
        """w <- round_storage(w + sigma * z_probe), every element of the arena."""
        kind = "bf16" if self.dtype == "bf16" else "f32"
        args = (_ptr(self.data), self.data.size, 0, seed, probe, float(np.float32(sigma)))
        if self.dirs == "q8":
            getattr(lib(), "oracle_q8_perturb_" + kind)(*args, _ptr(_q8()))
        else:
            getattr(lib(), "oracle_perturb_" + kind)(*args)

    def perturb_range(self, off: int, n: int, seed: int, probe: int, sigma: float) -> None:
        """The same on arena elements off .. off+n-1 only (direction elements
        off .. off+n-1)."""
        kind = "bf16" if self.dtype == "bf16" else "f32"
        view = self.data[off:off + n]
        args = (_ptr(view), n, off, seed, probe, float(np.float32(sigma)))
        if self.dirs == "q8":
            getattr(lib(), "oracle_q8_perturb_" + kind)(*args, _ptr(_q8()))
        else:
            getattr(lib(), "oracle_perturb_" + kind)(*args)

    def update_range(self, off: int, n: int, seed: int, coeffs: np.ndarray) -> None:
        """w <- round_storage(w + sum_i c_i z_i) on elements off .. off+n-1."""
        c = np.ascontiguousarray(coeffs, dtype=np.float64)
        kind = "bf16" if self.dtype == "bf16" else "f32"
        view = self.data[off:off + n]
        args = (_ptr(view), n, off, seed, c.size, _ptr(c))
        if self.dirs == "q8":
            getattr(lib(), "oracle_q8_update_" + kind)(*args, _ptr(_q8()))
        else:
            getattr(lib(), "oracle_update_" + kind)(*args)

    def update(self, seed: int, coeffs: np.ndarray) -> None:
        """w <- round_storage(w + sum_i c_i z_i), every element of the arena."""
        c = np.ascontiguousarray(coeffs, dtype=np.float64)
        kind = "bf16" if self.dtype == "bf16" else "f32"
        args = (_ptr(self.data), self.data.size, 0, seed, c.size, _ptr(c))
        if self.dirs == "q8":
            getattr(lib(), "oracle_q8_update_" + kind)(*args, _ptr(_q8()))
        else:
            getattr(lib(), "oracle_update_" + kind)(*args)


def fedspzo_step(arena: Arena, batch: dict, seed: int, p1: int, ps: int, eps: float, lr: float):
    """One split-perturbation step on the MLP (FedSPZO summary, section 2
    "방법론"); updates ``arena`` in place.

    The network is split into a first, larger block theta_1 = W1 (with the
    GELU) and a second, smaller block theta_2 = W2.  For each of p1 directions
    z1_i of theta_1 and each sign s: the block-1 output y_s = GELU(X D(W1 +
    s eps z1_i)^T) is computed once and reused by ps directions z2_m of
    theta_2, each evaluated at +eps and -eps: L(m, +-) = CE(y_s D(W2 +- eps
    z2_m)^T), m = (2 i + v) ps + k for sign index v (0: +, 1: -) and k < ps.
    So theta_2 gets p2 = 2 p1 ps directions.
      g2_m = (L(m, +) - L(m, -)) / (2 eps)      (losses sharing one y_s)
      g1_i = (Lbar(i, +) - Lbar(i, -)) / (2 eps), Lbar(i, s) the mean of the
             2 ps losses of branch s (the average of the f2 perturbations'
             loss differences)
    then W1 <- D(W1 - (lr/p1) sum_i g1_i z1_i), W2 <- D(W2 - (lr/p2) sum_m
    g2_m z2_m), nothing if any loss is not finite.  Directions: z1_i is probe
    i of the step seed on W1's elements, z2_m is probe p1 + m on W2's (arena
    element j uses direction element j); no other element is touched.
    Returns (losses [4 p1 ps] as L(m, +), L(m, -) for m = 0, 1, ..., g1 [p1],
    g2 [p2]).
    """
    assert arena.desc["kind"] == "mlp"
    lay = {name: (off, shape) for name, off, shape in param_layout(arena.desc)[0]}
    (o1, s1), (o2, s2) = lay["W1"], lay["W2"]
    n1, n2 = int(np.prod(s1)), int(np.prod(s2))
    sig = float(np.float32(eps))
    X = np.asarray(batch["X"], np.float64)
    labels = batch["labels"]
    p2 = 2 * p1 * ps
    losses = np.zeros(2 * p2)
    for i in range(p1):
        for v, s in enumerate((1.0, -1.0)):
            a = arena.copy()
            a.perturb_range(o1, n1, seed, i, s * sig)
            y = gelu_erf(X @ a.values()[o1:o1 + n1].reshape(s1).T)  # block-1 output, reused below
            for k in range(ps):
                m = (2 * i + v) * ps + k
                for t, u in enumerate((1.0, -1.0)):
                    b = arena.copy()
                    b.perturb_range(o2, n2, seed, p1 + m, u * sig)
                    losses[2 * m + t] = mean_ce(y @ b.values()[o2:o2 + n2].reshape(s2).T, labels)
    g2 = (losses[0::2] - losses[1::2]) / (2.0 * sig)
    branch = losses.reshape(p1, 2, 2 * ps).mean(axis=2)
    g1 = (branch[:, 0] - branch[:, 1]) / (2.0 * sig)
    if np.all(np.isfinite(losses)):
        arena.update_range(o1, n1, seed, -lr * g1 / p1)
        arena.update_range(o2, n2, seed, np.concatenate([np.zeros(p1), -lr * g2 / p2]))
    return losses, g1, g2


DUST_HIDDEN_STREAM, DUST_LOGIT_STREAM = 2, 3


def ce_rows(logits: np.ndarray, labels) -> np.ndarray:
    """Per-row cross-entropy."""
    return logsumexp_rows(logits) - logits[np.arange(logits.shape[0]), labels]


def dust_noise(seed: int, draw: int, stream: int, rows: int, width: int) -> np.ndarray:
    """Noise a[t][w] of one draw: element t * width + w of the stream."""
    return gauss_stream(seed, draw, stream, 0, rows * width).astype(np.float64).reshape(rows, width)


def dust_step(arena: Arena, batch: dict, seed: int, k1: int, sigma1: float, k2: int, sigma2: float, lr: float):
    """One Dust step on the MLP (Dust review page, "Dust: 역전파 없이
    트랜스포머를 사전학습하다", sections "Dust의 해법: 가상 개체군" and "신용
    할당(credit assignment): 보상에서 기울기까지", plus "간섭(interference)
    줄이기" for the separate forward per layer type and the head perturbed on
    cached logits); updates ``arena`` in place.

    Every sample t of the batch is a token.  The clean forward is cached:
    Y = X W1^T, A = GELU(Y), Z = A W2^T.
    Hidden layer (output y_t of W1), k1 draws with noise a ~ N(0, I) from
    stream 2 (draw i, element t * hidden + h):
      l[i][t] = CE(GELU(Y_t + sigma1 a_t^(i)) W2^T, label_t)   (per token)
      c = lbar_t - l[i][t], lbar_t the mean over the draws; the tokens are
      independent, so the reward is r = c (no later tokens to credit);
      ghat_t = -(1 / (k1 sigma1)) sum_i r a_t^(i),  G_W1 = sum_t ghat_t x_t^T.
    Head (output of W2, the logits), k2 draws on the cached logits with noise
    b ~ N(0, I) from stream 3 (element t * classes + c):
      l2[i][t] = CE(Z_t + sigma2 b_t^(i)), the same rewards,
      ghat2_t = -(1 / (k2 sigma2)) sum_i r2 b_t^(i),  G_W2 = sum_t ghat2_t A_t^T.
    Then W1 <- D(W1 - lr G_W1), W2 <- D(W2 - lr G_W2) (sigma and lr at fp32
    precision; both estimates from the same W), nothing if any loss is not
    finite.  The sums over tokens estimate the gradient of the summed token
    losses.  Returns (l [k1][M], l2 [k2][M], clean per-token losses [M],
    ghat [M][hidden], ghat2 [M][classes]).
    """
    assert arena.desc["kind"] == "mlp"
    lay = {name: (off, shape) for name, off, shape in param_layout(arena.desc)[0]}
    (o1, s1), (o2, s2) = lay["W1"], lay["W2"]
    n1, n2 = int(np.prod(s1)), int(np.prod(s2))
    vals = arena.values()
    W1 = vals[o1:o1 + n1].reshape(s1)
    W2 = vals[o2:o2 + n2].reshape(s2)
    X = np.asarray(batch["X"], np.float64)
    labels = batch["labels"]
    M, H, C = X.shape[0], s1[0], s2[0]
    sg1, sg2 = float(np.float32(sigma1)), float(np.float32(sigma2))
    Y = X @ W1.T
    A = gelu_erf(Y)
    Z = A @ W2.T
    l0 = ce_rows(Z, labels)
    # hidden layer: k1 draws, each a forward of the layers after W1
    noise1 = [dust_noise(seed, i, DUST_HIDDEN_STREAM, M, H) for i in range(k1)]
    l1 = np.stack([ce_rows(gelu_erf(Y + sg1 * a) @ W2.T, labels) for a in noise1])
    r1 = l1.mean(axis=0)[None, :] - l1
    ghat = -sum(r1[i][:, None] * noise1[i] for i in range(k1)) / (k1 * sg1)
    G1 = ghat.T @ X
    # head: k2 draws on the cached logits
    noise2 = [dust_noise(seed, i, DUST_LOGIT_STREAM, M, C) for i in range(k2)]
    l2 = np.stack([ce_rows(Z + sg2 * b, labels) for b in noise2])
    r2 = l2.mean(axis=0)[None, :] - l2
    ghat2 = -sum(r2[i][:, None] * noise2[i] for i in range(k2)) / (k2 * sg2)
    G2 = ghat2.T @ A
    if np.all(np.isfinite(l1)) and np.all(np.isfinite(l2)):
        lr32 = float(np.float32(lr))
        new = arena.data.copy()
        if arena.dtype != "f32":
            raise ValueError("the MLP arena is fp32")
        new[o1:o1 + n1] = (W1 - lr32 * G1).ravel().astype(np.float32)
        new[o2:o2 + n2] = (W2 - lr32 * G2).ravel().astype(np.float32)
        arena.data[:] = new
    return l1, l2, l0, ghat, ghat2


def model_loss(arena: Arena, batch: dict, round_bf16: bool = True) -> float:
    desc = arena.desc
    prm = unpack(desc, arena.values())
    if desc["kind"] == "lsq":
        return lsq_loss(prm["W"], batch["X"], batch["Y"])
    if desc["kind"] == "mlp":
        return mlp_loss(prm["W1"], prm["W2"], batch["X"], batch["labels"])
    return decoder_loss(desc, prm, batch["tokens"], round_bf16=round_bf16)


# ==================================================================== step
def probe_curvature(lp, lm, l0, sig):
    """Central second difference along each probe direction:
    (L(W + s z) + L(W - s z) - 2 L(W)) / s^2 = z^T H z + O(s^2)."""
    return ((np.asarray(lp) + np.asarray(lm)) - 2.0 * l0) / (sig * sig)


def spsa_step(arena: Arena, batch: dict, seed: int, n_probes: int, eps: float, lr: float,
              mode: str = "inplace", round_bf16: bool = True, precond: bool = False,
              curv_floor: float = 1.0):
    """One multi-probe SPSA step; updates ``arena`` in place.

    inplace: for each probe i, W += eps z_i; L+ ; W -= 2 eps z_i; L- ;
             W += eps z_i (restore), all on the stored weights.
    fused:   each evaluation sees round_storage(W_t +- eps z_i) of the same W_t.
    Then g_i = (L+_i - L-_i) / (2 eps) with eps taken at fp32 precision,
    c_i = -lr * g_i / N, and W <- round_storage(W + sum_i c_i z_i).
    Returns (losses [2N] as L+_0, L-_0, L+_1, ..., g [N]).

    precond (1.5-SPSA, ZOO blog, section on the first paper, probe-space
    preconditioning): one clean evaluation L0 at the stored weights, taken
    before any probe, gives each direction a curvature estimate
    h_i = (L+_i + L-_i - 2 L0) / eps^2 (the central second difference of
    L along z_i, i.e. z_i^T H z_i up to O(eps^2)); the step then uses
    g_i / max(h_i, curv_floor) in place of g_i (curv_floor at fp32 precision),
    and the returned losses hold 2N + 1 values, L0 last.
    """
    sig = float(np.float32(eps))
    losses = np.zeros(2 * n_probes + (1 if precond else 0))
    if precond:
        losses[2 * n_probes] = model_loss(arena, batch, round_bf16)
    for i in range(n_probes):
        if mode == "inplace":
            arena.perturb(seed, i, sig)
            losses[2 * i] = model_loss(arena, batch, round_bf16)
            arena.perturb(seed, i, -2.0 * sig)
            losses[2 * i + 1] = model_loss(arena, batch, round_bf16)
            arena.perturb(seed, i, sig)
        elif mode == "fused":
            a = arena.copy()
            a.perturb(seed, i, sig)
            losses[2 * i] = model_loss(a, batch, round_bf16)
            a = arena.copy()
            a.perturb(seed, i, -sig)
            losses[2 * i + 1] = model_loss(a, batch, round_bf16)
        else:
            raise ValueError(mode)
    lp, lm = losses[0:2 * n_probes:2], losses[1:2 * n_probes:2]
    g = (lp - lm) / (2.0 * sig)
    if precond:
        h = probe_curvature(lp, lm, losses[2 * n_probes], sig)
        with np.errstate(invalid="ignore"):
            g = np.where(np.isfinite(h), g / np.maximum(h, float(np.float32(curv_floor))), h)
    c = -lr * g / n_probes
    if np.all(np.isfinite(losses)):
        arena.update(seed, c)
    return losses, g
