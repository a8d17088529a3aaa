"""Python binding of libzo.so (ctypes).  Argument marshalling only: every step
of the path runs in the library's HIP kernels; torch supplies device memory and
the stream.  Importing this module loads the library and fails loudly when it
is missing or cannot be loaded -- there is no fallback."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libzo.so")

ZO_OK, ZO_ERR_INVALID, ZO_ERR_UNSUPPORTED, ZO_ERR_HIP, ZO_ERR_NONFINITE, ZO_ERR_WORKSPACE = 0, -1, -2, -3, -4, -5
ZO_F32, ZO_BF16 = 0, 1
ZO_MODEL_LSQ, ZO_MODEL_MLP, ZO_MODEL_DECODER = 0, 1, 2
ZO_ACT_GELU, ZO_ACT_RELU = 0, 1
ZO_MODE_INPLACE, ZO_MODE_FUSED, ZO_MODE_COPIES = 0, 1, 2
ZO_DIRS_GAUSS, ZO_DIRS_Q8 = 0, 1

EXPORTS = [
    "zo_param_layout", "zo_workspace_bytes", "zo_model_create", "zo_model_destroy", "zo_perturb",
    "zo_forward_loss", "zo_update", "zo_step", "zo_step_noalloc", "zo_step_split", "zo_step_dust", "zo_replay_step", "zo_perturb_buffer", "zo_update_buffer", "zo_gscalar",
    "zo_debug_rng", "zo_debug_box_muller", "zo_status_str", "zo_last_error",
    "zo_timing_enable", "zo_timing_select", "zo_timing_reset", "zo_timing_query",
    "zo_debug_gemm_bf16", "zo_debug_attention", "zo_debug_layernorm",
]


class ZoError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: status {status}: {msg}")
        self.status = status


class ModelDesc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("dtype", ctypes.c_int32), ("batch", ctypes.c_int64),
                ("seq", ctypes.c_int64), ("d_in", ctypes.c_int64), ("d_out", ctypes.c_int64),
                ("hidden", ctypes.c_int64), ("classes", ctypes.c_int64), ("layers", ctypes.c_int64),
                ("d_model", ctypes.c_int64), ("heads", ctypes.c_int64), ("ffn", ctypes.c_int64),
                ("vocab", ctypes.c_int64), ("max_seq", ctypes.c_int64), ("act", ctypes.c_int32),
                ("dirs", ctypes.c_int32)]


class ParamInfo(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("offset", ctypes.c_uint64), ("shape", ctypes.c_int64 * 2),
                ("ndim", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Batch(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("labels", ctypes.c_void_p),
                ("tokens", ctypes.c_void_p), ("batch", ctypes.c_int64), ("seq", ctypes.c_int64)]


class Pert(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("probe", ctypes.c_uint32), ("sigma", ctypes.c_float)]


class SplitCfg(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("p1", ctypes.c_uint32), ("ps", ctypes.c_uint32),
                ("eps", ctypes.c_float), ("lr", ctypes.c_float)]


class DustCfg(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("k1", ctypes.c_uint32), ("k2", ctypes.c_uint32),
                ("sigma1", ctypes.c_float), ("sigma2", ctypes.c_float), ("lr", ctypes.c_float)]


class StepCfg(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("n_probes", ctypes.c_uint32), ("eps", ctypes.c_float),
                ("lr", ctypes.c_float), ("mode", ctypes.c_int32), ("precond", ctypes.c_int32),
                ("curv_floor", ctypes.c_float)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first (zeroth_order_backprop_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    P, U64, U32, I32, F = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int32, ctypes.c_float
    sigs = {
        "zo_param_layout": [P, P, I32, P, P],
        "zo_workspace_bytes": [P, P],
        "zo_model_create": [P, P, U64, P, ctypes.c_size_t, P],
        "zo_model_destroy": [P],
        "zo_perturb": [P, U64, U32, F, P],
        "zo_forward_loss": [P, P, P, I32, P, P],
        "zo_update": [P, U64, U32, P, F, P],
        "zo_step": [P, P, P, P, P, P],
        "zo_step_noalloc": [P, P, U64, P, P, P, P, P],
        "zo_replay_step": [P, P, P, P],
        "zo_step_split": [P, P, P, P, P, P, P],
        "zo_step_dust": [P, P, P, P, P],
        "zo_perturb_buffer": [P, I32, I32, U64, U64, U64, U32, F, P],
        "zo_update_buffer": [P, I32, I32, U64, U64, U64, U32, P, F, P],
        "zo_gscalar": [P, U32, F, P, P],
        "zo_debug_rng": [U64, U32, U64, U64, P, P, P],
        "zo_debug_box_muller": [P, U64, P, P],
        "zo_debug_gemm_bf16": [P, P, P, I32, I32, I32, I32, P],
        "zo_debug_attention": [P, P, I32, I32, I32, I32, P],
        "zo_debug_layernorm": [P, P, P, P, I32, I32, P],
        "zo_timing_enable": [I32],
        "zo_timing_select": [ctypes.c_char_p],
        "zo_timing_reset": [],
        "zo_timing_query": [ctypes.c_char_p, P, P],
    }
    for name, args in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.zo_status_str.argtypes = [ctypes.c_int]
    L.zo_status_str.restype = ctypes.c_char_p
    L.zo_last_error.argtypes = []
    L.zo_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def check(status: int, where: str) -> None:
    if status != ZO_OK:
        raise ZoError(status, where, lib().zo_last_error().decode(errors="replace"))


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ------------------------------------------------------------ raw buffers
def perturb_buffer(w, n, j0, seed, probe, sigma, dtype, stream=None, dirs=ZO_DIRS_GAUSS):
    check(lib().zo_perturb_buffer(_ptr(w), dtype, dirs, n, j0, seed, probe, float(sigma), _stream(stream)),
          "zo_perturb_buffer")


def update_buffer(w, n, j0, seed, n_probes, g_dev, lr, dtype, stream=None, dirs=ZO_DIRS_GAUSS):
    check(lib().zo_update_buffer(_ptr(w), dtype, dirs, n, j0, seed, n_probes, _ptr(g_dev), float(lr),
                                 _stream(stream)), "zo_update_buffer")


def gscalar(losses_dev, n, eps, g_dev, stream=None):
    check(lib().zo_gscalar(_ptr(losses_dev), n, float(eps), _ptr(g_dev), _stream(stream)), "zo_gscalar")


def debug_rng(seed, probe, j0, n, words=None, z=None, stream=None):
    check(lib().zo_debug_rng(seed, probe, j0, n, _ptr(words), _ptr(z), _stream(stream)), "zo_debug_rng")


def debug_box_muller(pairs, n_pairs, z, stream=None):
    check(lib().zo_debug_box_muller(_ptr(pairs), n_pairs, _ptr(z), _stream(stream)), "zo_debug_box_muller")


def debug_gemm_bf16(A, W, C, M, N, K, epi=0, stream=None):
    check(lib().zo_debug_gemm_bf16(_ptr(A), _ptr(W), _ptr(C), M, N, K, epi, _stream(stream)), "zo_debug_gemm_bf16")


def debug_attention(qkv, out, B, S, H, dh, stream=None):
    check(lib().zo_debug_attention(_ptr(qkv), _ptr(out), B, S, H, dh, _stream(stream)), "zo_debug_attention")


def debug_layernorm(h, g, b, x, rows, d, stream=None):
    check(lib().zo_debug_layernorm(_ptr(h), _ptr(g), _ptr(b), _ptr(x), rows, d, _stream(stream)),
          "zo_debug_layernorm")


# ------------------------------------------------------------------ timing
def timing_enable(on: bool = True) -> None:
    check(lib().zo_timing_enable(1 if on else 0), "zo_timing_enable")


def timing_select(family=None) -> None:
    """Restrict timing to one kernel family (None: every family)."""
    check(lib().zo_timing_select(family.encode() if family else None), "zo_timing_select")


def timing_reset() -> None:
    check(lib().zo_timing_reset(), "zo_timing_reset")


def timing_query(family: str):
    """(total ms, launches) of one kernel family since the last reset."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    check(lib().zo_timing_query(family.encode(), ctypes.byref(ms), ctypes.byref(n)), "zo_timing_query")
    return ms.value, n.value


# ------------------------------------------------------------------ models
def make_desc(kind: int, **kw) -> ModelDesc:
    d = ModelDesc()
    d.kind = kind
    d.dtype = kw.pop("dtype", ZO_BF16 if kind == ZO_MODEL_DECODER else ZO_F32)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def param_layout(desc: ModelDesc):
    n = ctypes.c_int32()
    total = ctypes.c_uint64()
    check(lib().zo_param_layout(ctypes.byref(desc), None, 0, ctypes.byref(n), ctypes.byref(total)),
          "zo_param_layout")
    arr = (ParamInfo * n.value)()
    check(lib().zo_param_layout(ctypes.byref(desc), arr, n.value, ctypes.byref(n), ctypes.byref(total)),
          "zo_param_layout")
    out = []
    for p in arr:
        shape = tuple(p.shape[:p.ndim])
        out.append((p.name.decode(), int(p.offset), shape))
    return out, int(total.value)


def workspace_bytes(desc: ModelDesc) -> int:
    b = ctypes.c_size_t()
    check(lib().zo_workspace_bytes(ctypes.byref(desc), ctypes.byref(b)), "zo_workspace_bytes")
    return int(b.value)


class Model:
    """A model over a caller-owned parameter arena (torch tensor on cuda) and a
    workspace this object allocates through torch."""

    def __init__(self, desc: ModelDesc, arena):
        import torch
        self.desc = desc
        self.arena = arena
        self.layout, self.total = param_layout(desc)
        if arena.numel() != self.total:
            raise ValueError(f"arena has {arena.numel()} elements, layout needs {self.total}")
        nbytes = workspace_bytes(desc)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=arena.device)
        h = ctypes.c_void_p()
        check(lib().zo_model_create(ctypes.byref(desc), _ptr(arena), self.total, _ptr(self.workspace),
                                    nbytes, ctypes.byref(h)), "zo_model_create")
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.zo_model_destroy(h)
            self._h = None

    def perturb(self, seed, probe, sigma, stream=None):
        check(lib().zo_perturb(self._h, seed, probe, float(sigma), _stream(stream)), "zo_perturb")

    def forward_loss(self, batch: Batch, loss_dev, perts=None, stream=None):
        n = 0 if not perts else len(perts)
        arr = None
        if n:
            arr = (Pert * n)(*[Pert(int(s), int(i), float(sg)) for (s, i, sg) in perts])
        check(lib().zo_forward_loss(self._h, ctypes.byref(batch), arr, n, _ptr(loss_dev), _stream(stream)),
              "zo_forward_loss")

    def update(self, seed, n_probes, g_dev, lr, stream=None):
        check(lib().zo_update(self._h, seed, n_probes, _ptr(g_dev), float(lr), _stream(stream)), "zo_update")

    def step(self, batch: Batch, seed, n_probes, eps, lr, mode, losses_dev, g_dev, stream=None,
             precond=0, curv_floor=0.0):
        """One SPSA step; precond=1 selects 1.5-SPSA, and losses_dev then needs
        2 * n_probes + 1 entries (the clean loss last)."""
        need = 2 * int(n_probes) + (1 if precond else 0)
        if losses_dev.numel() < need or g_dev.numel() < int(n_probes):
            raise ValueError(f"zo_step: losses need {need} entries, g {int(n_probes)}")
        cfg = StepCfg(int(seed), int(n_probes), float(eps), float(lr), int(mode), int(precond), float(curv_floor))
        check(lib().zo_step(self._h, ctypes.byref(batch), ctypes.byref(cfg), _ptr(losses_dev), _ptr(g_dev),
                            _stream(stream)), "zo_step")

    def step_split(self, batch: Batch, seed, p1, ps, eps, lr, losses_dev, g1_dev, g2_dev, stream=None):
        """One split-perturbation (FedSPZO) step of the MLP: losses 4 p1 ps,
        g1 p1, g2 2 p1 ps entries (device fp64)."""
        p1, ps = int(p1), int(ps)
        if losses_dev.numel() < 4 * p1 * ps or g1_dev.numel() < p1 or g2_dev.numel() < 2 * p1 * ps:
            raise ValueError("zo_step_split: losses need 4 p1 ps entries, g1 p1, g2 2 p1 ps")
        cfg = SplitCfg(int(seed), p1, ps, float(eps), float(lr))
        check(lib().zo_step_split(self._h, ctypes.byref(batch), ctypes.byref(cfg), _ptr(losses_dev), _ptr(g1_dev),
                                  _ptr(g2_dev), _stream(stream)), "zo_step_split")

    def step_dust(self, batch: Batch, seed, k1, k2, sigma1, sigma2, lr, losses_dev, stream=None):
        """One Dust step of the MLP; losses_dev (device fp64) needs
        (1 + k1 + k2) * batch entries: clean, hidden draws, head draws."""
        need = (1 + int(k1) + int(k2)) * int(batch.batch)
        if losses_dev.numel() < need:
            raise ValueError(f"zo_step_dust: losses need {need} entries")
        cfg = DustCfg(int(seed), int(k1), int(k2), float(sigma1), float(sigma2), float(lr))
        check(lib().zo_step_dust(self._h, ctypes.byref(batch), ctypes.byref(cfg), _ptr(losses_dev), _stream(stream)),
              "zo_step_dust")

    def replay_step(self, seed, n_probes, eps, lr, mode, g_dev, stream=None):
        """The weight changes of a recorded step, given the g it produced."""
        if g_dev.numel() < int(n_probes):
            raise ValueError(f"zo_replay_step: g needs {int(n_probes)} entries")
        cfg = StepCfg(int(seed), int(n_probes), float(eps), float(lr), int(mode), 0, 0.0)
        check(lib().zo_replay_step(self._h, ctypes.byref(cfg), _ptr(g_dev), _stream(stream)), "zo_replay_step")


def step_noalloc(desc: ModelDesc, arena, batch: Batch, seed, n_probes, eps, lr, mode, losses_dev, g_dev,
                 stream=None, precond=0, curv_floor=0.0):
    """zo_step_noalloc: one SPSA step on `arena` (device tensor) with the
    library's static scratch as the workspace; no allocation."""
    cfg = StepCfg(int(seed), int(n_probes), float(eps), float(lr), int(mode), int(precond), float(curv_floor))
    check(lib().zo_step_noalloc(ctypes.byref(desc), _ptr(arena), arena.numel(), ctypes.byref(batch),
                                ctypes.byref(cfg), _ptr(losses_dev), _ptr(g_dev), _stream(stream)),
          "zo_step_noalloc")


def make_batch(x=None, y=None, labels=None, tokens=None, batch=0, seq=0) -> Batch:
    """A zo_batch over device tensors: x, y fp32, labels and tokens int32, all
    contiguous on a GPU.  The returned structure keeps references to the
    tensors, so they live as long as it does."""
    import torch
    b = Batch()
    for name, t, dt in (("x", x, torch.float32), ("y", y, torch.float32), ("labels", labels, torch.int32),
                        ("tokens", tokens, torch.int32)):
        if t is None:
            setattr(b, name, None)
            continue
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"make_batch: {name} must be a contiguous {dt} tensor on a GPU "
                             f"(got {t.dtype}, device {t.device}, contiguous={t.is_contiguous()})")
        setattr(b, name, t.data_ptr())
    b.batch = batch
    b.seq = seq
    b._keep = (x, y, labels, tokens)
    return b
