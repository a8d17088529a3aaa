"""CPU-side checks of the C ABI: the library loads, exports every function
include/zo.h declares, validates arguments before launching anything, and
reports the same parameter arena layout as the oracle states independently."""
import ctypes
import os
import re

import pytest

from oracle import oracle
from zeroth_order_backprop_amd import zo

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "zo.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zo_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = zo.lib()
    names = declared_functions()
    assert len(names) >= 15
    for name in names:
        assert hasattr(L, name), name
    assert sorted(zo.EXPORTS) == names


def test_status_strings():
    L = zo.lib()
    for st in (0, -1, -2, -3, -4, -5):
        assert L.zo_status_str(st)


DESCS = {
    "lsq": ({"kind": "lsq", "n": 512, "d_in": 256, "d_out": 256},
            dict(kind=zo.ZO_MODEL_LSQ, batch=512, d_in=256, d_out=256)),
    "mlp": ({"kind": "mlp", "batch": 256, "d_in": 1024, "hidden": 4096, "classes": 10},
            dict(kind=zo.ZO_MODEL_MLP, batch=256, d_in=1024, hidden=4096, classes=10)),
    "gpt": ({"kind": "decoder", "layers": 12, "d": 768, "heads": 12, "ffn": 3072, "vocab": 32000,
             "max_seq": 512, "act": "gelu"},
            dict(kind=zo.ZO_MODEL_DECODER, batch=8, seq=512, layers=12, d_model=768, heads=12, ffn=3072,
                 vocab=32000, max_seq=512, act=zo.ZO_ACT_GELU)),
    "odd": ({"kind": "decoder", "layers": 1, "d": 128, "heads": 2, "ffn": 192, "vocab": 33,
             "max_seq": 7, "act": "relu"},
            dict(kind=zo.ZO_MODEL_DECODER, batch=1, seq=7, layers=1, d_model=128, heads=2, ffn=192,
                 vocab=33, max_seq=7, act=zo.ZO_ACT_RELU)),
}


@pytest.mark.parametrize("name", sorted(DESCS))
def test_layout_matches_oracle(name):
    odesc, kw = DESCS[name]
    want, want_total = oracle.param_layout(odesc)
    desc = zo.make_desc(**kw)
    try:
        got, total = zo.param_layout(desc)
    except zo.ZoError as e:
        if e.status == zo.ZO_ERR_UNSUPPORTED:
            pytest.skip(str(e))
        raise
    assert total == want_total
    assert [(n, o, tuple(s)) for n, o, s in got] == [(n, o, tuple(s)) for n, o, s in want]


def test_parameter_counts():
    for name, count in (("lsq", 65_536), ("mlp", 4_235_264), ("gpt", 109_942_272)):
        _, total = oracle.param_layout(DESCS[name][0])
        assert total == count


def test_validation_rejects_before_launch():
    L = zo.lib()
    s = ctypes.c_void_p(0)
    G, Q = zo.ZO_DIRS_GAUSS, zo.ZO_DIRS_Q8
    assert L.zo_perturb_buffer(None, zo.ZO_F32, G, 16, 0, 1, 0, 1e-3, s) == zo.ZO_ERR_INVALID
    assert L.zo_perturb_buffer(ctypes.c_void_p(256), 7, G, 16, 0, 1, 0, 1e-3, s) == zo.ZO_ERR_UNSUPPORTED
    assert L.zo_perturb_buffer(ctypes.c_void_p(258), zo.ZO_F32, G, 16, 0, 1, 0, 1e-3, s) == zo.ZO_ERR_INVALID
    assert L.zo_perturb_buffer(ctypes.c_void_p(256), zo.ZO_F32, G, 16, 2, 1, 0, 1e-3, s) == zo.ZO_ERR_INVALID
    assert L.zo_perturb_buffer(ctypes.c_void_p(256), zo.ZO_F32, 2, 16, 0, 1, 0, 1e-3, s) == zo.ZO_ERR_INVALID
    assert L.zo_perturb_buffer(ctypes.c_void_p(256), zo.ZO_F32, Q, 16, 4, 1, 0, 1e-3, s) == zo.ZO_ERR_INVALID
    assert L.zo_update_buffer(ctypes.c_void_p(256), zo.ZO_F32, G, 16, 0, 1, 0, ctypes.c_void_p(512), 1e-3,
                              s) == zo.ZO_ERR_INVALID
    assert L.zo_update_buffer(ctypes.c_void_p(256), zo.ZO_F32, G, 16, 0, 1, 2, None, 1e-3, s) == zo.ZO_ERR_INVALID
    assert L.zo_update_buffer(ctypes.c_void_p(256), zo.ZO_BF16, Q, 16, 8, 1, 2, ctypes.c_void_p(512), 1e-3,
                              s) == zo.ZO_ERR_INVALID
    assert L.zo_debug_rng(0, 0, 0, 16, None, None, s) == zo.ZO_ERR_INVALID
    # debug GEMM: K % 64, N % 8, alignment, and every operand under 2 GiB
    A, W, C = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21), ctypes.c_void_p(1 << 22)
    gemm = L.zo_debug_gemm_bf16
    assert gemm(A, W, C, 256, 256, 96, 0, s) == zo.ZO_ERR_UNSUPPORTED
    assert gemm(A, W, C, 256, 260, 64, 0, s) == zo.ZO_ERR_UNSUPPORTED
    assert gemm(ctypes.c_void_p((1 << 20) + 8), W, C, 256, 256, 64, 0, s) == zo.ZO_ERR_INVALID
    assert gemm(A, W, C, 1 << 16, 1 << 14, 64, 0, s) == zo.ZO_ERR_UNSUPPORTED  # C: 2 GiB
    assert gemm(A, W, C, 1 << 15, 256, 1 << 15, 0, s) == zo.ZO_ERR_UNSUPPORTED  # A: 2 GiB
    assert gemm(None, W, C, 256, 256, 64, 0, s) == zo.ZO_ERR_INVALID
    # model creation: wrong arena size, misalignment, overlap, small workspace
    desc = zo.make_desc(**DESCS["lsq"][1])
    h = ctypes.c_void_p()
    _, total = zo.param_layout(desc)
    ws = zo.workspace_bytes(desc)
    base = 1 << 40
    assert L.zo_model_create(ctypes.byref(desc), ctypes.c_void_p(base), total + 64, ctypes.c_void_p(base << 1),
                             ws, ctypes.byref(h)) == zo.ZO_ERR_INVALID
    assert L.zo_model_create(ctypes.byref(desc), ctypes.c_void_p(base + 4), total, ctypes.c_void_p(base << 1),
                             ws, ctypes.byref(h)) == zo.ZO_ERR_INVALID
    if ws > 0:
        assert L.zo_model_create(ctypes.byref(desc), ctypes.c_void_p(base), total, ctypes.c_void_p(base << 1),
                                 ws - 1, ctypes.byref(h)) == zo.ZO_ERR_WORKSPACE
        assert L.zo_model_create(ctypes.byref(desc), ctypes.c_void_p(base), total, ctypes.c_void_p(base + 256),
                                 ws, ctypes.byref(h)) == zo.ZO_ERR_INVALID
    bad_dirs = zo.make_desc(**dict(DESCS["lsq"][1], dirs=3))
    assert L.zo_model_create(ctypes.byref(bad_dirs), ctypes.c_void_p(base), total, ctypes.c_void_p(base << 1),
                             ws, ctypes.byref(h)) == zo.ZO_ERR_INVALID
    bad = zo.make_desc(**dict(DESCS["gpt"][1], d_model=770))
    assert L.zo_workspace_bytes(ctypes.byref(bad), ctypes.byref(ctypes.c_size_t())) == zo.ZO_ERR_INVALID
    bad = zo.make_desc(**dict(DESCS["gpt"][1], heads=24))  # head dim 32: unsupported
    assert L.zo_workspace_bytes(ctypes.byref(bad), ctypes.byref(ctypes.c_size_t())) == zo.ZO_ERR_UNSUPPORTED
    bad = zo.make_desc(**dict(DESCS["lsq"][1], dtype=zo.ZO_BF16))
    assert L.zo_workspace_bytes(ctypes.byref(bad), ctypes.byref(ctypes.c_size_t())) == zo.ZO_ERR_UNSUPPORTED


def test_step_validation_without_gpu():
    L = zo.lib()
    desc = zo.make_desc(**DESCS["lsq"][1])
    _, total = zo.param_layout(desc)
    ws = zo.workspace_bytes(desc)
    h = ctypes.c_void_p()
    base = 1 << 40
    assert L.zo_model_create(ctypes.byref(desc), ctypes.c_void_p(base), total, ctypes.c_void_p(base << 1),
                             ws, ctypes.byref(h)) == zo.ZO_OK
    b = zo.Batch()
    b.x, b.y, b.batch = base << 2, base << 3, 512
    cfg = zo.StepCfg(0, 0, 1e-3, 1e-2, zo.ZO_MODE_FUSED)       # N = 0
    out = ctypes.c_void_p(base << 4)
    assert L.zo_step(h, ctypes.byref(b), ctypes.byref(cfg), out, out, None) == zo.ZO_ERR_INVALID
    cfg = zo.StepCfg(0, 4, 0.0, 1e-2, zo.ZO_MODE_FUSED)        # eps = 0
    assert L.zo_step(h, ctypes.byref(b), ctypes.byref(cfg), out, out, None) == zo.ZO_ERR_INVALID
    cfg = zo.StepCfg(0, 4, 1e-3, 1e-2, 9)                      # bad mode
    assert L.zo_step(h, ctypes.byref(b), ctypes.byref(cfg), out, out, None) == zo.ZO_ERR_INVALID
    b.batch = 513                                             # larger than the model's batch
    cfg = zo.StepCfg(0, 4, 1e-3, 1e-2, zo.ZO_MODE_FUSED)
    assert L.zo_step(h, ctypes.byref(b), ctypes.byref(cfg), out, out, None) == zo.ZO_ERR_INVALID
    assert L.zo_model_destroy(h) == zo.ZO_OK
