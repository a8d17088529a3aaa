"""Host logic of seed-replay checkpoints: the step log's file round trip and
its consistency checks (no GPU; replay itself is covered by the GPU tests)."""
import numpy as np
import pytest

from zeroth_order_backprop_amd import checkpoint


def test_step_log_round_trip(tmp_path):
    log = checkpoint.StepLog()
    rng = np.random.default_rng(0)
    for t, n in enumerate((4, 1, 16)):
        log.record(2**63 + t, n, 1e-3, 1e-2 * (t + 1), t % 2, rng.standard_normal(n + 2))
    p = tmp_path / "log.npz"
    log.save(p)
    back = checkpoint.StepLog.load(p)
    assert len(back) == 3
    for a, b in zip(log.steps, back.steps):
        assert a["seed"] == b["seed"] and a["n_probes"] == b["n_probes"] and a["mode"] == b["mode"]
        assert np.float32(a["eps"]) == np.float32(b["eps"]) and np.float32(a["lr"]) == np.float32(b["lr"])
        assert a["g"].tobytes() == b["g"].tobytes()  # fp64 scalars kept bit for bit


def test_step_log_rejects_inconsistent_files(tmp_path):
    log = checkpoint.StepLog()
    log.record(1, 2, 1e-3, 1e-3, 1, np.ones(2))
    with pytest.raises(ValueError):
        log.record(1, 3, 1e-3, 1e-3, 1, np.ones(2))
    p = tmp_path / "log.npz"
    log.save(p)
    with np.load(p) as f:
        d = dict(f)
    d["n_probes"] = np.array([3])
    np.savez(tmp_path / "bad.npz", **d)
    with pytest.raises(ValueError):
        checkpoint.StepLog.load(tmp_path / "bad.npz")


def test_empty_log(tmp_path):
    log = checkpoint.StepLog()
    log.save(tmp_path / "e.npz")
    assert len(checkpoint.StepLog.load(tmp_path / "e.npz")) == 0
