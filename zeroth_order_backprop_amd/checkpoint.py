"""Seed-replay checkpoints of SPSA training.

A trained model is fully determined by its initial weights and, per step, the
step's configuration and its N scalars g_i: every direction is regenerated from
(seed, probe, element), so no weight delta is ever stored (position paper
summary, P5; FedSPZO summary, "통신 프로토콜": the model is rebuilt from seeds
and scalar gradients).  `StepLog` records those scalars as the steps run and
writes them to an ``.npz`` of plain arrays; `replay` applies the recorded steps
to a model holding the initial weights through the library's
``zo_replay_step``, which rebuilds the trained weights bit for bit.

Host logic only: the weights are changed by the library's kernels alone.
"""
from __future__ import annotations

import numpy as np

from . import zo

_FIELDS = ("seed", "n_probes", "eps", "lr", "mode")


class StepLog:
    """Per-step (seed, n_probes, eps, lr, mode) and the fp64 scalars g_i that
    the step's update used (for 1.5-SPSA, the preconditioned ones)."""

    def __init__(self):
        self.steps = []

    def __len__(self):
        return len(self.steps)

    def record(self, seed, n_probes, eps, lr, mode, g):
        """g: the step's g buffer (device tensor or array) of >= n_probes values,
        read after the step has completed (this copies it to the host)."""
        if hasattr(g, "detach"):
            g = g.detach().cpu().numpy()
        g = np.asarray(g, np.float64)[:int(n_probes)].copy()
        if g.shape != (int(n_probes),):
            raise ValueError(f"need {int(n_probes)} scalars, got {g.shape}")
        self.steps.append({"seed": int(seed), "n_probes": int(n_probes), "eps": float(np.float32(eps)),
                           "lr": float(np.float32(lr)), "mode": int(mode), "g": g})

    def save(self, path):
        cfg = {k: np.array([s[k] for s in self.steps],
                           dtype=np.uint64 if k == "seed" else np.float32 if k in ("eps", "lr") else np.int64)
               for k in _FIELDS}
        offsets = np.cumsum([0] + [s["n_probes"] for s in self.steps]).astype(np.int64)
        g = np.concatenate([s["g"] for s in self.steps]) if self.steps else np.zeros(0)
        np.savez(path, g=g, offsets=offsets, **cfg)

    @classmethod
    def load(cls, path):
        log = cls()
        with np.load(path, allow_pickle=False) as f:
            offsets = f["offsets"]
            cols = {k: f[k] for k in _FIELDS}
            g = f["g"]
        if len(offsets) != len(cols["seed"]) + 1 or offsets[-1] != len(g):
            raise ValueError("inconsistent step log")
        for t in range(len(cols["seed"])):
            n = int(cols["n_probes"][t])
            if offsets[t + 1] - offsets[t] != n:
                raise ValueError(f"step {t}: {offsets[t + 1] - offsets[t]} scalars for {n} probes")
            log.steps.append({"seed": int(cols["seed"][t]), "n_probes": n, "eps": float(cols["eps"][t]),
                              "lr": float(cols["lr"][t]), "mode": int(cols["mode"][t]),
                              "g": g[offsets[t]:offsets[t + 1]].astype(np.float64)})
        return log


def replay(model: "zo.Model", log: StepLog, device="cuda"):
    """Apply every recorded step, in order, to `model` (which must hold the
    initial weights), on torch's current stream; synchronise before reading."""
    import torch

    if not len(log):
        return
    g = torch.from_numpy(np.concatenate([s["g"] for s in log.steps])).to(device)
    off = 0
    for s in log.steps:
        n = s["n_probes"]
        model.replay_step(s["seed"], n, s["eps"], s["lr"], s["mode"], g[off:off + n])
        off += n
