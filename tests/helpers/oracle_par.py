"""Process-parallel drivers of the CPU oracle for the larger parity cases.

The oracle itself stays single-threaded and plain; these helpers only split
independent work across processes: the element-wise passes over disjoint
ranges of one arena (each range is direction elements lo .. hi-1, exactly the
oracle's range routine), and whole loss evaluations of different weight
states.  Test infrastructure only.
"""
from __future__ import annotations

import multiprocessing
import os

import numpy as np


def workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _perturb_chunk(job):
    path, n, lo, hi, seed, probe, sigma = job
    from oracle import oracle
    data = np.memmap(path, dtype=np.uint16, mode="r+", shape=(n,))
    view = np.ascontiguousarray(data[lo:hi])
    oracle.lib().oracle_perturb_bf16(oracle._ptr(view), hi - lo, lo, seed, probe, float(np.float32(sigma)))
    data[lo:hi] = view
    data.flush()
    del data
    return hi - lo


def perturb_file(pool, path: str, n: int, seed: int, probe: int, sigma: float) -> None:
    """w <- bf16(w + sigma z_probe) over the bf16 arena stored in `path`
    (n elements), split into one range per worker."""
    k = workers()
    step = (n + k - 1) // k
    step = (step + 63) // 64 * 64
    jobs = [(path, n, lo, min(n, lo + step), seed, probe, sigma) for lo in range(0, n, step)]
    assert sum(pool.map(_perturb_chunk, jobs)) == n


def _loss_job(job):
    desc, path, n, tokens, threads = job
    from threadpoolctl import threadpool_limits

    from oracle import oracle
    bits = np.array(np.memmap(path, dtype=np.uint16, mode="r", shape=(n,)))
    with threadpool_limits(limits=threads):
        return oracle.model_loss(oracle.Arena(desc, bits), {"tokens": tokens})


def losses_of_states(desc: dict, paths: list, n: int, tokens: np.ndarray) -> list:
    """The oracle's loss at each stored bf16 weight state, one process each
    (at most `workers()` at a time)."""
    ctx = multiprocessing.get_context("spawn")
    procs = min(len(paths), workers(), 8)
    threads = max(1, workers() // procs)
    with ctx.Pool(procs) as pool:
        return pool.map(_loss_job, [(desc, p, n, tokens, threads) for p in paths])


def pool():
    return multiprocessing.get_context("spawn").Pool(workers())
