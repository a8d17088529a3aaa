"""GPU parity of the direction generator, perturbation and update against the
CPU oracle, through the C ABI.

Bars: Philox words bit-exact; |z_gpu - z| <= 1e-6 against the fp64 Box-Muller
definition (exhaustively over both 2^24-value uniform domains); perturbed and
updated weights within 1e-5 absolute (fp32), and for bf16 every mismatch must
be a rounding-boundary case: the oracle's exact pre-rounding value lies within
the z tolerance (times |sigma|) of a bf16 rounding midpoint.
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from zeroth_order_backprop_amd import zo

pytestmark = pytest.mark.gpu

DEV = "cuda"
ZTOL = 1e-6


def _sync():
    torch.cuda.synchronize()


# --------------------------------------------------------------- words / z
@pytest.mark.parametrize("seed,probe,j0,n", [
    (0, 0, 0, 100_000),
    (12345, 7, 4 * 1001, 65_537),
    (2**40 + 3, 31, 2**34 - 4 * 17, 4096),   # counter high word crosses zero -> one
    (2**64 - 1, 1023, 2**36, 999),
])
def test_rng_words_bit_exact_and_z(seed, probe, j0, n):
    words = torch.zeros(n, dtype=torch.int32, device=DEV)
    z = torch.zeros(n, dtype=torch.float32, device=DEV)
    zo.debug_rng(seed, probe, j0, n, words=words, z=z)
    _sync()
    want_w = oracle.rng_words(seed, probe, j0, n)
    got_w = words.cpu().numpy().view(np.uint32)
    assert (got_w == want_w).all()
    want_z = oracle.gauss(seed, probe, j0, n).astype(np.float64)
    got_z = z.cpu().numpy().astype(np.float64)
    assert np.abs(got_z - want_z).max() <= ZTOL


def _bm_gpu(pairs: np.ndarray) -> np.ndarray:
    p = torch.from_numpy(pairs.view(np.int32).copy()).to(DEV)
    out = torch.zeros(pairs.shape, dtype=torch.float32, device=DEV)
    zo.debug_box_muller(p, pairs.shape[0], out)
    _sync()
    return out.cpu().numpy().astype(np.float64)


def test_box_muller_exhaustive_radius():
    """Every one of the 2^24 radius inputs, at angle 0 (z_even = r, z_odd = 0)
    and at angle 1/8 turn (both components r / sqrt 2)."""
    a = np.arange(1 << 24, dtype=np.uint64).astype(np.uint32) << np.uint32(8)
    for b in (0, 1 << 21):
        pairs = np.stack([a, np.full_like(a, b << 8)], axis=1)
        got = _bm_gpu(pairs)
        want = oracle.box_muller_f64_array(pairs)
        err = np.abs(got - want).max()
        assert err <= ZTOL, err


def test_box_muller_exhaustive_angle():
    """Every one of the 2^24 angle inputs at the largest radius (a = 0, r = 5.77),
    at a mid radius, and at the two radius inputs where the hardware log2 errs
    most (a = 225: largest effect on r; a = 64456: largest error in ulps)."""
    b = np.arange(1 << 24, dtype=np.uint64).astype(np.uint32) << np.uint32(8)
    for a in (0, 225, 64456, 1 << 23):
        pairs = np.stack([np.full_like(b, a << 8), b], axis=1)
        got = _bm_gpu(pairs)
        want = oracle.box_muller_f64_array(pairs)
        err = np.abs(got - want).max()
        assert err <= ZTOL, err


def test_box_muller_random_pairs_and_special_cases():
    rng = np.random.default_rng(0)
    pairs = rng.integers(0, 2**32, size=(1 << 22, 2), dtype=np.uint64).astype(np.uint32)
    got = _bm_gpu(pairs)
    want = oracle.box_muller_f64_array(pairs)
    assert np.abs(got - want).max() <= ZTOL
    special = np.array([[(2**24 - 1) << 8, 12345 << 8], [0, 0], [0, (2**22) << 8], [0, (2**23) << 8]],
                       np.uint32)
    g = _bm_gpu(special)
    assert g[0, 0] == 0.0 and g[0, 1] == 0.0           # radius 0
    assert g[1, 1] == 0.0                               # angle 0: sin exactly 0
    assert g[2, 0] == 0.0 and g[3, 1] == 0.0            # quarter / half turn axes


# --------------------------------------------------------------- perturb
def _ulp_bf16(x):
    a = np.maximum(np.abs(x), 2.0**-126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _bf16_boundary_ok(w0, sigma, z, got, want):
    """Elements where GPU and oracle bf16 results differ must be rounding
    boundary cases: the exact w0 + sigma z lies within |sigma| * ZTOL (+ one
    fp32 rounding) of the midpoint between the two results."""
    bad = got != want
    if not bad.any():
        return True
    exact = w0[bad] + np.float64(np.float32(sigma)) * z[bad]
    mid = 0.5 * (got[bad] + want[bad])
    slack = abs(float(np.float32(sigma))) * ZTOL + np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64)
    adjacent = np.abs(got[bad] - want[bad]) <= _ulp_bf16(np.maximum(np.abs(got[bad]), np.abs(want[bad]))) * 1.0001
    return bool((np.abs(exact - mid) <= slack).all() and adjacent.all())


@pytest.mark.parametrize("n,j0", [(1 << 20, 0), ((1 << 16) + 1237, 4 * 333), (2047, 8), (5, 0)])
def test_perturb_f32_parity(n, j0):
    rng = np.random.default_rng(n)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    wd = torch.from_numpy(w.copy()).to(DEV)
    L = oracle.lib()

    def both(seed, probe, sigma):
        zo.perturb_buffer(wd, n, j0, seed, probe, sigma, zo.ZO_F32)
        L.oracle_perturb_f32(oracle._ptr(w), n, j0, seed, probe, float(np.float32(sigma)))

    w0 = w.astype(np.float64)
    both(3, 0, 1e-3)
    _sync()
    got = wd.cpu().numpy().astype(np.float64)
    # sigma * (z difference <= 1e-6) can only move elements whose exact value
    # sits next to an fp32 rounding midpoint, and then by one ulp
    z = oracle.gauss(3, 0, j0, n).astype(np.float64)
    bad = got != w
    exact = w0[bad] + float(np.float32(1e-3)) * z[bad]
    mid = 0.5 * (got[bad] + w[bad])
    assert (np.abs(exact - mid) <= 1e-3 * ZTOL * 1.01).all()
    big = np.maximum(np.abs(got[bad]), np.abs(w[bad])).astype(np.float32)
    assert (np.abs(got - w)[bad] <= np.spacing(big) + 1e-3 * ZTOL).all()
    both(3, 5, -2e-3)
    _sync()
    got = wd.cpu().numpy().astype(np.float64)
    big = np.maximum(np.abs(got), np.abs(w)).astype(np.float32)
    assert (np.abs(got - w) <= 2 * np.spacing(big) + 3e-3 * ZTOL).all()
    both(99, 2, 0.5)  # large sigma: every element may round differently, bound only
    _sync()
    got = wd.cpu().numpy().astype(np.float64)
    ulp = np.spacing(np.abs(w)).astype(np.float64)
    assert (np.abs(got - w) <= 3 * ulp + 0.504 * ZTOL).all()
    assert np.abs(got - w).max() <= 1e-5


@pytest.mark.parametrize("n,j0", [(1 << 20, 0), ((1 << 16) + 1237, 4 * 333), (7, 4)])
def test_perturb_bf16_parity(n, j0):
    from zeroth_order_backprop_amd import inputs
    rng = np.random.default_rng(n + 1)
    w = inputs.f32_to_bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
    wd = torch.from_numpy(w.view(np.int16).copy()).to(DEV)
    sigma = 1e-3
    w0 = oracle.bf16_bits_to_f64(w)
    zo.perturb_buffer(wd, n, j0, 17, 3, sigma, zo.ZO_BF16)
    want_bits = w.copy()
    oracle.lib().oracle_perturb_bf16(oracle._ptr(want_bits), n, j0, 17, 3, float(np.float32(sigma)))
    _sync()
    got = oracle.bf16_bits_to_f64(wd.cpu().numpy().view(np.uint16))
    want = oracle.bf16_bits_to_f64(want_bits)
    z = oracle.gauss(17, 3, j0, n).astype(np.float64)
    assert _bf16_boundary_ok(w0, sigma, z, got, want)
    assert np.mean(got == want) > 0.999


@pytest.mark.parametrize("dtype", [zo.ZO_F32, zo.ZO_BF16])
def test_restore_sequence_on_gpu(dtype):
    from zeroth_order_backprop_amd import inputs
    n = 1 << 20
    w32 = (np.random.default_rng(5).standard_normal(n) * 0.02).astype(np.float32)
    if dtype == zo.ZO_BF16:
        host = inputs.f32_to_bf16_bits(w32)
        wd = torch.from_numpy(host.view(np.int16).copy()).to(DEV)
        vals = lambda t: oracle.bf16_bits_to_f64(t.cpu().numpy().view(np.uint16))
        ulp = _ulp_bf16
    else:
        wd = torch.from_numpy(w32.copy()).to(DEV)
        vals = lambda t: t.cpu().numpy().astype(np.float64)
        ulp = lambda x: np.spacing(np.abs(x).astype(np.float32)).astype(np.float64)
    w0 = vals(wd)
    zo.perturb_buffer(wd, n, 0, 8, 1, 1e-3, dtype)
    wp = vals(wd)
    zo.perturb_buffer(wd, n, 0, 8, 1, -2e-3, dtype)
    wm = vals(wd)
    zo.perturb_buffer(wd, n, 0, 8, 1, 1e-3, dtype)
    wr = vals(wd)
    mx = np.maximum(np.maximum(np.abs(w0), np.abs(wp)), np.abs(wm))
    assert (np.abs(wr - w0) <= 1.5 * ulp(mx)).all()


# ---------------------------------------------------------------- update
@pytest.mark.parametrize("n,j0,N", [(1 << 20, 0, 4), ((1 << 15) + 999, 4 * 21, 16), (3, 0, 1)])
def test_update_f32_parity(n, j0, N):
    rng = np.random.default_rng(N)
    w = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = rng.standard_normal(N) * 20.0
    lr = np.float32(1e-2)
    wd = torch.from_numpy(w.copy()).to(DEV)
    gd = torch.from_numpy(g).to(DEV)
    zo.update_buffer(wd, n, j0, 41, N, gd, lr, zo.ZO_F32)
    c = -float(lr) * g / N
    oracle.lib().oracle_update_f32(oracle._ptr(w), n, j0, 41, N, oracle._ptr(np.ascontiguousarray(c)))
    _sync()
    got = wd.cpu().numpy().astype(np.float64)
    assert np.abs(got - w).max() <= 1e-5
    step = np.abs(c).sum() * 6.0
    assert (np.abs(got - w) <= np.spacing(np.abs(w)) * 1.5 + step * (2 * ZTOL + N * 2**-23)).all()


@pytest.mark.parametrize("n,N", [(1 << 20, 1), ((1 << 15) + 999, 8)])
def test_update_bf16_parity(n, N):
    from zeroth_order_backprop_amd import inputs
    rng = np.random.default_rng(N + 7)
    w = inputs.f32_to_bf16_bits((rng.standard_normal(n) * 0.02).astype(np.float32))
    g = rng.standard_normal(N) * 20.0
    lr = np.float32(1e-3)
    wd = torch.from_numpy(w.view(np.int16).copy()).to(DEV)
    gd = torch.from_numpy(g).to(DEV)
    zo.update_buffer(wd, n, 0, 42, N, gd, lr, zo.ZO_BF16)
    c = -float(lr) * g / N
    want_bits = w.copy()
    oracle.lib().oracle_update_bf16(oracle._ptr(want_bits), n, 0, 42, N, oracle._ptr(np.ascontiguousarray(c)))
    _sync()
    got = oracle.bf16_bits_to_f64(wd.cpu().numpy().view(np.uint16))
    want = oracle.bf16_bits_to_f64(want_bits)
    bad = got != want
    assert np.mean(bad) < 1e-3
    # one bf16 ulp (a rounding flip) plus the z tolerance carried by sum |c_i|
    slack = np.abs(c).sum() * (ZTOL + 6.0 * N * 2.0**-24)
    assert (np.abs(got - want)[bad] <= _ulp_bf16(np.maximum(np.abs(got), np.abs(want)))[bad] * 1.0001 + slack).all()


def test_update_skips_nonfinite_g():
    n = 4096
    w = torch.randn(n, device=DEV)
    before = w.clone()
    g = torch.tensor([1.0, float("nan"), 2.0], dtype=torch.float64, device=DEV)
    zo.update_buffer(w, n, 0, 1, 3, g, 1e-2, zo.ZO_F32)
    _sync()
    assert torch.equal(w, before)


def test_gscalar():
    L = torch.tensor([3.0, 1.0, 0.5, 0.75], dtype=torch.float64, device=DEV)
    g = torch.zeros(2, dtype=torch.float64, device=DEV)
    zo.gscalar(L, 2, 1e-3, g)
    _sync()
    sig = float(np.float32(1e-3))
    assert g.cpu().tolist() == [(3.0 - 1.0) / (2 * sig), (0.5 - 0.75) / (2 * sig)]


def test_determinism_bitwise():
    n = (1 << 18) + 100
    a = torch.randn(n, device=DEV)
    b = a.clone()
    g = torch.randn(5, dtype=torch.float64, device=DEV)
    for t in (a, b):
        zo.perturb_buffer(t, n, 0, 9, 2, 1e-3, zo.ZO_F32)
        zo.update_buffer(t, n, 0, 9, 5, g, 1e-2, zo.ZO_F32)
    _sync()
    assert torch.equal(a, b)
