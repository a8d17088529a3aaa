"""Pins of the oracle's direction generator, Gaussian map and bf16 rounding
against things other than itself: published known-answer vectors, an
independent Philox implementation (rocRAND, used as a black box), closed-form
special cases, sampling statistics and an exhaustive library comparison."""
import ctypes
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch
from scipy import stats

from oracle import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _kat_lines():
    rows = []
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(x, 16) for x in line.split()])
    return rows


@pytest.fixture(scope="module")
def rocrand_ref():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND reference")
    d = tempfile.mkdtemp()
    so = os.path.join(d, "librr.so")
    subprocess.check_call([hipcc, "-O1", "-fPIC", "-shared", "-o", so,
                           os.path.join(HERE, "helpers", "rocrand_philox_ref.cpp")],
                          cwd=d, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    lib = ctypes.CDLL(so)
    lib.rocrand_ref_philox.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_uint64, ctypes.c_void_p]

    def run(ctr, key):
        ctr = np.ascontiguousarray(ctr, np.uint32)
        key = np.ascontiguousarray(key, np.uint32)
        n = ctr.shape[0]
        out = np.zeros((n, 4), np.uint32)
        lib.rocrand_ref_philox(ctr.ctypes.data, key.ctypes.data, n, out.ctypes.data)
        return out
    return run


def test_philox_known_answers():
    for row in _kat_lines():
        ctr, key, want = row[0:4], row[4:6], row[6:10]
        assert list(oracle.philox4x32_10(ctr, key)) == want


def test_philox_known_answers_rocrand(rocrand_ref):
    rows = np.array(_kat_lines(), dtype=np.uint64).astype(np.uint32)
    got = rocrand_ref(rows[:, 0:4], rows[:, 4:6])
    assert (got == rows[:, 6:10]).all()


def test_philox_matches_rocrand_random_inputs(rocrand_ref):
    rng = np.random.default_rng(123)
    n = 4000
    ctr = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    key = rng.integers(0, 2**32, size=(n, 2), dtype=np.uint64).astype(np.uint32)
    ref = rocrand_ref(ctr, key)
    mine = np.stack([oracle.philox4x32_10(ctr[t], key[t]) for t in range(n)])
    assert (ref == mine).all()


def test_stream_layout_against_rocrand(rocrand_ref):
    """Element j of probe i under seed s is word j%4 of Philox(ctr=(q lo, q hi,
    i, 0), key=(s lo, s hi)), q = j//4 -- including q beyond 2^32."""
    for seed, probe, j0 in [(0, 0, 0), (7, 3, 1022), (2**40 + 5, 31, (2**34) - 6), (2**64 - 1, 2, 12345)]:
        n = 24
        words = oracle.rng_words(seed, probe, j0, n)
        js = np.arange(j0, j0 + n, dtype=np.uint64)
        q = js >> np.uint64(2)
        ctr = np.stack([(q & np.uint64(0xFFFFFFFF)).astype(np.uint32), (q >> np.uint64(32)).astype(np.uint32),
                        np.full(n, probe, np.uint32), np.zeros(n, np.uint32)], axis=1)
        key = np.tile(np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint64).astype(np.uint32), (n, 1))
        ref = rocrand_ref(ctr, key)
        want = ref[np.arange(n), (js & np.uint64(3)).astype(np.int64)]
        assert (words == want).all()


def test_philox_no_repeats_and_bit_balance():
    # bijection spot check + per-bit balance on 2^16 consecutive counters
    w = oracle.rng_words(99, 0, 0, 4 * 65536).reshape(-1, 4)
    as_tuples = {tuple(r) for r in w.tolist()}
    assert len(as_tuples) == w.shape[0]
    bits = np.unpackbits(w.view(np.uint8)).reshape(-1)
    ones = bits.sum()
    n = bits.size
    assert abs(ones - n / 2) < 5 * np.sqrt(n / 4)


# ------------------------------------------------------------- Box-Muller map
def test_box_muller_special_cases():
    # a = 2^24-1 -> u_r = 1 -> radius 0 exactly
    ze, zo = oracle.box_muller_f64((2**24 - 1) << 8, 12345 << 8)
    assert ze == 0.0 and zo == 0.0
    rmax = np.sqrt(-2.0 * np.log(2.0**-24))
    # a = 0 gives the largest radius; b = 0, 2^22, 2^23, 3*2^22 are the axes
    ze, zo = oracle.box_muller_f64(0, 0)
    assert ze == rmax and zo == 0.0
    ze, zo = oracle.box_muller_f64(0, (2**22) << 8)
    assert abs(ze) < 1e-14 and zo == pytest.approx(rmax, abs=1e-14)
    ze, zo = oracle.box_muller_f64(0, (2**23) << 8)
    assert ze == pytest.approx(-rmax, abs=1e-14) and abs(zo) < 1e-14
    ze, zo = oracle.box_muller_f64(0, (3 * 2**22) << 8)
    assert abs(ze) < 1e-14 and zo == pytest.approx(-rmax, abs=1e-14)
    # the low 8 bits of each word are ignored
    assert oracle.box_muller_f64(0x123456FF, 0xABCDEF01) == oracle.box_muller_f64(0x12345600, 0xABCDEF00)


def test_box_muller_radius_closed_form():
    # u_r = 1/2 (a = 2^23 - 1) -> r = sqrt(2 ln 2); angle 1/8 turn -> z = r/sqrt(2) each
    ze, zo = oracle.box_muller_f64((2**23 - 1) << 8, (2**21) << 8)
    r = np.sqrt(2.0 * np.log(2.0))
    assert ze == pytest.approx(r / np.sqrt(2.0), rel=1e-15)
    assert zo == pytest.approx(r / np.sqrt(2.0), rel=1e-15)


def test_gaussian_moments_and_ks():
    z = oracle.gauss(seed=2024, probe=0, j0=0, n=2_000_000).astype(np.float64)
    n = z.size
    assert abs(z.mean()) < 5 / np.sqrt(n)
    assert abs(z.var() - 1.0) < 5 * np.sqrt(2.0 / n)
    kurt = stats.kurtosis(z, fisher=False)
    assert abs(kurt - 3.0) < 5 * np.sqrt(24.0 / n)
    assert stats.kstest(z, "norm").pvalue > 1e-4
    assert np.abs(z).max() <= np.sqrt(-2.0 * np.log(2.0**-24)) + 1e-6


def test_directions_independent_across_probes_and_seeds():
    n = 1_000_000
    a = oracle.gauss(5, 0, 0, n).astype(np.float64)
    b = oracle.gauss(5, 1, 0, n).astype(np.float64)
    c = oracle.gauss(6, 0, 0, n).astype(np.float64)
    for x, y in ((a, b), (a, c)):
        r = np.corrcoef(x, y)[0, 1]
        assert abs(r) < 5 / np.sqrt(n)
    # even/odd members of one Box-Muller pair are uncorrelated too
    assert abs(np.corrcoef(a[0::2], a[1::2])[0, 1]) < 5 / np.sqrt(n / 2)


def test_gauss_at_matches_range():
    idx = np.array([0, 1, 2, 3, 4, 1001, 2**33 + 7], np.uint64)
    z = oracle.gauss_at(3, 4, idx)
    for t, j in enumerate(idx.tolist()):
        assert z[t] == oracle.gauss(3, 4, j, 1)[0]


# -------------------------------------------------------------------- bf16
@pytest.mark.slow
def test_bf16_rne_exhaustive_vs_torch():
    """All 2^32 fp32 bit patterns against torch's fp32 -> bfloat16 conversion."""
    L = oracle.lib()
    chunk = 1 << 24
    bad = 0
    for k in range(1 << 8):
        u = np.arange(k * chunk, (k + 1) * chunk, dtype=np.uint64).astype(np.uint32)
        f = torch.from_numpy(u.view(np.float32))
        expect = f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        expect = np.ascontiguousarray(expect)
        bad += L.oracle_bf16_compare_range(k * chunk, chunk, expect.ctypes.data)
    assert bad == 0


def _bf16_neighbours(x):
    """The two bf16 values bracketing x > 0, by walking bit patterns."""
    f = np.float32(x)
    h = (np.array([f], np.float32).view(np.uint32)[0] >> 16).astype(np.uint32)
    cand = []
    for hh in (h - 1, h, h + 1, h + 2):
        v = np.array([hh << 16], np.uint32).view(np.float32)[0]
        cand.append((float(v), int(hh)))
    lo = max((c for c in cand if c[0] <= x), key=lambda c: c[0])
    hi = min((c for c in cand if c[0] >= x), key=lambda c: c[0])
    return lo, hi


def test_bf16_from_f64_nearest_ties_even():
    rng = np.random.default_rng(7)
    xs = list(rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000))
    # exact ties and near-ties at several magnitudes
    for e in (-20, -3, 0, 5, 40):
        base = 2.0**e
        step = base * 2.0**-7
        for m in range(0, 128, 9):
            xs += [base + (m + 0.5) * step, base + (m + 0.5) * step * (1 + 2**-40),
                   base + (m + 0.5) * step * (1 - 2**-40)]
    for x in xs:
        if x == 0:
            continue
        got = oracle.bf16_round(np.array([abs(x)]))[0]
        (lo, hlo), (hi, hhi) = _bf16_neighbours(abs(x))
        dlo, dhi = abs(x) - lo, hi - abs(x)
        if dlo < dhi:
            want = lo
        elif dhi < dlo:
            want = hi
        else:
            want = lo if hlo % 2 == 0 else hi
        assert got == want, (x, got, want)
        assert oracle.bf16_round(np.array([-abs(x)]))[0] == -want


def test_bf16_from_f64_subnormal_and_overflow():
    tiny = 2.0**-133
    assert oracle.bf16_round(np.array([tiny]))[0] == tiny
    assert oracle.bf16_round(np.array([tiny * 0.5]))[0] == 0.0          # tie -> even (0)
    assert oracle.bf16_round(np.array([tiny * 0.75]))[0] == tiny
    assert oracle.bf16_round(np.array([tiny * 1.5]))[0] == 2 * tiny     # tie -> even
    big = 3.3895313892515355e38
    assert oracle.bf16_round(np.array([big]))[0] == big
    assert np.isinf(oracle.bf16_round(np.array([2.0**128]))[0])
