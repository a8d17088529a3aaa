"""Pins of the oracle's update rounding and of its sampled-index routines.

The update w <- D(w + sum_i c_i z_i) (ZOO blog "Backprop 없이 Transformer를
학습시킨다", section "backprop의 메모리 세금", the loop's last box: W <- W - eta
g_hat with g_hat = (1/N) sum_i g_i z_i) is read as one rounding of the exact
value to the storage type.  These tests check the oracle against that exact
value, computed here with rational arithmetic and a neighbour search, on
random elements, on exact ties (which must go to the even neighbour) and on
values a hair off a tie (where rounding first to fp32 and then to bf16 would
pick the wrong side).

The "_at" routines (the same passes at scattered element indices, the
checkers of every full-size GPU test) are compared bit for bit with the range
routines at the same indices, counters past 2^32 included.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle


def _f32_bits(x: float) -> int:
    return int(np.array([x], np.float32).view(np.uint32)[0])


def _bf16_value(bits: int) -> Fraction:
    return Fraction(float(np.array([bits << 16], np.uint32).view(np.float32)[0]))


def _nearest_even_bf16(v: Fraction) -> int:
    """bf16 bit pattern nearest to the exact value v, ties to the even
    pattern, by searching the patterns around v's truncation (finite, normal
    results only)."""
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    t = _f32_bits(float(a)) >> 16  # within a couple of patterns of the answer
    best = None
    for b in range(max(t - 3, 0), t + 4):
        d = abs(_bf16_value(b) - a)
        if best is None or d < best[0] or (d == best[0] and b % 2 == 0):
            best = (d, b)
    return best[1] | sign


def _nearest_even_f32(v: Fraction) -> int:
    sign = 0x80000000 if v < 0 else 0
    a = abs(v)
    t = _f32_bits(float(a))
    best = None
    for b in range(t - 2, t + 3):
        d = abs(Fraction(float(np.array([b], np.uint32).view(np.float32)[0])) - a)
        if best is None or d < best[0] or (d == best[0] and b % 2 == 0):
            best = (d, b)
    return best[1] | sign


def _update_one_bf16(wbits: int, j: int, seed: int, c) -> int:
    w = np.array([wbits], np.uint16)
    cc = np.ascontiguousarray(c, np.float64)
    oracle.lib().oracle_update_bf16(oracle._ptr(w), 1, j, seed, cc.size, oracle._ptr(cc))
    return int(w[0])


def test_update_bf16_is_nearest_even_of_exact_sum():
    rng = np.random.default_rng(21)
    n, N, seed, j0 = 3000, 4, 77, 1_000_003
    w = oracle.bf16_round(rng.standard_normal(n) * 0.05)
    bits = (w.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    c = rng.standard_normal(N) * 1e-3
    got = bits.copy()
    oracle.lib().oracle_update_bf16(oracle._ptr(got), n, j0, seed, N, oracle._ptr(np.ascontiguousarray(c)))
    Z = [oracle.gauss(seed, i, j0, n) for i in range(N)]
    cf = [Fraction(float(x)) for x in c]
    for t in range(n):
        exact = Fraction(float(w[t])) + sum(cf[i] * Fraction(float(Z[i][t])) for i in range(N))
        assert int(got[t]) == _nearest_even_bf16(exact), t


def test_update_f32_is_nearest_even_of_exact_sum():
    rng = np.random.default_rng(22)
    n, N, seed, j0 = 2000, 3, 5, 4096
    w = (rng.standard_normal(n) * 0.05).astype(np.float32)
    c = rng.standard_normal(N) * 1e-4
    got = w.copy()
    oracle.lib().oracle_update_f32(oracle._ptr(got), n, j0, seed, N, oracle._ptr(np.ascontiguousarray(c)))
    Z = [oracle.gauss(seed, i, j0, n) for i in range(N)]
    cf = [Fraction(float(x)) for x in c]
    for t in range(n):
        exact = Fraction(float(w[t])) + sum(cf[i] * Fraction(float(Z[i][t])) for i in range(N))
        assert _f32_bits(float(got[t])) == _nearest_even_f32(exact), t


def _short_directions(seed: int, probe: int, n: int, max_bits: int = 6):
    """Elements j whose direction value has at most `max_bits` significant
    bits and 1/4 <= |z| < 4: z = m 2^p with m odd, m < 2^max_bits."""
    z = oracle.gauss(seed, probe, 0, n)
    u = z.view(np.uint32)
    mag = np.abs(z)
    ok = ((u & ((1 << (24 - max_bits)) - 1)) == 0) & (mag >= 0.25) & (mag < 4.0)
    return [(int(j), float(z[j])) for j in np.nonzero(ok)[0]]


@pytest.fixture(scope="module")
def short_dirs():
    found = []
    for probe in range(3):
        found += [(probe, j, z) for j, z in _short_directions(9, probe, 1 << 22)]
    assert len(found) >= 8, len(found)
    return found


def _odd_part(z: float):
    """z = m 2^p with m an odd integer: returns (m, p)."""
    f = Fraction(z)
    p = 0
    while f.denominator != 1:
        f *= 2
        p -= 1
    m = f.numerator
    while m % 2 == 0:
        m //= 2
        p += 1
    return m, p


@pytest.mark.parametrize("w0", [1.5, -0.75, 3.0, 0.0234375, -40.0])
def test_update_bf16_exact_ties_go_to_even(short_dirs, w0):
    """c z = m u / 2 exactly (u = the bf16 spacing at w, m odd): w + c z lies
    exactly half way between two bf16 values, and the update must return the
    one with the even pattern."""
    wbits = _f32_bits(w0) >> 16
    assert float(_bf16_value(wbits)) == w0
    u = Fraction(2) ** (int(np.floor(np.log2(abs(w0)))) - 7)
    ties = 0
    for probe, j, z in short_dirs:
        m, p = _odd_part(z)
        if abs(m) * u / 2 >= abs(Fraction(w0)) / 4:
            continue  # keep w + c z in w's binade
        cpow = u / 2 / Fraction(2) ** p  # a power of two: c z = m u / 2 exactly
        c = np.zeros(probe + 1)
        c[probe] = float(cpow)
        assert Fraction(c[probe]) == cpow
        exact = Fraction(w0) + Fraction(c[probe]) * Fraction(z)
        lo = (exact // u) * u
        assert exact - lo == u / 2  # exactly a tie
        want = _nearest_even_bf16(exact)
        assert want % 2 == 0
        assert _update_one_bf16(wbits, j, 9, c) == want
        ties += 1
    assert ties >= 4


@pytest.mark.parametrize("w0", [1.5, -0.75, 3.0])
def test_update_bf16_rounds_once_near_ties(short_dirs, w0):
    """Two probes: the first puts w + c z exactly on a tie, the second adds a
    term about 2^-30 u of either sign.  The exact sum is then just off the
    tie and must round towards it; rounding first to fp32 (whose spacing is
    2^-16 u) would land on the tie and take the even side instead."""
    wbits = _f32_bits(w0) >> 16
    u = Fraction(2) ** (int(np.floor(np.log2(abs(w0)))) - 7)
    checked = 0
    for probe, j, z in short_dirs:
        if probe != 0:
            continue
        m, p = _odd_part(z)
        if abs(m) * u / 2 >= abs(Fraction(w0)) / 4:
            continue
        z1 = float(oracle.gauss(9, 1, j, 1)[0])
        if z1 == 0.0:
            continue
        for sgn in (1, -1):
            c = np.array([float(u / 2 / Fraction(2) ** p), sgn * float(u) * 2.0**-30 / z1])
            exact = Fraction(w0) + Fraction(c[0]) * Fraction(z) + Fraction(c[1]) * Fraction(z1)
            want = _nearest_even_bf16(exact)
            assert abs(float(exact - (exact // u) * u - u / 2)) > 0  # not a tie
            assert _update_one_bf16(wbits, j, 9, c) == want
            # the two neighbours of the tie differ, so this checks the side
            checked += 1
    assert checked >= 2


# ------------------------------------------------ sampled-index routines
def _ranges():
    # element ranges at the start, unaligned, and with q = j / 4 (j / 16 for
    # 8-bit directions) beyond 2^32
    return [(0, 40), (1001, 37), (2**34 - 12, 40), (2**36 + 3, 33), (2**40 + 16, 48)]


@pytest.mark.parametrize("dirs", ["gauss", "q8"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_at_routines_equal_range_routines(dirs, dtype):
    L = oracle.lib()
    q8 = oracle._q8()
    pre = "oracle_q8_" if dirs == "q8" else "oracle_"
    tail = (oracle._ptr(q8),) if dirs == "q8" else ()
    rng = np.random.default_rng(5)
    seed, probe, sigma = 2**33 + 7, 3, float(np.float32(-2e-3))
    c = np.ascontiguousarray(rng.standard_normal(5) * 1e-3)
    for j0, n in _ranges():
        if dtype == "f32":
            w = (rng.standard_normal(n) * 0.05).astype(np.float32)
        else:
            w = (oracle.bf16_round(rng.standard_normal(n) * 0.05).astype(np.float32).view(np.uint32) >> 16
                 ).astype(np.uint16)
        idx = np.ascontiguousarray(np.arange(j0, j0 + n, dtype=np.uint64))
        # perturb
        a, b = w.copy(), w.copy()
        getattr(L, pre + "perturb_" + dtype)(oracle._ptr(a), n, j0, seed, probe, sigma, *tail)
        getattr(L, pre + "perturb_" + dtype + "_at")(oracle._ptr(b), oracle._ptr(idx), n, seed, probe, sigma, *tail)
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (j0, "perturb")
        # update with 5 probes
        a, b = w.copy(), w.copy()
        getattr(L, pre + "update_" + dtype)(oracle._ptr(a), n, j0, seed, c.size, oracle._ptr(c), *tail)
        getattr(L, pre + "update_" + dtype + "_at")(oracle._ptr(b), oracle._ptr(idx), n, seed, c.size,
                                                    oracle._ptr(c), *tail)
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (j0, "update")
        # scattered indices, each against the range routine on that one element
        sc = np.ascontiguousarray(np.sort(rng.choice(np.arange(j0, j0 + 10 * n, dtype=np.uint64), n, replace=False)))
        b = w.copy()
        getattr(L, pre + "update_" + dtype + "_at")(oracle._ptr(b), oracle._ptr(sc), n, seed, c.size,
                                                    oracle._ptr(c), *tail)
        for t in range(n):
            one = w[t:t + 1].copy()
            getattr(L, pre + "update_" + dtype)(oracle._ptr(one), 1, int(sc[t]), seed, c.size, oracle._ptr(c), *tail)
            assert one.view(np.uint8).tobytes() == b[t:t + 1].view(np.uint8).tobytes(), (j0, t)


@pytest.mark.parametrize("dirs", ["gauss", "q8"])
def test_value_at_equals_range(dirs):
    for j0, n in _ranges():
        idx = np.arange(j0, j0 + n, dtype=np.uint64)
        if dirs == "gauss":
            a = oracle.gauss(2**63 + 1, 7, j0, n)
            b = oracle.gauss_at(2**63 + 1, 7, idx)
        else:
            a = oracle.directions("q8", 2**63 + 1, 7, j0, n)
            b = np.zeros(n, np.float32)
            oracle.lib().oracle_q8_values_at(2**63 + 1, 7, oracle._ptr(np.ascontiguousarray(idx)), n,
                                             oracle._ptr(b), oracle._ptr(oracle._q8()))
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("sigma", [1e-3, -2e-3, 0.37])
def test_perturb_is_nearest_even_of_exact_value(sigma):
    """w <- D(w + sigma z) rounded once from the exact value (fp32: the fma;
    bf16: nearest even of the exact sum), sigma taken at fp32 precision."""
    rng = np.random.default_rng(31)
    n, seed, probe, j0 = 3000, 12, 5, 2**35 + 8
    s32 = float(np.float32(sigma))
    z = oracle.gauss(seed, probe, j0, n)
    w = oracle.bf16_round(rng.standard_normal(n) * 0.05)
    bits = (w.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    got = bits.copy()
    oracle.lib().oracle_perturb_bf16(oracle._ptr(got), n, j0, seed, probe, s32)
    w32 = (rng.standard_normal(n) * 0.05).astype(np.float32)
    got32 = w32.copy()
    oracle.lib().oracle_perturb_f32(oracle._ptr(got32), n, j0, seed, probe, s32)
    sf = Fraction(s32)
    for t in range(n):
        zt = Fraction(float(z[t]))
        assert int(got[t]) == _nearest_even_bf16(Fraction(float(w[t])) + sf * zt), t
        assert _f32_bits(float(got32[t])) == _nearest_even_f32(Fraction(float(w32[t])) + sf * zt), t
