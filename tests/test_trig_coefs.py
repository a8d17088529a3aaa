"""Host check of the generator's quarter-turn polynomial coefficients.

The direction generator evaluates K sin(pi t / 2) and K cos(pi t / 2),
K = sqrt(2 ln 2), on the reduced angle t = i 2^-22 in [-1/2, 1/2] with fp32
Horner polynomials (Box-Muller, with the radius taken in base-2 logarithms).
This reads the coefficients from the device header and evaluates them in
emulated fp32 (one rounding per fma) over every reduced angle, against the
exact functions.  A dropped or mistyped coefficient fails it by orders of
magnitude; the GPU sweeps over all 2^24 angles check the kernel itself.
"""
import pathlib
import re

import numpy as np

HDR = pathlib.Path(__file__).resolve().parents[1] / "zeroth_order_backprop_amd" / "csrc" / "zo_rng.hpp"
K = np.sqrt(2.0 * np.log(2.0))


def _coefs():
    text = HDR.read_text()
    vals = {}
    for name, lit in re.findall(r"constexpr float (k[SC]\d+) = ([-0-9a-fx.p+]+)f;", text):
        vals[name] = np.float32(float.fromhex(lit))
    return [vals[f"kS{k}"] for k in (1, 3, 5, 7)], [vals[f"kC{k}"] for k in (0, 2, 4, 6, 8)]


def _horner(cs, t2):
    p = np.full_like(t2, np.float64(cs[-1]))
    for c in cs[-2::-1]:
        p = (p * t2 + np.float64(c)).astype(np.float32).astype(np.float64)
    return p


def test_quarter_turn_polynomials_fp32():
    s, c = _coefs()
    t = np.arange(-(1 << 21), (1 << 21) + 1, dtype=np.float64) * 2.0 ** -22
    t32 = t.astype(np.float32)
    t2 = (t32 * t32).astype(np.float32).astype(np.float64)
    st = (_horner(s, t2).astype(np.float32) * t32).astype(np.float64)
    ct = _horner(c, t2)
    assert np.abs(st - K * np.sin(np.pi * t / 2)).max() <= 6.5e-8
    assert np.abs(ct - K * np.cos(np.pi * t / 2)).max() <= 7.7e-8
    assert st[t == 0] == 0.0                       # the axes stay exact
    assert c[0] == np.float32(K)                   # constant term: the fp32 value nearest K


def test_quarter_turn_polynomials_full_turn():
    """Both components at the quadrant edges t = +-1/2 agree with the
    neighbouring quadrant's polynomials (continuity of the rotation)."""
    s, c = _coefs()
    t2 = (np.float32(0.5) * np.float32(0.5)).astype(np.float64) * np.ones(1)
    sin_h = float(_horner(s, t2)[0] * 0.5)
    cos_h = float(_horner(c, t2)[0])
    assert abs(sin_h - cos_h) <= 1.2e-7            # sin(pi/4) = cos(pi/4)
    assert abs(sin_h - K * np.sqrt(0.5)) <= 1e-7
