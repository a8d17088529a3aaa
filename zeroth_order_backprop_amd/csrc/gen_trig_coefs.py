"""Derive the quarter-turn sin/cos polynomial coefficients used by zo_rng.hpp.

The Box-Muller transform (Box and Muller, 1958) needs cos and sin of 2 pi u_t.
After the exact quadrant reduction, t is in [-1/2, 1/2] and the generator
evaluates

    K sin(pi t / 2) ~ t * (s1 + s3 t^2 + s5 t^4 + s7 t^6)
    K cos(pi t / 2) ~ c0 + c2 t^2 + c4 t^4 + c6 t^6 + c8 t^8,   K = sqrt(2 ln 2),

so the radius factor sqrt(-2 ln u) = K sqrt(-log2 u) only needs sqrt(-log2 u).
The coefficients are fitted by the Remez exchange for the smallest maximum
absolute error on [0, 1/2] (f64), rounded to fp32, then every coefficient but
c0 is moved by up to two fp32 steps to minimise the error of the fp32 Horner
evaluation over every reduced angle the generator can see (t = i 2^-22).
c0 is the fp32 value nearest K.  Run: python gen_trig_coefs.py  (about 90 s).
"""
import itertools

import numpy as np

K = np.sqrt(2.0 * np.log(2.0))
f32, f64 = np.float32, np.float64


def remez_even(f, weight, deg, lo, hi, iters=40):
    """Coefficients of p(x^2) of degree `deg` in x^2 minimising max |weight (f - p)|."""
    x = np.linspace(lo, hi, 200001)
    n = deg + 2
    ref = (lo + hi) / 2 + (hi - lo) / 2 * np.cos(np.pi * np.arange(n)[::-1] / (n - 1))
    c = None
    for _ in range(iters):
        a = np.array([[weight(xi) * xi ** (2 * k) for k in range(deg + 1)] + [(-1) ** i]
                      for i, xi in enumerate(ref)])
        c = np.linalg.solve(a, np.array([weight(xi) * f(xi) for xi in ref]))[:deg + 1]
        e = weight(x) * (f(x) - sum(c[k] * x ** (2 * k) for k in range(deg + 1)))
        sgn = np.sign(e)
        idx, start = [], 0
        for j in range(1, len(x) + 1):
            if j == len(x) or sgn[j] != sgn[start]:
                seg = np.arange(start, j)
                idx.append(seg[np.argmax(np.abs(e[seg]))])
                start = j
        while len(idx) > n:
            idx = idx[1:] if abs(e[idx[0]]) < abs(e[idx[-1]]) else idx[:-1]
        if len(idx) < n:
            break
        ref = x[np.array(idx)]
    return c


T = np.arange(0, (1 << 21) + 1, dtype=np.float64) * 2.0 ** -22
T32 = T.astype(f32)
T2 = (T32 * T32).astype(f32).astype(f64)


def horner(cs):
    p = np.full_like(T2, f64(cs[-1]))
    for c in cs[-2::-1]:
        p = (p * T2 + f64(c)).astype(f32).astype(f64)     # one fp32 rounding per fma
    return p


def err_sin(cs):
    return np.abs((horner(cs).astype(f32) * T32).astype(f64) - K * np.sin(np.pi * T / 2)).max()


def err_cos(cs):
    return np.abs(horner(cs) - K * np.cos(np.pi * T / 2)).max()


def nudge(v, k):
    v = f32(v)
    for _ in range(abs(k)):
        v = np.nextafter(v, f32(np.inf) if k > 0 else f32(-np.inf))
    return f32(v)


def tune(cs, err, free):
    best = (err(cs), cs)
    for d in itertools.product(range(-2, 3), repeat=len(free)):
        c = list(cs)
        for i, k in zip(free, d):
            c[i] = nudge(cs[i], k)
        e = err(c)
        if e < best[0]:
            best = (e, c)
    return best


def main():
    sinc = lambda x: K * np.sin(np.pi * x / 2) / x
    s = [f32(v) for v in remez_even(sinc, lambda x: x, 3, 1e-6, 0.5)]
    c = [f32(v) for v in remez_even(lambda x: K * np.cos(np.pi * x / 2), lambda x: 1.0 + 0 * x, 4, 0.0, 0.5)]
    c[0] = f32(K)
    es, s = tune(s, err_sin, [0, 1, 2, 3])
    ec, c = tune(c, err_cos, [1, 2, 3, 4])
    print("// max abs error of the fp32 evaluation: sin %.3e, cos %.3e" % (es, ec))
    for name, vals in (("kS", s), ("kC", c)):
        for k, v in enumerate(vals):
            deg = 2 * k + 1 if name == "kS" else 2 * k
            mant, exp = float(v).hex().split("p")
            print("constexpr float %s%d = %sp%sf;  // %.9g" % (name, deg, mant.rstrip("0"), exp, float(v)))


if __name__ == "__main__":
    main()
