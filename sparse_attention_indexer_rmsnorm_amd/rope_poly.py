"""Coefficients of the key store's RoPE cosine and sine polynomials (not run at build time).

On [-pi/4, pi/4], sin r = r + r^3 P(z) and cos r = 1 + z Q(z) with z = r^2; P (degree 5) and Q
(degree 6) interpolate (sin r - r) / r^3 and (cos r - 1) / z at Chebyshev nodes on [0, (pi/4)^2],
which is close to the minimax fit.  Everything is computed in 80-digit decimal arithmetic (sin and
cos by their Taylor series) and the coefficients are printed as fp64 hex literals, lowest degree
first, with the largest error of each polynomial on a fine grid.
"""
import math
from decimal import Decimal as D, getcontext

getcontext().prec = 80
PI = D("3.14159265358979323846264338327950288419716939937510582097494459230781640628620899863")
ZMAX = (PI / 4) ** 2


def _series(x, first, start):
    s, t, k = D(0), first, start
    while abs(t) > D(10) ** -70:
        s += t
        t = -t * x * x / ((k + 1) * (k + 2))
        k += 2
    return s


def sin_d(x):
    return _series(x, x, 1)


def cos_d(x):
    return _series(x, D(1), 0)


def f_sin(z):
    r = z.sqrt()
    return (sin_d(r) - r) / (r * z)


def f_cos(z):
    return (cos_d(z.sqrt()) - 1) / z


def fit(f, deg):
    """Coefficients (lowest first) of the degree-deg polynomial through f at Chebyshev nodes."""
    n = deg + 1
    nodes = [ZMAX / 2 * (1 - D(math.cos((2 * i + 1) * math.pi / (2 * n)))) for i in range(n)]
    a = [[x ** j for j in range(n)] + [f(x)] for x in nodes]
    for c in range(n):
        p = max(range(c, n), key=lambda r: abs(a[r][c]))
        a[c], a[p] = a[p], a[c]
        for r in range(n):
            if r != c:
                m = a[r][c] / a[c][c]
                a[r] = [u - m * v for u, v in zip(a[r], a[c])]
    return [a[i][n] / a[i][i] for i in range(n)]


def horner(c, z):
    s = D(0)
    for v in reversed(c):
        s = s * z + v
    return s


if __name__ == "__main__":
    for name, f, deg in (("P (sin)", f_sin, 5), ("Q (cos)", f_cos, 6)):
        c = fit(f, deg)
        err = max(abs((horner(c, ZMAX * i / 400) - f(ZMAX * i / 400)) * (ZMAX * i / 400))
                  for i in range(1, 401))
        print(name, "max error x z:", float(err))
        print("  ", ", ".join(float(v).hex() for v in c))
