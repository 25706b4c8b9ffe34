"""Lloyd-Max codebooks for one coordinate of a rotated unit vector (oracle, fp64).

Follows: turboquant-serve 0.1.2, "Architecture" (keys are normalised to the unit sphere and
Lloyd-Max quantised, MSE-optimal for the Beta prior on rotated unit vectors; codebooks are
fitted once and shared), and the TorbuQuant docs, "Current Status" table (Lloyd-Max
codebooks for the exact Beta-sphere law and its Gaussian approximation).

Densities (textbook, not on the pages)
--------------------------------------
beta      one coordinate X of a uniform point on S^{D-1}:
          f(x) = C (1 - x^2)^((D-3)/2) on [-1, 1],  C = Gamma(D/2) / (sqrt(pi) Gamma((D-1)/2)),
          equivalently (X + 1)/2 ~ Beta((D-1)/2, (D-1)/2).
gaussian  N(0, 1/D), the large-D limit of the above.

Lloyd-Max conditions for L = 2^bits levels c_0 < ... < c_{L-1} and boundaries t_1 < ... < t_{L-1}:
  midpoint condition   t_j = (c_{j-1} + c_j) / 2
  centroid condition   c_j = E[X | t_j < X <= t_{j+1}]      (t_0 = lower end, t_L = upper end)
The solver alternates the two conditions (Lloyd's method) from quantile start points and then
polishes the same fixed point with Newton steps on the boundary equations, because plain
alternation needs very many sweeps at 256 levels.  Each sweep is made exactly symmetric
(c_{L-1-j} = -c_j), which makes the middle boundary exactly 0.

The fp32 arrays handed to the quantizer are the fp64 fixed point rounded to nearest, centroids
and boundaries rounded independently.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
from scipy import special
from scipy.linalg import solve_banded

FAMILIES = ("beta", "gaussian")


# --------------------------------------------------------------------------------------------
# The two densities: pdf, cdf, survival function, quantile and partial first moment.
# --------------------------------------------------------------------------------------------
class _Beta:
    """One coordinate of a uniform point on S^{D-1}."""

    def __init__(self, D: int):
        self.D = D
        self.a = (D - 1) / 2.0            # Beta shape of (X+1)/2
        self.beta = (D - 3) / 2.0         # exponent of (1 - x^2)
        self.logC = math.lgamma(D / 2.0) - 0.5 * math.log(math.pi) - math.lgamma((D - 1) / 2.0)
        self.lo, self.hi = -1.0, 1.0

    def pdf(self, x):
        x = np.asarray(x, dtype=np.float64)
        return np.exp(self.logC) * np.power(np.clip(1.0 - x * x, 0.0, None), self.beta)

    def cdf(self, x):
        return special.betainc(self.a, self.a, (1.0 + np.asarray(x, np.float64)) / 2.0)

    def sf(self, x):
        return special.betainc(self.a, self.a, (1.0 - np.asarray(x, np.float64)) / 2.0)

    def ppf(self, p):
        return 2.0 * special.betaincinv(self.a, self.a, np.asarray(p, np.float64)) - 1.0

    def first_moment(self, a, b):
        """Integral of x f(x) over [a, b] (closed form: d/dx (1-x^2)^(beta+1) = -2(beta+1) x (1-x^2)^beta)."""
        a = np.asarray(a, np.float64)
        b = np.asarray(b, np.float64)
        k = self.beta + 1.0
        ga = np.power(np.clip(1.0 - a * a, 0.0, None), k)
        gb = np.power(np.clip(1.0 - b * b, 0.0, None), k)
        return np.exp(self.logC) * (ga - gb) / (2.0 * k)

    def second_moment(self):
        return 1.0 / self.D


class _Gauss:
    """N(0, sigma^2) with sigma^2 = 1/D."""

    def __init__(self, D: int):
        self.D = D
        self.sigma = 1.0 / math.sqrt(D)
        self.lo, self.hi = -np.inf, np.inf

    def pdf(self, x):
        z = np.asarray(x, np.float64) / self.sigma
        return np.exp(-0.5 * z * z) / (self.sigma * math.sqrt(2.0 * math.pi))

    def cdf(self, x):
        return special.ndtr(np.asarray(x, np.float64) / self.sigma)

    def sf(self, x):
        return special.ndtr(-np.asarray(x, np.float64) / self.sigma)

    def ppf(self, p):
        return self.sigma * special.ndtri(np.asarray(p, np.float64))

    def first_moment(self, a, b):
        """Integral of x f(x) over [a, b] = sigma^2 (f(a) - f(b))."""
        fa = np.where(np.isfinite(a), self.pdf(np.where(np.isfinite(a), a, 0.0)), 0.0)
        fb = np.where(np.isfinite(b), self.pdf(np.where(np.isfinite(b), b, 0.0)), 0.0)
        return self.sigma ** 2 * (fa - fb)

    def second_moment(self):
        return self.sigma ** 2


def density(D: int, family: str):
    if family == "beta":
        return _Beta(D)
    if family == "gaussian":
        return _Gauss(D)
    raise ValueError(f"unknown codebook family {family!r}")


# --------------------------------------------------------------------------------------------
# Cell probabilities and centroids for a boundary vector.
# --------------------------------------------------------------------------------------------
def cell_probabilities(dist, t_inner: np.ndarray) -> np.ndarray:
    """P_j = Pr[t_j < X <= t_{j+1}] for the L cells cut by the L-1 inner boundaries.

    Cells in the upper half use differences of the survival function and cells in the lower
    half differences of the cdf, so that tail cells keep their relative precision.
    """
    t = np.concatenate(([dist.lo], t_inner, [dist.hi]))
    lower_half = t[1:] <= 0.0
    p_cdf = dist.cdf(t[1:]) - dist.cdf(t[:-1])
    p_sf = dist.sf(t[:-1]) - dist.sf(t[1:])
    return np.where(lower_half, p_cdf, p_sf)


def centroids_for(dist, t_inner: np.ndarray):
    """Centroid condition: c_j = (integral of x f over cell j) / P_j."""
    t = np.concatenate(([dist.lo], t_inner, [dist.hi]))
    P = cell_probabilities(dist, t_inner)
    M = dist.first_moment(t[:-1], t[1:])
    return M / P, P


def midpoints(c: np.ndarray) -> np.ndarray:
    """Midpoint (nearest-neighbour) condition: t_j = (c_{j-1} + c_j) / 2."""
    return 0.5 * (c[:-1] + c[1:])


def _symmetrize(c: np.ndarray) -> np.ndarray:
    return 0.5 * (c - c[::-1])


@dataclass
class Codebook:
    D: int
    bits: int
    family: str
    centroids: np.ndarray        # fp64, length 2^bits, ascending
    boundaries: np.ndarray       # fp64, length 2^bits - 1, ascending
    probabilities: np.ndarray    # fp64 cell probabilities
    mse: float                   # E[(X - Q(X))^2] per coordinate
    residual: float              # max |c - centroid condition(midpoints(c))|
    iterations: int

    @property
    def centroids32(self) -> np.ndarray:
        return self.centroids.astype(np.float32)

    @property
    def boundaries32(self) -> np.ndarray:
        return self.boundaries.astype(np.float32)


def _newton_step(dist, t: np.ndarray) -> np.ndarray:
    """One Newton step on G_j(t) = t_j - (c_{j-1}(t) + c_j(t))/2 = 0, j = 1..L-1.

    dc_j/dt_j = f(t_j)(c_j - t_j)/P_j and dc_j/dt_{j+1} = f(t_{j+1})(t_{j+1} - c_j)/P_j,
    so the Jacobian is tridiagonal.
    """
    c, P = centroids_for(dist, t)
    f = dist.pdf(t)
    n = t.size
    # derivative of c_j (cell j = [t_j, t_{j+1}], inner boundary index j-1 .. j in 't')
    dc_lower = f * (c[1:] - t) / P[1:]        # d c_{j} / d t_j      for cells 1..L-1 (lower end t_j)
    dc_upper = f * (t - c[:-1]) / P[:-1]      # d c_{j-1} / d t_j    for cells 0..L-2 (upper end t_j)
    G = t - 0.5 * (c[:-1] + c[1:])
    diag = 1.0 - 0.5 * (dc_upper + dc_lower)
    sub = -0.5 * dc_lower[:-1]                # dG_{j+1}/dt_j  = -0.5 dc_j/dt_j      (c_j lower end)
    sup = -0.5 * dc_upper[1:]                 # dG_{j}/dt_{j+1} = -0.5 dc_j/dt_{j+1} (c_j upper end)
    ab = np.zeros((3, n))
    ab[0, 1:] = sup
    ab[1, :] = diag
    ab[2, :-1] = sub
    step = solve_banded((1, 1), ab, G)
    return step


def lloyd_max(D: int, bits: int, family: str = "beta", tol: float = 1e-13,
              max_lloyd: int = 400, max_newton: int = 60) -> Codebook:
    """Lloyd-Max fixed point for 2^bits levels (fp64)."""
    if bits < 1 or bits > 8:
        raise ValueError("bits must be in 1..8")
    dist = density(D, family)
    L = 1 << bits
    c = dist.ppf((np.arange(L) + 0.5) / L)
    c = _symmetrize(c)
    it = 0
    residual = np.inf
    # Lloyd's alternation of the two conditions.
    for _ in range(max_lloyd):
        it += 1
        t = midpoints(c)
        c_new, _ = centroids_for(dist, t)
        c_new = _symmetrize(c_new)
        residual = float(np.max(np.abs(c_new - c)))
        c = c_new
        if residual <= tol:
            break
    # Newton polishing of the same fixed point (boundary form), kept symmetric.  It runs to the
    # floating-point floor (not just to `tol`) so that independent solvers round the fixed point
    # to the same fp32 values.
    if residual > tol or bits >= 3:
        t = midpoints(c)
        best, stall = residual, 0
        for _ in range(max_newton):
            it += 1
            step = _newton_step(dist, t)
            lam = 1.0
            while True:
                t_try = t - lam * step
                t_try = 0.5 * (t_try - t_try[::-1])
                ext = np.concatenate(([dist.lo], t_try, [dist.hi]))
                if np.all(np.diff(ext) > 0):
                    break
                lam *= 0.5
            t = t_try
            c_new, _ = centroids_for(dist, t)
            c_new = _symmetrize(c_new)
            c_chk, _ = centroids_for(dist, midpoints(c_new))
            residual = float(np.max(np.abs(_symmetrize(c_chk) - c_new)))
            c = c_new
            if residual < best:
                best, stall = residual, 0
            else:
                stall += 1
            if residual <= 1e-17 or stall >= 3:
                break
    t = midpoints(c)
    t[L // 2 - 1] = 0.0 if L > 1 else t[L // 2 - 1]   # exact by symmetry; removes a +-0 ulp
    c_chk, P = centroids_for(dist, t)
    residual = float(np.max(np.abs(c_chk - c)))
    mse = float(dist.second_moment() - np.sum(P * c * c))
    return Codebook(D=D, bits=bits, family=family, centroids=c, boundaries=t,
                    probabilities=P, mse=mse, residual=residual, iterations=it)


_CACHE: dict = {}


def codebook(D: int, bits: int, family: str = "beta") -> Codebook:
    """Memoised lloyd_max()."""
    key = (D, bits, family)
    if key not in _CACHE:
        _CACHE[key] = lloyd_max(D, bits, family)
    return _CACHE[key]
