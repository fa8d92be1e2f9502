"""FP64 CPU oracle for Wasserstein distances between output distributions.

TEST INFRASTRUCTURE ONLY (see ``oracle.attention``): only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use
it, and it shares nothing with the HIP library.

What it computes, and the passages it follows
---------------------------------------------
"Is Flash Attention Stable?" (abstract) measures how numeric deviation
matters with the Wasserstein distance, citing "Statistical Aspects of
Wasserstein Distances" (its reference list).  Applied here without training,
the distributions compared are the empirical distributions of the values of
two output tensors of the same forward pass (a low-precision one and the
FP64 one, or two low-precision ones): each tensor of n elements is the
uniform distribution on its n values.  The pages fix neither the order p nor
the ground metric; the reading is the real line with |x - y| and
p = 1, 2, infinity.  For distributions on the real line the optimal coupling
pairs equal quantiles, so

    W_p(mu, nu)^p = integral over t in (0, 1] of |F^-1(t) - G^-1(t)|^p dt
    W_inf(mu, nu) = sup over t of |F^-1(t) - G^-1(t)|

with F^-1, G^-1 the quantile functions.  For p = 1 this equals the area
between the two distribution functions, integral |F(x) - G(x)| dx, computed
separately by :func:`wasserstein1_cdf` (a different formula, used to pin the
quantile one).

Non-finite values: if either input holds a NaN or an infinity the distances
are NaN (they are undefined or infinite) and the count of such elements is
reported.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["wasserstein", "wasserstein1_cdf"]


def _finite_sorted(x):
    a = np.asarray(x, dtype=np.float64).ravel()
    bad = int((~np.isfinite(a)).sum())
    return np.sort(a), bad


def wasserstein(u, v) -> dict:
    """W_1, W_2 and W_inf between the empirical distributions of u and v
    (any sizes >= 1), from the quantile functions.

    The quantile function of n sorted values u_(1) <= ... <= u_(n) is
    u_(i) on ((i-1)/n, i/n].  Both step functions are constant between
    consecutive points of {i/n} and {j/m}; with the common denominator n*m
    these are the integers i*m and j*n, so the intervals are exact."""
    a, bad_a = _finite_sorted(u)
    b, bad_b = _finite_sorted(v)
    n, m = a.size, b.size
    assert n >= 1 and m >= 1
    bad = bad_a + bad_b
    if bad:
        nan = float("nan")
        return dict(w1=nan, w2=nan, winf=nan, n_nonfinite=bad)
    ends = np.union1d(np.arange(1, n + 1, dtype=np.int64) * m,
                      np.arange(1, m + 1, dtype=np.int64) * n)   # right ends, in (0, nm]
    starts = np.concatenate(([0], ends[:-1]))
    width = (ends - starts).astype(np.float64) / (float(n) * float(m))
    ia = -(-ends // m) - 1          # quantile index ceil(T/m) - 1 of u at t = T/(nm)
    ib = -(-ends // n) - 1
    gap = np.abs(a[ia] - b[ib])
    w1 = float((width * gap).sum())
    w2 = float(math.sqrt((width * gap * gap).sum()))
    winf = float(gap.max())
    return dict(w1=w1, w2=w2, winf=winf, n_nonfinite=0)


def wasserstein1_cdf(u, v) -> float:
    """W_1 as the area between the distribution functions:
    sum over consecutive distinct values z_k < z_{k+1} of the pooled sample
    of (z_{k+1} - z_k) * |F(z_k) - G(z_k)|, F(z) = #{u_i <= z} / n."""
    a, bad_a = _finite_sorted(u)
    b, bad_b = _finite_sorted(v)
    if bad_a + bad_b:
        return float("nan")
    z = np.unique(np.concatenate((a, b)))
    if z.size < 2:
        return 0.0
    fa = np.searchsorted(a, z[:-1], side="right") / a.size
    fb = np.searchsorted(b, z[:-1], side="right") / b.size
    return float((np.diff(z) * np.abs(fa - fb)).sum())
