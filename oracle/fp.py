"""Floating-point building blocks of the oracle's canonical fp32 chain.

TEST INFRASTRUCTURE (see the package docstring).

The pages state the method over the reals. To compare a GPU implementation
code for code, the oracle fixes one fp32 evaluation order (the reading is
listed with each use). The pieces here are:

  fma32(a, b, c)     float32 fused multiply-add, RN(a*b + c) with one rounding
  pairwise_sum       cascade (pairwise) summation along an axis whose length
                     is a power of two: level 1 adds neighbours (x0+x1),
                     (x2+x3), ..., level 2 adds neighbouring pairs, and so on.
  f16_round          IEEE binary16 round-to-nearest-even (numpy's conversion)
  f16_of_exact       the same from float64, for exact float32 x binary16 products

Arith bundles the operations so that the recurrence is written once and run
in 'f32' (canonical) or 'f64' (definitional) mode.
"""
import numpy as np

f32 = np.float32
f64 = np.float64


def fma32(a, b, c):
    """Exact float32 fused multiply-add: round(a*b + c) once, to nearest-even.

    a*b of two float32 values is exact in float64 (48 significant bits). The
    float64 sum s = a*b + c may round; TwoSum gives its exact error e. The
    only way float32(s) can differ from the correctly rounded result is when s
    lies exactly on a float32 rounding midpoint and e != 0; then the exact
    value lies on e's side of the midpoint and that neighbour is taken.
    """
    a64 = np.asarray(a, dtype=f32).astype(f64)
    b64 = np.asarray(b, dtype=f32).astype(f64)
    c64 = np.asarray(c, dtype=f32).astype(f64)
    p = a64 * b64
    s = p + c64
    bb = s - p
    err = (p - (s - bb)) + (c64 - bb)
    with np.errstate(over="ignore", invalid="ignore"):
        r = s.astype(f32)
        rd = r.astype(f64)
        d = s - rd
        toward = np.where(d > 0, np.float32(np.inf), np.float32(-np.inf)).astype(f32)
        other = np.nextafter(r, toward)
        half = (other.astype(f64) - rd) * 0.5
        mid = (d != 0) & (d == half) & (err != 0) & np.isfinite(s)
        up = np.maximum(r, other)
        dn = np.minimum(r, other)
        fixed = np.where(err > 0, up, dn)
    return np.where(mid, fixed, r).astype(f32)


def pairwise_sum(x, axis, add):
    """Cascade summation of x along `axis` (length a power of two).

    Level by level: y_i = x_{2i} + x_{2i+1}; repeat until one value is left.
    `add` is the elementwise addition of the arithmetic in use.
    """
    x = np.moveaxis(np.asarray(x), axis, -1)
    n = x.shape[-1]
    if n & (n - 1):
        raise ValueError("pairwise_sum needs a power-of-two length, got %d" % n)
    while x.shape[-1] > 1:
        x = add(x[..., 0::2], x[..., 1::2])
    return x[..., 0]


def f16_round(x):
    """IEEE binary16 round-to-nearest-even (overflow gives inf), as float32 values."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=f32).astype(np.float16).astype(f32)


def f16_of_exact(x64):
    """Round float64 values (exact products) once to binary16, nearest-even, as float32."""
    with np.errstate(over="ignore"):
        return np.asarray(x64, dtype=np.float64).astype(np.float16).astype(f32)


class Arith:
    """Elementwise arithmetic of one evaluation mode."""

    def __init__(self, name):
        assert name in ("f32", "f64")
        self.name = name
        self.dt = f32 if name == "f32" else f64

    def c(self, x):
        return np.asarray(x, dtype=self.dt)

    def mul(self, a, b):
        return self.c(a) * self.c(b)

    def add(self, a, b):
        return self.c(a) + self.c(b)

    def sub(self, a, b):
        return self.c(a) - self.c(b)

    def div(self, a, b):
        with np.errstate(divide="ignore", invalid="ignore"):
            return self.c(a) / self.c(b)

    def fma(self, a, b, c):
        if self.name == "f32":
            return fma32(a, b, c)
        return self.c(a) * self.c(b) + self.c(c)

    def tree_sum(self, x, axis):
        if self.name == "f32":
            return pairwise_sum(self.c(x), axis, self.add)
        return np.sum(self.c(x), axis=axis)


F32 = Arith("f32")
F64 = Arith("f64")
