"""INT4+Had: the state stored after a Walsh-Hadamard rotation of each scale
group, written out.

TEST INFRASTRUCTURE (see the package docstring).

Source: "Preserving Updates in Low-Bit Recurrent State Quantization",
Table 2: the INT4+Had baseline applies a Hadamard rotation before INT4
quantization, at the same 4.50 bits per element as INT4 (group 32 with a
16-bit step size).

Readings (the design notes list them):
  H1  The rotation acts on each scale group: the g consecutive columns of one
      row (the d_v axis, along which the groups run). Stored codes and steps
      describe y = x H_g, with H_g the g x g Sylvester-Hadamard matrix
      (entries +-1, unnormalised); the step rule and rounding act on y.
  H2  Dequantization inverts the rotation: x_hat = (c s) H_g / g; g is a power
      of two, so the 1/g is an exact scaling.
  H3  The step runs in the rotated basis. The rotation acts on the value
      axis only, while the decay scales rows and the update is rank one, so
      (A X + k w^T) H_g = A (X H_g) + k (H_g w)^T. With y_hat = fl(c s) the
      stored (rotated) state:
        r = fl(c fl(a_i s))                     decay, as without the rotation
        u~ = sum_i k_i y_hat_i                  retrieval in the rotated basis
                                                (pairwise tree of exact products)
        u = fl(u~ H_g) / g                      Gated DeltaNet: back to the state's basis
        w = fl(beta fl(v - fl(alpha u)))        (w = v for the other rows)
        y = fma(k_i, fl(H_g w)_j, r_ij)         the new rotated state
        o = (sum_i q_i y_i) H_g / g             the readout, in the state's basis
      and y is requantized. In exact arithmetic this is the same map as
      un-rotating, stepping and rotating again; it transforms three vectors
      per tile instead of the whole state, twice.
  H4  The transform runs in float32 as the radix-2 butterfly with pair
      distance h = 1, 2, 4, ..., g/2 in that order, each butterfly
      (a, b) -> (fl(a + b), fl(a - b)) on positions (j, j + h), j & h = 0.
  H5  BDR and the low-rank bypass are not combined with the rotation (the
      pages evaluate INT4+Had as a plain baseline).
"""
from typing import Dict

import numpy as np

from .fp import Arith, F32, F64
from .recurrence import (OState, NONFINITE, SCALE_OVERFLOW, CLIPPED, decay_rows, qrange, scale_rule,
                         quantize_group_codes, _expand, _flat, _retrieval, _group_absmax, _fp16_midpoint_near,
                         FORGIVE)


def fwht(x, g, A: Arith = F32):
    """Unnormalised Walsh-Hadamard transform of each group of g consecutive
    entries along the last axis, butterflies in the order of H4."""
    x = A.c(x)
    shp = x.shape
    y = x.reshape(shp[:-1] + (shp[-1] // g, g)).copy()
    h = 1
    while h < g:
        idx = np.arange(g)
        lo = idx[(idx & h) == 0]
        hi = lo + h
        a = y[..., lo]
        b = y[..., hi]
        y[..., lo] = A.add(a, b)
        y[..., hi] = A.sub(a, b)
        h *= 2
    return y.reshape(shp)


def inverse(y, g, A: Arith = F32):
    """x = (y H_g) / g (H2)."""
    return A.mul(fwht(y, g, A), 1.0 / g)


def dequant(st: OState, w, A: Arith = F32) -> np.ndarray:
    """x_hat of every tile: fl(c s) rotated back (H2)."""
    yhat = A.mul(st.codes.astype(A.dt), _expand(st.scales, w.group))
    return inverse(yhat, w.group, A)


def step(st: OState, inp: Dict, w, A: Arith = F32, static=None):
    """One decode step of an INT4+Had state (H1-H4). Same return convention
    as recurrence.step: (new state, o [T, d_v] float64, diag)."""
    if w.bdr or w.lrb_m > 0 or w.scale_mode == "yoked":
        raise ValueError("the rotation runs without BDR, bypass or yoked scales (H5)")
    T, g = w.tiles, w.group
    q = A.c(_flat(w, inp["q"]))
    k = A.c(_flat(w, inp["k"]))
    v = A.c(_flat(w, inp["v"]))
    a = decay_rows(w, inp, static)
    new = st.copy()
    new.t = st.t + 1
    codes_f = st.codes.astype(A.dt)
    s_full = _expand(st.scales, g)
    # decay in the rotated basis: r = fl(c fl(a_i s))
    c1 = A.mul(a[:, :, None], st.scales)
    r = A.mul(codes_f, _expand(c1, g))
    if w.model == "gdn":
        alpha = A.c(_flat(w, inp["alpha"])).reshape(T)
        beta = A.c(_flat(w, inp["beta"])).reshape(T)
        yhat = A.mul(codes_f, s_full)
        u = inverse(_retrieval(w, A, k, yhat), g, A)
        wv = A.mul(beta[:, None], A.sub(v, A.mul(alpha[:, None], u)))
    else:
        wv = v
    y = A.c(A.fma(k[:, :, None], fwht(wv, g, A)[:, None, :], r))
    if not np.all(np.isfinite(y)):
        new.flags |= NONFINITE
    # the readout in the state's basis: (q^T y) H / g, in float64
    o = fwht(np.einsum("ti,tij->tj", q.astype(np.float64), y.astype(np.float64)), g, F64) / g
    x = inverse(y, g, F64)      # the unquantized new state in its own basis (diagnostics)
    bits_full = st.bits[:, None, None]
    _, _, qmax = qrange(bits_full)
    m = _group_absmax(y, g)
    s_new, grew, thr = scale_rule(m, st.scales, qmax, w, A)
    if w.scale_dtype == "f16" and np.any(np.isinf(s_new)):
        new.flags |= SCALE_OVERFLOW
    c, yq, clipped = quantize_group_codes(y, _expand(s_new, g), bits_full, A)
    if np.any(clipped):
        new.flags |= CLIPPED
    new.codes, new.scales = c, s_new
    # decision windows, as in recurrence._requantize
    frac = yq - np.floor(yq)
    near = np.abs(frac - 0.5) < FORGIVE
    gnear = np.zeros(m.shape, bool)
    if thr is not None:
        with np.errstate(invalid="ignore", divide="ignore"):
            gnear |= np.abs(m.astype(np.float64) - thr.astype(np.float64)) <= FORGIVE * np.abs(thr.astype(np.float64))
    if w.scale_dtype == "f16":
        ratio = A.div(m, A.c(qmax)).astype(np.float32)
        gnear |= _fp16_midpoint_near(ratio) & (grew if thr is not None else True)
    near |= _expand(gnear, g)
    diag = dict(x=x, y=y, r=r, w=wv, m=m, grew=grew, thr=thr, s_new=s_new, near=near, group_near=gnear,
                clipped=clipped)
    return new, o, diag
