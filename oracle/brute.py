"""Brute-force and scalar-loop versions of the oracle's pieces, for tiny shapes.

TEST INFRASTRUCTURE (see the package docstring).

These are written independently of recurrence.py, with explicit Python loops
over every index, so that an indexing, transposition or sign mistake in the
vectorized oracle shows up as a disagreement:

  nearest_code   enumerate every code, keep the nearest, ties to the even one
  bdr_code       enumerate the codes on the update's side of the no-update
                 value r and keep the nearest to x (Fig. 4 of "Preserving
                 Updates in Low-Bit Recurrent State Quantization": BDR moves a
                 reversed element to the update's side)
  step_tile      one decode step of one tile with scalar arithmetic, in the
                 same fp32 chain as the vectorized oracle (or float64); with
                 bypass columns (U, W) it also runs the bypass side of the
                 step: for Gated DeltaNet the retrieval reads s_hat + U W^T,
                 every update goes to a new fp16 column pair and the state
                 only decays
"""
from fractions import Fraction
import math
import numpy as np

from .fp import fma32

f32 = np.float32


def nearest_code(y, lo, hi):
    """argmin over integer codes c in [lo, hi] of |y - c|; exact ties go to the even code."""
    y = Fraction(y) if not isinstance(y, Fraction) else y
    best, bestd = None, None
    for c in range(lo, hi + 1):
        d = abs(y - c)
        if best is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    return best


def bdr_code(x, r, sigma, s, lo, hi):
    """Nearest code to x among codes whose value c*s is not on the far side of r.

    sigma = +1: keep c*s >= r; sigma = -1: keep c*s <= r. The nearest-code
    rule is applied within that set (ties to even); if the set is empty the
    plain nearest code is returned.
    """
    x, r, s = Fraction(float(x)), Fraction(float(r)), Fraction(float(s))
    cands = [c for c in range(lo, hi + 1)
             if (sigma > 0 and c * s >= r) or (sigma < 0 and c * s <= r)]
    if not cands:
        return nearest_code(x / s, lo, hi)
    best, bestd = None, None
    for c in cands:
        d = abs(x - c * s)
        if best is None or d < bestd or (d == bestd and c % 2 == 0):
            best, bestd = c, d
    return best


def _pairwise(vals, add):
    if len(vals) == 1:
        return vals[0]
    h = len(vals) // 2
    return add(_pairwise(vals[:h], add), _pairwise(vals[h:], add))


def _round_half_even(y):
    fl = math.floor(y)
    d = y - fl
    if d < 0.5:
        return fl
    if d > 0.5:
        return fl + 1
    return fl if fl % 2 == 0 else fl + 1


def _f16(x):
    return float(np.float16(x))


def step_tile(codes, scales, bits, a, q, k, v, model, group, scale_mode,
              scale_dtype, trigger=1.0, alpha=None, beta=None, bdr=False,
              bdr_eps=0.5, mode="f32", U=None, W=None):
    """One decode step of one tile with scalar loops.

    codes [d_k][d_v] ints, scales [d_k][d_v/group] floats, a [d_k] row decays,
    q, k [d_k], v [d_v]. Returns (codes, scales, o list, x matrix); with a
    bypass, U and W are lists of columns (U[c][i], W[c][j], binary16 values)
    and the new U, W are returned after x.
    """
    dk, dv = len(codes), len(codes[0])
    ng = dv // group
    lo, hi = -(2 ** (bits - 1)), 2 ** (bits - 1) - 1
    qmax = hi
    if mode == "f32":
        F = f32
        mul = lambda p, q_: f32(F(p) * F(q_))
        add = lambda p, q_: f32(F(p) + F(q_))
        sub = lambda p, q_: f32(F(p) - F(q_))
        div = lambda p, q_: f32(F(p) / F(q_))
        fma = lambda p, q_, r_: f32(fma32(np.float32(p), np.float32(q_), np.float32(r_)))
    else:
        F = float
        mul = lambda p, q_: float(p) * float(q_)
        add = lambda p, q_: float(p) + float(q_)
        sub = lambda p, q_: float(p) - float(q_)
        div = lambda p, q_: float(p) / float(q_)
        fma = lambda p, q_, r_: float(p) * float(q_) + float(r_)

    def store(x):
        if scale_dtype == "f16":
            return float(np.float16(x))
        return float(np.float32(x))

    bypass = U is not None
    n = len(U) if bypass else 0
    wv = [v[j] for j in range(dv)]
    if model == "gdn":
        # the bypass's projections of k: z_c = sum_i U_ic k_i
        zk = []
        for c in range(n):
            terms = [mul(U[c][i], k[i]) for i in range(dk)]
            zk.append(_pairwise(terms, add) if mode == "f32" else math.fsum(terms))
        for j in range(dv):
            terms = [mul(k[i], mul(codes[i][j], scales[i][j // group])) for i in range(dk)]
            u = _pairwise(terms, add) if mode == "f32" else math.fsum(terms)
            if n:
                b = F(0.0)
                for c in range(n):
                    b = fma(W[c][j], zk[c], b)
                u = add(u, b)
            wv[j] = mul(beta, sub(v[j], mul(alpha, u)))
    x = [[None] * dv for _ in range(dk)]
    r = [[None] * dv for _ in range(dk)]
    for i in range(dk):
        for j in range(dv):
            c1 = mul(a[i], scales[i][j // group])
            r[i][j] = mul(codes[i][j], c1)
            x[i][j] = r[i][j] if bypass else fma(k[i], wv[j], r[i][j])
    o = [sum(float(q[i]) * float(x[i][j]) for i in range(dk)) for j in range(dv)]
    if bypass:
        # decay the held columns (the exact product rounded once to binary16),
        # append the update as a new column pair, read the bypass out
        U2 = [[_f16(float(a[i]) * float(U[c][i])) for i in range(dk)] for c in range(n)]
        W2 = [list(W[c]) for c in range(n)]
        U2.append([_f16(k[i]) for i in range(dk)])
        W2.append([_f16(wv[j]) for j in range(dv)])
        for j in range(dv):
            o[j] += sum(float(W2[c][j]) * sum(float(U2[c][i]) * float(q[i]) for i in range(dk))
                        for c in range(n + 1))
    new_codes = [[0] * dv for _ in range(dk)]
    new_scales = [[0.0] * ng for _ in range(dk)]
    for i in range(dk):
        for G in range(ng):
            cols = range(G * group, (G + 1) * group)
            m = max(abs(float(x[i][j])) for j in cols)
            s_old = scales[i][G]
            if scale_mode == "dynamic":
                s_new = store(div(m, qmax))
            else:
                thr = mul(mul(trigger, qmax), s_old)
                s_new = store(div(m, qmax)) if m > float(thr) else s_old
            new_scales[i][G] = s_new
            for j in cols:
                if s_new == 0:
                    c = 0
                else:
                    if mode == "f32":
                        inv = f32(f32(1) / f32(s_new))
                        y = float(np.float64(x[i][j]) * np.float64(inv))
                    else:
                        y = float(x[i][j]) / s_new
                    c = min(max(_round_half_even(y), lo), hi)
                if bdr and s_new != 0 and not bypass:
                    sg = int(np.sign(k[i]) * np.sign(wv[j]))
                    if sg != 0:
                        val = float(mul(c, s_new))
                        if (sg > 0 and val < float(r[i][j])) or (sg < 0 and val > float(r[i][j])):
                            cand = min(max(c + sg, lo), hi)
                            err = abs(float(sub(x[i][j], mul(cand, s_new))))
                            if err <= float(mul(add(0.5, bdr_eps), s_new)):
                                c = cand
                new_codes[i][j] = c
    if bypass:
        return new_codes, new_scales, o, x, U2, W2
    return new_codes, new_scales, o, x
