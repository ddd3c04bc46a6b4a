"""Pure-write sliding window (PW) for the Gated DeltaNet state, written out.

TEST INFRASTRUCTURE (see the package docstring).

Source: abstract of "Low-Bit GDN Recurrent-State Quantization: Global
Gradient-aware Allocation and Pure-Write Sliding Windows": PW keeps the most
recent pure writes as FP8 vector pairs, carries them through the full GDN
state transition, and merges them into the low-bit historical state only once
they leave the window. The recurrence itself is the GDN row of Table 1 of
"Preserving Updates in Low-Bit Recurrent State Quantization":
S_t = alpha (S - beta k (k^T S)) + beta k v^T, i.e. S_t = A_t S_{t-1} + beta k v^T
with the transition A_t = alpha_t (I - beta_t k_t k_t^T) acting on key rows.

Readings (the design notes list them):
  W1  S_t = H_t + sum_{c in window} u_c w_c^T. H is the low-bit history
      (codes and steps, requantized every step); the window holds the last W
      pure writes beta_t k_t v_t^T as FP8 pairs (u, w) = (fp8(k_t),
      fp8(fl(beta_t v_t))), in ring slot (t - 1) mod W.
  W2  A pair that stays in the window takes the transition:
        d = pairwise sum over i (row order) of fl(k_i u_i), b = fl(beta d),
        u_i <- fp8(fl(alpha fl(u_i - fl(b k_i)))).
  W3  At step t > W the pair written at step t - W leaves and joins the
      history. The transition T(S) = alpha (S - beta k (k^T S)) is linear, so
      T(H + u w^T) = T(H) + T(u) w^T: the history and the leaving pair take
      the transition separately and the pair is added after it. The history
      takes the GDN step with v = 0 on y_hat = fl(c s), as a state without a
      window does: r = fl(c fl(alpha s)), g_j = pairwise sum over i of
      fl(k_i y_hat_ij) (exact products), w_j = fl(beta fl(0 - fl(alpha g_j))),
      x = fma(k_i, w_j, r). The leaving pair's key takes the W2 transition
      without the FP8 rounding, u'_i = fl(alpha fl(u_i - fl(b k_i))), and
      joins: x = fma(u'_i, w_leave_j, x). x is then requantized by the
      history's scale rule. (An fp32 history uses r = fl(alpha S).)
  W4  The new pair takes the slot the leaving pair freed (or the next empty
      slot while the window fills).
  W5  o_t = x^T q + sum_c w_c (u_c^T q) over the window after the step.
  W6  FP8 is the OCP E4M3 format (exponent bias 7, 3 mantissa bits, largest
      finite 448, no infinities), rounded to nearest-even and saturated to
      +-448 on overflow; NaN stays NaN.
"""
from typing import Dict

import numpy as np

from .fp import Arith, F32, pairwise_sum
from .recurrence import (OState, NONFINITE, SCALE_OVERFLOW, CLIPPED, qrange, scale_rule, quantize_group_codes,
                         _expand, _flat, _retrieval, _group_absmax, _fp16_midpoint_near, FORGIVE)

E4M3_MAX = 448.0


def e4m3_values():
    """The 256 E4M3 codes as float64 (NaN for 0x7F and 0xFF), from the format."""
    out = np.empty(256)
    for b in range(256):
        s = -1.0 if b & 0x80 else 1.0
        e, m = (b >> 3) & 15, b & 7
        if e == 15 and m == 7:
            out[b] = np.nan
        elif e == 0:
            out[b] = s * m * 2.0 ** -9
        else:
            out[b] = s * (1 + m / 8.0) * 2.0 ** (e - 7)
    return out


def fp8_round(x):
    """Round float32 values to E4M3 (W6); returns float32 values."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        _, ex = np.frexp(np.where(np.isfinite(a) & (a > 0), a, 1.0))
        e = np.maximum(ex.astype(np.float64) - 1.0, -6.0)   # binade; below 2^-6 the spacing stays 2^-9
        step = 2.0 ** (e - 3)
        q = np.rint(a / step) * step                 # exact: a / step and back are power-of-two scalings
        q = np.minimum(q, E4M3_MAX)
    r = np.where(np.isnan(x), np.nan, np.copysign(q, x))
    return r.astype(np.float32)


def fp8_encode(x):
    """E4M3 bytes of values already on the grid (fp8_round output)."""
    pos = e4m3_values()[:127]                     # codes 0x00 .. 0x7E, increasing
    x = np.asarray(x, np.float64)
    a = np.where(np.isnan(x), 0.0, np.abs(x))
    idx = np.searchsorted(pos, a).astype(np.int64)
    if np.any(pos[np.minimum(idx, 126)] != a):
        raise ValueError("value not on the E4M3 grid")
    out = (idx | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), out)


def fp8_decode(b):
    """float32 values of E4M3 bytes."""
    return e4m3_values()[np.asarray(b, np.int64)].astype(np.float32)


def zero_state(w) -> OState:
    """Empty history and window (reading: codes 0, steps 0, no pairs)."""
    from .recurrence import zero_state as zs
    if w.model != "gdn" or w.pw_window < 1:
        raise ValueError("the pure-write window is a Gated DeltaNet option with W >= 1")
    st = zs(w.with_(lrb_k=0, lrb_m=0))
    W = w.pw_window
    st.U = np.zeros((w.tiles, w.d_k, W), np.float32)
    st.W = np.zeros((w.tiles, w.d_v, W), np.float32)
    st.n = 0
    return st


def state_dense(st: OState, w) -> np.ndarray:
    """H + sum of the window's pairs, float64 [T, d_k, d_v]."""
    g = w.group
    H = st.codes.astype(np.float64) * np.repeat(st.scales.astype(np.float64), g, axis=2)
    n = min(st.n, w.pw_window)
    return H + np.einsum("tic,tjc->tij", st.U[:, :, :n].astype(np.float64), st.W[:, :, :n].astype(np.float64))


def step(st: OState, inp: Dict, w, A: Arith = F32, static=None, rounding=True):
    """One decode step of a GDN state with a pure-write window (W1-W6).

    rounding=False keeps the window pairs unrounded (no FP8); with an fp32
    history and the 'f64' arithmetic the step is then the exact recurrence
    split into history and window.
    """
    T, dk, dv, g, W = w.tiles, w.d_k, w.d_v, w.group, w.pw_window
    rnd = fp8_round if rounding else (lambda v: A.c(v))
    q = A.c(_flat(w, inp["q"]))
    k = A.c(_flat(w, inp["k"]))
    v = A.c(_flat(w, inp["v"]))
    alpha = A.c(_flat(w, inp["alpha"])).reshape(T)
    beta = A.c(_flat(w, inp["beta"])).reshape(T)
    new = st.copy()
    new.t = st.t + 1
    n = min(st.t, W)
    slot = st.t % W
    leaving = st.t >= W
    # the history takes the transition with v = 0 (W3)
    if st.S32 is not None:
        H = A.c(st.S32)
        r = A.mul(alpha[:, None, None], H)
    else:
        codes_f = st.codes.astype(A.dt)
        H = A.mul(codes_f, _expand(st.scales, g))
        r = A.mul(codes_f, _expand(A.mul(alpha[:, None, None], st.scales), g))
    gsum = _retrieval(w, A, k, H)
    wv = A.mul(beta[:, None], A.sub(A.c(0.0), A.mul(alpha[:, None], gsum)))
    x = A.c(A.fma(k[:, :, None], wv[:, None, :], r))
    # the leaving pair: its key takes the transition (W2 without FP8) and joins (W3)
    if leaving:
        u = A.c(st.U[:, :, slot])
        d = pairwise_sum(A.mul(k, u), 1, A.add) if A.name == "f32" else np.sum(k * u, axis=1)
        b = A.mul(beta, d)
        up = A.mul(alpha[:, None], A.sub(u, A.mul(b[:, None], k)))
        x = A.c(A.fma(up[:, :, None], st.W[:, :, slot][:, None, :], x))
    if not np.all(np.isfinite(x)):
        new.flags |= NONFINITE
    # window pairs that stay take the transition (W2)
    stay = [c for c in range(n) if not (leaving and c == slot)]
    for c in stay:
        u = A.c(st.U[:, :, c])
        d = pairwise_sum(A.mul(k, u), 1, A.add) if A.name == "f32" else np.sum(k * u, axis=1)
        b = A.mul(beta, d)
        new.U[:, :, c] = rnd(A.mul(alpha[:, None], A.sub(u, A.mul(b[:, None], k))))
    # the new pair (W1, W4)
    new.U[:, :, slot] = rnd(k)
    new.W[:, :, slot] = rnd(A.mul(beta[:, None], v))
    new.n = min(st.t + 1, W)
    # readout (W5)
    o = np.einsum("ti,tij->tj", q.astype(np.float64), x.astype(np.float64))
    nn = new.n
    z = np.einsum("tic,ti->tc", new.U[:, :, :nn].astype(np.float64), q.astype(np.float64))
    o = o + np.einsum("tjc,tc->tj", new.W[:, :, :nn].astype(np.float64), z)
    diag = dict(x=x, r=r, w=wv, leaving=leaving, slot=slot)
    if st.S32 is not None:
        new.S32 = x
        return new, o, diag
    # requantize the history (scale rule and rounding as for the plain state)
    bits_full = st.bits[:, None, None]
    _, _, qmax = qrange(bits_full)
    m = _group_absmax(x, g)
    s_new, grew, thr = scale_rule(m, st.scales, qmax, w, A)
    if w.scale_dtype == "f16" and np.any(np.isinf(s_new)):
        new.flags |= SCALE_OVERFLOW
    c_, y, clipped = quantize_group_codes(x, _expand(s_new, g), bits_full, A)
    if np.any(clipped):
        new.flags |= CLIPPED
    new.codes, new.scales = c_, s_new
    frac = y - np.floor(y)
    near = np.abs(frac - 0.5) < FORGIVE
    gnear = np.zeros(m.shape, bool)
    if thr is not None:
        with np.errstate(invalid="ignore", divide="ignore"):
            gnear |= np.abs(m.astype(np.float64) - thr.astype(np.float64)) <= FORGIVE * np.abs(thr.astype(np.float64))
    if w.scale_dtype == "f16":
        ratio = A.div(m, A.c(qmax)).astype(np.float32)
        gnear |= _fp16_midpoint_near(ratio) & (grew if thr is not None else True)
    near |= _expand(gnear, g)
    diag.update(y=y, m=m, grew=grew, thr=thr, s_new=s_new, near=near, group_near=gnear, clipped=clipped)
    return new, o, diag
