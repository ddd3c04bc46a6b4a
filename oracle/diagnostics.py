"""Error accounting of the quantized recurrence, written out.

TEST INFRASTRUCTURE (see the package docstring).

Sources: "Preserving Updates in Low-Bit Recurrent State Quantization":
  * Fig. 1: the per-step rounding errors R_tau, their decayed sum
    E_T = sum_tau a_{tau:T} R_tau (a_{tau:T} the decay accumulated from step
    tau to T), and the coherent gain g_T = ||E_T||_F^2 over the sum of its
    diagonal terms sum_tau ||a_{tau:T} R_tau||_F^2;
  * Fig. 2: the same gain restricted to the errors of elements whose update
    was lost (g^lost) or moved to another grid point (g^moved);
  * Fig. 4: rounding loses an update, moves it, or reverses it;
  * Table 5 (appendix): quartiles of |b| / Delta_t (an update element over
    the step size) and the fraction of lost updates.

Readings (the design notes list them):
  D1  R_tau = s_hat_tau - x_tau: the stored value minus the value before
      rounding, every element of the state.
  D2  a_{tau:T} is the product of the row decays of steps tau+1 .. T (the
      Table 1 decay only; the Gated DeltaNet retrieval is not part of it), so
      E_T = a_T E_{T-1} + R_T and D_T = a_T^2 D_{T-1} + R_T^2 elementwise with
      g_T = sum E_T^2 / sum D_T.
  D3  b = k_i w_j (B_t of Table 1) and Delta_t = the group's step after the
      scale rule; an element is updated when b != 0.
  D4  Lost: updated, and the stored code equals the code the no-update value
      r = a s_hat_{t-1} rounds to on the same grid (the update changed
      nothing). Moved: updated and not lost. Reversed: updated and the stored
      value lies strictly on the other side of r from b (the BDR test).
      Lost and moved partition the updated elements; reversed is counted
      apart and overlaps them.
  D5  |b| / Delta_t is counted for updated elements with a finite step
      Delta_t > 0; others carry -1.

In 'f32' mode every quantity follows one float32 chain:
  b = fl(k w), s_hat = c s (exact), R = fl(s_hat - x), ratio = fl(|b| RN(1/s)),
  a2 = fl(a a), E <- fl(fl(a E) + R_m), D <- fl(fl(a2 D) + fl(R_m R_m))
with R_m = R on the elements of the mask m (all, lost, moved) and 0 elsewhere.
"""
from typing import Dict

import numpy as np

from .fp import Arith, F32
from .recurrence import decay_rows, quantize_group_codes, _expand, _flat

PLANES = ("E", "D", "E_lost", "D_lost", "E_moved", "D_moved")
COUNTS = ("updated", "lost", "moved", "reversed")


def zero_accumulators(w, A: Arith = F32) -> Dict[str, np.ndarray]:
    shape = (w.tiles, w.d_k, w.d_v)
    return {p: np.zeros(shape, A.dt) for p in PLANES}


def classify(new, diag, inp, w, A: Arith = F32, static=None):
    """Per-element quantities of one step from the oracle's own step results
    (new state and the diag dict of oracle.step). Returns a dict with
    b, R, ratio, updated, lost, moved, reversed and the decay rows a."""
    g = w.group
    k = A.c(_flat(w, inp["k"]))
    x, r, wv = diag["x"], diag["r"], diag["w"]
    s_full = _expand(new.scales, g).astype(np.float32)
    bits_full = new.bits[:, None, None]
    c = new.codes
    b = A.mul(k[:, :, None], A.c(wv)[:, None, :])
    shat = A.mul(c.astype(A.dt), s_full)
    R = A.sub(shat, x)
    c0, _, _ = quantize_group_codes(r, s_full, bits_full, A)
    updated = b != 0
    lost = updated & (c == c0)
    moved = updated & (c != c0)
    rev = updated & (s_full > 0) & (((b > 0) & (shat < r)) | ((b < 0) & (shat > r)))
    ok = updated & (s_full > 0) & np.isfinite(s_full)
    with np.errstate(divide="ignore", invalid="ignore"):
        if A.name == "f32":
            inv = (np.float32(1) / np.where(ok, s_full, np.float32(1))).astype(np.float32)
            ratio = np.where(ok, A.mul(np.abs(b), inv), np.float32(-1)).astype(np.float32)
        else:
            ratio = np.where(ok, np.abs(b) / np.where(ok, s_full, 1.0), -1.0)
    a = decay_rows(w, inp, static)
    return dict(b=b, R=R, ratio=ratio, updated=updated, lost=lost, moved=moved,
                reversed=rev, a=a)


def accumulate(acc, R, a, masks, A: Arith = F32):
    """One step of E <- a E + R_m, D <- a^2 D + R_m^2 for every mask (D2)."""
    a3 = A.c(a)[:, :, None]
    a2 = A.mul(a3, a3)
    out = {}
    for name, m in masks.items():
        Rm = A.c(np.where(m, R, 0))
        sfx = "" if name == "all" else "_" + name
        out["E" + sfx] = A.add(A.mul(a3, acc["E" + sfx]), Rm)
        out["D" + sfx] = A.add(A.mul(a2, acc["D" + sfx]), A.mul(Rm, Rm))
    return out


def step_diagnostics(acc, counts, new, diag, inp, w, A: Arith = F32, static=None):
    """Fold one oracle step into the accumulators. counts: int64 [T, 4]
    (updated, lost, moved, reversed), added to in place. Returns (acc, ratio)."""
    q = classify(new, diag, inp, w, A, static)
    masks = {"all": np.ones(q["R"].shape, bool), "lost": q["lost"], "moved": q["moved"]}
    acc = accumulate(acc, q["R"], q["a"], masks, A)
    for i, name in enumerate(COUNTS):
        counts[:, i] += q[name].reshape(w.tiles, -1).sum(axis=1)
    return acc, q["ratio"]


def gain(E, D, axis=None):
    """g = sum E^2 / sum D (float64)."""
    e = np.sum(np.asarray(E, np.float64) ** 2, axis=axis)
    d = np.sum(np.asarray(D, np.float64), axis=axis)
    with np.errstate(divide="ignore", invalid="ignore"):
        return e / d


def explicit_error_sum(R_hist, a_hist):
    """E_T = sum_tau (prod_{t = tau+1}^{T} a_t) R_tau in float64, written as
    the sum over tau (not the recursion); a_hist[t] are row decays [T, d_k]."""
    T = len(R_hist)
    E = np.zeros_like(np.asarray(R_hist[0], np.float64))
    for tau in range(T):
        w = np.ones(np.asarray(a_hist[0]).shape, np.float64)
        for t in range(tau + 1, T):
            w = w * np.asarray(a_hist[t], np.float64)
        E = E + w[:, :, None] * np.asarray(R_hist[tau], np.float64)
    return E
