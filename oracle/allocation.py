"""Decay-aware choice of per-head state widths, written out.

TEST INFRASTRUCTURE (see the package docstring).

Source: abstract of "Low-Bit Recurrent States in Hybrid Language Models":
bits are allocated across recurrent states, without calibration data, from
distortion weights given by the observability Gramian combined with
normalised state ranges.

Reading (the page gives no formula; this is the plainest one for a scalar
decay observed directly, and the design notes list it):
  * head h's state decays by a_t each step; an error e put into it at step t
    is still a_{t+1} ... a_{t+n} e after n steps, so its expected total energy
    over the future is e^2 * sum_n E[a^2]^n = e^2 / (1 - E[a^2]) (the
    observability Gramian of x_{t+1} = a_t x_t, y_t = x_t, with independent
    a_t of second moment E[a^2] < 1);
  * rounding to a b-bit symmetric grid over range rho has step
    rho / (2^(b-1) - 1), and the error energy is proportional to its square;
  * so head h at width b costs J_h(b) = w_h / (2^(b-1) - 1)^2 with
    w_h = rho_h^2 / (1 - E[a_h^2]);
  * widths are in {4, 6, 8} (the widths the state codes come in) and the sum
    of widths is at most floor(mean_bits * heads).
The allocation is the minimiser of sum_h J_h. allocate() finds it by upgrades
of 2 bits taken largest saving first (ties: lower head index); min_cost()
finds the minimum by enumeration, which pins allocate() on small cases.
"""
import itertools

import numpy as np

WIDTHS = (4, 6, 8)


def qmax(b):
    """Largest code of a b-bit symmetric grid: 2^(b-1) - 1."""
    return float(2 ** (b - 1) - 1)


def weights(decay_sq, ranges):
    """w_h = rho_h^2 / (1 - E[a_h^2]) in float64 from the float32 inputs."""
    d = np.asarray(decay_sq, dtype=np.float32).astype(np.float64)
    r = np.asarray(ranges, dtype=np.float32).astype(np.float64)
    if np.any(~(d >= 0.0) | ~(d < 1.0)):
        raise ValueError("decay_sq must be in [0, 1)")
    if np.any(~np.isfinite(r) | (r < 0.0)):
        raise ValueError("ranges must be finite and >= 0")
    return (r * r) / (1.0 - d)


def cost(bits, w):
    """sum_h w_h / qmax(b_h)^2."""
    return float(sum(wh / (qmax(b) * qmax(b)) for wh, b in zip(w, bits)))


def budget(heads, mean_bits):
    return int(np.floor(np.float64(np.float32(mean_bits)) * heads))


def allocate(decay_sq, ranges, mean_bits):
    """Greedy upgrades, largest saving J_h(b) - J_h(b+2) first, while the
    budget allows and the saving is positive."""
    w = weights(decay_sq, ranges)
    H = len(w)
    if not (4.0 <= float(np.float32(mean_bits)) <= 8.0):
        raise ValueError("mean_bits must be in [4, 8]")
    bits = [4] * H
    left = (budget(H, mean_bits) - 4 * H) // 2
    while left > 0:
        best, best_gain = -1, 0.0
        for h in range(H):
            b = bits[h]
            if b == 8:
                continue
            gain = w[h] / (qmax(b) * qmax(b)) - w[h] / (qmax(b + 2) * qmax(b + 2))
            if gain > best_gain:
                best, best_gain = h, gain
        if best < 0:
            break
        bits[best] += 2
        left -= 1
    return bits


def min_cost(decay_sq, ranges, mean_bits):
    """Minimum of sum_h J_h over every assignment in {4,6,8}^H within the
    budget, by enumeration (small H only)."""
    w = weights(decay_sq, ranges)
    H = len(w)
    cap = budget(H, mean_bits)
    best = None
    for bits in itertools.product(WIDTHS, repeat=H):
        if sum(bits) > cap:
            continue
        c = cost(bits, w)
        best = c if best is None else min(best, c)
    return best
