"""Decay-aware head widths: the oracle against enumeration, a simulation of
its cost model and its special cases; the C entry point against the oracle.

Source: abstract of "Low-Bit Recurrent States in Hybrid Language Models"
(bits allocated across recurrent states from observability-Gramian distortion
weights and normalised state ranges). No GPU is used."""
import ctypes

import numpy as np
import pytest

from oracle import allocation as A

bitrsq = pytest.importorskip("bit_recurrent_state_rsq_amd")
from bit_recurrent_state_rsq_amd import Error, allocate_head_bits, _abi  # noqa: E402
from bit_recurrent_state_rsq_amd._abi import lib  # noqa: E402


def _case(rng, H):
    d = rng.uniform(0.0, 0.9999, H).astype(np.float32)
    r = rng.uniform(0.0, 4.0, H).astype(np.float32)
    return d, r


# ---- oracle pins ---------------------------------------------------------

def test_gramian_weight_matches_a_simulated_error_lifetime():
    """An error e put into a state decaying by random a_t ~ U[0.5, 0.95] keeps
    sum_n prod a^2 of its energy; the mean over many paths is 1/(1 - E[a^2])."""
    rng = np.random.default_rng(7)
    lo, hi = 0.5, 0.95
    ea2 = (hi ** 3 - lo ** 3) / (3.0 * (hi - lo))
    paths, n = 20000, 400
    a = rng.uniform(lo, hi, (paths, n))
    energy = np.cumprod(a * a, axis=1).sum(axis=1) + 1.0   # n = 0 term: the error itself
    w = A.weights([np.float32(ea2)], [1.0])[0]
    assert abs(energy.mean() / w - 1.0) < 0.02


@pytest.mark.parametrize("rho", [0.3, 2.5])
def test_width_cost_matches_simulated_rounding_error(rho):
    """Mean squared rounding error on the b-bit grid of range rho scales as
    (rho / (2^(b-1) - 1))^2: the cost ratios of widths 4, 6, 8 follow it."""
    rng = np.random.default_rng(3)
    x = rng.uniform(-rho, rho, 400000)
    mse = {}
    for b in A.WIDTHS:
        step = rho / (2 ** (b - 1) - 1)
        mse[b] = np.mean((np.round(x / step) * step - x) ** 2)
        assert abs(mse[b] / (step * step / 12.0) - 1.0) < 0.02
    w = A.weights([0.0], [rho])
    for b in (6, 8):
        ratio_cost = A.cost([4], w) / A.cost([b], w)
        assert abs((mse[4] / mse[b]) / ratio_cost - 1.0) < 0.03


@pytest.mark.parametrize("seed", range(6))
def test_greedy_reaches_the_enumerated_minimum(seed):
    rng = np.random.default_rng(seed)
    for _ in range(40):
        H = int(rng.integers(1, 7))
        d, r = _case(rng, H)
        mb = float(rng.uniform(4.0, 8.0))
        bits = A.allocate(d, r, mb)
        assert sum(bits) <= A.budget(H, mb) and set(bits) <= set(A.WIDTHS)
        got = A.cost(bits, A.weights(d, r))
        best = A.min_cost(d, r, mb)
        assert got <= best * (1 + 1e-12) + 1e-300


def test_special_cases():
    d = [0.5, 0.9, 0.99, 0.0]
    r = [1.0, 1.0, 1.0, 1.0]
    assert A.allocate(d, r, 4.0) == [4, 4, 4, 4]
    assert A.allocate(d, r, 8.0) == [8, 8, 8, 8]
    # equal weights: lower indices first
    assert A.allocate([0.5] * 4, [1.0] * 4, 5.0) == [6, 6, 4, 4]
    # a slower decay earns its width first; a head of zero range never gains
    assert A.allocate(d, r, 5.0) == [4, 6, 6, 4]
    assert A.allocate([0.9, 0.9], [0.0, 1.0], 8.0) == [4, 8]
    # the odd bit of a budget is left unused
    assert sum(A.allocate([0.5] * 3, [1.0] * 3, 4.9)) == 14


def test_each_upgrade_goes_to_the_largest_saving():
    """Equal weights fill 4 -> 6 everywhere before any 6 -> 8 (the 4 -> 6
    saving is the larger), in head order."""
    H = 5
    seq = [A.allocate([0.3] * H, [1.0] * H, 4.0 + 2.0 * u / H) for u in range(2 * H + 1)]
    assert seq[H] == [6] * H
    assert seq[H + 2] == [8, 8, 6, 6, 6]
    assert seq[2 * H] == [8] * H


def test_monotone_in_decay_and_range():
    rng = np.random.default_rng(11)
    for _ in range(30):
        H = 12
        d, r = _case(rng, H)
        bits = A.allocate(d, r, float(rng.uniform(4.5, 7.5)))
        w = A.weights(d, r)
        for i in range(H):
            for j in range(H):
                if w[i] > w[j]:
                    assert bits[i] >= bits[j]


def test_oracle_rejects_bad_inputs():
    with pytest.raises(ValueError):
        A.weights([1.0], [1.0])
    with pytest.raises(ValueError):
        A.weights([-0.1], [1.0])
    with pytest.raises(ValueError):
        A.weights([0.5], [np.inf])
    with pytest.raises(ValueError):
        A.allocate([0.5], [1.0], 3.5)


# ---- C entry point against the oracle ------------------------------------

@pytest.mark.parametrize("seed", range(8))
def test_c_allocation_equals_the_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    for H in (1, 2, 3, 7, 16, 64, 1000):
        d, r = _case(rng, H)
        mb = float(np.float32(rng.uniform(4.0, 8.0)))
        assert allocate_head_bits(d, r, mb) == A.allocate(d, r, mb)


def test_c_allocation_ties_and_extremes():
    assert allocate_head_bits([0.5] * 4, [1.0] * 4, 5.0) == [6, 6, 4, 4]
    assert allocate_head_bits([0.5] * 4, [1.0] * 4, 4.0) == [4] * 4
    assert allocate_head_bits([0.5] * 4, [1.0] * 4, 8.0) == [8] * 4
    assert allocate_head_bits([0.9, 0.9], [0.0, 1.0], 8.0) == [4, 8]
    # quantised-looking inputs with many exact ties
    d = np.array([0.5, 0.75, 0.5, 0.75, 0.0, 0.0] * 4, np.float32)
    r = np.array([1.0, 0.5, 1.0, 0.5, 2.0, 2.0] * 4, np.float32)
    for mb in (4.25, 5.0, 5.5, 6.0, 6.75, 7.5):
        assert allocate_head_bits(d, r, mb) == A.allocate(d, r, mb)


@pytest.mark.parametrize("d,r,mb", [
    ([1.0], [1.0], 6.0),
    ([-0.01], [1.0], 6.0),
    ([float("nan")], [1.0], 6.0),
    ([0.5], [float("inf")], 6.0),
    ([0.5], [-1.0], 6.0),
    ([0.5], [1.0], 3.99),
    ([0.5], [1.0], 8.01),
    ([0.5], [1.0], float("nan")),
])
def test_c_allocation_rejects_bad_inputs(d, r, mb):
    with pytest.raises(Error):
        allocate_head_bits(d, r, mb)


def test_c_allocation_null_and_empty():
    out = (ctypes.c_int32 * 1)()
    f = (ctypes.c_float * 1)(0.5)
    assert lib.rsq_allocate_head_bits(None, f, 1, 6.0, out) == _abi.RSQ_E_INVALID
    assert lib.rsq_allocate_head_bits(f, f, 0, 6.0, out) == _abi.RSQ_E_INVALID
    assert lib.rsq_allocate_head_bits(f, f, 1, 6.0, None) == _abi.RSQ_E_INVALID


# ---- what the allocation buys, measured on the oracle -------------------

def _mamba2_decay_sq(a_log, lo=0.001, hi=0.1):
    """E[alpha^2] for alpha = exp(-dt e^a), dt ~ U(lo, hi) (the Mamba2 gate of
    the synthetic inputs), integrated in closed form."""
    c = np.exp(np.asarray(a_log, np.float64))
    return (np.exp(-2 * lo * c) - np.exp(-2 * hi * c)) / (2 * c * (hi - lo))


def test_mamba2_decay_moment_matches_sampling():
    rng = np.random.default_rng(5)
    for a in (0.0, 1.0, 2.0):
        dt = rng.uniform(0.001, 0.1, 200000)
        assert abs(np.mean(np.exp(-2 * dt * np.exp(a))) / _mamba2_decay_sq([a])[0] - 1) < 3e-3


def test_gramian_allocation_lowers_state_error():
    """Mamba2 heads with decays spread by a ~ U(0, 2), 160 steps in float64.
    Relative state error sum ||S_q - S||^2 / sum ||S||^2 over steps 41..160
    against the unquantized state: the Gramian allocation beats the same
    budget spent on protecting the first heads, and matches or beats
    uniform widths. Ranges are the stationary scale sqrt(1/(1 - E[a^2])) of
    a state driven by unit-variance writes (no calibration data)."""
    import oracle
    from rsq_workloads import CONFIGS, static_params, step_inputs
    w = CONFIGS[2].with_(batch=1, heads=16, d_k=64, d_v=64, group=64, steps=160,
                         mixed_bits=None, scale_mode="dynamic", scale_dtype="f32")
    sp = static_params(w)
    d = _mamba2_decay_sq(sp["a_log"]).astype(np.float32)
    rho = np.sqrt(1.0 / (1.0 - d.astype(np.float64))).astype(np.float32)
    H = w.heads
    policies = {
        "uniform 6": [6] * H,
        "gramian 6": allocate_head_bits(d, rho, 6.0),
        "first heads 5": [8] * (H // 4) + [4] * (H - H // 4),
        "gramian 5": allocate_head_bits(d, rho, 5.0),
    }
    for name, b in policies.items():
        assert sum(b) <= (6 if name.endswith("6") else 5) * H, name
    wr = w.with_(bits=32)
    ref = oracle.zero_state(wr)
    sts = {k: oracle.zero_state(w, head_bits=v) for k, v in policies.items()}
    err = dict.fromkeys(policies, 0.0)
    den = 0.0
    for t in range(1, w.steps + 1):
        inp = step_inputs(w, t, sp)
        ref, _, _ = oracle.step(ref, inp, wr, oracle.F64, sp)
        S = ref.S32.astype(np.float64)
        for k in policies:
            sts[k], _, _ = oracle.step(sts[k], inp, w, oracle.F64, sp)
            if t > 40:
                err[k] += float(np.sum((sts[k].dequant() - S) ** 2))
        if t > 40:
            den += float(np.sum(S * S))
    rel = {k: v / den for k, v in err.items()}
    print("relative state error:", {k: "%.4g" % v for k, v in rel.items()})
    assert rel["gramian 6"] <= rel["uniform 6"]
    assert rel["gramian 5"] < 0.5 * rel["first heads 5"]
