"""Pins of the error-accounting oracle (oracle/diagnostics.py): the decayed
error sum against the gap between the quantized and the unquantized
trajectories, the coherent gain on constructed error sequences, and the
lost / moved / reversed classification against enumeration.

Sources: "Preserving Updates in Low-Bit Recurrent State Quantization",
Figs. 1, 2, 4 and Table 5."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import diagnostics as dg
from oracle.brute import nearest_code
from rsq_workloads import CONFIGS, static_params, step_inputs


def _w(model, bits=4, g=8, dk=16, dv=16, batch=1, heads=2, mode="dynamic", sdt="f32", seed=55, **kw):
    base = {"retnet": CONFIGS[0], "gdn": CONFIGS[1], "mamba2": CONFIGS[2], "gla": CONFIGS[3]}[model]
    return base.with_(batch=batch, heads=heads, d_k=dk, d_v=dv, group=g, bits=bits, mixed_bits=None,
                      lrb_k=0, lrb_m=0, bdr=False, scale_mode=mode, scale_dtype=sdt, seed=seed, **kw)


def _run(w, T, A, static=None, keep=False):
    static = static or static_params(w)
    st = oracle.zero_state(w)
    acc = dg.zero_accumulators(w, A)
    counts = np.zeros((w.tiles, 4), np.int64)
    hist = []
    for t in range(1, T + 1):
        inp = step_inputs(w, t, static)
        new, _, diag = oracle.step(st, inp, w, A, static)
        q = dg.classify(new, diag, inp, w, A, static)
        acc, _ = dg.step_diagnostics(acc, counts, new, diag, inp, w, A, static)
        if keep:
            hist.append((q, inp))
        st = new
    return st, acc, counts, hist


@pytest.mark.parametrize("model", ["retnet", "mamba2", "gla"])
def test_error_sum_is_the_gap_to_the_unquantized_state(model):
    """For the rows whose update does not read the state, the quantized and
    unquantized recurrences differ by exactly sum_tau a_{tau:T} R_tau."""
    w = _w(model, gamma=0.9)
    T = 40
    st, acc, counts, hist = _run(w, T, oracle.F64, keep=True)
    wr = w.with_(bits=32)
    ref = oracle.zero_state(wr)
    sp = static_params(w)
    for t in range(1, T + 1):
        ref, _, _ = oracle.step(ref, step_inputs(w, t, sp), wr, oracle.F64, sp)
    gap = st.dequant() - np.asarray(ref.S32, np.float64)
    rel = np.linalg.norm(acc["E"] - gap) / np.linalg.norm(gap)
    assert rel < 1e-10
    explicit = dg.explicit_error_sum([q["R"] for q, _ in hist], [q["a"] for q, _ in hist])
    assert np.linalg.norm(explicit - gap) / np.linalg.norm(gap) < 1e-10
    # the masked sums split the total: lost + moved + (errors of elements with no update)
    assert np.all(counts[:, 1] + counts[:, 2] == counts[:, 0])


def test_f32_chain_tracks_f64():
    w = _w("gla", dk=32, dv=32, g=16)
    _, a32, c32, _ = _run(w, 30, oracle.F32)
    _, a64, c64, _ = _run(w, 30, oracle.F64)
    for p in dg.PLANES:
        n = np.linalg.norm(a64[p])
        assert np.linalg.norm(a32[p] - a64[p]) <= 1e-3 * n + 1e-30, p
    assert abs(dg.gain(a32["E"], a32["D"]) / dg.gain(a64["E"], a64["D"]) - 1) < 1e-3


def _acc_run(Rs, a):
    shape = Rs[0].shape
    acc = {p: np.zeros(shape) for p in dg.PLANES}
    for R in Rs:
        acc = dg.accumulate(acc, R, np.full(shape[:2], a), {"all": np.ones(shape, bool)}, oracle.F64)
    return acc


def test_gain_of_constructed_error_sequences():
    rng = np.random.default_rng(0)
    R = rng.standard_normal((1, 4, 4))
    T = 12
    # identical errors, no decay: fully coherent, g = T
    acc = _acc_run([R] * T, 1.0)
    assert abs(dg.gain(acc["E"], acc["D"]) - T) < 1e-12
    # alternating signs cancel
    acc = _acc_run([R if t % 2 == 0 else -R for t in range(T)], 1.0)
    assert dg.gain(acc["E"], acc["D"]) < 1e-24
    # disjoint supports: no cross terms, g = 1
    Rs = []
    for t in range(T):
        m = np.zeros((1, 4, 4))
        m.reshape(-1)[t] = rng.standard_normal()
        Rs.append(m)
    acc = _acc_run(Rs, 0.7)
    assert abs(dg.gain(acc["E"], acc["D"]) - 1.0) < 1e-12
    # identical errors under decay a: (sum a^n)^2 / sum a^(2n)
    a = 0.8
    acc = _acc_run([R] * T, a)
    n = np.arange(T)
    assert abs(dg.gain(acc["E"], acc["D"]) - (a ** n).sum() ** 2 / (a ** (2 * n)).sum()) < 1e-9


def test_explicit_sum_equals_recursion_on_random_sequences():
    rng = np.random.default_rng(1)
    Rs = [rng.standard_normal((2, 3, 5)) for _ in range(9)]
    As = [rng.uniform(0.2, 1.0, (2, 3)) for _ in range(9)]
    acc = {p: np.zeros((2, 3, 5)) for p in dg.PLANES}
    for R, a in zip(Rs, As):
        acc = dg.accumulate(acc, R, a, {"all": np.ones(R.shape, bool)}, oracle.F64)
    assert np.allclose(acc["E"], dg.explicit_error_sum(Rs, As), rtol=1e-13, atol=0)


@pytest.mark.parametrize("model,mode", [("mamba2", "dynamic"), ("gla", "persistent"), ("gdn", "dynamic"),
                                        ("retnet", "persistent")])
def test_classification_against_enumeration(model, mode):
    """Every element of a few steps: the code of r and of x by enumeration
    over the code range in exact rationals, the reversal by exact comparison."""
    w = _w(model, bits=4, g=4, dk=8, dv=8, mode=mode, sdt="f16", seed=9)
    sp = static_params(w)
    st = oracle.zero_state(w)
    lo, hi = -8, 7
    seen = dict(lost=0, moved=0, reversed=0)
    for t in range(1, 13):
        inp = step_inputs(w, t, sp)
        new, _, diag = oracle.step(st, inp, w, oracle.F32, sp)
        q = dg.classify(new, diag, inp, w, oracle.F32, sp)
        s_full = np.repeat(new.scales, w.group, axis=2)
        for idx in np.ndindex(*q["b"].shape):
            b = float(q["b"][idx])
            s = float(s_full[idx])
            if b == 0 or s == 0:
                assert not (q["lost"][idx] or q["moved"][idx] or q["reversed"][idx])
                continue
            inv = Fraction(float(np.float32(1) / np.float32(s)))
            c0 = nearest_code(Fraction(float(diag["r"][idx])) * inv, lo, hi)
            c = int(new.codes[idx])
            assert c == nearest_code(Fraction(float(diag["x"][idx])) * inv, lo, hi)
            assert bool(q["lost"][idx]) == (c == c0)
            assert bool(q["moved"][idx]) == (c != c0)
            val, r = Fraction(c) * Fraction(s), Fraction(float(diag["r"][idx]))
            assert bool(q["reversed"][idx]) == ((b > 0 and val < r) or (b < 0 and val > r))
            want = Fraction(abs(b)) * inv
            assert abs(Fraction(float(q["ratio"][idx])) - want) <= want * Fraction(1, 2 ** 24)
            for k in seen:
                seen[k] += bool(q[k][idx])
        st = new
    assert seen["lost"] > 0 and seen["moved"] > 0


def test_on_grid_states_never_reverse():
    """gamma = 1 and a persistent step: where a group's step did not grow,
    r = s_hat is on the grid, so rounding x = r + b never lands on the far
    side of r (and an update smaller than half a step is always lost)."""
    w = _w("retnet", bits=4, g=8, dk=16, dv=16, mode="persistent", sdt="f16", gamma=1.0, trigger=1.0)
    sp = static_params(w)
    st = oracle.zero_state(w)
    kept = lost_small = 0
    for t in range(1, 31):
        inp = step_inputs(w, t, sp)
        new, _, diag = oracle.step(st, inp, w, oracle.F32, sp)
        q = dg.classify(new, diag, inp, w, oracle.F32, sp)
        same = np.repeat(new.scales == st.scales, w.group, axis=2) & (np.repeat(new.scales, w.group, axis=2) > 0)
        assert not np.any(q["reversed"] & same)
        small = same & q["updated"] & (q["ratio"] < 0.5)
        assert np.all(q["lost"][small])
        kept += int(same.sum())
        lost_small += int(small.sum())
        st = new
    assert kept > 1000 and lost_small > 100


def test_bdr_leaves_only_reversals_at_the_range_end():
    """With eps_B >= 0.5 BDR corrects every reversed element whose corrected
    code is in range. What stays reversed sits at the end of the code range:
    a binary16 step fl16(m / qmax) can round below m / qmax, so qmax s can
    fall just short of the no-update value r."""
    w = _w("gla", bits=4, g=8, dk=16, dv=16, mode="dynamic", sdt="f16")
    _, _, plain, _ = _run(w, 24, oracle.F32)
    assert plain[:, 3].sum() > 20
    wb = w.with_(bdr=True, bdr_eps=0.5)
    sp = static_params(wb)
    st = oracle.zero_state(wb)
    left = 0
    for t in range(1, 25):
        inp = step_inputs(wb, t, sp)
        new, _, diag = oracle.step(st, inp, wb, oracle.F32, sp)
        q = dg.classify(new, diag, inp, wb, oracle.F32, sp)
        c = new.codes[q["reversed"]]
        b = q["b"][q["reversed"]]
        assert np.all(((b > 0) & (c == 7)) | ((b < 0) & (c == -8)))
        left += int(q["reversed"].sum())
        st = new
    assert left <= 2


def test_persistent_inputs_make_lost_updates_coherent():
    """Fig. 2's finding on synthetic inputs: when the same small update keeps
    arriving (inputs with a persistent direction), its rounding errors add
    up coherently (g_T well above 1), and mostly on the elements whose
    update is lost; independent steps give g_T close to 1."""
    def run(rho):
        w = _w("retnet", bits=4, g=8, dk=32, dv=32, mode="dynamic", sdt="f16", gamma=0.97,
               coherence=rho, seed=77)
        _, acc, _, _ = _run(w, 400, oracle.F32)
        return (dg.gain(acc["E"], acc["D"]), dg.gain(acc["E_lost"], acc["D_lost"]),
                dg.gain(acc["E_moved"], acc["D_moved"]))
    g0, _, _ = run(0.0)
    g, gl, gm = run(0.9)
    assert g0 < 1.3
    assert g > 3.0 and gl > 2.0 * gm
