"""Brute force on tiny shapes: the vectorized oracle against enumeration and a
scalar triple-loop implementation (the oracle's readings R3, R6, R7, R9)."""
from fractions import Fraction
import numpy as np
import pytest

import oracle
from oracle import brute, recurrence as R
from rsq_workloads import CONFIGS, step_inputs, static_params

N_SEEDS = 10000


def test_rne_formula_matches_code_enumeration():
    rng = np.random.default_rng(11)
    for bits in (2, 3, 4, 6, 8):
        lo, hi = -(2 ** (bits - 1)), 2 ** (bits - 1) - 1
        ys = np.concatenate([rng.uniform(lo - 2, hi + 2, 400),
                             np.arange(lo * 2 - 2, hi * 2 + 3) / 2.0])      # every exact tie
        x = ys.astype(np.float32).reshape(1, 1, -1)
        s = np.ones_like(x)
        c, _, _ = R.quantize_group_codes(x, s, np.full((1, 1, 1), bits), oracle.F64)
        for yi, ci in zip(x.ravel(), c.ravel()):
            assert ci == brute.nearest_code(Fraction(float(yi)), lo, hi)


def test_bdr_matches_enumeration_on_the_update_side():
    rng = np.random.default_rng(12)
    checked = 0
    for _ in range(3000):
        bits = int(rng.choice([2, 3, 4]))
        lo, hi = -(2 ** (bits - 1)), 2 ** (bits - 1) - 1
        s = np.float32(2.0 ** rng.integers(-3, 2)) * np.float32(rng.uniform(0.6, 1.4))
        r = np.float32(rng.uniform(lo + 0.5, hi - 0.5) * s)
        sigma = int(rng.choice([-1, 1]))
        x = np.float32(r + sigma * abs(rng.standard_normal()) * s * rng.choice([0.05, 0.3, 1.0]))
        xa = np.array([[[x]]], np.float32)
        sa = np.array([[[s]]], np.float32)
        bitsa = np.full((1, 1, 1), bits)
        c, _, _ = R.quantize_group_codes(xa, sa, bitsa, oracle.F32)
        c2, rev, fix = R.bdr_apply(c, xa, np.array([[[r]]], np.float32), np.full((1, 1, 1), sigma),
                                   sa, bitsa, 0.5, oracle.F32)
        want = brute.bdr_code(x, r, sigma, s, lo, hi)
        if abs(float(x) / float(s)) > hi + 0.5 or abs(float(x) / float(s)) > -lo + 0.5:
            continue          # outside the covered range the clamp decides
        assert c2.ravel()[0] == want, (x, r, sigma, s, bits)
        checked += 1
    assert checked > 2000


def _tiny_workload(rng, seed):
    model = str(rng.choice(["retnet", "mamba2", "gla", "gdn"]))
    dk = int(rng.choice([1, 2, 4] if model == "gdn" else [1, 2, 3]))
    dv = int(rng.choice([2, 4]))
    g = int(rng.choice([1, 2, dv]))
    bits = int(rng.choice([2, 3, 4]))
    mode = str(rng.choice(["dynamic", "persistent"]))
    sdt = str(rng.choice(["f32", "f16"]))
    bdr = bool(rng.integers(0, 2)) and model != "retnet"
    base = {"retnet": CONFIGS[0], "gdn": CONFIGS[1], "mamba2": CONFIGS[2], "gla": CONFIGS[3]}[model]
    return base.with_(batch=1, heads=1, d_k=dk, d_v=dv, group=g, bits=bits, mixed_bits=None,
                      scale_mode=mode, scale_dtype=sdt, bdr=bdr, bdr_eps=float(rng.choice([0.25, 0.5])),
                      lrb_k=0, lrb_m=0, in_dtype="f32", seed=seed,
                      gamma=float(rng.uniform(0.8, 1.0)))


@pytest.mark.parametrize("arith", ["f32", "f64"])
def test_vectorized_step_matches_scalar_loops(arith):
    A = oracle.F32 if arith == "f32" else oracle.F64
    rng = np.random.default_rng(2024 if arith == "f32" else 2025)
    n_seeds = N_SEEDS if arith == "f32" else N_SEEDS // 5
    for case in range(n_seeds):
        w = _tiny_workload(rng, seed=50_000 + case)
        static = static_params(w)
        st = oracle.zero_state(w)
        T = int(rng.integers(1, 9))
        codes = [[0] * w.d_v for _ in range(w.d_k)]
        scales = [[0.0] * (w.d_v // w.group) for _ in range(w.d_k)]
        for t in range(1, T + 1):
            inp = step_inputs(w, t, static)
            st, o, d = oracle.step(st, inp, w, A, static)
            a = oracle.decay_rows(w, inp, static)[0]
            kw = dict(alpha=float(inp["alpha"].ravel()[0]), beta=float(inp["beta"].ravel()[0])) \
                if w.model == "gdn" else {}
            codes, scales, o_s, x_s = brute.step_tile(
                codes, scales, w.bits, a, inp["q"][0, 0], inp["k"][0, 0], inp["v"][0, 0],
                w.model, w.group, w.scale_mode, w.scale_dtype, w.trigger,
                bdr=w.bdr, bdr_eps=w.bdr_eps, mode=arith, **kw)
            if arith == "f64":
                # float64 sums may associate differently: compare codes away from ties
                ok = ~d["near"][0] & ~(np.abs(d["y"][0] - np.round(d["y"][0])) > 0.5 - 1e-9)
                assert np.array_equal(np.array(codes)[ok], st.codes[0][ok]), (case, w)
                codes = st.codes[0].tolist()
                scales = st.scales[0].astype(float).tolist()
            else:
                assert np.array_equal(np.array(codes), st.codes[0]), (case, t, w)
                assert np.array_equal(np.array(scales, np.float32), st.scales[0]), (case, t, w)
                assert np.array_equal(np.array(x_s, np.float32), d["x"][0].astype(np.float32))
            assert np.allclose(o_s, o[0], rtol=1e-9, atol=1e-12)
