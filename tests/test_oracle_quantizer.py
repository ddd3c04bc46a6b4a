"""Pins of the oracle's quantizer, scale rules and BDR (invariants that follow
from the definitions; see the oracle's reading list R3-R7)."""
import numpy as np
import pytest

import oracle
from oracle import recurrence as R
from rsq_workloads import CONFIGS, step_inputs, static_params


def _small(ci, **kw):
    w = CONFIGS[ci]
    d = dict(batch=2)
    if w.heads > 4:
        d["heads"] = 4
        if w.mixed_bits:
            d["mixed_bits"] = (1, 2, 1)
    d.update(kw)
    return w.with_(**d)


def _trajectory(w, T):
    static = static_params(w)
    st = oracle.zero_state(w)
    for t in range(1, T + 1):
        inp = step_inputs(w, t, static)
        prev = st
        st, o, d = oracle.step(st, inp, w, oracle.F32, static)
        yield prev, st, d


@pytest.mark.parametrize("ci", [0, 1, 2, 4])
def test_codes_in_range_and_group_absmax_maps_to_qmax(ci):
    w = _small(ci)
    for prev, st, d in _trajectory(w, 24):
        lo, hi, qmax = R.qrange(st.bits[:, None, None])
        assert np.all(st.codes >= lo) and np.all(st.codes <= hi)
        if w.scale_mode == "dynamic":
            T, dk, dv = st.codes.shape
            g = w.group
            ca = np.abs(st.codes.reshape(T, dk, dv // g, g)).max(axis=3)
            nz = st.scales > 2.0 ** -14          # normal-range scales
            assert np.all(ca[nz] == np.broadcast_to(qmax, ca.shape)[nz])


@pytest.mark.parametrize("ci", [0, 2, 3])
def test_dynamic_requantization_is_idempotent(ci):
    w = _small(ci, lrb_k=0, lrb_m=0, bdr=False, model="mamba2" if ci != 3 else "gla")
    static = static_params(w)
    st = None
    for _, st, _ in _trajectory(w, 8):
        pass
    # a step with unit decay and a zero update requantizes deq(Q(x)) only
    inp = step_inputs(w, 99, static)
    inp = dict(inp, k=np.zeros_like(inp["k"]), alpha=np.ones_like(inp["alpha"]))
    new, _, _ = oracle.step(st, inp, w, oracle.F32, static)
    assert np.array_equal(new.codes, st.codes)
    ulp = np.spacing(st.scales)
    assert np.all(np.abs(new.scales - st.scales) <= ulp)


@pytest.mark.parametrize("ci", [0, 1, 2, 4])
def test_rounding_error_within_half_step(ci):
    w = _small(ci)
    for prev, st, d in _trajectory(w, 16):
        s = np.repeat(st.scales, w.group, axis=2).astype(np.float64)
        x = d["x"].astype(np.float64)
        ok = ~d["clipped"] & (s > 0)
        err = np.abs(x - st.codes * s)
        # y = x * RN(1/s) with |RN(1/s) s - 1| <= 2^-24: the grid point c/RN(1/s) sits within
        # |c| s 2^-24 of c s
        slack = (np.abs(st.codes) + 1) * s * 2.0 ** -23
        assert np.all(err[ok] <= 0.5 * s[ok] + slack[ok])


def test_exact_ties_round_to_even():
    s = np.full((1, 1, 16), 2.0 ** -4, np.float32)
    n = np.arange(-8, 8)
    x = ((n + 0.5) * 2.0 ** -4).astype(np.float32).reshape(1, 1, 16)
    bits = np.full((1, 1, 1), 6)
    for A in (oracle.F32, oracle.F64):
        c, y, _ = R.quantize_group_codes(x, s, bits, A)
        assert np.all(c % 2 == 0)
        assert np.all(np.abs(c - (n + 0.5)) == 0.5)


def test_zero_scale_gives_zero_codes():
    x = np.zeros((1, 2, 4), np.float32)
    s = np.zeros((1, 2, 4), np.float32)
    c, y, _ = R.quantize_group_codes(x, s, np.full((1, 1, 1), 4), oracle.F32)
    assert np.all(c == 0)


@pytest.mark.parametrize("ci", [1, 4])
def test_persistent_scale_grows_only_past_threshold(ci):
    w = _small(ci)
    grew_any = False
    for prev, st, d in _trajectory(w, 48):
        assert np.all(st.scales >= prev.scales)
        changed = st.scales != prev.scales
        lo, hi, qmax = R.qrange(st.bits[:, None, None])
        m = d["m"].astype(np.float64)
        thr = (np.float32(w.trigger) * qmax.astype(np.float32)).astype(np.float32) * prev.scales
        assert np.all(m[changed] > thr[changed])
        grew_any |= bool(changed.any())
        # the covered range: |y| <= qmax (1 + 2^-11) where the scale is a normal binary16
        s = np.repeat(st.scales, w.group, axis=2)
        normal = s >= 2.0 ** -14
        q = np.broadcast_to(qmax, d["y"].shape)
        assert np.all(np.abs(d["y"][normal]) <= q[normal] * (1 + 2.0 ** -11))
    assert grew_any


def _bdr_workload(eps=0.5, model="gdn"):
    base = CONFIGS[1] if model == "gdn" else CONFIGS[3]
    return base.with_(batch=2, heads=2, d_k=32, d_v=32, bdr=True, bdr_eps=eps, lrb_k=0, lrb_m=0,
                      scale_mode="dynamic", scale_dtype="f16", seed=4242)


@pytest.mark.parametrize("model", ["gdn", "gla"])
def test_bdr_never_leaves_an_element_opposite_to_its_update(model):
    w = _bdr_workload(0.5, model)
    seen_fix = 0
    for prev, st, d in _trajectory(w, 40):
        sig = d["sigma"]
        s = np.repeat(st.scales, w.group, axis=2)
        val = (st.codes.astype(np.float32) * s).astype(np.float32)
        r = d["r"]
        lo, hi, _ = R.qrange(st.bits[:, None, None])
        # the one exception: the stored step rounds below absmax/qmax, the absmax element
        # rounds to the range edge, and c + sigma would leave the code range
        edge = (d["c_rtn"] + sig < lo) | (d["c_rtn"] + sig > hi)
        live = (sig != 0) & (s > 0) & ~edge
        assert np.all(sig[live] * (val[live].astype(np.float64) - r[live].astype(np.float64)) >= 0)
        assert np.all(np.abs(st.codes - d["c_rtn"]) <= 1)
        assert np.all(d["reversed"][st.codes != d["c_rtn"]])
        err = np.abs(d["x"].astype(np.float64) - st.codes * s.astype(np.float64))
        assert np.all(err[s > 0] <= s[s > 0].astype(np.float64) * (1 + 2.0 ** -20))
        # a correction never crosses the clamp
        fixed = d["corrected"]
        assert np.all(st.codes[fixed] == d["c_rtn"][fixed] + sig[fixed])
        seen_fix += int(fixed.sum())
    assert seen_fix > 0


def test_bdr_gate_below_half_step_leaves_large_moves():
    w = _bdr_workload(0.3, "gdn")
    n_gated = 0
    for prev, st, d in _trajectory(w, 40):
        s = np.repeat(st.scales, w.group, axis=2).astype(np.float64)
        sig = d["sigma"]
        rev = d["reversed"]
        unfixed = rev & ~d["corrected"]
        cand = d["c_rtn"] + sig
        err = np.abs(d["x"].astype(np.float64) - cand * s)
        assert np.all(err[unfixed] > 0.8 * s[unfixed] * (1 - 2.0 ** -20))
        assert np.all(rev[d["corrected"]])
        n_gated += int(unfixed.sum())
    assert n_gated > 0
