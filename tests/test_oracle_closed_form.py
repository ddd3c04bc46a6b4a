"""Pins of the oracle's unquantized (fp32-state) path: closed forms of the
unrolled recurrence and the delta rule's special cases (Table 1 of
"Preserving Updates in Low-Bit Recurrent State Quantization")."""
import numpy as np
import pytest

import oracle
from oracle import closed_form as cf
from rsq_workloads import CONFIGS, step_inputs, static_params


def _fp32_workload(model, dk=16, dv=8, batch=2, heads=2, seed=77):
    base = {"retnet": CONFIGS[0], "gdn": CONFIGS[1], "mamba2": CONFIGS[2], "gla": CONFIGS[3]}[model]
    return base.with_(batch=batch, heads=heads, d_k=dk, d_v=dv, bits=32, group=dv,
                      mixed_bits=None, lrb_k=0, lrb_m=0, bdr=False,
                      scale_mode="dynamic", seed=seed)


def _run(w, T, arith, static=None, first=None):
    static = static or static_params(w)
    st = oracle.zero_state(w)
    if first is not None:
        st.S32 = first.copy()
    outs, states, inps = [], [], []
    for t in range(1, T + 1):
        inp = step_inputs(w, t, static)
        st, o, _ = oracle.step(st, inp, w, arith, static)
        outs.append(o)
        states.append(st.S32.astype(np.float64))
        inps.append(inp)
    return states, outs, inps


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("model", ["retnet", "mamba2", "gla"])
def test_fp32_path_matches_unrolled_sum(model):
    w = _fp32_workload(model)
    T = 24
    static = static_params(w)
    s64, o64, inps = _run(w, T, oracle.F64, static)
    s32, o32, _ = _run(w, T, oracle.F32, static)
    for tile in range(w.tiles):
        b, h = divmod(tile, w.heads)
        a_seq = [oracle.decay_rows(w, inp, static)[tile] for inp in inps]
        k_seq = [inp["k"][b, h] for inp in inps]
        v_seq = [inp["v"][b, h] for inp in inps]
        for t in (1, 2, 7, T):
            S = cf.unrolled_diag(a_seq[:t], k_seq[:t], v_seq[:t])
            o = cf.readout(S, inps[t - 1]["q"][b, h])
            assert np.allclose(s64[t - 1][tile], S, rtol=1e-12, atol=1e-14)
            assert np.allclose(o64[t - 1][tile], o, rtol=1e-11, atol=1e-13)
            assert _rel(s32[t - 1][tile], S) <= (1e-4 if t < T else 1e-3)
            assert _rel(o32[t - 1][tile], o) <= (1e-4 if t < T else 1e-3)


def test_fp32_gdn_matches_ordered_product():
    w = _fp32_workload("gdn", dk=8, dv=4)
    T = 12
    static = static_params(w)
    s64, o64, inps = _run(w, T, oracle.F64, static)
    s32, _, _ = _run(w, T, oracle.F32, static)
    for tile in range(w.tiles):
        b, h = divmod(tile, w.heads)
        al = [inp["alpha"][b, h] for inp in inps]
        be = [inp["beta"][b, h] for inp in inps]
        ks = [inp["k"][b, h] for inp in inps]
        vs = [inp["v"][b, h] for inp in inps]
        for t in (1, 3, T):
            S = cf.unrolled_gdn(al[:t], be[:t], ks[:t], vs[:t])
            assert np.allclose(s64[t - 1][tile], S, rtol=1e-11, atol=1e-13)
            assert _rel(s32[t - 1][tile], S) <= 1e-4


def test_gdn_writes_exactly_when_beta_one_and_unit_key():
    # beta = 1 and |k| = 1: S_t^T k_t = alpha(S^T k - S^T k) + v = v.
    w = _fp32_workload("gdn", dk=8, dv=4)
    static = static_params(w)
    st = oracle.zero_state(w)
    rng = np.random.default_rng(5)
    st.S32 = rng.standard_normal((w.tiles, w.d_k, w.d_v)).astype(np.float32)
    for t in range(1, 6):
        inp = step_inputs(w, t, static)
        k = inp["k"].astype(np.float64)
        k = k / np.linalg.norm(k, axis=-1, keepdims=True)
        inp = dict(inp, k=k, beta=np.ones_like(inp["beta"]))
        st64, _, _ = oracle.step(st, inp, w, oracle.F64, static)
        kt = k.reshape(w.tiles, w.d_k)
        got = np.einsum("tij,ti->tj", st64.S32.astype(np.float64), kt)
        assert np.allclose(got, inp["v"].reshape(w.tiles, w.d_v), atol=1e-5)
        st = st64


def test_gdn_identity_when_alpha_one_beta_zero():
    w = _fp32_workload("gdn", dk=8, dv=4)
    static = static_params(w)
    st = oracle.zero_state(w)
    st.S32 = np.random.default_rng(9).standard_normal((w.tiles, w.d_k, w.d_v)).astype(np.float32)
    inp = step_inputs(w, 1, static)
    inp = dict(inp, alpha=np.ones_like(inp["alpha"]), beta=np.zeros_like(inp["beta"]))
    new, _, _ = oracle.step(st, inp, w, oracle.F32, static)
    assert np.array_equal(new.S32, st.S32)


def test_retnet_gamma_one_is_running_sum():
    w = _fp32_workload("retnet", dk=8, dv=4).with_(gamma=1.0)
    static = static_params(w)
    s64, _, inps = _run(w, 10, oracle.F64, static)
    S = sum(np.einsum("bhi,bhj->bhij", inp["k"].astype(np.float64), inp["v"].astype(np.float64))
            for inp in inps).reshape(w.tiles, w.d_k, w.d_v)
    assert np.allclose(s64[-1], S, rtol=1e-12, atol=1e-14)
