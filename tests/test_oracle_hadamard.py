"""Pins of the INT4+Had oracle (oracle/hadamard.py): the transform against
scipy's Hadamard matrix, its inverse and energy, the exact reconstruction of
a constant group, the per-group error bound, and a definitional step written
with explicit matrix products.

Source: "Preserving Updates in Low-Bit Recurrent State Quantization",
Table 2 (INT4+Had: a Hadamard rotation before INT4, 4.50 bits)."""
import numpy as np
import pytest
from scipy.linalg import hadamard

import oracle
from oracle import hadamard as hd
from oracle.brute import nearest_code
from rsq_workloads import CONFIGS, static_params, step_inputs


@pytest.mark.parametrize("g", [8, 16, 32, 64, 128])
def test_transform_is_the_hadamard_matrix(g):
    rng = np.random.default_rng(g)
    x = rng.integers(-1000, 1000, (3, 5, 256)).astype(np.float64)
    y = hd.fwht(x, g, oracle.F64)
    ref = (x.reshape(3, 5, 256 // g, g) @ hadamard(g)).reshape(x.shape)
    assert np.array_equal(y, ref)
    assert np.array_equal(hd.inverse(y, g, oracle.F64), x)
    xf = rng.standard_normal((2, 3, 256))
    yf = hd.fwht(xf, g, oracle.F64)
    assert np.allclose(yf, (xf.reshape(2, 3, 256 // g, g) @ hadamard(g)).reshape(xf.shape), rtol=0, atol=1e-12)
    e_in = (xf.reshape(2, 3, -1, g) ** 2).sum(-1)
    e_out = (yf.reshape(2, 3, -1, g) ** 2).sum(-1)
    assert np.allclose(e_out, g * e_in, rtol=1e-13)


def test_f32_transform_rounds_each_butterfly():
    """float32 butterflies: the result equals the float64 transform of the
    same values rounded level by level."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 2, 32)).astype(np.float32)
    y = x.astype(np.float64).reshape(2, 2, 1, 32)
    h = 1
    while h < 32:
        idx = np.arange(32)
        lo, hi = idx[(idx & h) == 0], idx[(idx & h) == 0] + h
        a, b = y[..., lo].copy(), y[..., hi].copy()
        y[..., lo] = (a + b).astype(np.float32)
        y[..., hi] = (a - b).astype(np.float32)
        h *= 2
    assert np.array_equal(hd.fwht(x, 32, oracle.F32), y.reshape(2, 2, 32).astype(np.float32))


def _w(model, g=32, bits=4, mode="dynamic", sdt="f16", dk=16, dv=64, seed=31, **kw):
    base = {"retnet": CONFIGS[0], "gdn": CONFIGS[1], "mamba2": CONFIGS[2], "gla": CONFIGS[3]}[model]
    return base.with_(batch=1, heads=2, d_k=dk, d_v=dv, group=g, bits=bits, mixed_bits=None, lrb_k=0,
                      lrb_m=0, bdr=False, scale_mode=mode, scale_dtype=sdt, hadamard=True, seed=seed, **kw)


def test_constant_group_is_reconstructed():
    """A group of equal values rotates to one non-zero coefficient, which
    the quantizer stores as +-qmax: the group comes back up to the step's
    storage rounding."""
    w = _w("retnet", g=32, dk=8, dv=32, sdt="f32", gamma=1.0)
    st = oracle.zero_state(w)
    inp = step_inputs(w, 1, static_params(w))
    inp["k"] = np.zeros_like(inp["k"])
    inp["k"][..., 0] = 1.0
    inp["v"] = np.full_like(inp["v"], 0.375)
    new, _, _ = hd.step(st, inp, w, oracle.F64)
    xh = hd.dequant(new, w, oracle.F64)
    assert np.allclose(xh[:, 0, :], 0.375, rtol=1e-7)
    assert np.all(xh[:, 1:, :] == 0)
    assert set(np.unique(new.codes[:, 0, :])) <= {0, 7}


@pytest.mark.parametrize("model", ["mamba2", "gla", "gdn"])
def test_group_error_bound(model):
    """Dynamic scales never clip, so each rotated element is within s/2 and
    the group's L2 error in the state's own basis is at most s/2 (the
    rotation divided by g is sqrt(g) times an orthogonal map)."""
    w = _w(model, sdt="f32")
    sp = static_params(w)
    st = oracle.zero_state(w)
    for t in range(1, 12):
        new, _, diag = hd.step(st, step_inputs(w, t, sp), w, oracle.F64, sp)
        err = (hd.dequant(new, w, oracle.F64) - diag["x"]).reshape(w.tiles, w.d_k, -1, w.group)
        l2 = np.sqrt((err ** 2).sum(-1))
        assert np.all(l2 <= 0.5 * new.scales * (1 + 1e-9) + 1e-300)
        st = new


@pytest.mark.parametrize("model,mode", [("retnet", "dynamic"), ("mamba2", "persistent"), ("gla", "dynamic"),
                                        ("gdn", "persistent")])
def test_step_matches_a_definitional_loop(model, mode):
    """The step in float64, written per tile and row with explicit products
    by the Hadamard matrix and nearest-code enumeration, matches the oracle's
    step code for code."""
    w = _w(model, g=16, bits=4, mode=mode, sdt="f32", dk=8, dv=32)
    sp = static_params(w)
    st = oracle.zero_state(w)
    Hm = hadamard(w.group).astype(np.float64)
    g, ng = w.group, w.d_v // w.group
    for t in range(1, 7):
        inp = step_inputs(w, t, sp)
        new, _, diag = hd.step(st, inp, w, oracle.F64, sp)
        a_rows = oracle.decay_rows(w, inp, sp)
        for ti in range(w.tiles):
            b, h = divmod(ti, w.heads)
            k, v = inp["k"][b, h].astype(np.float64), inp["v"][b, h].astype(np.float64)
            S = np.zeros((w.d_k, w.d_v))
            for i in range(w.d_k):
                for G in range(ng):
                    yhat = st.codes[ti, i, G * g:(G + 1) * g] * float(st.scales[ti, i, G])
                    S[i, G * g:(G + 1) * g] = yhat @ Hm / g
            R = a_rows[ti][:, None] * S
            if w.model == "gdn":
                al, be = float(inp["alpha"][b, h]), float(inp["beta"][b, h])
                wv = be * (v - al * (k @ S))
            else:
                wv = v
            X = np.outer(k, wv) + R
            for i in range(w.d_k):
                for G in range(ng):
                    y = X[i, G * g:(G + 1) * g] @ Hm
                    m = np.max(np.abs(y))
                    s_old = float(st.scales[ti, i, G])
                    s = float(np.float32(m / 7))
                    if mode == "persistent" and not m > 7 * s_old:
                        s = s_old
                    assert float(new.scales[ti, i, G]) == s
                    for jj in range(g):
                        want = 0 if s == 0 else nearest_code(y[jj] / s, -8, 7)
                        got = new.codes[ti, i, G * g + jj]
                        assert got == want or diag["near"][ti, i, G * g + jj]
        st = new


@pytest.mark.parametrize("model", ["mamba2", "gdn"])
def test_rotation_protects_the_small_channels_of_an_outlier_group(model):
    """What the rotation is for: with one value channel 20x larger in every
    group, plain INT4 sets the group's step by the outlier and rounds the
    other channels away; rotated groups spread the outlier over the group,
    and the other channels keep well under half of plain INT4's error."""
    base = {"gdn": CONFIGS[1], "mamba2": CONFIGS[2]}[model]
    w = base.with_(batch=1, heads=2, d_k=16, d_v=64, group=32, bits=4, scale_mode="dynamic", scale_dtype="f16",
                   mixed_bits=None, lrb_k=0, lrb_m=0, bdr=False, seed=5)
    wh, wr = w.with_(hadamard=True), w.with_(bits=32)
    sp = static_params(w)
    a, h, r = oracle.zero_state(w), oracle.zero_state(wh), oracle.zero_state(wr)
    ea = eh = den = 0.0
    for t in range(1, 121):
        inp = step_inputs(w, t, sp)
        inp["v"] = inp["v"].copy()
        inp["v"][..., ::32] *= 20.0
        a, _, _ = oracle.step(a, inp, w, oracle.F64, sp)
        h, _, _ = hd.step(h, inp, wh, oracle.F64, sp)
        r, _, _ = oracle.step(r, inp, wr, oracle.F64, sp)
        if t > 40:
            S = np.asarray(r.S32, np.float64)
            keep = np.ones(S.shape, bool)
            keep[..., ::32] = False
            ea += np.sum(((a.dequant() - S) ** 2)[keep])
            eh += np.sum(((hd.dequant(h, wh, oracle.F64) - S) ** 2)[keep])
            den += np.sum((S ** 2)[keep])
    assert np.sqrt(eh / den) < 0.6 * np.sqrt(ea / den)
