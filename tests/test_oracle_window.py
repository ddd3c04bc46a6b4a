"""Pins of the pure-write window oracle (oracle/window.py): the E4M3 rounding
against enumeration of the format, and the history + window split against
the closed-form Gated DeltaNet recurrence.

Sources: abstract of "Low-Bit GDN Recurrent-State Quantization: Global
Gradient-aware Allocation and Pure-Write Sliding Windows"; Table 1 of
"Preserving Updates in Low-Bit Recurrent State Quantization"."""
import numpy as np
import pytest

import oracle
from oracle import window as pw
from oracle import closed_form as cf
from rsq_workloads import CONFIGS, static_params, step_inputs


def test_e4m3_table():
    v = pw.e4m3_values()
    fin = v[np.isfinite(v)]
    assert np.sum(np.isnan(v)) == 2 and fin.max() == 448.0 and fin.min() == -448.0
    pos = np.sort(np.unique(fin[fin > 0]))
    assert len(pos) == 126 and pos[0] == 2.0 ** -9 and pos[7] == 2.0 ** -6
    # 8 values per binade above the subnormals, spacing 2^(e-3)
    assert np.all(np.diff(pos[7:15]) == 2.0 ** -9)
    assert np.array_equal(pw.fp8_decode(pw.fp8_encode(pos)), pos.astype(np.float32))


def _nearest_brute(x):
    v = pw.e4m3_values()
    codes = [b for b in range(256) if np.isfinite(v[b]) and not (b == 0x80)]
    out = []
    for xi in np.asarray(x, np.float64):
        if np.isnan(xi):
            out.append(np.nan)
            continue
        if abs(xi) > 448.0:
            out.append(np.copysign(448.0, xi))
            continue
        best, bd = None, None
        for b in codes:
            d = abs(xi - v[b])
            if best is None or d < bd or (d == bd and (b & 1) == 0):
                best, bd = b, d
        out.append(v[best] if v[best] != 0 else np.copysign(0.0, xi))
    return np.array(out)


def test_fp8_rounding_against_enumeration():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(400) * 10.0 ** rng.uniform(-4, 2.5, 400),
        pw.e4m3_values()[np.isfinite(pw.e4m3_values())],                      # on the grid
        (pw.e4m3_values()[1:126] + pw.e4m3_values()[2:127]) / 2,             # exact ties
        [447.0, 449.0, 463.9, 464.0, 500.0, 1e30, -1e30, 2.0 ** -10, 2.0 ** -10 * 3, np.nan, 0.0, -0.0],
    ]).astype(np.float32)
    got = pw.fp8_round(x).astype(np.float64)
    want = _nearest_brute(x.astype(np.float64))
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all(), x[~same][:5]


def _w(W, bits=32, seed=21, **kw):
    return CONFIGS[1].with_(batch=1, heads=2, d_k=16, d_v=8, group=8, bits=bits, mixed_bits=None,
                            scale_mode="dynamic", scale_dtype="f32", pw_window=W, seed=seed, **kw)


@pytest.mark.parametrize("W", [1, 3, 8])
def test_history_plus_window_is_the_exact_recurrence(W):
    """Unrounded pairs and an fp32 history in float64: H + sum u w^T is the
    ordered-product sum of the GDN recurrence at every step, before and after
    pairs start leaving the window, and o_t is S_t^T q_t."""
    w = _w(W)
    sp = static_params(w)
    st = pw.zero_state(w)
    st.S32, st.U, st.W = (a.astype(np.float64) for a in (st.S32, st.U, st.W))   # keep everything in float64
    ks, vs, als, bes = [], [], [], []
    for t in range(1, 15):
        inp = step_inputs(w, t, sp)
        st, o, _ = pw.step(st, inp, w, oracle.F64, sp, rounding=False)
        ks.append(inp["k"].reshape(w.tiles, -1))
        vs.append(inp["v"].reshape(w.tiles, -1))
        als.append(inp["alpha"].reshape(-1))
        bes.append(inp["beta"].reshape(-1))
        dense = st.S32.astype(np.float64) + np.einsum(
            "tic,tjc->tij", st.U[:, :, :st.n].astype(np.float64), st.W[:, :, :st.n].astype(np.float64))
        assert st.n == min(t, W)
        for ti in range(w.tiles):
            ref = cf.unrolled_gdn([a[ti] for a in als], [b[ti] for b in bes], [k[ti] for k in ks],
                                  [v[ti] for v in vs])
            assert np.allclose(dense[ti], ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))
            q = inp["q"].reshape(w.tiles, -1)[ti].astype(np.float64)
            assert np.allclose(o[ti], ref.T @ q, rtol=0, atol=1e-11)


def test_pairs_sit_in_ring_slots():
    """The pair written at step t is (fp8(k_t), fp8(beta_t v_t)) in slot
    (t - 1) mod W until it leaves W steps later."""
    W = 3
    w = _w(W, bits=4)
    sp = static_params(w)
    st = pw.zero_state(w)
    for t in range(1, 8):
        inp = step_inputs(w, t, sp)
        st, _, _ = pw.step(st, inp, w, oracle.F32, sp)
        s = (t - 1) % W
        assert np.array_equal(st.U[:, :, s], pw.fp8_round(inp["k"].reshape(w.tiles, -1)))
        bv = (inp["beta"].reshape(-1, 1).astype(np.float32) * inp["v"].reshape(w.tiles, -1).astype(np.float32))
        assert np.array_equal(st.W[:, :, s], pw.fp8_round(bv))


def test_window_reduces_the_error_of_a_low_bit_history():
    """What the window is for: with an INT4 history, keeping the last 8
    writes as FP8 pairs leaves the full state closer to the exact recurrence
    than plain INT4 (relative error over steps 41-120)."""
    base = CONFIGS[1].with_(batch=2, heads=2, d_k=32, d_v=32, group=32, bits=4, mixed_bits=None,
                            scale_mode="persistent", scale_dtype="f16", seed=8)
    wp = base.with_(pw_window=8)
    wr = base.with_(bits=32)
    sp = static_params(base)
    a, p, r = oracle.zero_state(base), pw.zero_state(wp), oracle.zero_state(wr)
    ea = ep = den = 0.0
    for t in range(1, 121):
        inp = step_inputs(base, t, sp)
        a, _, _ = oracle.step(a, inp, base, oracle.F32, sp)
        p, _, _ = pw.step(p, inp, wp, oracle.F32, sp)
        r, _, _ = oracle.step(r, inp, wr, oracle.F32, sp)
        if t > 40:
            S = r.S32.astype(np.float64)
            ea += np.sum((a.dequant() - S) ** 2)
            ep += np.sum((pw.state_dense(p, wp) - S) ** 2)
            den += np.sum(S * S)
    assert ep < 0.8 * ea
