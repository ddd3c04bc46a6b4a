"""Pins of the Gated DeltaNet step with a Low-Rank Bypass ("Preserving Updates
in Low-Bit Recurrent State Quantization": Table 1's delta rule, the bypass of
the abstract and Fig. 3, run on GDN in Tables 2, 6, 7 and 8).

The delta rule reads the state it updates: u = S_{t-1}^T k. With a bypass the
state is the stored codes plus the bypass, s_hat + U W^T, so the retrieval must
see both. These tests fix that against things other than the oracle's own
formula: the dense matrix product, a scalar-loop implementation, and the
closed form of the unquantized delta rule (the bypass alone carries it when the
stored codes stay zero)."""
import numpy as np
import pytest

import oracle
from oracle import brute, closed_form as cf
from rsq_workloads import CONFIGS, static_params, step_inputs


def _gdn_lrb(**kw):
    # Table 6's GDN row: k = 1, m = 15, eps_L = 0.5, eps_B = 0.3
    d = dict(batch=2, heads=2, d_k=16, d_v=8, group=8, bdr=True, bdr_eps=0.3,
             lrb_k=1, lrb_m=15, lrb_eps=0.5, scale_mode="dynamic", seed=4242)
    d.update(kw)
    return CONFIGS[1].with_(**d)


def _random_bypass_state(w, n, seed):
    rng = np.random.default_rng(seed)
    st = oracle.zero_state(w)
    st.codes = rng.integers(-7, 8, size=st.codes.shape).astype(np.int32)
    st.scales = oracle.f16_round(rng.uniform(0.01, 0.05, size=st.scales.shape))
    st.U[:, :, :n] = oracle.f16_round(0.3 * rng.standard_normal((w.tiles, w.d_k, n)))
    st.W[:, :, :n] = oracle.f16_round(0.3 * rng.standard_normal((w.tiles, w.d_v, n)))
    st.n = n
    return st


@pytest.mark.parametrize("n", [1, 5, 15])
def test_retrieval_reads_the_stored_state_plus_the_bypass(n):
    """f64: u = (s_hat + U W^T)^T k exactly as the dense product gives it."""
    w = _gdn_lrb()
    st = _random_bypass_state(w, n, seed=n)
    inp = step_inputs(w, 3, static_params(w))
    new, o, d = oracle.step(st, inp, w, oracle.F64)
    k = inp["k"].reshape(w.tiles, -1).astype(np.float64)
    dense = st.dequant()                                  # c s + U W^T, float64
    u_ref = np.einsum("tij,ti->tj", dense, k)
    assert np.allclose(d["u"], u_ref, rtol=1e-12, atol=1e-14)
    # and without the bypass term the retrieval would be visibly different
    shat_only = np.einsum("tij,ti->tj", dense - np.einsum("tic,tjc->tij", st.U[:, :, :n].astype(np.float64),
                                                          st.W[:, :, :n].astype(np.float64)), k)
    assert np.linalg.norm(d["u"] - shat_only) > 1e-3 * np.linalg.norm(u_ref)
    # w = beta (v - alpha u), the delta rule
    al = inp["alpha"].reshape(-1)[:, None].astype(np.float64)
    be = inp["beta"].reshape(-1)[:, None].astype(np.float64)
    v = inp["v"].reshape(w.tiles, -1).astype(np.float64)
    assert np.allclose(d["w"], be * (v - al * u_ref), rtol=1e-12, atol=1e-14)


def test_f32_retrieval_is_the_f64_one_to_rounding():
    w = _gdn_lrb()
    st = _random_bypass_state(w, 9, seed=99)
    inp = step_inputs(w, 5, static_params(w))
    _, _, d32 = oracle.step(st, inp, w, oracle.F32)
    _, _, d64 = oracle.step(st, inp, w, oracle.F64)
    err = np.abs(d32["u"].astype(np.float64) - d64["u"])
    scale = np.abs(d64["u"]) + 1e-3
    assert np.max(err / scale) < 1e-5


def test_empty_bypass_retrieves_like_the_plain_step():
    """n = 0 (just after a k = 0 merge, or a fresh state): no bypass term."""
    w = _gdn_lrb(lrb_k=0)
    st = _random_bypass_state(w, 0, seed=5)
    inp = step_inputs(w, 2, static_params(w))
    _, _, d = oracle.step(st, inp, w, oracle.F32)
    plain = w.with_(lrb_k=0, lrb_m=0)
    st2 = oracle.zero_state(plain)
    st2.codes, st2.scales = st.codes.copy(), st.scales.copy()
    _, _, d2 = oracle.step(st2, inp, plain, oracle.F32)
    assert np.array_equal(d["u"], d2["u"]) and np.array_equal(d["w"], d2["w"])


@pytest.mark.parametrize("arith", ["f32", "f64"])
def test_bypass_carries_the_delta_rule_while_the_codes_stay_zero(arith):
    """Fresh state, no merge: every update lands in the bypass and the stored
    codes stay zero, so U W^T alone must follow the unquantized delta rule
    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T (closed
    form, ordered product), up to the binary16 rounding of the factors. A
    retrieval that missed the bypass would write beta v instead of
    beta (v - alpha S^T k)."""
    A = oracle.F32 if arith == "f32" else oracle.F64
    w = _gdn_lrb(batch=1, heads=3, d_k=8, d_v=8, lrb_k=0, lrb_m=12, bdr=False)
    static = static_params(w)
    st = oracle.zero_state(w)
    inps = []
    for t in range(1, 13):
        inp = step_inputs(w, t, static)
        inps.append(inp)
        st, o, d = oracle.step(st, inp, w, A, static)
        assert not st.codes.any()
        for tile in range(w.tiles):
            S = cf.unrolled_gdn([i["alpha"].reshape(-1)[tile] for i in inps],
                                [i["beta"].reshape(-1)[tile] for i in inps],
                                [i["k"].reshape(w.tiles, -1)[tile] for i in inps],
                                [i["v"].reshape(w.tiles, -1)[tile] for i in inps])
            got = st.dequant()[tile]
            rel = np.linalg.norm(got - S) / np.linalg.norm(S)
            assert rel < 4e-3, (t, tile, rel)
            # the readout is S^T q of that state
            q = inps[-1]["q"].reshape(w.tiles, -1)[tile]
            assert np.linalg.norm(o[tile] - cf.readout(S, q)) <= 4e-3 * np.linalg.norm(cf.readout(S, q)) + 1e-6


def _tiny_gdn_bypass(rng, seed):
    dk = int(rng.choice([1, 2, 4]))
    dv = int(rng.choice([2, 4]))
    g = int(rng.choice([1, 2, dv]))
    k = int(rng.integers(0, 3))
    m = int(rng.integers(1, 4))
    return CONFIGS[1].with_(batch=1, heads=1, d_k=dk, d_v=dv, group=g, bits=int(rng.choice([2, 3, 4])),
                            mixed_bits=None, scale_mode=str(rng.choice(["dynamic", "persistent"])),
                            scale_dtype=str(rng.choice(["f32", "f16"])), bdr=False, lrb_k=k, lrb_m=m,
                            lrb_eps=0.5, in_dtype=str(rng.choice(["f32", "bf16"])), seed=seed)


@pytest.mark.parametrize("arith", ["f32", "f64"])
def test_vectorized_gdn_bypass_step_matches_scalar_loops(arith):
    """A scalar-loop step (oracle/brute.py, written apart from the vectorized
    code) on tiny shapes over many seeds: codes, steps, bypass factors and the
    readout agree. Merges run between steps as the capacity requires."""
    A = oracle.F32 if arith == "f32" else oracle.F64
    rng = np.random.default_rng(77 if arith == "f32" else 78)
    cases = 3000 if arith == "f32" else 600
    compared = 0
    for case in range(cases):
        w = _tiny_gdn_bypass(rng, 60_000 + case)
        static = static_params(w)
        st = oracle.zero_state(w)
        cap = w.lrb_k + w.lrb_m
        for t in range(1, int(rng.integers(2, 9))):
            if st.n == cap:
                st, _ = oracle.merge(st, w, oracle.F32)
            inp = step_inputs(w, t, static)
            n = st.n
            U = [st.U[0, :, c].tolist() for c in range(n)]
            W = [st.W[0, :, c].tolist() for c in range(n)]
            codes, scales = st.codes[0].tolist(), st.scales[0].astype(float).tolist()
            a = oracle.decay_rows(w, inp, static)[0]
            new, o, d = oracle.step(st, inp, w, A, static)
            c_s, s_s, o_s, x_s, U2, W2 = brute.step_tile(
                codes, scales, w.bits, a, inp["q"][0, 0], inp["k"][0, 0], inp["v"][0, 0], w.model, w.group,
                w.scale_mode, w.scale_dtype, w.trigger, alpha=float(inp["alpha"].ravel()[0]),
                beta=float(inp["beta"].ravel()[0]), mode=arith, U=U, W=W)
            assert np.allclose(o_s, o[0], rtol=1e-9, atol=1e-12)
            if arith == "f32":
                assert np.array_equal(np.array(c_s), new.codes[0]), (case, t)
                assert np.array_equal(np.array(s_s, np.float32), new.scales[0]), (case, t)
                assert np.array_equal(np.array(U2, np.float32).T, new.U[0, :, :n + 1]), (case, t)
                assert np.array_equal(np.array(W2, np.float32).T, new.W[0, :, :n + 1]), (case, t)
                compared += 1
            else:
                # float64 sums may associate differently: the appended w to binary16 rounding
                assert np.allclose(np.array(W2, np.float64).T, new.W[0, :, :n + 1], rtol=2e-3, atol=1e-6)
            st = new
    if arith == "f32":
        assert compared > 5000
