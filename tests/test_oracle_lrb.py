"""Pins of the Low-Rank Bypass: storage accounting against the pages' printed
bits (Tables 2, 6, 8, 9 of "Preserving Updates in Low-Bit Recurrent State
Quantization"), and the merge's rank-k compression against Eckart-Young."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import accounting as acc, recurrence as R
from rsq_workloads import CONFIGS, step_inputs, static_params

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "bits_tables.json")))

# Head shapes are not printed. GDN and RetNet follow (d_k + d_v)/(d_k d_v) = 3/512
# (e.g. d_k = 256, d_v = 512); Mamba2 uses d_state 128 x head_dim 64.
GDN_SHAPE = (256, 512)
MAMBA2_SHAPE = (128, 64)


def test_int4_group32_fp16_scale_is_4_50_bits():
    avg, peak = acc.bits_per_element(4, 32, 16, *GDN_SHAPE)
    assert avg == peak == GOLD["table2_bits"]["INT4"]


@pytest.mark.parametrize("row", GOLD["table8_gdn"]["rows"])
def test_table8_average_bits(row):
    k, m, printed = row
    avg, peak = acc.bits_per_element(4, 32, 16, *GDN_SHAPE, k=k, m=m)
    assert abs(avg - printed) <= 0.005 + 1e-12
    assert abs(peak - GOLD["table8_gdn"]["peak"]) <= 0.005


@pytest.mark.parametrize("row", GOLD["table9"]["rows"])
def test_table9_bits(row):
    model, km, avg_p, peak_p = row
    avg, peak = acc.bits_per_element(4, 32, 16, *GDN_SHAPE, k=1, m=km - 1)
    if model == "GDN":
        assert abs(avg - avg_p) <= 0.005 + 1e-12
        # 6.76 is printed for k+m = 24 where the formula gives 6.75
        assert abs(peak - peak_p) <= (0.0101 if km == 24 else 0.005 + 1e-12)
    else:
        # GLA's printed bits sit 0.06-0.07 above this shape's formula; see
        # test_gla_bits_fit_no_head_shape for why the GLA row stays unpinned
        assert 0.055 < avg_p - avg < 0.07 and 0.055 < peak_p - peak < 0.075


def test_gla_bits_fit_no_head_shape():
    """The GLA entries of Table 6 (k = 1, m = 15: 5.31 / 6.07) and Table 9
    (k + m = 8: 4.94 / 5.31) are not reproduced by the storage formula
    4 bits + scale bits / g + n * 16 (d_k + d_v) / (d_k d_v) at any head shape,
    group size or scale width: the four values need a slope per bypass column
    and an intercept that no (d_k, d_v, g, scale bits) gives together. They sit
    0.06-0.07 bits above the GDN entries at the same k and m, as if a GLA head
    stored something more than its codes, step sizes and fp16 bypass columns,
    which the page does not describe. The GLA storage bits are therefore
    parity unpinned; GDN, RetNet (Tables 6, 8, 9) and Mamba2 (Table 6) are
    pinned above."""
    t6, t9 = GOLD["table6"]["GLA"], [r for r in GOLD["table9"]["rows"] if r[0] == "GLA"][0]
    want = [(1 + (t6["m"] - 1) / 2, t6["avg"]), (1 + t6["m"], t6["peak"]),
            (1 + (t9[1] - 2) / 2, t9[2]), (t9[1], t9[3])]
    sizes = [16, 32, 48, 64, 96, 128, 192, 256, 384, 512, 768, 1024, 2048, 4096]
    fits = []
    for dk in sizes:
        for dv in sizes:
            for g in (8, 16, 32, 64, 128, 256):
                for sb in (8, 16, 32):
                    rho = (dk + dv) / (dk * dv)
                    if all(abs(4 + sb / g + n * 16 * rho - v) <= 0.005 + 1e-9 for n, v in want):
                        fits.append((dk, dv, g, sb))
    assert fits == []
    # while the GDN entries at the same k, m fit the reading's shape
    gdn = GOLD["table6"]["GDN"]
    avg, peak = acc.bits_per_element(4, 32, 16, *GDN_SHAPE, k=gdn["k"], m=gdn["m"])
    assert (round(avg, 2), round(peak, 2)) == (gdn["avg"], gdn["peak"])


def test_table6_bits():
    t6 = GOLD["table6"]
    for name in ("GDN", "RetNet"):
        avg, peak = acc.bits_per_element(4, 32, 16, *GDN_SHAPE, k=t6[name]["k"], m=t6[name]["m"])
        assert abs(avg - t6[name]["avg"]) <= 0.005 and abs(peak - t6[name]["peak"]) <= 0.005
    avg, peak = acc.bits_per_element(4, 32, 16, *MAMBA2_SHAPE, k=1, m=5)
    assert abs(avg - t6["Mamba2"]["avg"]) <= 0.02 and abs(peak - t6["Mamba2"]["peak"]) <= 0.035


def test_memory_reduction_up_to_5_3x():
    _, peak = acc.bits_per_element(4, 32, 16, *GDN_SHAPE, k=1, m=15)
    assert round(32.0 / peak, 1) == GOLD["abstract_memory_reduction"]["value"]


def test_step_bytes_match_the_workload_budget():
    # per-tile bytes per step for the four throughput workloads
    want = {1: 19720, 2: 18308, 3: 55168, 4: 25352}
    for ci, b in want.items():
        w = CONFIGS[ci]
        sb = 2 if w.scale_dtype == "f16" else 4
        inb = 2 if w.in_dtype == "bf16" else 4
        gate = {"retnet": 0, "mamba2": 4, "gdn": 8, "gla": 4 * w.d_k}[w.model]
        bits = oracle.recurrence.tile_bits(w)[: w.heads]
        per = np.mean([acc.step_bytes_per_tile(int(bb), w.group, sb, w.d_k, w.d_v, inb, gate,
                                               w.lrb_k, w.lrb_m) for bb in bits])
        assert per == b


# ---------------------------------------------------------------- merge (Eckart-Young)

def _lrb_workload(**kw):
    d = dict(batch=2, heads=2, d_k=32, d_v=16, group=8, seed=321)
    d.update(kw)
    return CONFIGS[3].with_(**d)


def _run_to_merge(w, T=None):
    static = static_params(w)
    st = oracle.zero_state(w)
    cap = w.lrb_k + w.lrb_m
    merges = []
    t = 0
    while len(merges) < 3:
        t += 1
        st, o, d = oracle.step(st, step_inputs(w, t, static), w, oracle.F32, static)
        if st.n == cap:
            before = st
            st, md = oracle.merge(st, w, oracle.F32)
            merges.append((before, st, md))
    return merges


def test_merge_keeps_the_best_rank_k_residual():
    w = _lrb_workload()
    for before, after, md in _run_to_merge(w):
        R_ = md["R"]
        sv = md["svals"]
        k = w.lrb_k
        for ti in range(R_.shape[0]):
            approx = after.U[ti, :, :k].astype(np.float64) @ after.W[ti, :, :k].astype(np.float64).T
            err = np.linalg.norm(R_[ti] - approx)
            tail = np.sqrt(np.sum(sv[ti, k:] ** 2))
            fp16 = 2.0 ** -10 * np.sum(sv[ti, :k])            # factor storage rounding
            assert err <= (1 + 1e-3) * tail + fp16 + 1e-12
        assert after.n == k
        # each U column's largest-magnitude entry is positive
        U = after.U[:, :, :k]
        idx = np.argmax(np.abs(U), axis=1)
        top = np.take_along_axis(U, idx[:, None, :], axis=1)
        assert np.all(top >= 0)


def test_merge_of_a_rank_k_residual_is_exact():
    w = _lrb_workload(lrb_eps=1e30)        # nothing merges: R = L = U W^T of rank <= n
    st = oracle.zero_state(w)
    st.scales[:] = 1.0                     # the threshold eps_L * s is then huge
    rng = np.random.default_rng(3)
    k = w.lrb_k
    st.U[:, :, :2] = oracle.f16_round(rng.standard_normal((w.tiles, w.d_k, 2)))
    st.W[:, :, :2] = oracle.f16_round(rng.standard_normal((w.tiles, w.d_v, 2)))
    st.n = 2
    after, md = oracle.merge(st, w, oracle.F32)
    L = md["L"].astype(np.float64)
    for ti in range(w.tiles):
        approx = after.U[ti, :, :k].astype(np.float64) @ after.W[ti, :, :k].astype(np.float64).T
        assert np.linalg.norm(L[ti] - approx) <= 2.0 ** -10 * np.linalg.norm(L[ti]) * 4
    assert np.all(after.codes == 0)


def test_merge_threshold_zero_merges_everything_and_infinite_merges_nothing():
    w0 = _lrb_workload(lrb_eps=0.0)
    for before, after, md in _run_to_merge(w0):
        assert np.all(md["M"] | (md["L"] == 0))
        assert np.all(after.U == 0) or np.allclose(md["R"], 0)
    winf = _lrb_workload(lrb_eps=np.inf)
    for before, after, md in _run_to_merge(winf):
        assert not md["M"].any()
        assert np.array_equal(after.codes, before.codes)      # requantizing s_hat alone is idempotent


def test_rank_zero_bypass_drops_the_residual():
    w = _lrb_workload(lrb_k=0)
    for before, after, md in _run_to_merge(w):
        assert after.n == 0 and np.all(after.U == 0) and np.all(after.W == 0)


def test_decode_steps_with_bypass_only_decay_the_state():
    w = _lrb_workload()
    static = static_params(w)
    st = oracle.zero_state(w)
    merges = _run_to_merge(w)
    st = merges[0][1]
    inp = step_inputs(w, 100, static)
    new, o, d = oracle.step(st, inp, w, oracle.F32, static)
    a = oracle.decay_rows(w, inp, static)
    s = np.repeat(st.scales, w.group, axis=2)
    c1 = np.repeat((a[:, :, None] * st.scales).astype(np.float32), w.group, axis=2)
    assert np.array_equal(d["x"], (st.codes.astype(np.float32) * c1).astype(np.float32))
    assert new.n == st.n + 1
    assert np.array_equal(new.U[:, :, st.n], oracle.f16_round(inp["k"].reshape(w.tiles, -1)))
    # the readout includes the bypass: S_t = x + U W^T
    S = d["x"].astype(np.float64) + np.einsum("tic,tjc->tij", new.U[:, :, :new.n].astype(np.float64),
                                              new.W[:, :, :new.n].astype(np.float64))
    assert np.allclose(o, np.einsum("ti,tij->tj", inp["q"].reshape(w.tiles, -1).astype(np.float64), S))
