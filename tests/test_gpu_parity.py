"""GPU parity: the HIP decode step against the CPU oracle, through the C ABI.

Every test is teacher-forced (see harness.py): codes and step sizes bit-exact
outside the 1e-6 decision windows, o_t and the dequantized state within
rel-L2 1e-4 per step. The five workloads run at their full shapes; where the
oracle cannot follow every tile at every step, a seeded sample of tiles that
covers every head (and so every bit width) is checked at a spread of steps.
"""
import numpy as np
import pytest

from harness import (InputPool, Tally, compare, gpu_step, log, make_state, rel_l2, run_parity,
                     sub_inputs, sub_static, sub_workload, tile_bits, to_device, to_oracle)
import oracle
from rsq_workloads import CONFIGS, static_params, step_inputs

pytestmark = pytest.mark.gpu


def _sample_tiles(w, per_head, seed=0):
    rng = np.random.default_rng([seed, w.seed])
    rows = rng.choice(w.batch, size=min(per_head, w.batch), replace=False)
    return sorted(int(b) * w.heads + h for b in rows for h in range(w.heads))


def test_cfg0_retnet_int4_every_step():
    w = CONFIGS[0]
    log("cfg0", w.name)
    tally, st = run_parity(w, w.steps, check_steps=range(1, w.steps + 1))
    tally.check()
    assert st.counters() == (w.steps, 0)
    assert st.get_status() == 0


def test_cfg1_gdn_int4_persistent():
    w = CONFIGS[1]
    log("cfg1", w.name)
    checks = list(range(1, 9)) + list(range(32, w.steps + 1, 64)) + [w.steps]
    tiles = _sample_tiles(w, 4)
    tally, st = run_parity(w, w.steps, check_steps=checks, tiles=tiles)
    tally.check()
    log("cfg1 forgiven", tally.forgiven, "of", tally.elements)


def test_cfg1_gdn_all_tiles_first_steps():
    w = CONFIGS[1]
    tally, st = run_parity(w, 3, check_steps=[1, 2, 3])
    tally.check()


def test_cfg2_mamba2_int8_rows():
    w = CONFIGS[2]
    log("cfg2", w.name)
    pool = InputPool.build(w, 16)
    checks = [1, 2, 3, 100, 500, 1000, 1500, w.steps]
    tally, st = run_parity(w, w.steps, check_steps=checks, tiles=_sample_tiles(w, 2), pool=pool)
    tally.check()


def test_cfg4_gdn_mixed_bits():
    w = CONFIGS[4]
    log("cfg4", w.name)
    pool = InputPool.build(w, 8)
    checks = [1, 2, 3, 64, 512, 1024, 2048, 3000, w.steps]
    tally, st = run_parity(w, w.steps, check_steps=checks, tiles=_sample_tiles(w, 4), pool=pool)
    tally.check()


def test_cfg3_gla_bypass_decode_steps():
    """Decode steps of the bypass workload up to the first merge point."""
    w = CONFIGS[3]
    tally, st = run_parity(w, w.lrb_k + w.lrb_m, check_steps=range(1, w.lrb_k + w.lrb_m + 1),
                           tiles=_sample_tiles(w, 4), merge_check=lambda *a: None)
    tally.check()
    assert st.counters()[1] == w.lrb_k + w.lrb_m


@pytest.mark.parametrize("model", ["retnet", "mamba2", "gla", "gdn"])
def test_fp32_state_matches_oracle_bitwise(model):
    base = {"retnet": CONFIGS[0], "gdn": CONFIGS[1], "mamba2": CONFIGS[2], "gla": CONFIGS[3]}[model]
    w = base.with_(batch=3, heads=2, d_k=128, d_v=64, group=32, bits=32, mixed_bits=None,
                   lrb_k=0, lrb_m=0, bdr=False, scale_mode="dynamic", seed=555)
    tally, st = run_parity(w, 40, check_steps=range(1, 41))
    assert tally.steps == 40


@pytest.mark.parametrize("model,bits,g,mode,sdt", [
    ("gdn", 8, 16, "dynamic", "f32"),
    ("gdn", 6, 32, "persistent", "f16"),
    ("mamba2", 4, 8, "persistent", "f32"),
    ("retnet", 6, 64, "dynamic", "f16"),
    ("gla", 8, 128, "dynamic", "f16"),
    ("gla", 4, 32, "persistent", "f16"),
])
def test_small_variants(model, bits, g, mode, sdt):
    base = {"retnet": CONFIGS[0], "gdn": CONFIGS[1], "mamba2": CONFIGS[2], "gla": CONFIGS[3]}[model]
    dk = 128 if g <= 32 else (64 if g == 64 else 256)
    dv = max(g, 32) * 2 if g < 128 else 128
    w = base.with_(batch=2, heads=3, d_k=dk, d_v=dv, group=g, bits=bits, mixed_bits=None,
                   scale_mode=mode, scale_dtype=sdt, lrb_k=0, lrb_m=0, bdr=False, seed=777 + bits)
    tally, st = run_parity(w, 24, check_steps=range(1, 25))
    tally.check()


@pytest.mark.parametrize("model", ["gdn", "gla"])
def test_bdr_without_bypass(model):
    base = CONFIGS[1] if model == "gdn" else CONFIGS[3]
    w = base.with_(batch=2, heads=4, d_k=128, d_v=64, group=32, bits=4, bdr=True, bdr_eps=0.3,
                   lrb_k=0, lrb_m=0, scale_mode="dynamic", scale_dtype="f16", seed=991)
    tally, st = run_parity(w, 32, check_steps=range(1, 33))
    tally.check()


@pytest.mark.parametrize("model", ["gdn", "mamba2"])
def test_yoked_scales(model):
    base = CONFIGS[1] if model == "gdn" else CONFIGS[2]
    w = base.with_(batch=2, heads=2, d_k=128, d_v=64, group=32, bits=4, scale_mode="yoked",
                   scale_dtype="f16", lrb_k=0, lrb_m=0, seed=4321, bdr=(model == "gdn"))
    tally, st = run_parity(w, 40, check_steps=range(1, 41))
    tally.check()
    from bit_recurrent_state_rsq_amd import _abi
    assert st.get_status() & _abi.F_CLIPPED      # the scale follows the reference, codes clip


def test_allocated_head_widths_drive_the_decode_step():
    """Widths from rsq_allocate_head_bits (Mamba2 decays, mean 5 bits: a mix
    of INT4, INT6 and INT8 heads) run through the decode step bit-exact."""
    from bit_recurrent_state_rsq_amd import allocate_head_bits
    base = CONFIGS[2]
    w = base.with_(batch=4, heads=16, d_k=128, d_v=64, group=64, mixed_bits=None, seed=2468)
    c = np.exp(static_params(w)["a_log"])
    d = ((np.exp(-0.002 * c) - np.exp(-0.2 * c)) / (2 * c * 0.099)).astype(np.float32)
    rho = np.sqrt(1.0 / (1.0 - d.astype(np.float64))).astype(np.float32)
    rho[:2] *= 8.0                                   # two wide-range heads earn INT8
    hb = allocate_head_bits(d, rho, 5.0)
    log("allocated widths", hb)
    assert {4, 6, 8} <= set(hb)
    w = w.with_(head_bits=tuple(hb))
    tally, st = run_parity(w, 48, check_steps=list(range(1, 9)) + [24, 47, 48])
    tally.check()


def test_gdn_with_d_k_256_crosses_wavefronts():
    w = CONFIGS[1].with_(batch=2, heads=2, d_k=256, d_v=64, seed=31)
    tally, st = run_parity(w, 16, check_steps=range(1, 17))
    tally.check()


def test_readout_call_matches_dequantized_state():
    import torch
    w = CONFIGS[4].with_(batch=4)
    tally, st = run_parity(w, 10, check_steps=[10], tiles=list(range(w.tiles)))
    arrs = st.read_tiles()
    inp = step_inputs(w, 11, static_params(w))
    dev = to_device(inp, w)
    o = st.readout(dev["q"]).reshape(w.tiles, -1).cpu().numpy()
    ost = to_oracle(arrs, w, list(range(w.tiles)), 0)
    o_ref = oracle.readout(ost, inp["q"], w)
    assert rel_l2(o, o_ref) <= 1e-5


def test_nonfinite_input_sets_the_status_flag():
    import torch
    from bit_recurrent_state_rsq_amd import _abi
    w = CONFIGS[1].with_(batch=1, heads=2)
    st = make_state(w)
    inp = step_inputs(w, 1, static_params(w))
    dev = to_device(inp, w)
    gpu_step(st, dev)
    assert st.get_status() == 0
    dev["v"][0, 1, 3] = float("inf")
    gpu_step(st, dev)
    assert st.get_status() & _abi.F_NONFINITE
    assert st.get_status() == 0          # reading clears the word


def test_attach_restores_a_saved_state():
    import torch
    import bit_recurrent_state_rsq_amd as rsq
    w = CONFIGS[4].with_(batch=2)
    st = make_state(w)
    static = static_params(w)
    for t in range(1, 6):
        gpu_step(st, to_device(step_inputs(w, t, static), w))
    saved = st.buf.clone()
    kw = dict(st.kw)
    st2 = rsq.State(buffer=saved, attach=True, **kw)
    assert st2.counters() == (5, 0)
    d6 = to_device(step_inputs(w, 6, static), w)
    o1 = gpu_step(st, d6)
    o2 = gpu_step(st2, d6)
    assert torch.equal(o1, o2)
    assert torch.equal(st.buf, saved)
    # a different configuration does not attach
    with pytest.raises(rsq.Error) as e:
        rsq.State(buffer=saved, attach=True, **dict(kw, group=16))
    assert e.value.code in (rsq._abi.RSQ_E_ATTACH, rsq._abi.RSQ_E_BUFFER)


def test_full_bypass_refuses_a_decode_step():
    import bit_recurrent_state_rsq_amd as rsq
    w = CONFIGS[3].with_(batch=1, heads=2, lrb_k=1, lrb_m=2)
    st = make_state(w)
    static = static_params(w)
    for t in range(1, 4):
        gpu_step(st, to_device(step_inputs(w, t, static), w))
    with pytest.raises(rsq.Error) as e:
        gpu_step(st, to_device(step_inputs(w, 4, static), w))
    assert e.value.code == rsq._abi.RSQ_E_BYPASS_FULL


def test_bound_and_timed_steps_match_the_plain_call():
    """State.bind_step and rsq_decode_step_timed run the same step as rsq_decode_step."""
    import ctypes
    import torch
    w = CONFIGS[1].with_(batch=4)
    a, b = make_state(w), make_state(w)
    static = static_params(w)
    rt = ctypes.CDLL("libamdhip64.so.7")
    P = ctypes.c_void_p
    rt.hipEventCreate.argtypes = [ctypes.POINTER(P)]
    rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
    rt.hipEventDestroy.argtypes = [P]
    ev = [P(), P()]
    for e in ev:
        assert rt.hipEventCreate(ctypes.byref(e)) == 0
    stream = torch.cuda.current_stream()
    try:
        for t in range(1, 5):
            d = to_device(step_inputs(w, t, static), w)
            o1 = gpu_step(a, d)
            o2 = torch.empty_like(o1)
            issue = b.bind_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], out=o2, stream=stream)
            if t % 2:
                issue(ev[0], ev[1])
            else:
                issue()
            torch.cuda.synchronize()
            assert torch.equal(o1, o2)
            assert torch.equal(a.buf, b.buf)
            if t % 2:
                ms = ctypes.c_float()
                assert rt.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
                assert 0.0 < ms.value < 1000.0
        assert a.counters() == b.counters() == (4, 0)
    finally:
        for e in ev:
            rt.hipEventDestroy(e)


def _merge_checker(w, results):
    """Teacher-forced check of rsq_merge_bypass: the oracle merges the GPU's
    pre-merge state of the sampled tiles. Codes and step sizes must match
    outside the decision windows; the GPU's bypass factors must satisfy the
    Eckart-Young bound on the oracle's residual (the factors of a rank-k
    truncation are not unique, their product's error is)."""
    def check(st, t, tiles, tally):
        sw = sub_workload(w, tiles)
        _, n = st.counters()
        pre = st.read_tiles(tiles)
        ost = to_oracle(pre, w, tiles, n)
        ost.bits = tile_bits(w, tiles)
        new, md = oracle.merge(ost, sw, oracle.F32)
        st.merge_bypass()
        post = st.read_tiles(tiles)
        near, gnear = md["near"], md["group_near"]
        diff = post["codes"] != new.codes
        bad = diff & ~near
        sbad = (post["scales"] != new.scales) & ~gnear
        tally.elements += diff.size
        tally.forgiven += int((diff & near).sum())
        tally.mismatch += int(bad.sum()) + int(sbad.sum())
        assert not bad.any(), "merge after step %d: codes differ at %s" % (t, np.argwhere(bad)[:4].tolist())
        assert not sbad.any(), "merge after step %d: step sizes differ" % t
        k = w.lrb_k
        assert st.counters()[1] == k
        U = post["U"].astype(np.float64)
        W = post["W"].astype(np.float64)
        assert not U[:, :, k:].any() and not W[:, :, k:].any(), "columns past k must be empty"
        worst = 0.0
        for ti in range(U.shape[0]):
            sv = md["svals"][ti]
            tail = np.sqrt(np.sum(sv[k:] ** 2))
            err = np.linalg.norm(md["R"][ti] - U[ti, :, :k] @ W[ti, :, :k].T)
            bound = (1 + 1e-3) * tail + 2.0 ** -10 * np.sum(sv[:k]) + 1e-12
            assert err <= bound, "merge after step %d tile %d: |R - UW^T| %g > %g" % (t, ti, err, bound)
            worst = max(worst, err / tail - 1 if tail > 0 else 0.0)
            if k:
                col = U[ti, :, :k]
                top = col[np.argmax(np.abs(col), axis=0), np.arange(k)]
                assert np.all(top >= 0), "U columns must have a positive largest entry"
        results.append(worst)
    return check


def test_cfg3_gla_merges_match_oracle():
    """Decode steps and four bypass merges of the GLA workload, teacher-forced."""
    w = CONFIGS[3]
    steps = w.lrb_k + w.lrb_m + 3 * w.lrb_m
    merges = []
    tally, st = run_parity(w, steps, check_steps=range(1, steps + 1), tiles=_sample_tiles(w, 4),
                           merge_check=_merge_checker(w, merges))
    tally.check()
    assert len(merges) == 4
    log("merge: worst Eckart-Young excess %.2e" % max(merges))


def test_cfg3_gla_full_horizon_with_merges():
    """The full 1024-step GLA workload: every merge checked on the sampled tiles."""
    w = CONFIGS[3]
    merges = []
    checks = [1, 2, 20, 21, 37, 300, 517, 1000, w.steps]
    tally, st = run_parity(w, w.steps, check_steps=checks, tiles=_sample_tiles(w, 2),
                           merge_check=_merge_checker(w, merges))
    tally.check()
    assert len(merges) == (w.steps - w.lrb_k) // w.lrb_m
    log("%d merges, worst Eckart-Young excess %.2e" % (len(merges), max(merges)))


@pytest.mark.parametrize("model,bits,g,mode,sdt,dk,dv,k,m,bdr", [
    ("retnet", 4, 32, "dynamic", "f16", 128, 128, 2, 5, True),
    ("mamba2", 8, 64, "dynamic", "f32", 128, 64, 4, 8, False),
    ("gla", 6, 16, "persistent", "f16", 128, 64, 3, 4, True),
    ("gla", 4, 128, "dynamic", "f16", 64, 128, 1, 3, True),
    ("retnet", 8, 32, "dynamic", "f32", 256, 32, 0, 4, True),
    # the bypass column loop: one wavefront with more than four columns, and d_k > 256
    ("gla", 4, 64, "dynamic", "f16", 64, 64, 2, 6, True),
    ("retnet", 4, 32, "dynamic", "f16", 512, 32, 2, 3, False),
    # more than 8 kept columns: the basis keeps all 17 - 32 bypass columns and
    # Rayleigh-Ritz runs on all threads (two sizes of its unrolled factor)
    ("gla", 4, 32, "dynamic", "f16", 128, 64, 9, 12, True),
    ("gla", 4, 32, "dynamic", "f16", 128, 64, 10, 8, True),
])
def test_merge_variants(model, bits, g, mode, sdt, dk, dv, k, m, bdr):
    base = {"retnet": CONFIGS[0], "mamba2": CONFIGS[2], "gla": CONFIGS[3]}[model]
    w = base.with_(batch=2, heads=3, d_k=dk, d_v=dv, bits=bits, group=g, scale_mode=mode, scale_dtype=sdt,
                   lrb_k=k, lrb_m=m, lrb_eps=0.5, bdr=bdr, bdr_eps=0.5, in_dtype="bf16", mixed_bits=None)
    merges = []
    steps = k + 3 * m
    tally, st = run_parity(w, steps, check_steps=range(1, steps + 1), merge_check=_merge_checker(w, merges))
    tally.check()
    assert len(merges) == 3


def test_decode_steps_replay_from_a_hip_graph():
    """Eight decode steps captured once in a graph (torch.cuda.CUDAGraph over
    the caller's stream) and replayed three times give the same codes, step
    sizes and outputs as 24 eager steps. The host-side step counter advances
    only at capture, so this holds for states whose arithmetic does not read
    it (no bypass, no window)."""
    import torch
    w = CONFIGS[1].with_(batch=4)
    sp = static_params(w)
    pool = [to_device(step_inputs(w, t, sp), w) for t in range(1, 9)]
    eager, graphed = make_state(w), make_state(w)
    outs_e = []
    for rep in range(3):
        for d in pool:
            outs_e.append(gpu_step(eager, d).clone())
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    outs = [torch.empty((w.batch, w.heads, w.d_v), dtype=torch.float32, device="cuda") for _ in pool]
    issues = [graphed.bind_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], out=o, stream=side)
              for d, o in zip(pool, outs)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for issue in issues:
            issue()
    torch.cuda.synchronize()
    # capture recorded the launches without running them
    assert not graphed.read_tiles()["codes"].any()
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for s in range(8):
            assert torch.equal(outs[s], outs_e[8 * rep + s]), "replay %d step %d" % (rep, s)
    a, b = eager.read_tiles(), graphed.read_tiles()
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])


@pytest.mark.parametrize("base,over", [
    (3, dict(batch=2)),                                                      # GLA, rank-4 bypass, m = 16
    (1, dict(batch=2, lrb_k=1, lrb_m=15, lrb_eps=0.5, bdr=True, bdr_eps=0.3)),   # GDN, Table 6's setting
])
def test_readout_call_on_a_bypass_state_mid_cycle(base, over):
    """rsq_readout of a state whose bypass holds columns (k kept by a merge
    plus seven decode steps' appends): o = deq(S)^T q + W (U^T q) against the
    oracle's dense state (codes, steps and the bypass product)."""
    w = CONFIGS[base].with_(**over)
    steps = w.lrb_k + w.lrb_m + 7
    tally, st = run_parity(w, steps, check_steps=[steps], tiles=list(range(w.tiles)))
    t_done, n = st.counters()
    assert n == w.lrb_k + 7
    arrs = st.read_tiles()
    inp = step_inputs(w, steps + 1, static_params(w))
    dev = to_device(inp, w)
    o = st.readout(dev["q"]).reshape(w.tiles, -1).cpu().numpy()
    ost = to_oracle(arrs, w, list(range(w.tiles)), n)
    o_ref = oracle.readout(ost, inp["q"], w)
    assert rel_l2(o, o_ref) <= 1e-5
    # the bypass term matters here: without it the readout is visibly different
    plain = np.einsum("ti,tij->tj", inp["q"].reshape(w.tiles, -1).astype(np.float64),
                      arrs["codes"] * np.repeat(arrs["scales"].astype(np.float64), w.group, axis=2))
    assert rel_l2(plain, o_ref) > 1e-3


@pytest.mark.parametrize("model", ["gdn", "gla"])
def test_fp32_state_free_run_matches_closed_form(model):
    """The fp32 state (bits = 32) runs 48 steps on its own and is compared with
    the closed form of the unrolled recurrence (ordered product for GDN) in
    float64: rel-L2 within 1e-4 per step and 1e-3 at the end."""
    from oracle import closed_form as cf
    base = CONFIGS[1] if model == "gdn" else CONFIGS[3]
    w = base.with_(batch=2, heads=2, d_k=128, d_v=64, group=32, bits=32, mixed_bits=None, lrb_k=0, lrb_m=0,
                   bdr=False, scale_mode="dynamic", seed=808)
    st = make_state(w)
    sp = static_params(w)
    inps = []
    for t in range(1, 49):
        inp = step_inputs(w, t, sp)
        inps.append(inp)
        o = gpu_step(st, to_device(inp, w)).reshape(w.tiles, -1).cpu().numpy()
        if t in (1, 2, 8, 24, 48):
            S32 = st.read_tiles()["S32"]
            for tile in range(w.tiles):
                b, h = divmod(tile, w.heads)
                k_seq = [i["k"][b, h] for i in inps]
                v_seq = [i["v"][b, h] for i in inps]
                if model == "gdn":
                    S = cf.unrolled_gdn([i["alpha"][b, h] for i in inps], [i["beta"][b, h] for i in inps],
                                        k_seq, v_seq)
                else:
                    S = cf.unrolled_diag([i["alpha"][b, h] for i in inps], k_seq, v_seq)
                tol = 1e-4 if t < 48 else 1e-3
                assert rel_l2(S32[tile], S) <= tol, (t, tile, rel_l2(S32[tile], S))
                assert rel_l2(o[tile], cf.readout(S, inp["q"][b, h])) <= tol


def test_bypass_steps_refuse_graph_capture():
    """A bypass state's step takes its column from the host handle, so
    capturing it in a graph is refused (RSQ_E_UNSUPPORTED); outside a capture
    the same call runs."""
    import torch
    import bit_recurrent_state_rsq_amd as rsq
    w = CONFIGS[3].with_(batch=1, heads=2)
    st = make_state(w)
    d = to_device(step_inputs(w, 1, static_params(w)), w)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(rsq.Error) as e:
        with torch.cuda.graph(g, stream=side):
            st.decode_step(d["q"], d["k"], d["v"], d["alpha"], None, stream=side)
    assert e.value.code == rsq._abi.RSQ_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert st.counters() == (0, 0)
    gpu_step(st, d)
    assert st.counters() == (1, 1)
