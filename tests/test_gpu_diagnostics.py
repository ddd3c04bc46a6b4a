"""GPU parity of the error-accounting step (rsq_decode_step_diag) against the
oracle's accounting (oracle/diagnostics.py), teacher-forced like the decode
parity tests: before each step the GPU state and accumulators are read back,
the oracle advances both from them, and the results are compared.

Accumulator planes, ratios and counters are bit-exact except at elements
whose code decision lies in the oracle's 1e-6 decision window (`near`),
where the two sides may legitimately round differently."""
import numpy as np
import pytest

from harness import Tally, compare, log, make_state, to_device, to_oracle
import oracle
from oracle import diagnostics as dg
from rsq_workloads import CONFIGS, static_params, step_inputs

pytestmark = pytest.mark.gpu


def _w(model, **kw):
    base = {"retnet": CONFIGS[0], "gdn": CONFIGS[1], "mamba2": CONFIGS[2], "gla": CONFIGS[3]}[model]
    d = dict(batch=2, heads=2, d_k=128, d_v=64, group=32, bits=4, mixed_bits=None, lrb_k=0, lrb_m=0,
             bdr=False, scale_mode="dynamic", scale_dtype="f16", seed=4242)
    d.update(kw)
    return base.with_(**d)


def _run(w, steps):
    import bit_recurrent_state_rsq_amd as rsq
    st = make_state(w)
    ea = rsq.ErrorAccounting(st)
    sp = static_params(w)
    tiles = list(range(w.tiles))
    tally = Tally()
    worst = 0
    for t in range(1, steps + 1):
        inp = step_inputs(w, t, sp)
        dev = to_device(inp, w)
        pre = st.read_tiles(tiles)
        ost = to_oracle(pre, w, tiles, 0)
        acc0 = {p: ea.plane(p) for p in dg.PLANES}
        cnt0 = ea.count_table().astype(np.int64)
        new, o_ref, diag = oracle.step(ost, inp, w, oracle.F32, sp)
        o = ea.step(dev["q"], dev["k"], dev["v"], dev.get("alpha"), dev.get("beta"))
        post = st.read_tiles(tiles)
        compare(post, new, diag, o.reshape(w.tiles, -1).cpu().numpy(), o_ref, w, tally, what="step %d" % t)
        cnt = cnt0.copy()
        acc, ratio = dg.step_diagnostics(acc0, cnt, new, diag, inp, w, oracle.F32, sp)
        near = diag["near"]
        for p in dg.PLANES:
            g = ea.plane(p)
            bad = (g != acc[p]) & ~near
            assert not bad.any(), "step %d plane %s differs at %s" % (t, p, np.argwhere(bad)[:3].tolist())
        gr = ea.ratios()
        bad = (gr != ratio) & ~near
        assert not bad.any(), "step %d ratio differs at %s" % (t, np.argwhere(bad)[:3].tolist())
        gc = ea.count_table().astype(np.int64)
        slack = near.reshape(w.tiles, -1).sum(axis=1)
        assert np.all(np.abs(gc - cnt) <= slack[:, None]), "step %d counts %s vs %s" % (t, gc, cnt)
        worst = max(worst, int(slack.max()))
    tally.check()
    return st, ea, worst


@pytest.mark.parametrize("model,kw", [
    ("retnet", dict(gamma=0.97)),
    ("mamba2", dict(bits=8, group=64, scale_dtype="f32", in_dtype="bf16")),
    ("gla", dict(bdr=True, bdr_eps=0.3)),
    ("gdn", dict(scale_mode="persistent")),
    ("gdn", dict(bits=6, group=16, d_k=128, d_v=32)),
])
def test_accounting_matches_oracle(model, kw):
    w = _w(model, **kw)
    log("diag", model, kw)
    st, ea, worst = _run(w, 20)
    c = ea.count_table()
    assert c[:, 0].sum() > 0 and np.all(c[:, 1] + c[:, 2] == c[:, 0])
    log("  counts", c.sum(axis=0).tolist(), "gains", np.round(ea.gains().mean(axis=0), 3).tolist())


def test_accounting_step_advances_the_state_like_the_plain_step():
    import torch
    import bit_recurrent_state_rsq_amd as rsq
    w = _w("gla", bdr=True, batch=3)
    a, b = make_state(w), make_state(w)
    ea = rsq.ErrorAccounting(b, keep_ratio=False)
    sp = static_params(w)
    for t in range(1, 9):
        dev = to_device(step_inputs(w, t, sp), w)
        oa = a.decode_step(dev["q"], dev["k"], dev["v"], dev.get("alpha"), dev.get("beta"))
        ob = ea.step(dev["q"], dev["k"], dev["v"], dev.get("alpha"), dev.get("beta"))
        assert torch.equal(oa, ob)
    torch.cuda.synchronize()
    assert torch.equal(a.buf, b.buf)


@pytest.mark.parametrize("kw", [dict(bits=32), dict(lrb_k=2, lrb_m=4), dict(scale_mode="yoked")])
def test_accounting_rejects_unsupported_states(kw):
    import bit_recurrent_state_rsq_amd as rsq
    w = _w("gla", **kw)
    st = make_state(w)
    ea = rsq.ErrorAccounting(st)
    dev = to_device(step_inputs(w, 1, static_params(w)), w)
    with pytest.raises(rsq.Error):
        ea.step(dev["q"], dev["k"], dev["v"], dev.get("alpha"), dev.get("beta"))
