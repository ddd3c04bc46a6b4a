"""GPU parity of the Gated DeltaNet pure-write window ("Low-Bit GDN
Recurrent-State Quantization: Global Gradient-aware Allocation and Pure-Write
Sliding Windows", abstract) against oracle/window.py, teacher-forced: history
codes and steps bit-exact outside the decision windows, the E4M3 window pairs
bit-exact, o_t within rel-L2 1e-4; plus the readout call, attach/restore of
a state with a full window, and the E4M3 conversion over every input class."""
import numpy as np
import pytest

from harness import log, make_state, rel_l2, run_parity, to_device, to_oracle
import oracle
from rsq_workloads import CONFIGS, static_params, step_inputs

pytestmark = pytest.mark.gpu


def _w(**kw):
    d = dict(batch=2, heads=3, d_k=128, d_v=64, group=32, bits=4, mixed_bits=None, scale_mode="persistent",
             scale_dtype="f16", in_dtype="bf16", pw_window=8, seed=717)
    d.update(kw)
    return CONFIGS[1].with_(**d)


@pytest.mark.parametrize("kw", [
    dict(),
    dict(pw_window=1),
    dict(pw_window=3, scale_mode="dynamic"),
    dict(pw_window=16, d_v=128),
    dict(d_k=256, d_v=128, pw_window=5),
    dict(bits=8, group=64, scale_dtype="f32", pw_window=4),
    dict(bits=6, group=16, d_v=32, pw_window=2, in_dtype="f32"),
    dict(d_k=64, group=64, d_v=64, pw_window=6),
    dict(d_k=32, group=128, d_v=128, pw_window=7, scale_dtype="f32"),
    # the general pair transition: eight rows per lane (d_k = 512), and more
    # pairs than four per wavefront (one wavefront, W = 6)
    dict(d_k=512, d_v=32, pw_window=4),
    dict(d_v=32, pw_window=6),
])
def test_window_step_matches_oracle(kw):
    w = _w(**kw)
    log("pw", kw)
    W = w.pw_window
    steps = 2 * W + 6
    tally, st = run_parity(w, steps, check_steps=range(1, steps + 1))
    tally.check()
    assert st.counters() == (steps, W)
    # every step is checked, so the sticky status word holds exactly the bits
    # the oracle raised (a decayed history with tiny binary16 steps can clip)
    assert st.get_status() == tally.oracle_flags


def test_window_cfg1_shape_sampled():
    """The default workload's shape (64 x 16 tiles of 128 x 128) with W = 8,
    sampled tiles over 64 steps."""
    w = CONFIGS[1].with_(pw_window=8)
    rng = np.random.default_rng(3)
    tiles = sorted(int(b) * w.heads + h for b in rng.choice(w.batch, 2, replace=False) for h in range(w.heads))
    tally, st = run_parity(w, 64, check_steps=list(range(1, 12)) + [31, 32, 63, 64], tiles=tiles)
    tally.check()


def test_window_readout_call():
    w = _w()
    tally, st = run_parity(w, 11, check_steps=[11])
    arrs = st.read_tiles()
    inp = step_inputs(w, 12, static_params(w))
    o = st.readout(to_device(inp, w)["q"]).reshape(w.tiles, -1).cpu().numpy()
    t, n = st.counters()
    ost = to_oracle(arrs, w, list(range(w.tiles)), n)
    ost.t = t
    S = oracle.window.state_dense(ost, w)
    q = inp["q"].reshape(w.tiles, -1).astype(np.float64)
    assert rel_l2(o, np.einsum("ti,tij->tj", q, S)) <= 1e-5


def test_attach_restores_a_window_state():
    import torch
    import bit_recurrent_state_rsq_amd as rsq
    w = _w(pw_window=4)
    a = make_state(w)
    sp = static_params(w)
    for t in range(1, 7):
        d = to_device(step_inputs(w, t, sp), w)
        a.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    torch.cuda.synchronize()
    buf = a.buf.clone()
    b = rsq.State(buffer=buf, attach=True, **rsq.config_kwargs_from(w))
    assert b.counters() == (6, 4)
    d = to_device(step_inputs(w, 7, sp), w)
    oa = a.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    ob = b.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(a.buf, b.buf)


# bf16 values around every decision of the E4M3 encoding (OCP E4M3 of
# "Low-Bit GDN Recurrent-State Quantization ...", abstract; reading of its
# rounding and saturation): zeros, the subnormal grid m 2^-9 and its ties,
# the subnormal/normal boundary, ties in the normal range, the largest
# finite value 448, the tie 464 with the NaN pattern above it, and beyond
_E4M3_EDGES = [0.0, 2.0 ** -12, 2.0 ** -10, 2.0 ** -9, 3 * 2.0 ** -10, 5 * 2.0 ** -10, 7 * 2.0 ** -9,
               15 * 2.0 ** -10, 2.0 ** -6, 1.0, 1.0625, 1.1875, 1.25, 3.0, 240.0, 416.0, 432.0, 440.0,
               448.0, 456.0, 464.0, 472.0, 480.0, 496.0, 512.0, 1.0e4, 3.0e38, 1.0e-30]


def test_window_e4m3_edge_cases():
    """The new pair (e4m3(k_t), e4m3(fl(beta_t v_t))) byte for byte against the
    oracle's encoder on inputs that hit every class of the conversion; v also
    carries infinities and NaNs of both signs (v feeds only the pair and the
    readout, so the history stays finite)."""
    import torch
    from oracle.window import fp8_encode, fp8_round
    w = _w(batch=1, heads=1, d_k=128, d_v=128, pw_window=8)
    st = make_state(w)
    edges = np.array(_E4M3_EDGES, np.float32)
    rng = np.random.default_rng(11)
    kv = np.concatenate([edges, -edges])
    k = np.concatenate([kv, (rng.standard_normal(w.d_k - kv.size) * 0.1).astype(np.float32)])
    kb = (k.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)   # bf16 of k (edges are exact)
    vb = kb.copy()
    vb[-6:] = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7FC1, 0xFF81], np.uint16)   # +-inf, NaNs
    qb = (rng.standard_normal(w.d_k).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    dev = lambda bits: torch.from_numpy(bits.astype(np.int16)).cuda().view(torch.bfloat16).reshape(1, 1, -1)
    alpha = torch.full((1, 1), 0.9, dtype=torch.float32, device="cuda")
    beta = torch.ones((1, 1), dtype=torch.float32, device="cuda")
    st.decode_step(dev(qb), dev(kb), dev(vb), alpha, beta)
    torch.cuda.synchronize()
    sec = st._sections[0]
    base = st.tile_offset(0, 0)
    raw = st.buf.view(-1)[: st.nbytes].view(torch.uint8).cpu().numpy()
    u_gpu = raw[base + sec["bypass_u"]: base + sec["bypass_u"] + w.d_k]
    w_gpu = raw[base + sec["bypass_w"]: base + sec["bypass_w"] + w.d_v]
    kf = (kb.astype(np.uint32) << 16).view(np.float32)
    vf = (vb.astype(np.uint32) << 16).view(np.float32)     # fl(1 * v) = v
    with np.errstate(invalid="ignore"):   # (casting the NaN inputs)
        u_ref = fp8_encode(fp8_round(kf))
        w_ref = fp8_encode(fp8_round(vf))
    bad_u = np.nonzero(u_gpu != u_ref)[0]
    bad_w = np.nonzero(w_gpu != w_ref)[0]
    log("e4m3 edges: %d u and %d w bytes differ" % (bad_u.size, bad_w.size))
    assert bad_u.size == 0, [(float(kf[i]), int(u_gpu[i]), int(u_ref[i])) for i in bad_u[:8]]
    assert bad_w.size == 0, [(float(vf[i]), int(w_gpu[i]), int(w_ref[i])) for i in bad_w[:8]]
