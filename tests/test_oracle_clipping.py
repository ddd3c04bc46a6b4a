"""Where codes clip under persistent binary16 step sizes (the scale policy of
the abstract of "When Dynamic Scaling Fails ...", as the Gated DeltaNet
workloads run it).

A group's new step is s' = fp16(m / qmax) when its maximum m outgrows the
covered range, else the old one. For a normal binary16 s' the rounding is
relative (at most 2^-11), so the largest element lands at most
qmax (1 + 2^-11) (1 + 2^-24) < qmax + 1/2 from zero in code units and no code
leaves the range. A subnormal s' (below 2^-14) has an absolute spacing of
2^-24, so m / qmax can round down by far more than 2^-11 of itself and the
largest elements then clip. That happens only in groups whose maximum is
tiny, i.e. on a fresh state's first steps, in rows with a tiny key. These
tests pin that: on the workloads' own inputs every clipped element sits in
a group with a subnormal step, and a constructed subnormal case clips
exactly as the arithmetic says."""
import numpy as np
import pytest

import oracle
from oracle import recurrence as R
from rsq_workloads import CONFIGS, head_bits_for, static_params, step_inputs

SUBNORMAL = 2.0 ** -14


@pytest.mark.parametrize("ci,tiles,steps", [(1, 16, 48), (4, 32, 24)])
def test_clipping_happens_only_in_groups_with_a_subnormal_step(ci, tiles, steps):
    w = CONFIGS[ci]
    sw = w.with_(batch=1, heads=tiles, mixed_bits=None, head_bits=None)
    sp = static_params(sw)
    st = oracle.zero_state(sw)
    st.bits = head_bits_for(w)[np.arange(tiles) % w.heads].astype(np.int32)
    clipped = 0
    for t in range(1, steps + 1):
        st, o, d = oracle.step(st, step_inputs(sw, t, sp), sw, oracle.F32, sp)
        c = d["clipped"]
        if c.any():
            s_full = np.repeat(d["s_new"], w.group, axis=2)
            assert np.all(s_full[c] < SUBNORMAL), "a clipped element has a normal binary16 step"
            assert bool(st.flags & R.CLIPPED)
            clipped += int(c.sum())
    # and it is rare: at most a few elements per million over these steps
    assert clipped <= 5e-6 * steps * sw.tiles * w.d_k * w.d_v


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_normal_steps_never_clip(bits):
    """Random groups at every binary16 exponent from 2^-14 up: the persistent
    and dynamic rules never produce an out-of-range code."""
    rng = np.random.default_rng(bits)
    qmax = 2 ** (bits - 1) - 1
    for e in range(-14, 15):
        m = np.float32(qmax * 2.0 ** e) * rng.uniform(1.0, 2.0, size=(64, 1, 1)).astype(np.float32)
        x = (m * rng.uniform(-1, 1, size=(64, 1, 32))).astype(np.float32)
        x[:, :, 0] = m[:, :, 0]                       # the maximum is present
        w = CONFIGS[1].with_(batch=1, heads=64, d_k=1, d_v=32, group=32, bits=bits, scale_mode="dynamic")
        s_new, _, _ = R.scale_rule(np.abs(x).max(axis=2, keepdims=True), np.zeros((64, 1, 1), np.float32),
                                   np.full((64, 1, 1), qmax), w, oracle.F32)
        assert np.all(s_new >= SUBNORMAL)
        c, y, clipped = R.quantize_group_codes(x, np.repeat(s_new, 32, axis=2), np.full((64, 1, 1), bits), oracle.F32)
        assert not clipped.any() and np.all(np.abs(y) <= qmax + 0.5)


def test_a_subnormal_step_that_rounds_down_clips():
    """m / qmax = 1.45 * 2^-24 rounds to the binary16 subnormal 2^-24, so the
    maximum sits at 1.45 qmax code units: it clips to qmax."""
    qmax = 7
    m = np.float32(1.45 * 2.0 ** -24 * qmax)
    x = np.array([[[m, -m / 2, 0.0, m / 8] + [0.0] * 28]], np.float32)
    w = CONFIGS[1].with_(batch=1, heads=1, d_k=1, d_v=32, group=32, bits=4, scale_mode="dynamic")
    s_new, _, _ = R.scale_rule(np.abs(x).max(axis=2, keepdims=True), np.zeros((1, 1, 1), np.float32),
                               np.full((1, 1, 1), qmax), w, oracle.F32)
    assert s_new[0, 0, 0] == np.float32(2.0 ** -24)
    c, y, clipped = R.quantize_group_codes(x, np.repeat(s_new, 32, axis=2), np.full((1, 1, 1), 4), oracle.F32)
    assert clipped[0, 0, 0] and c[0, 0, 0] == qmax
    assert c[0, 0, 1] == -5 and not clipped[0, 0, 1]     # -0.725 qmax = -5.075 -> -5
