"""Pins of reference-yoked scaling (abstract of "When Dynamic Scaling Fails: A
Scale-State Feedback Governs Recurrent-State Quantization in Linear-Attention
and SSM LLMs"): the reference follows the unquantized recurrence exactly, and
codes clip only where the quantized state leaves the reference's range."""
import numpy as np
import pytest

import oracle
from oracle import recurrence as R
from rsq_workloads import CONFIGS, step_inputs, static_params


@pytest.mark.parametrize("ci", [1, 2])
def test_reference_equals_the_fp32_state_path(ci):
    w = CONFIGS[ci].with_(batch=2, heads=2, d_k=32, d_v=32, group=32 if ci == 1 else 32,
                          scale_mode="yoked", bits=4)
    wf = w.with_(bits=32, scale_mode="dynamic")
    static = static_params(w)
    sq, sf = oracle.zero_state(w), oracle.zero_state(wf)
    clipped_seen = 0
    for t in range(1, 40):
        inp = step_inputs(w, t, static)
        sq, oq, dq = oracle.step(sq, inp, w, oracle.F32, static)
        sf, of, _ = oracle.step(sf, inp, wf, oracle.F32, static)
        assert np.array_equal(sq.ref, sf.S32)
        # clipping happens exactly where RNE(y) leaves the code range
        lo, hi, _ = R.qrange(sq.bits[:, None, None])
        rn = np.rint(dq["y"])
        assert np.array_equal(dq["clipped"], (rn < lo) | (rn > hi))
        clipped_seen += int(dq["clipped"].sum())
        if dq["clipped"].any():
            assert sq.flags & R.CLIPPED
    # the scale follows the reference, so the quantized state does leave its range
    assert clipped_seen > 0
