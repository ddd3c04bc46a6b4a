"""GPU parity of the INT4+Had decode step ("Preserving Updates ...",
Table 2: a Hadamard rotation before INT4) against oracle/hadamard.py,
teacher-forced like the other parity tests (codes and steps bit-exact outside
the decision windows, o_t within rel-L2 1e-4), and of the readout call."""
import numpy as np
import pytest

from harness import log, rel_l2, run_parity, to_device, to_oracle
import oracle
from rsq_workloads import CONFIGS, static_params, step_inputs

pytestmark = pytest.mark.gpu

BASE = {"retnet": CONFIGS[0], "gdn": CONFIGS[1], "mamba2": CONFIGS[2], "gla": CONFIGS[3]}


def _w(model, **kw):
    d = dict(batch=2, heads=3, d_k=128, d_v=64, group=32, bits=4, mixed_bits=None, lrb_k=0, lrb_m=0, bdr=False,
             scale_mode="dynamic", scale_dtype="f16", in_dtype="bf16", hadamard=True, seed=515)
    d.update(kw)
    return BASE[model].with_(**d)


@pytest.mark.parametrize("model,kw", [
    ("retnet", dict()),
    ("mamba2", dict(scale_mode="persistent")),
    ("gla", dict(d_k=256, d_v=128)),
    ("gdn", dict()),
    ("gdn", dict(scale_mode="persistent", d_v=128)),
    ("gdn", dict(bits=8, group=64, scale_dtype="f32")),
    ("mamba2", dict(bits=6, group=16, d_v=32)),
    ("gla", dict(group=8, d_v=32)),
    ("retnet", dict(group=128, d_k=32, d_v=128, in_dtype="f32", scale_dtype="f32")),
])
def test_hadamard_step_matches_oracle(model, kw):
    w = _w(model, **kw)
    log("had", model, kw)
    tally, st = run_parity(w, 24, check_steps=range(1, 25))
    tally.check()
    assert st.get_status() == 0


def test_hadamard_readout_call():
    w = _w("gla")
    tally, st = run_parity(w, 6, check_steps=[6])
    arrs = st.read_tiles()
    inp = step_inputs(w, 7, static_params(w))
    o = st.readout(to_device(inp, w)["q"]).reshape(w.tiles, -1).cpu().numpy()
    ost = to_oracle(arrs, w, list(range(w.tiles)), 0)
    S = oracle.hadamard.dequant(ost, w, oracle.F64)
    q = inp["q"].reshape(w.tiles, -1).astype(np.float64)
    o_ref = np.einsum("ti,tij->tj", q, S)
    assert rel_l2(o, o_ref) <= 1e-5


@pytest.mark.parametrize("ci", [1, 4])
def test_hadamard_at_the_workload_shapes_sampled(ci):
    """The default workload (64 x 16 tiles of 128 x 128) and the mixed-width
    one (512 x 32 tiles, INT8/INT6/INT4 heads) with rotated groups: sampled
    tiles covering every head, checked at a spread of steps."""
    w = CONFIGS[ci].with_(hadamard=True)
    rng = np.random.default_rng([ci, 5])
    rows = rng.choice(w.batch, size=2, replace=False)
    tiles = sorted(int(b) * w.heads + h for b in rows for h in range(w.heads))
    tally, st = run_parity(w, 48, check_steps=[1, 2, 3, 16, 47, 48], tiles=tiles)
    tally.check()
