"""GPU parity of the decode step's less common settings, against the CPU oracle.

The workload-shaped tests leave some forms of the staged decode step
unreached: RetNet's gamma rows with bf16 inputs, fp32 inputs with fp32 steps,
6- and 8-bit codes with 32-column groups, and a persistent trigger above 1,
under which codes can leave the range and are clipped (the only case where
the clamp runs with normal steps). Every step is checked: codes and step
sizes bit-exact outside the 1e-6 decision windows, o_t within rel-L2 1e-4,
the same teacher-forced protocol as the other parity tests.
"""
import pytest

from harness import log, run_parity
from rsq_workloads import CONFIGS

pytestmark = pytest.mark.gpu

_BASE = {"retnet": CONFIGS[0], "gdn": CONFIGS[1], "mamba2": CONFIGS[2], "gla": CONFIGS[3]}


@pytest.mark.parametrize("model,bits,g,mode,sdt,idt,dk,dv,trigger", [
    ("retnet", 8, 32, "dynamic", "f16", "bf16", 128, 64, 1.0),
    ("retnet", 6, 64, "dynamic", "f32", "f32", 128, 128, 1.0),
    ("mamba2", 8, 64, "dynamic", "f32", "f32", 128, 64, 1.0),
    ("gla", 6, 32, "persistent", "f16", "bf16", 256, 128, 1.0),
    ("gla", 4, 32, "persistent", "f16", "bf16", 128, 64, 1.5),
    ("mamba2", 8, 32, "persistent", "f16", "bf16", 128, 64, 1.5),
    ("gdn", 4, 32, "persistent", "f16", "bf16", 128, 128, 1.5),
])
def test_less_common_settings(model, bits, g, mode, sdt, idt, dk, dv, trigger):
    w = _BASE[model].with_(batch=2, heads=3, d_k=dk, d_v=dv, group=g, bits=bits, mixed_bits=None,
                           scale_mode=mode, scale_dtype=sdt, in_dtype=idt, trigger=trigger, lrb_k=0, lrb_m=0,
                           bdr=False, seed=4242 + bits)
    steps = 24
    tally, st = run_parity(w, steps, check_steps=range(1, steps + 1))
    tally.check()
    assert tally.steps == steps
    log("%s %d-bit g%d %s trigger %g: %d elements, %d forgiven" % (model, bits, g, mode, trigger, tally.elements,
                                                                  tally.forgiven))
