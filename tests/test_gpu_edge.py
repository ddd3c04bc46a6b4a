"""GPU parity on degenerate inputs: the HIP decode step against the CPU oracle.

The workloads' seeded inputs with one edit applied at chosen steps:
  * zero updates: k = v = 0, so a fresh state stays at zero with zero step
    sizes, then grows from them when the inputs come back;
  * zero decay: the transition A_t = 0 drops the whole state, leaving the update;
  * decay underflow: a subnormal gate, so that the folded dequantization factor
    a s is subnormal and the step takes its exact long form;
  * identity (Gated DeltaNet): alpha = 1 and beta = 0, so the recurrence is the
    identity and a dynamic requantization must reproduce the stored codes;
  * large values: v scaled by 2^12, far up the binary16 step-size range.

Each case is compared step by step under the same teacher-forced protocol as
the other parity tests (codes and step sizes bit-exact outside the 1e-6
decision windows, o_t within rel-L2 1e-4).
"""
import numpy as np
import pytest

from harness import log, run_parity
from rsq_workloads import CONFIGS, static_params, step_inputs

pytestmark = pytest.mark.gpu

_BASE = {"retnet": CONFIGS[0], "gdn": CONFIGS[1], "mamba2": CONFIGS[2], "gla": CONFIGS[3]}


def _set(inp, name, vals):
    """Replace input `name` by float32 `vals` (bf16-exact), bit patterns too."""
    vals = np.ascontiguousarray(vals, np.float32)
    inp[name] = vals
    if name + "_bits" in inp:
        inp[name + "_bits"] = (vals.view(np.uint32) >> 16).astype(np.uint16)


def _zero_updates(inp, t):
    if t <= 6:
        _set(inp, "k", np.zeros_like(inp["k"]))
        _set(inp, "v", np.zeros_like(inp["v"]))


def _zero_decay(inp, t):
    if t % 3 == 0:
        inp["alpha"] = np.zeros_like(inp["alpha"])


def _decay_underflow(inp, t):
    if t % 4 == 0:
        inp["alpha"] = np.full_like(inp["alpha"], np.float32(2.0 ** -140))


def _identity(inp, t):
    if t > 4:
        inp["alpha"] = np.ones_like(inp["alpha"])
        inp["beta"] = np.zeros_like(inp["beta"])


def _large_values(inp, t):
    _set(inp, "v", inp["v"] * np.float32(4096.0))


_EDITS = {"zero_updates": _zero_updates, "zero_decay": _zero_decay, "decay_underflow": _decay_underflow,
          "identity": _identity, "large_values": _large_values}


class EditedInputs:
    """The workload's seeded inputs with an edit applied (an InputPool stand-in)."""

    def __init__(self, w, edit):
        self.w, self.edit, self.static = w, edit, static_params(w)

    def at(self, t):
        inp = step_inputs(self.w, t, self.static)
        self.edit(inp, t)
        return inp


@pytest.mark.parametrize("model,bits,g,mode,sdt,edit", [
    ("retnet", 4, 32, "dynamic", "f16", "zero_updates"),
    ("gdn", 4, 32, "persistent", "f16", "zero_updates"),
    ("mamba2", 8, 64, "dynamic", "f32", "zero_updates"),
    ("gla", 4, 32, "dynamic", "f16", "zero_decay"),
    ("gdn", 4, 32, "persistent", "f16", "zero_decay"),
    ("mamba2", 6, 32, "persistent", "f16", "decay_underflow"),
    ("gdn", 6, 32, "dynamic", "f32", "decay_underflow"),
    ("gla", 6, 64, "dynamic", "f32", "decay_underflow"),
    ("gdn", 4, 32, "dynamic", "f16", "identity"),
    ("gdn", 4, 32, "persistent", "f16", "large_values"),
])
def test_degenerate_inputs(model, bits, g, mode, sdt, edit):
    w = _BASE[model].with_(batch=2, heads=2, d_k=128, d_v=64, group=g, bits=bits, mixed_bits=None,
                           scale_mode=mode, scale_dtype=sdt, lrb_k=0, lrb_m=0, bdr=False, seed=2024 + bits)
    steps = 16
    tally, st = run_parity(w, steps, check_steps=range(1, steps + 1), pool=EditedInputs(w, _EDITS[edit]))
    tally.check()
    assert tally.steps == steps
    log("%s %s: %d elements, %d forgiven" % (model, edit, tally.elements, tally.forgiven))


def test_identity_steps_keep_the_codes():
    """alpha = 1, beta = 0 under dynamic scales: every stored code and step
    size comes back unchanged (requantizing a dequantized state is exact)."""
    w = _BASE["gdn"].with_(batch=2, heads=2, d_k=128, d_v=64, group=32, bits=4, mixed_bits=None,
                           scale_mode="dynamic", scale_dtype="f16", lrb_k=0, lrb_m=0, bdr=False, seed=77)
    pool = EditedInputs(w, _identity)
    tally, st = run_parity(w, 4, check_steps=[4], pool=pool)
    tiles = list(range(w.tiles))
    before = st.read_tiles(tiles)
    from harness import gpu_step, to_device
    for t in range(5, 9):
        gpu_step(st, to_device(pool.at(t), w))
    after = st.read_tiles(tiles)
    assert np.array_equal(before["codes"], after["codes"])
    assert np.array_equal(before["scales"], after["scales"])
