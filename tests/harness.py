"""GPU-vs-oracle parity harness (test infrastructure).

Teacher-forced protocol: before a checked step, the GPU state of the sampled
tiles is read back and the oracle runs the same step from it on the CPU (the
canonical fp32 chain); after the GPU step the two results are compared.

  * codes must be bit-exact except at elements whose pre-rounding value lies
    within 1e-6 of a decision boundary (the oracle reports them as `near`);
  * stored step sizes must be bit-exact except in groups the oracle marks;
  * the forgiven count must stay at or below 1e-5 of the compared elements;
  * o_t and the dequantized state must agree to rel-L2 <= 1e-4.

Because the next step starts from the GPU's state, forgiven elements are
adopted automatically (reconciliation).
"""
import sys

import numpy as np

import oracle
from rsq_workloads import head_bits_for, static_params, step_inputs, InputPool

REL_STEP = 1e-4
REL_HORIZON = 1e-3
FORGIVEN_MAX = 1e-5


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / nb if nb > 0 else np.linalg.norm(a)


def make_state(w, **over):
    import bit_recurrent_state_rsq_amd as rsq
    hb = head_bits_for(w) if (w.mixed_bits or w.head_bits) else None
    kw = rsq.config_kwargs_from(w, head_bits=hb)
    kw.update(over)
    return rsq.State(**kw)


def to_device(inp, w):
    import torch
    dev = "cuda"
    out = {}
    for name in ("q", "k", "v"):
        if w.in_dtype == "bf16":
            bits = np.ascontiguousarray(inp[name + "_bits"]).view(np.int16)
            out[name] = torch.from_numpy(bits).to(dev).view(torch.bfloat16)
        else:
            out[name] = torch.from_numpy(np.ascontiguousarray(inp[name], np.float32)).to(dev)
    for name in ("alpha", "beta"):
        if name in inp:
            out[name] = torch.from_numpy(np.ascontiguousarray(inp[name], np.float32)).to(dev)
    return out


def gpu_step(st, dev_inp):
    return st.decode_step(dev_inp["q"], dev_inp["k"], dev_inp["v"], dev_inp.get("alpha"), dev_inp.get("beta"))


def sub_workload(w, tiles):
    return w.with_(batch=1, heads=len(tiles), mixed_bits=None, head_bits=None)


def sub_inputs(inp, w, tiles):
    b = np.asarray(tiles) // w.heads
    h = np.asarray(tiles) % w.heads
    out = {}
    for name in ("q", "k", "v", "alpha", "beta"):
        if name in inp:
            out[name] = np.asarray(inp[name])[b, h][None]
    return out


def sub_static(w, tiles):
    sp = static_params(w)
    out = {}
    if "gamma" in sp:
        out["gamma"] = np.asarray(sp["gamma"])[np.asarray(tiles) % w.heads]
    return out


def tile_bits(w, tiles):
    hb = head_bits_for(w)
    return hb[np.asarray(tiles) % w.heads].astype(np.int32)


def to_oracle(arrs, w, tiles, n):
    bits = tile_bits(w, tiles)
    if "S32" in arrs:
        st = oracle.OState(codes=np.zeros_like(arrs["S32"], dtype=np.int32),
                           scales=np.zeros((len(tiles), w.d_k, w.d_v // w.group), np.float32),
                           bits=bits, S32=arrs["S32"].copy())
    else:
        st = oracle.OState(codes=arrs["codes"].copy(), scales=arrs["scales"].copy(), bits=bits)
    if "U" in arrs:
        st.U, st.W, st.n = arrs["U"].copy(), arrs["W"].copy(), n
    if "ref" in arrs:
        st.ref = arrs["ref"].copy()
    return st


class Tally:
    def __init__(self):
        self.elements = 0
        self.forgiven = 0
        self.mismatch = 0
        self.steps = 0
        self.oracle_flags = 0   # status bits the oracle raised on the checked steps

    def check(self):
        assert self.mismatch == 0, "%d code/scale mismatches outside the decision windows" % self.mismatch
        assert self.forgiven <= FORGIVEN_MAX * max(self.elements, 1), \
            "forgiven %d of %d elements" % (self.forgiven, self.elements)


def compare(post, new, diag, o_gpu, o_ref, w, tally, what=""):
    """Compare one checked step. `post` GPU arrays, `new` oracle OState."""
    tally.oracle_flags |= int(getattr(new, "flags", 0))
    if "S32" in post:
        assert np.array_equal(post["S32"], new.S32.astype(np.float32)), what + " fp32 state differs"
        assert rel_l2(o_gpu, o_ref) <= REL_STEP, what + " o rel-L2 %g" % rel_l2(o_gpu, o_ref)
        tally.steps += 1
        return
    near = diag["near"]
    gnear = diag["group_near"]
    diff = post["codes"] != new.codes
    bad = diff & ~near
    sdiff = post["scales"] != new.scales
    sbad = sdiff & ~gnear
    tally.elements += diff.size
    tally.forgiven += int((diff & near).sum())
    tally.mismatch += int(bad.sum()) + int(sbad.sum())
    if bad.any() or sbad.any():
        idx = np.argwhere(bad)[:5] if bad.any() else np.argwhere(sbad)[:5]
        log(what, "mismatch at", idx.tolist(), "gpu", post["codes"][tuple(idx[0])] if bad.any() else None,
            "oracle", new.codes[tuple(idx[0])] if bad.any() else None)
        if bad.any():
            t, i, j = idx[0]
            log("  x", diag["x"][t, i, j], "y", diag["y"][t, i, j], "s_new", new.scales[t, i, j // w.group],
                "gpu scale", post["scales"][t, i, j // w.group])
    if "ref" in post:
        assert np.array_equal(post["ref"], new.ref), what + " yoked reference differs"
    if "U" in post:
        n = new.n
        assert np.array_equal(post["U"][:, :, :n], new.U[:, :, :n]), what + " bypass U differs"
        assert np.array_equal(post["W"][:, :, :n], new.W[:, :, :n]), what + " bypass W differs"
    r = rel_l2(o_gpu, o_ref)
    assert r <= REL_STEP, what + " o rel-L2 %g" % r
    tally.steps += 1
    assert tally.mismatch == 0, what + " %d mismatches" % tally.mismatch


def run_parity(w, steps, check_steps, tiles=None, pool=None, st=None, merge_check=None):
    """Run `steps` GPU decode steps of workload w; teacher-force-check the steps
    in `check_steps` on `tiles` (default: all). Returns the tally and the state."""
    import torch
    T = w.tiles
    tiles = list(range(T)) if tiles is None else list(tiles)
    st = make_state(w) if st is None else st
    sw = sub_workload(w, tiles)
    ss = sub_static(w, tiles)
    static = static_params(w)
    tally = Tally()
    check_steps = set(check_steps)
    cap = w.lrb_k + w.lrb_m if w.lrb_m else 0
    for t in range(1, steps + 1):
        inp = pool.at(t) if pool is not None else step_inputs(w, t, static)
        dev = to_device(inp, w)
        if t in check_steps:
            t_done, n = st.counters()
            pre = st.read_tiles(tiles)
            ost = to_oracle(pre, w, tiles, n)
            ost.t = t_done
            ost.bits = tile_bits(w, tiles)
            ostep = (oracle.hadamard.step if w.hadamard else oracle.window.step if w.pw_window
                     else oracle.step)
            new, o_ref, diag = ostep(ost, sub_inputs(inp, w, tiles), sw, oracle.F32, ss)
            o = gpu_step(st, dev)
            post = st.read_tiles(tiles)
            o_gpu = o.reshape(T, -1)[tiles].cpu().numpy()
            compare(post, new, diag, o_gpu, o_ref, w, tally, what="step %d" % t)
        else:
            gpu_step(st, dev)
        if t % 512 == 0:
            log("  step", t, "of", steps)
        if cap and st.counters()[1] == cap:
            if merge_check is not None:
                merge_check(st, t, tiles, tally)
            else:
                st.merge_bypass()
    torch.cuda.synchronize()
    return tally, st
