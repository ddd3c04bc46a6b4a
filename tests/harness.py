"""GPU-vs-oracle parity harness (test infrastructure).

Two protocols.

run_parity (teacher-forced, sampled steps): before a checked step, the GPU
state of the sampled tiles is read back and the oracle runs the same step
from it on the CPU (the canonical fp32 chain); after the GPU step the two
results are compared.

run_horizon (every step, full horizon): the oracle keeps its own state of the
sampled tiles and steps it alongside the GPU at every step. After each step
the results are compared as above; the oracle then adopts the GPU's values
only at the forgiven elements and groups (reconciliation), and at merges the
GPU's bypass factors (a rank-k truncation's factors are not unique; they are
checked against the Eckart-Young bound instead). At the end, the final
dequantized state and the whole o_t sequence must agree to rel-L2 <= 1e-3.

Checks at every compared step:
  * codes must be bit-exact except at elements whose pre-rounding value lies
    within 1e-6 of a decision boundary (the oracle reports them as `near`);
  * stored step sizes must be bit-exact except in groups the oracle marks;
  * bypass factors / window pairs and the yoked reference bit-exact;
  * the forgiven count must stay at or below 1e-5 of the compared elements;
  * o_t and the dequantized state must agree to rel-L2 <= 1e-4.
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
        self.worst_state = 0.0  # largest per-step dequantized-state rel-L2
        self.merges = 0

    def check(self):
        assert self.mismatch == 0, "%d code/scale mismatches outside the decision windows" % self.mismatch
        assert self.forgiven <= FORGIVEN_MAX * max(self.elements, 1), \
            "forgiven %d of %d elements" % (self.forgiven, self.elements)


def dequant_gpu(post, w, n):
    """Dense float64 state of read-back tiles: c s (+ U W^T over n bypass
    columns; + u w^T over the window's pairs). Rotated (INT4+Had) tiles are
    compared in their stored, rotated basis."""
    if "S32" in post:
        return post["S32"].astype(np.float64)
    g = post["codes"].shape[2] // post["scales"].shape[2]
    S = post["codes"].astype(np.float64) * np.repeat(post["scales"].astype(np.float64), g, axis=2)
    if "U" in post and n > 0:
        S = S + np.einsum("tic,tjc->tij", post["U"][:, :, :n].astype(np.float64),
                          post["W"][:, :, :n].astype(np.float64))
    return S


def dequant_oracle(st):
    if st.S32 is not None:
        return st.S32.astype(np.float64)
    g = st.codes.shape[2] // st.scales.shape[2]
    S = st.codes.astype(np.float64) * np.repeat(st.scales.astype(np.float64), g, axis=2)
    if st.U is not None and st.n > 0:
        S = S + np.einsum("tic,tjc->tij", st.U[:, :, :st.n].astype(np.float64),
                          st.W[:, :, :st.n].astype(np.float64))
    return S


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
    rs = rel_l2(dequant_gpu(post, w, new.n), dequant_oracle(new))
    assert rs <= REL_STEP, what + " dequantized state rel-L2 %g" % rs
    tally.worst_state = max(tally.worst_state, rs)
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


def _oracle_step_fn(w):
    return oracle.hadamard.step if w.hadamard else oracle.window.step if w.pw_window else oracle.step


def check_merge_factors(post, md, k, what=""):
    """Pi8 on the GPU's factors: ||R - U W^T||_F within the Eckart-Young
    optimum sqrt(sum_{i>k} sigma_i^2) (1 + 1e-3) plus the binary16 factor
    rounding; columns past k empty; each U column's largest entry positive.
    Returns the worst relative excess over the optimum."""
    U = post["U"].astype(np.float64)
    W = post["W"].astype(np.float64)
    assert not U[:, :, k:].any() and not W[:, :, k:].any(), what + " columns past k must be empty"
    worst = 0.0
    for ti in range(U.shape[0]):
        sv = md["svals"][ti]
        tail = np.sqrt(np.sum(sv[k:] ** 2))
        err = np.linalg.norm(md["R"][ti] - U[ti, :, :k] @ W[ti, :, :k].T)
        bound = (1 + 1e-3) * tail + 2.0 ** -10 * np.sum(sv[:k]) + 1e-12
        assert err <= bound, what + " tile %d: |R - UW^T| %g > %g" % (ti, err, bound)
        worst = max(worst, err / tail - 1 if tail > 0 else 0.0)
        if k:
            col = U[ti, :, :k]
            top = col[np.argmax(np.abs(col), axis=0), np.arange(k)]
            assert np.all(top >= 0), what + " U columns must have a positive largest entry"
    return worst


class DeviceInputs:
    """Fresh inputs at every step, drawn on the device by the shared input
    generator (rsq_workloads.gen_device: the workload's distributions, torch's
    generator, no arithmetic of the method). The GPU step takes the full
    device tensors; the oracle gets the sampled tiles' values, copied back to
    the host exactly (bf16 values widen to fp32 without rounding)."""

    def __init__(self, w):
        self.w = w
        self.a_log = static_params(w).get("a_log")

    def at_device(self, t, tiles):
        import torch
        from rsq_workloads.gen_device import device_step_inputs
        d = device_step_inputs(self.w, t, a_log=self.a_log)
        dev = {k: v for k, v in d.items() if v is not None}
        T = self.w.tiles
        idx = torch.as_tensor(list(tiles), device="cuda", dtype=torch.long)
        sub = {}
        for name, x in dev.items():
            rows = x.reshape(T, -1)[idx].float().cpu().numpy()
            sub[name] = (rows[:, 0] if x.dim() == 2 else rows)[None]
        return dev, sub


def run_horizon(w, steps, tiles, pool=None, st=None, log_every=256):
    """Every step of the horizon on the sampled tiles, with the oracle kept
    in step (reconciled only at forgiven elements and at merges' factors),
    then the full-horizon bars: final dequantized state and the whole o_t
    sequence within rel-L2 1e-3. Returns (tally, GPU state, report dict)."""
    import torch
    T = w.tiles
    tiles = list(tiles)
    st = make_state(w) if st is None else st
    sw = sub_workload(w, tiles)
    ss = sub_static(w, tiles)
    static = static_params(w)
    ost = oracle.window.zero_state(sw) if w.pw_window else oracle.zero_state(sw)
    ost.bits = tile_bits(w, tiles)
    ostep = _oracle_step_fn(w)
    cap = w.lrb_k + w.lrb_m if w.lrb_m else 0
    tally = Tally()
    num = den = 0.0
    worst_merge = 0.0
    for t in range(1, steps + 1):
        if isinstance(pool, DeviceInputs):
            dev, sub = pool.at_device(t, tiles)
        else:
            inp = pool.at(t) if pool is not None else step_inputs(w, t, static)
            dev, sub = to_device(inp, w), sub_inputs(inp, w, tiles)
        new, o_ref, diag = ostep(ost, sub, sw, oracle.F32, ss)
        o = gpu_step(st, dev)
        post = st.read_tiles(tiles)
        o_gpu = o.reshape(T, -1)[tiles].cpu().numpy()
        compare(post, new, diag, o_gpu, o_ref, w, tally, what="step %d" % t)
        num += float(np.sum((o_gpu.astype(np.float64) - o_ref) ** 2))
        den += float(np.sum(np.asarray(o_ref, np.float64) ** 2))
        if "codes" in post:
            # reconciliation: the GPU's value where the oracle's decision was
            # within the window of a boundary, the oracle's own elsewhere
            new.codes = np.where(diag["near"], post["codes"], new.codes).astype(np.int32)
            new.scales = np.where(diag["group_near"], post["scales"], new.scales).astype(np.float32)
        ost = new
        if cap and st.counters()[1] == cap:
            mnew, md = oracle.merge(ost, sw, oracle.F32)
            st.merge_bypass()
            post = st.read_tiles(tiles)
            bad = (post["codes"] != mnew.codes) & ~md["near"]
            sbad = (post["scales"] != mnew.scales) & ~md["group_near"]
            tally.elements += bad.size
            tally.forgiven += int(((post["codes"] != mnew.codes) & md["near"]).sum())
            tally.mismatch += int(bad.sum()) + int(sbad.sum())
            assert not bad.any(), "merge after step %d: codes differ at %s" % (t, np.argwhere(bad)[:4].tolist())
            assert not sbad.any(), "merge after step %d: step sizes differ" % t
            worst_merge = max(worst_merge, check_merge_factors(post, md, w.lrb_k, "merge after step %d" % t))
            mnew.codes = np.where(md["near"], post["codes"], mnew.codes).astype(np.int32)
            mnew.scales = np.where(md["group_near"], post["scales"], mnew.scales).astype(np.float32)
            mnew.U, mnew.W = post["U"].copy(), post["W"].copy()   # the GPU's factors (Pi8 checked)
            ost = mnew
            tally.merges += 1
        if t % log_every == 0:
            log("  step", t, "of", steps, "forgiven", tally.forgiven)
    torch.cuda.synchronize()
    post = st.read_tiles(tiles)
    n = st.counters()[1]
    final = rel_l2(dequant_gpu(post, w, n), dequant_oracle(ost))
    o_seq = np.sqrt(num / den) if den > 0 else np.sqrt(num)
    assert final <= REL_HORIZON, "final dequantized state rel-L2 %g" % final
    assert o_seq <= REL_HORIZON, "o_t sequence rel-L2 %g" % o_seq
    tally.check()
    report = dict(final_state_rel_l2=final, o_sequence_rel_l2=o_seq, worst_step_state_rel_l2=tally.worst_state,
                  forgiven=tally.forgiven, elements=tally.elements, merges=tally.merges,
                  worst_merge_excess=worst_merge)
    log("  horizon", w.name, report)
    return tally, st, report
