"""Throughput of the fused low-bit recurrent-state decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config I] [--warm]

A step is one decode step of every (batch, head) tile of the workload: load
and dequantize the state, decay, update (the Gated DeltaNet delta rule for the
default workload), read out o_t, rescale, requantize, store in place; with a
low-rank bypass, a merge follows every m-th step and is part of the step's
cost. The default workload is the large-batch Gated DeltaNet serving step
(512 x 32 heads of 128 x 128, per-head INT8/INT6/INT4). Inputs for 64
distinct steps are generated once and cycled; they sit in HBM before the
timed region starts. The state is rotated over enough independent state sets
(>= 1 GiB) that the 256 MB Infinity Cache cannot hold them, so every step
streams its state from HBM ("cold"; --warm times a single state set). Each
state set is first brought to decode step `--age` (untimed set-up), so the
timed steps see a decoding state rather than a fresh zero one.

Prints one JSON line (rank 0). `value` is state-updates per second
(batch * heads * steps / wall time). `roofline.achieved` is the algorithmic
bytes of one step (decode launch plus the amortized merges) divided by the
mean device time of one step from HIP events on the launch stream;
`roofline.frac` is against the 8 TB/s HBM peak and `frac_of_copy` against a
plain device copy measured on the same GPU. `roofline.traffic` comes from
committed rocprofv3 counter summaries when they were taken on the current
kernel sources, else null. `fp32_state` times the same step on an fp32 state
(bits = 32, no quantizer) of the same shape under the same protocol: the
quantized step's speed-up over it. `quality` (default workload) runs a
quantized state and an fp32 state from zero on the same device-drawn inputs
for the whole horizon and reports the relative L2 error of o_t at a quarter,
half and all of it, per bit width and overall. `cpu_baseline` times the CPU
oracle (test infrastructure) on a bounded sample.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
GROUP = 16          # launches per timed event pair
METRIC = "quantized state-update steps/sec (batch*heads*steps) and achieved HBM GB/s vs peak"


DECODE_SOURCES = ("decode_impl.hpp", "lane_ops.hpp", "rsq_device.hpp", "rsq_kernels.hpp", "decode_dispatch.hip",
                  "decode_retnet.hip", "decode_mamba2.hip", "decode_gla.hip", "decode_gdn.hip")


def kernel_source_hash():
    """Hash of the sources that define the decode kernel (counter summaries are
    only used while it matches)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_recurrent_state_rsq_amd", "csrc")
    for f in DECODE_SOURCES:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(workload_name, bytes_per_launch):
    """HBM bytes per launch from a committed counter summary, if it matches the sources."""
    p = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload_name)
    if not os.path.exists(p):
        return None, None
    d = json.load(open(p))
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None, d
    return d.get("hbm_bytes_per_launch"), d


def cpu_baseline(w, tiles_per_worker=64, steps=256):
    """The oracle's fp32-canonical step, as it stands, on a bounded sample of tiles.

    One worker process per host core (at most 16), each with one BLAS thread,
    steps `tiles_per_worker` tiles of the workload's shape for `steps` steps
    (with bypass merges where the workload has them). Only the step loop is
    timed; the rate is the sum of updates over the slowest worker's loop time.
    """
    import multiprocessing as mp
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    args = [(w, i, tiles_per_worker, steps) for i in range(cores)]
    ctx = mp.get_context("fork")
    with ctx.Pool(cores) as pool:
        done = pool.map(_oracle_worker, args)
    updates = sum(u for u, _ in done)
    loop_s = max(t for _, t in done)
    return {"value": updates / loop_s, "unit": "state-updates/s", "cores": cores, "kind": "oracle",
            "sample": "%d worker processes x %d tiles (%dx%d, the workload's heads cycled) x %d steps; "
                      "oracle fp32-canonical step in numpy, one thread per process; slowest step loop %.1f s"
                      % (cores, tiles_per_worker, w.d_k, w.d_v, steps, loop_s)}


def _oracle_worker(a):
    os.environ["OMP_NUM_THREADS"] = "1"
    os.environ["OPENBLAS_NUM_THREADS"] = "1"
    w, wid, ntiles, steps = a
    import oracle
    from rsq_workloads import static_params, step_inputs
    sw = w.with_(batch=1, heads=ntiles, mixed_bits=None, head_bits=None, seed=w.seed + 17 * wid)
    static = static_params(sw)
    inps = [step_inputs(sw, t, static) for t in range(1, steps + 1)]
    st = oracle.zero_state(sw)
    hb = oracle.recurrence.tile_bits(w)
    st.bits = hb[np.arange(ntiles) % w.heads].astype(np.int32)
    t0 = time.perf_counter()
    for t, inp in enumerate(inps, 1):
        st, o, d = (oracle.hadamard.step if w.hadamard else oracle.step)(st, inp, sw, oracle.F32, static)
        if w.lrb_m and t % w.lrb_m == 0:
            st, _ = oracle.merge(st, sw, oracle.F32)
    return ntiles * steps, time.perf_counter() - t0


def copy_reference(torch, nbytes=1 << 30, reps=10):
    """Bandwidth of a plain device-to-device copy (read + write bytes / time)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return {"bytes_per_copy": 2 * nbytes, "ms": ms, "gbs": 2 * nbytes / (ms * 1e-3) / 1e9}


class _HipEvents:
    """HIP events (through the runtime PyTorch loaded) that the decode kernel's
    dispatch records itself via rsq_decode_step_timed: they time each launch
    on its own stream without putting marker commands between the launches."""

    def __init__(self, n):
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        P = ctypes.c_void_p
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(P)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
        self.rt.hipEventDestroy.argtypes = [P]
        self.ev = []
        for _ in range(n):
            e = P()
            if self.rt.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e)

    def elapsed(self, a, b):
        ms = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(ms), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self):
        for e in self.ev:
            self.rt.hipEventDestroy(e)
        self.ev = []


def accounting_report(torch, steps, batch=4, heads=4):
    """Error accounting on synthetic inputs ("Preserving Updates ...", Figs. 1,
    2, 4 and Table 5; the scale-state feedback of "When Dynamic Scaling
    Fails ..."): for each Table 1 row at its workload's head shape, INT4
    group 32 with dynamic binary16 steps, run `steps` decode steps with the
    accounting step next to yoked-scale and fp32 states fed the same inputs,
    once with independent steps and once with inputs that keep a persistent
    per-tile direction (coherence 0.9). Prints one JSON line per run."""
    import bit_recurrent_state_rsq_amd as rsq
    from rsq_workloads import CONFIGS, static_params, step_inputs

    def dev_inputs(w, inp):
        d = {}
        for name in ("q", "k", "v"):
            d[name] = torch.from_numpy(np.ascontiguousarray(inp[name + "_bits"]).view(np.int16)).cuda().view(torch.bfloat16)
        for name in ("alpha", "beta"):
            if name in inp:
                d[name] = torch.from_numpy(np.ascontiguousarray(inp[name], np.float32)).cuda()
        return d

    def dense(st, rotated=False):
        t = st.read_tiles()
        if "S32" in t:
            return t["S32"].astype(np.float64)
        s = np.repeat(t["scales"].astype(np.float64), st.group, axis=2)
        y = t["codes"] * s
        if st.pw:
            n = st.counters()[1]
            y = y + np.einsum("tic,tjc->tij", t["U"][:, :, :n].astype(np.float64), t["W"][:, :, :n].astype(np.float64))
        if rotated:
            # stored groups are y = x H (Sylvester-Hadamard): x = y H / g
            g = st.group
            hm = np.array([[(-1.0) ** bin(a & b).count("1") for b in range(g)] for a in range(g)])
            y = (y.reshape(y.shape[0], y.shape[1], -1, g) @ hm / g).reshape(y.shape)
        return y

    for (model, ci), rho in ((m, r) for m in (("retnet", 0), ("mamba2", 2), ("gla", 3), ("gdn", 1))
                             for r in (0.0, 0.9)):
        base = CONFIGS[ci]
        w = base.with_(batch=batch, heads=heads, d_k=max(base.d_k, 128), bits=4, group=32, scale_mode="dynamic",
                       scale_dtype="f16", in_dtype="bf16", mixed_bits=None, head_bits=None, lrb_k=0, lrb_m=0,
                       bdr=False, seed=9000 + ci, coherence=rho)
        kw = rsq.config_kwargs_from(w)
        dyn = rsq.State(**kw)
        yok = rsq.State(**dict(kw, scale_mode="yoked"))
        had = rsq.State(**dict(kw, hadamard=True))
        f32 = rsq.State(**dict(kw, bits=32))
        # Gated DeltaNet: the same INT4 history with an 8-pair pure-write window, and INT6
        extra = {}
        if model == "gdn":
            extra = {"pw8": rsq.State(**dict(kw, pw_window=8)), "int6": rsq.State(**dict(kw, bits=6))}
        ea = rsq.ErrorAccounting(dyn)
        sp = static_params(w)
        norms = []
        for t in range(1, steps + 1):
            d = dev_inputs(w, step_inputs(w, t, sp))
            args = (d["q"], d["k"], d["v"], d.get("alpha"), d.get("beta"))
            if t == steps:
                ea.counts.zero_()          # counters of the last step only
            ea.step(*args)
            yok.decode_step(*args)
            had.decode_step(*args)
            f32.decode_step(*args)
            for xs in extra.values():
                xs.decode_step(*args)
            if t in (steps // 8, steps // 4, steps // 2, steps):
                S, Sd, Sy, Sh = dense(f32), dense(dyn), dense(yok), dense(had, rotated=True)
                nS = np.linalg.norm(S)
                norms.append(dict(t=t, norm_dynamic=np.linalg.norm(Sd) / nS, norm_yoked=np.linalg.norm(Sy) / nS,
                                  norm_had=np.linalg.norm(Sh) / nS,
                                  err_dynamic=np.linalg.norm(Sd - S) / nS, err_yoked=np.linalg.norm(Sy - S) / nS,
                                  err_had=np.linalg.norm(Sh - S) / nS,
                                  **{"err_" + k: np.linalg.norm(dense(xs) - S) / nS for k, xs in extra.items()}))
        torch.cuda.synchronize()
        c = ea.count_table().astype(np.int64).sum(axis=0)
        g = ea.gains()
        # cost of the accounting step next to the plain step, same state shape
        d = dev_inputs(w, step_inputs(w, 1, sp))
        args = (d["q"], d["k"], d["v"], d.get("alpha"), d.get("beta"))
        timing = {}
        runs = [("plain", lambda: dyn.decode_step(*args)), ("accounting", lambda: ea.step(*args)),
                ("hadamard", lambda: had.decode_step(*args))]
        runs += [(k, (lambda xs=xs: xs.decode_step(*args))) for k, xs in extra.items()]
        for name, fn in runs:
            for _ in range(20):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(200):
                fn()
            e1.record()
            torch.cuda.synchronize()
            timing[name + "_us"] = e0.elapsed_time(e1) / 200 * 1e3
        q25, q50, q75 = ea.ratio_quartiles()
        print(json.dumps({
            "accounting": model, "coherence": rho, "steps": steps, "tiles": w.tiles, "d_k": w.d_k, "d_v": w.d_v,
            "state": "int4 g32 dynamic fp16", "data": "synthetic",
            "ratio_quartiles_last_step": [q25, q50, q75],
            "lost_fraction_last_step": float(c[1] / max(c[0], 1)),
            "reversed_fraction_last_step": float(c[3] / max(c[0], 1)),
            "g_T": float(np.mean(g[:, 0])), "g_lost_T": float(np.mean(g[:, 1])), "g_moved_T": float(np.mean(g[:, 2])),
            "state_norms": norms, "step_time": timing,
        }), flush=True)


def _dev_inputs(torch, w, inp):
    d = {}
    for name in ("q", "k", "v"):
        if w.in_dtype == "bf16":
            d[name] = torch.from_numpy(np.ascontiguousarray(inp[name + "_bits"]).view(np.int16)).cuda().view(torch.bfloat16)
        else:
            d[name] = torch.from_numpy(np.ascontiguousarray(inp[name], np.float32)).cuda()
    for name in ("alpha", "beta"):
        d[name] = torch.from_numpy(np.ascontiguousarray(inp[name], np.float32)).cuda() if name in inp else None
    return d


def time_steps(torch, rsq, w, kw, dev, K, warmup, age, warm, min_set_bytes, out):
    """The timed protocol for one state configuration: rotate over state sets
    of >= min_set_bytes (one set if warm), bring each to decode step `age`,
    run `warmup` untimed steps, then time K steps. Decode launches are timed in
    groups of up to GROUP consecutive steps by HIP events on their first and
    last dispatch; each merge carries its own pair. Returns a dict."""
    per_state = rsq.state_bytes(**kw)
    nsets = 1 if warm else int(np.ceil(min_set_bytes / per_state))
    states = [rsq.State(**kw) for _ in range(nsets)]
    cap = w.lrb_k + w.lrb_m if w.lrb_m else 0
    stream = torch.cuda.current_stream()
    bound = {}

    def step_fn(i, s):
        key = (i, s % len(dev))
        if key not in bound:
            d = dev[key[1]]
            bound[key] = states[i].bind_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], out=out, stream=stream)
        return bound[key]

    def maybe_merge(i):
        if cap and states[i].counters()[1] == cap:
            states[i].merge_bypass(stream=stream)

    for i in range(nsets):
        for s in range(age):
            step_fn(i, s)()
            maybe_merge(i)
    for s in range(warmup):
        step_fn(s % nsets, age + s // nsets)()
        maybe_merge(s % nsets)
    torch.cuda.synchronize()

    # which timed steps are followed by a merge (fills evolve deterministically)
    merge_after = set()
    fill = [st.counters()[1] for st in states]
    if cap:
        for s in range(K):
            i = s % nsets
            fill[i] += 1
            if fill[i] == cap:
                merge_after.add(s)
                fill[i] = w.lrb_k
    groups = []
    g0 = 0
    for s in range(K):
        if s - g0 + 1 == GROUP or s in merge_after or s == K - 1:
            groups.append((g0, s + 1))
            g0 = s + 1
    hip = _HipEvents(2 * len(groups) + 2 * len(merge_after))
    base = [st.counters()[0] for st in states]
    calls = [step_fn(s % nsets, base[s % nsets] + s // nsets) for s in range(K)]
    ev_of = {}
    for gi, (a0, a1) in enumerate(groups):
        ev_of[a0] = [hip.ev[2 * gi], None]
        ev_of.setdefault(a1 - 1, [None, None])[1] = hip.ev[2 * gi + 1]
    mev = {s: (hip.ev[2 * len(groups) + 2 * mi], hip.ev[2 * len(groups) + 2 * mi + 1])
           for mi, s in enumerate(sorted(merge_after))}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        e = ev_of.get(s)
        if e is None:
            calls[s]()
        else:
            calls[s](e[0], e[1])
        if s in merge_after:
            states[s % nsets].merge_bypass(stream=stream, start_event=mev[s][0], stop_event=mev[s][1])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if cap and [st.counters()[1] for st in states] != fill:
        raise RuntimeError("bypass fill differs from the merge schedule")
    group_ms = np.array([hip.elapsed(2 * gi, 2 * gi + 1) for gi in range(len(groups))])
    group_n = np.array([a1 - a0 for a0, a1 in groups])
    merge_ms = np.array([hip.elapsed(2 * len(groups) + 2 * mi, 2 * len(groups) + 2 * mi + 1)
                         for mi in range(len(merge_after))])
    hip.destroy()
    flags = [st.get_status() for st in states[: min(4, nsets)]]
    extra_merges = 0
    if cap and len(merge_ms) < 8:
        # too few state sets filled inside the timed region: after it, fill up
        # to 8 of them (untimed decode steps) and time their merges alone
        nm = min(8, nsets)
        ev = _HipEvents(2 * nm)
        for i in range(nm):
            while states[i].counters()[1] < cap:
                step_fn(i, states[i].counters()[0])()
        torch.cuda.synchronize()
        for i in range(nm):
            states[i].merge_bypass(stream=stream, start_event=ev.ev[2 * i], stop_event=ev.ev[2 * i + 1])
        torch.cuda.synchronize()
        merge_ms = np.concatenate([merge_ms, [ev.elapsed(2 * i, 2 * i + 1) for i in range(nm)]])
        ev.destroy()
        extra_merges = nm
    decode_ms = float(group_ms.sum() / group_n.sum())
    merge_mean = float(merge_ms.mean()) if len(merge_ms) else None
    res = {"nsets": nsets, "per_state": per_state, "wall": wall, "decode_ms": decode_ms,
           "decode_median_ms": float(np.median(group_ms / group_n)),
           "merges": len(merge_after), "extra_merges": extra_merges, "merge_ms": merge_mean,
           # device time of one step: a decode launch plus 1/m of a merge
           "step_ms": decode_ms + (merge_mean / w.lrb_m if cap else 0.0), "flags": flags}
    del states, bound, calls
    return res


def quality_report(torch, rsq, w, hb, steps):
    """o_t of a quantized state against an fp32 state (bits = 32) of the same
    shape fed the same device-drawn inputs from a zero state, for `steps`
    steps: relative L2 error over [B, H, d_v] at a quarter, half and all of the
    horizon, overall and per bit width."""
    from rsq_workloads import static_params
    from rsq_workloads.gen_device import device_step_inputs
    kwq = rsq.config_kwargs_from(w, head_bits=hb if (w.mixed_bits or w.head_bits) else None)
    w32 = w.with_(bits=32, mixed_bits=None, head_bits=None, lrb_k=0, lrb_m=0, bdr=False, scale_mode="dynamic",
                  hadamard=False, pw_window=0)
    kw32 = rsq.config_kwargs_from(w32)
    sq, s32 = rsq.State(**kwq), rsq.State(**kw32)
    cap = w.lrb_k + w.lrb_m if w.lrb_m else 0
    a_log = static_params(w).get("a_log")
    oq = torch.empty((w.batch, w.heads, w.d_v), dtype=torch.float32, device="cuda")
    o32 = torch.empty_like(oq)
    marks = sorted({steps // 4, steps // 2, steps})
    classes = {b: torch.as_tensor(np.flatnonzero(hb == b), device="cuda") for b in sorted(set(int(x) for x in hb))}
    rep = {}
    for t in range(1, steps + 1):
        d = device_step_inputs(w, t, a_log=a_log)
        args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"])
        sq.decode_step(*args, out=oq)
        s32.decode_step(*args, out=o32)
        if cap and sq.counters()[1] == cap:
            sq.merge_bypass()
        if t in marks:
            def rel(a, b):
                return float(torch.linalg.vector_norm((a - b).double()) / torch.linalg.vector_norm(b.double()))
            r = {"all": rel(oq, o32)}
            if len(classes) > 1:
                for b, idx in classes.items():
                    r["int%d" % b] = rel(oq[:, idx], o32[:, idx])
            rep[str(t)] = r
    torch.cuda.synchronize()
    flags = sq.get_status()
    del sq, s32
    return {"reference": "fp32 state (bits = 32) of the same shape, same inputs", "steps": steps,
            "o_rel_l2": rep, "status_flags": flags,
            "inputs": "drawn on the device (rsq_workloads.gen_device, the workload's distributions, fresh every step)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500,
                    help="timed steps (with a bypass: raised to a whole number of merge periods over all state sets)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before timing (default: 4 per rotated state set, at least 16)")
    ap.add_argument("--age", type=int, default=32,
                    help="untimed set-up: bring every state set to this decode step first")
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--warm", action="store_true", help="time one state set in place (cache-warm)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-fp32", action="store_true", help="skip the fp32-state comparator")
    ap.add_argument("--quality", type=int, default=None, metavar="T",
                    help="steps of the quantized-vs-fp32 o_t report (default: the workload's horizon for "
                         "the default workload, 0 = skip)")
    ap.add_argument("--min-set-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--copy-only", action="store_true",
                    help="only time a plain 1 GiB device copy (the reference for HBM counters)")
    ap.add_argument("--hadamard", action="store_true",
                    help="store the state rotated per group (the INT4+Had baseline)")
    ap.add_argument("--pw", type=int, default=0, metavar="W",
                    help="Gated DeltaNet: keep a pure-write window of W FP8 pairs beside the history")
    ap.add_argument("--lrb", type=str, default=None, metavar="K,M",
                    help="add a low-rank bypass of rank K merged every M steps (with BDR, eps_L 0.5, eps_B 0.3)")
    ap.add_argument("--accounting", type=int, default=0, metavar="T",
                    help="instead of timing, run the error accounting for T steps per Table 1 row")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the decode step has no cross-GPU exchange (tiles shard "
              "by batch row with nothing to communicate), so --gpus %d is not run." % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_only:
        torch.cuda.set_device(0)
        print(json.dumps({"copy_reference": copy_reference(torch)}), flush=True)
        return
    if args.accounting:
        torch.cuda.set_device(0)
        accounting_report(torch, args.accounting)
        return
    import bit_recurrent_state_rsq_amd as rsq
    from rsq_workloads import CONFIGS, head_bits_for, InputPool

    w = CONFIGS[args.config]
    if args.hadamard:
        w = w.with_(hadamard=True)
    if args.pw:
        w = w.with_(pw_window=args.pw)
    if args.lrb:
        k, m = (int(x) for x in args.lrb.split(","))
        w = w.with_(lrb_k=k, lrb_m=m, lrb_eps=0.5, bdr=True, bdr_eps=0.3)
    # the CPU baseline forks worker processes: do it before this process touches the GPU
    cpu = None if args.no_cpu else cpu_baseline(w)
    torch.cuda.set_device(0)
    copy_ref = copy_reference(torch)
    hb = head_bits_for(w)
    kw = rsq.config_kwargs_from(w, head_bits=hb if (w.mixed_bits or w.head_bits) else None)

    pool = InputPool.build(w, 64)
    dev = [_dev_inputs(torch, w, inp) for inp in pool.steps]
    out = torch.empty((w.batch, w.heads, w.d_v), dtype=torch.float32, device="cuda")
    K = args.steps
    nsets_guess = 1 if args.warm else int(np.ceil(args.min_set_bytes / rsq.state_bytes(**kw)))
    if args.warmup is None:
        args.warmup = max(16, 4 * nsets_guess)
    if w.lrb_m:
        # a whole number of merge periods over every state set, so that the
        # wall clock holds exactly one merge per m steps of each set
        period = nsets_guess * w.lrb_m
        K = -(-K // period) * period
    q = time_steps(torch, rsq, w, kw, dev, K, args.warmup, args.age, args.warm, args.min_set_bytes, out)
    if w.lrb_m and q["merges"] != K // w.lrb_m:
        raise RuntimeError("timed region holds %d merges, not one per %d steps" % (q["merges"], w.lrb_m))

    bytes_step = rsq.workload_step_bytes(w.model, w.batch, hb, w.group, w.scale_dtype, w.d_k, w.d_v,
                                         w.in_dtype, w.lrb_k, w.lrb_m, w.pw_window)
    merge_bytes = rsq.workload_merge_bytes(w.batch, hb, w.group, w.scale_dtype, w.d_k, w.d_v, w.lrb_k,
                                           w.lrb_m) if w.lrb_m else 0
    # one step's algorithmic bytes: the decode launch plus 1/m of a merge
    bytes_e2e = bytes_step + (merge_bytes / w.lrb_m if w.lrb_m else 0)
    updates = w.batch * w.heads * K
    achieved = bytes_e2e / (q["step_ms"] * 1e-3) / 1e9
    traffic, tinfo = load_traffic(w.name + ("_had" if w.hadamard else "") + ("_pw%d" % w.pw_window if w.pw_window else "")
                                  + ("_lrb%d_%d" % (w.lrb_k, w.lrb_m) if args.lrb else ""), bytes_step)

    res = {
        "metric": METRIC,
        "value": updates / q["wall"],
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": q["wall"] / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "model": w.model, "batch": w.batch, "heads": w.heads,
            "d_k": w.d_k, "d_v": w.d_v,
            "state": "int%s%s%s%s" % ("/".join(str(b) for b in sorted(set(hb))), "+had" if w.hadamard else "",
                                      "+pw%d" % w.pw_window if w.pw_window else "",
                                      "+lrb%d/%d" % (w.lrb_k, w.lrb_m) if w.lrb_m else ""),
            "group": w.group, "scale": "%s %s" % (w.scale_mode, w.scale_dtype), "inputs": w.in_dtype,
            "protocol": "warm (one state set)" if args.warm else
                        "cold (%d state sets, %.2f GiB)" % (q["nsets"], q["nsets"] * q["per_state"] / 2 ** 30),
            "state_age": args.age,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "frac_of_copy": achieved / copy_ref["gbs"],
        },
        "kernel": {"name": "rsq::decode_kernel", "mean_us": q["decode_ms"] * 1e3,
                   "median_us": q["decode_median_ms"] * 1e3,
                   "timing": "HIP events on the dispatches of the first and last launch of each "
                             "group of up to %d consecutive decode steps in the timed region "
                             "(groups end at bypass merges; each merge has its own pair)" % GROUP,
                   "algorithmic_bytes_per_launch": bytes_step,
                   "decode_only_gbs": bytes_step / (q["decode_ms"] * 1e-3) / 1e9,
                   "hbm_gbs_wall": bytes_e2e * K / q["wall"] / 1e9},
        "status_flags": q["flags"],
        "copy_reference": copy_ref,
    }
    if w.lrb_m:
        res["merge"] = {"name": "rsq::merge_kernel", "merges_in_timed_region": q["merges"],
                        "merges_timed_after": q["extra_merges"],
                        "mean_us": q["merge_ms"] * 1e3 if q["merge_ms"] is not None else None,
                        "algorithmic_bytes_per_merge": merge_bytes,
                        "step_us_with_amortized_merge": q["step_ms"] * 1e3}
    if not args.no_fp32:
        w32 = w.with_(bits=32, mixed_bits=None, head_bits=None, lrb_k=0, lrb_m=0, bdr=False,
                      scale_mode="dynamic", hadamard=False, pw_window=0)
        kw32 = rsq.config_kwargs_from(w32)
        f = time_steps(torch, rsq, w32, kw32, dev, K, args.warmup, args.age, args.warm, args.min_set_bytes, out)
        b32 = rsq.workload_step_bytes(w.model, w.batch, [32] * w.heads, w.group, w.scale_dtype, w.d_k, w.d_v,
                                      w.in_dtype)
        res["fp32_state"] = {"step_us": f["step_ms"] * 1e3, "algorithmic_bytes_per_launch": b32,
                             "gbs": b32 / (f["step_ms"] * 1e-3) / 1e9,
                             "protocol": "cold (%d state sets, %.2f GiB)" % (f["nsets"], f["nsets"] * f["per_state"] / 2 ** 30),
                             "speedup_of_quantized": f["step_ms"] / q["step_ms"],
                             "state_bytes_ratio": f["per_state"] / q["per_state"]}
    qsteps = args.quality if args.quality is not None else (w.steps if args.config == 4 else 0)
    if qsteps:
        res["quality"] = quality_report(torch, rsq, w, hb, qsteps)
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
