"""Throughput of the fused low-bit recurrent-state decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config I] [--warm]

A step is one decode step of every (batch, head) tile of the workload: load
and dequantize the state, decay, update (the Gated DeltaNet delta rule for the
default workload), read out o_t, rescale, requantize, store in place. Inputs
for 64 distinct steps are generated once and cycled; they sit in HBM before
the timed region starts. The state is rotated over enough independent state
sets (>= 1 GiB) that the 256 MB Infinity Cache cannot hold them, so every
step streams its state from HBM ("cold"; --warm times a single state set).

Prints one JSON line (rank 0). `value` is state-updates per second
(batch * heads * steps / wall time). `roofline.achieved` is the algorithmic
bytes of one launch divided by the mean kernel duration from HIP events on the
launch stream; `roofline.traffic` comes from committed rocprofv3 counter
summaries when they were taken on the current kernel sources, else null.
`cpu_baseline` times the CPU oracle (test infrastructure) on a bounded sample.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "quantized state-update steps/sec (batch*heads*steps) and achieved HBM GB/s vs peak"


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_recurrent_state_rsq_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
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


def cpu_baseline(w, budget_s=15.0):
    """The oracle's canonical fp32 step on a bounded sample of tiles, on the host cores."""
    import multiprocessing as mp
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    tiles_per_worker, steps = 8, 4
    args = [(w, i, tiles_per_worker, steps) for i in range(cores)]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        done = pool.map(_oracle_worker, args)
    wall = time.perf_counter() - t0
    updates = sum(done)
    return {"value": updates / wall, "unit": "state-updates/s", "cores": cores, "kind": "oracle",
            "sample": "%d worker processes x %d tiles x %d steps of the same workload "
                      "(oracle fp32-canonical step, numpy, one thread each); %.1f s wall"
                      % (cores, tiles_per_worker, steps, wall)}


def _oracle_worker(a):
    os.environ["OMP_NUM_THREADS"] = "1"
    w, wid, ntiles, steps = a
    import oracle
    from rsq_workloads import static_params, step_inputs
    sw = w.with_(batch=1, heads=ntiles, mixed_bits=None, seed=w.seed + 17 * wid)
    static = static_params(sw)
    inps = [step_inputs(sw, t, static) for t in range(1, steps + 1)]
    st = oracle.zero_state(sw)
    hb = oracle.recurrence.tile_bits(w)
    st.bits = hb[np.arange(ntiles) % w.heads].astype(np.int32)
    t0 = time.perf_counter()
    for inp in inps:
        st, o, d = oracle.step(st, inp, sw, oracle.F32, static)
    _ = time.perf_counter() - t0
    return ntiles * steps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before timing (default: 24 per rotated state set, at least 64)")
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--warm", action="store_true", help="time one state set in place (cache-warm)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--min-set-bytes", type=float, default=float(1 << 30))
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the decode step has no cross-GPU exchange (tiles shard "
              "by batch row with nothing to communicate), so --gpus %d is not run." % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_recurrent_state_rsq_amd as rsq
    from rsq_workloads import CONFIGS, head_bits_for, InputPool

    w = CONFIGS[args.config]
    # the CPU baseline forks worker processes: do it before this process touches the GPU
    cpu = None if args.no_cpu else cpu_baseline(w)
    torch.cuda.set_device(0)
    hb = head_bits_for(w)
    kw = rsq.config_kwargs_from(w, head_bits=hb if w.mixed_bits else None)
    per_state = rsq.state_bytes(**kw)
    nsets = 1 if args.warm else int(np.ceil(args.min_set_bytes / per_state))
    states = [rsq.State(**kw) for _ in range(nsets)]

    pool = InputPool.build(w, 64)
    dev = []
    for inp in pool.steps:
        d = {}
        for name in ("q", "k", "v"):
            if w.in_dtype == "bf16":
                d[name] = torch.from_numpy(np.ascontiguousarray(inp[name + "_bits"]).view(np.int16)).cuda().view(torch.bfloat16)
            else:
                d[name] = torch.from_numpy(np.ascontiguousarray(inp[name], np.float32)).cuda()
        for name in ("alpha", "beta"):
            d[name] = torch.from_numpy(np.ascontiguousarray(inp[name], np.float32)).cuda() if name in inp else None
        dev.append(d)
    out = torch.empty((w.batch, w.heads, w.d_v), dtype=torch.float32, device="cuda")
    cap = w.lrb_k + w.lrb_m if w.lrb_m else 0

    def one_step(s, st):
        d = dev[s % len(dev)]
        st.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], out=out)
        if cap and st.counters()[1] == cap:
            st.merge_bypass()

    if args.warmup is None:
        args.warmup = max(64, 24 * nsets)
    for s in range(args.warmup):
        one_step(s, states[s % nsets])
    torch.cuda.synchronize()

    K = args.steps
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        st = states[s % nsets]
        d = dev[s % len(dev)]
        ev[s][0].record(stream)
        st.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], out=out)
        ev[s][1].record(stream)
        if cap and st.counters()[1] == cap:
            st.merge_bypass()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = np.array([a.elapsed_time(b) for a, b in ev])

    bytes_step = rsq.workload_step_bytes(w.model, w.batch, hb, w.group, w.scale_dtype, w.d_k, w.d_v,
                                         w.in_dtype, w.lrb_k, w.lrb_m)
    updates = w.batch * w.heads * K
    value = updates / wall
    mean_ms = float(kernel_ms.mean())
    achieved = bytes_step / (mean_ms * 1e-3) / 1e9
    traffic, tinfo = load_traffic(w.name, bytes_step)
    flags = [st.get_status() for st in states[: min(4, nsets)]]

    res = {
        "metric": METRIC,
        "value": value,
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "model": w.model, "batch": w.batch, "heads": w.heads,
            "d_k": w.d_k, "d_v": w.d_v, "state": "int%s" % ("/".join(str(b) for b in sorted(set(hb)))),
            "group": w.group, "scale": "%s %s" % (w.scale_mode, w.scale_dtype), "inputs": w.in_dtype,
            "protocol": "warm (one state set)" if args.warm else "cold (%d state sets, %.2f GiB)" % (nsets, nsets * per_state / 2 ** 30),
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
        },
        "kernel": {"name": "rsq::decode_kernel", "mean_us": mean_ms * 1e3,
                   "median_us": float(np.median(kernel_ms)) * 1e3,
                   "algorithmic_bytes_per_launch": bytes_step,
                   "hbm_gbs_wall": bytes_step * K / wall / 1e9},
        "status_flags": flags,
    }
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
