"""Low-bit recurrent-state decode step for MI355X (gfx950).

Python binding of librsq.so (include/rsq.h). PyTorch supplies device memory
and the current stream; every arithmetic step runs in the HIP kernels.

    st = State(model="gdn", batch=64, heads=16, d_k=128, d_v=128, group=32,
               bits=4, scale_mode="persistent", scale_dtype="f16",
               in_dtype="bf16")
    o = st.decode_step(q, k, v, alpha=alpha, beta=beta)     # torch tensors on cuda

The recurrence is Table 1 of "Preserving Updates in Low-Bit Recurrent State
Quantization" (RetNet, Mamba2, GLA, Gated DeltaNet); requantization, BDR and
the low-rank bypass follow the same page, the scale policies the abstract of
"When Dynamic Scaling Fails: A Scale-State Feedback Governs Recurrent-State
Quantization in Linear-Attention and SSM LLMs".
"""
import ctypes
from typing import Dict, Optional, Sequence

import numpy as np

from . import _abi
from ._abi import Error, check, lib
from . import codec
from .accounting import step_bytes_per_tile, workload_step_bytes, workload_merge_bytes

__all__ = ["State", "Error", "state_bytes", "make_config", "step_bytes_per_tile",
           "workload_step_bytes", "workload_merge_bytes", "allocate_head_bits", "ErrorAccounting"]


def make_config(model, batch, heads, d_k, d_v, group, bits=4, head_bits=None,
                scale_mode="dynamic", scale_dtype="f32", trigger=1.0, bdr=False,
                bdr_eps=0.5, lrb_k=0, lrb_m=0, lrb_eps=0.5, gamma=None, in_dtype="f32", hadamard=False,
                pw_window=0):
    """Build an rsq_config. Returns (config, keep-alive list of host arrays)."""
    keep = []
    cfg = _abi.Config()
    cfg.abi_version = _abi.ABI_VERSION
    cfg.model = _abi.MODELS[model] if isinstance(model, str) else int(model)
    cfg.batch, cfg.heads, cfg.d_k, cfg.d_v = int(batch), int(heads), int(d_k), int(d_v)
    cfg.group = int(group)
    cfg.bits = int(bits)
    if head_bits is not None:
        hb = (ctypes.c_int32 * heads)(*[int(b) for b in head_bits])
        keep.append(hb)
        cfg.head_bits = ctypes.cast(hb, ctypes.POINTER(ctypes.c_int32))
    cfg.scale_mode = _abi.SCALE_MODES[scale_mode] if isinstance(scale_mode, str) else int(scale_mode)
    cfg.scale_dtype = _abi.DTYPES[scale_dtype] if isinstance(scale_dtype, str) else int(scale_dtype)
    cfg.persist_trigger = float(trigger)
    cfg.bdr = int(bool(bdr))
    cfg.bdr_eps = float(bdr_eps)
    cfg.lrb_k, cfg.lrb_m = int(lrb_k), int(lrb_m)
    cfg.lrb_eps = float(lrb_eps)
    if gamma is not None:
        g = (ctypes.c_float * heads)(*[float(x) for x in np.broadcast_to(np.asarray(gamma, np.float32), (heads,))])
        keep.append(g)
        cfg.gamma = ctypes.cast(g, ctypes.POINTER(ctypes.c_float))
    cfg.in_dtype = _abi.DTYPES[in_dtype] if isinstance(in_dtype, str) else int(in_dtype)
    cfg.hadamard = int(bool(hadamard))
    cfg.pw_window = int(pw_window)
    return cfg, keep


def config_kwargs_from(w, head_bits=None) -> Dict:
    """Keyword arguments of make_config for a workload description object
    (attributes model, batch, heads, d_k, d_v, group, bits, ... as in rsq_workloads)."""
    kw = dict(model=w.model, batch=w.batch, heads=w.heads, d_k=w.d_k, d_v=w.d_v, group=w.group,
              bits=w.bits, scale_mode=w.scale_mode, scale_dtype=w.scale_dtype, trigger=w.trigger,
              bdr=w.bdr, bdr_eps=w.bdr_eps, lrb_k=w.lrb_k, lrb_m=w.lrb_m, lrb_eps=w.lrb_eps,
              in_dtype=w.in_dtype)
    if head_bits is not None:
        kw["head_bits"] = list(head_bits)
    if w.model == "retnet":
        kw["gamma"] = [w.gamma] * w.heads
    if getattr(w, "hadamard", False):
        kw["hadamard"] = True
    if getattr(w, "pw_window", 0):
        kw["pw_window"] = int(w.pw_window)
    return kw


def state_bytes(**kw) -> int:
    cfg, keep = make_config(**kw)
    n = ctypes.c_size_t()
    check(lib.rsq_state_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def allocate_head_bits(decay_sq: Sequence[float], ranges: Sequence[float], mean_bits: float):
    """Per-head widths in {4, 6, 8} with mean at most mean_bits that minimise
    sum_h range_h^2 / (1 - decay_sq_h) / (2^(b_h-1) - 1)^2 (rsq_allocate_head_bits).
    decay_sq[h] = E[a_t^2] of head h's decay; ranges[h] = its typical group absmax."""
    d = np.ascontiguousarray(decay_sq, dtype=np.float32).reshape(-1)
    r = np.ascontiguousarray(ranges, dtype=np.float32).reshape(-1)
    if d.size != r.size:
        raise ValueError("decay_sq and ranges must have one entry per head")
    out = np.zeros(max(d.size, 1), dtype=np.int32)
    fp = ctypes.POINTER(ctypes.c_float)
    check(lib.rsq_allocate_head_bits(d.ctypes.data_as(fp), r.ctypes.data_as(fp), int(d.size),
                                     float(mean_bits), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
    return [int(b) for b in out[:d.size]]


def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


class State:
    """A quantized recurrent state of batch x heads tiles in caller-owned device memory.

    The buffer is a torch uint8 tensor owned by this object (or passed in);
    the library keeps only a small host handle.
    """

    def __init__(self, device="cuda", buffer=None, attach=False, stream=None, **kw):
        torch = _torch()
        self.kw = dict(kw)
        self.cfg, self._keep = make_config(**kw)
        n = ctypes.c_size_t()
        check(lib.rsq_state_bytes(ctypes.byref(self.cfg), ctypes.byref(n)))
        self.nbytes = n.value
        if buffer is None:
            raw = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=device)
            off = (-raw.data_ptr()) % 256
            buffer = raw[off: off + self.nbytes]
            self._raw = raw
        self.buf = buffer
        self.device = buffer.device
        h = ctypes.c_void_p()
        check(lib.rsq_state_alloc(ctypes.byref(self.cfg), ctypes.c_void_p(buffer.data_ptr()),
                                  buffer.numel(), _abi.ATTACH if attach else _abi.INIT_ZERO,
                                  _stream_ptr(stream), ctypes.byref(h)))
        self.h = h
        self.layout = _abi.Layout()
        check(lib.rsq_state_layout(self.h, ctypes.byref(self.layout)))
        self.model = kw["model"]
        self.batch, self.heads = int(kw["batch"]), int(kw["heads"])
        self.d_k, self.d_v, self.group = int(kw["d_k"]), int(kw["d_v"]), int(kw["group"])
        self.in_bf16 = kw.get("in_dtype", "f32") == "bf16"
        self.scale_f16 = kw.get("scale_dtype", "f32") == "f16"
        self.cap = int(kw.get("lrb_k", 0)) + int(kw.get("lrb_m", 0)) if int(kw.get("lrb_m", 0)) > 0 else 0
        # a pure-write window keeps its W pairs in the same sections, as E4M3 bytes
        self.pw = int(kw.get("pw_window", 0))
        if self.pw:
            self.cap = self.pw
        self.yoked = kw.get("scale_mode") == "yoked"
        self._sections = [self._tile_sections(hh) for hh in range(self.heads)]

    def close(self):
        """Free the host handle (the device buffer stays with its tensor)."""
        h = getattr(self, "h", None)
        if h is not None and h.value:
            _abi.lib.rsq_state_free(h)
        self.h = None

    def __del__(self):
        # at interpreter exit the binding may already be torn down; the handle
        # is a small host allocation that the exiting process releases anyway
        try:
            self.close()
        except (AttributeError, TypeError):
            pass

    # ------------------------------------------------------------------ calls
    def _ptr(self, t, dtype, shape, name):
        torch = _torch()
        if t is None:
            return None
        if t.device != self.device:
            raise ValueError("%s must be on %s" % (name, self.device))
        if t.dtype != dtype:
            raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if tuple(t.shape) != tuple(shape):
            raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
        return ctypes.c_void_p(t.data_ptr())

    def decode_step(self, q, k, v, alpha=None, beta=None, out=None, stream=None):
        """One decode step; returns o_t (fp32 [batch, heads, d_v])."""
        torch = _torch()
        B, H, dk, dv = self.batch, self.heads, self.d_k, self.d_v
        idt = torch.bfloat16 if self.in_bf16 else torch.float32
        if out is None:
            out = torch.empty((B, H, dv), dtype=torch.float32, device=self.device)
        ashape = (B, H, dk) if self.model == "gla" else (B, H)
        check(lib.rsq_decode_step(
            self.h, self._ptr(q, idt, (B, H, dk), "q"), self._ptr(k, idt, (B, H, dk), "k"),
            self._ptr(v, idt, (B, H, dv), "v"),
            self._ptr(alpha, torch.float32, ashape, "alpha"), self._ptr(beta, torch.float32, (B, H), "beta"),
            self._ptr(out, torch.float32, (B, H, dv), "o"), _stream_ptr(stream)))
        return out

    def decode_step_diag(self, q, k, v, alpha, beta, acc, counts, ratio=None, out=None, stream=None):
        """One decode step with error accounting (rsq_decode_step_diag).

        acc: fp32 device tensor [tiles, 6, d_k*d_v], counts: int32 device
        tensor [tiles, 4] (read as u32), ratio: optional fp32 [tiles, d_k*d_v].
        Returns o_t like decode_step."""
        torch = _torch()
        B, H, dk, dv = self.batch, self.heads, self.d_k, self.d_v
        idt = torch.bfloat16 if self.in_bf16 else torch.float32
        if out is None:
            out = torch.empty((B, H, dv), dtype=torch.float32, device=self.device)
        ashape = (B, H, dk) if self.model == "gla" else (B, H)
        T = B * H
        check(lib.rsq_decode_step_diag(
            self.h, self._ptr(q, idt, (B, H, dk), "q"), self._ptr(k, idt, (B, H, dk), "k"),
            self._ptr(v, idt, (B, H, dv), "v"),
            self._ptr(alpha, torch.float32, ashape, "alpha"), self._ptr(beta, torch.float32, (B, H), "beta"),
            self._ptr(out, torch.float32, (B, H, dv), "o"),
            self._ptr(acc, torch.float32, (T, 6, dk * dv), "acc"),
            self._ptr(ratio, torch.float32, (T, dk * dv), "ratio"),
            self._ptr(counts, torch.int32, (T, 4), "counts"), _stream_ptr(stream)))
        return out

    def bind_step(self, q, k, v, alpha=None, beta=None, out=None, stream=None):
        """Check the step's arguments once; return a callable that issues that step.

        Each call of the returned function is one rsq_decode_step with the same
        tensors (which it keeps alive) on the same stream, without re-checking
        them: the lean form for a tight launch loop.
        """
        torch = _torch()
        B, H, dk, dv = self.batch, self.heads, self.d_k, self.d_v
        idt = torch.bfloat16 if self.in_bf16 else torch.float32
        ashape = (B, H, dk) if self.model == "gla" else (B, H)
        args = (self.h, self._ptr(q, idt, (B, H, dk), "q"), self._ptr(k, idt, (B, H, dk), "k"),
                self._ptr(v, idt, (B, H, dv), "v"),
                self._ptr(alpha, torch.float32, ashape, "alpha"), self._ptr(beta, torch.float32, (B, H), "beta"),
                self._ptr(out, torch.float32, (B, H, dv), "o"), _stream_ptr(stream))
        keep = (q, k, v, alpha, beta, out, stream)
        f, ft = lib.rsq_decode_step, lib.rsq_decode_step_timed

        def issue(start_event=None, stop_event=None, _keep=keep):
            """start_event / stop_event: optional hipEvent_t handles (ctypes.c_void_p)
            recorded by the decode kernel's own dispatch (rsq_decode_step_timed)."""
            if start_event is None and stop_event is None:
                code = f(*args)
            else:
                code = ft(*args, start_event, stop_event)
            if code:
                check(code)
        return issue

    def merge_bypass(self, stream=None, start_event=None, stop_event=None):
        """rsq_merge_bypass; with events, rsq_merge_bypass_timed (recorded by
        the merge kernel's own dispatch)."""
        if start_event is None and stop_event is None:
            check(lib.rsq_merge_bypass(self.h, _stream_ptr(stream)))
        else:
            check(lib.rsq_merge_bypass_timed(self.h, _stream_ptr(stream), start_event, stop_event))

    def readout(self, q, out=None, stream=None):
        torch = _torch()
        B, H, dk, dv = self.batch, self.heads, self.d_k, self.d_v
        idt = torch.bfloat16 if self.in_bf16 else torch.float32
        if out is None:
            out = torch.empty((B, H, dv), dtype=torch.float32, device=self.device)
        check(lib.rsq_readout(self.h, self._ptr(q, idt, (B, H, dk), "q"),
                              self._ptr(out, torch.float32, (B, H, dv), "o"), _stream_ptr(stream)))
        return out

    def get_status(self, stream=None) -> int:
        f = ctypes.c_uint32()
        check(lib.rsq_get_status(self.h, ctypes.byref(f), _stream_ptr(stream)))
        return f.value

    def counters(self):
        t, n = ctypes.c_int64(), ctypes.c_int32()
        check(lib.rsq_state_counters(self.h, ctypes.byref(t), ctypes.byref(n)))
        return t.value, n.value

    # ------------------------------------------------------------------ layout
    def _tile_sections(self, head):
        vals = [ctypes.c_size_t() for _ in range(6)]
        bits = ctypes.c_int32()
        check(lib.rsq_tile_sections(self.h, head, *[ctypes.byref(v) for v in vals], ctypes.byref(bits)))
        ho, co, so, bu, bw, rf = [v.value for v in vals]
        return dict(head_offset=ho, codes=co, scales=so, bypass_u=bu, bypass_w=bw, ref=rf, bits=bits.value)

    def head_bits(self):
        return [s["bits"] for s in self._sections]

    def tile_offset(self, b, h):
        return self.layout.tiles + b * self.layout.batch_stride + self._sections[h]["head_offset"]

    def _tile_bytes(self, h):
        s = self._sections[h]
        end = self._sections[h + 1]["head_offset"] if h + 1 < self.heads else self.layout.batch_stride
        return end - s["head_offset"]

    def read_tiles(self, tiles: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
        """Copy tiles (flat indices b*heads + h) to the host and decode them.

        Returns codes int32 [n, d_k, d_v] (or S32 float32 for an fp32 state),
        scales float32 [n, d_k, d_v/group], U/W float32 [n, d_k|d_v, cap],
        ref float32 [n, d_k, d_v] when present, and the tile list.
        """
        torch = _torch()
        T = self.batch * self.heads
        tiles = list(range(T)) if tiles is None else [int(t) for t in tiles]
        torch.cuda.synchronize(self.device)
        out = {"tiles": np.array(tiles)}
        by_head = {}
        for pos, t in enumerate(tiles):
            by_head.setdefault(t % self.heads, []).append((pos, t))
        n = len(tiles)
        dk, dv, g = self.d_k, self.d_v, self.group
        codes = np.zeros((n, dk, dv), np.int32)
        s32 = None
        scales = np.zeros((n, dk, dv // g), np.float32)
        U = np.zeros((n, dk, self.cap), np.float32) if self.cap else None
        W = np.zeros((n, dv, self.cap), np.float32) if self.cap else None
        ref = np.zeros((n, dk, dv), np.float32) if self.yoked else None
        for h, lst in by_head.items():
            sec = self._sections[h]
            nb = self._tile_bytes(h)
            offs = [self.tile_offset(t // self.heads, h) for _, t in lst]
            idx = torch.tensor([o + i for o in offs for i in range(0, nb, 256)], device=self.device)
            rows = self.buf.view(-1)[: self.nbytes]
            # gather whole tiles as 256-byte rows
            flat = rows[: (self.nbytes // 256) * 256].view(-1, 256)
            raw = flat.index_select(0, idx // 256).cpu().numpy().reshape(len(lst), nb)
            pos = [p for p, _ in lst]
            bits = sec["bits"]
            cbytes = dk * dv * bits // 8
            dec = codec.decode_codes(raw[:, :cbytes], bits, dk, dv)
            if bits == 32:
                if s32 is None:
                    s32 = np.zeros((n, dk, dv), np.float32)
                s32[pos] = dec
            else:
                codes[pos] = dec
                scales[pos] = codec.decode_scales(raw[:, sec["scales"]:], dk, dv, g, self.scale_f16)
            if self.pw:
                U[pos] = codec.decode_e4m3_columns(raw[:, sec["bypass_u"]:], self.cap, dk)
                W[pos] = codec.decode_e4m3_columns(raw[:, sec["bypass_w"]:], self.cap, dv)
            elif self.cap:
                U[pos] = codec.decode_fp16_columns(raw[:, sec["bypass_u"]:], self.cap, dk)
                W[pos] = codec.decode_fp16_columns(raw[:, sec["bypass_w"]:], self.cap, dv)
            if self.yoked:
                ref[pos] = codec.decode_codes(raw[:, sec["ref"]: sec["ref"] + 4 * dk * dv], 32, dk, dv)
        if s32 is not None:
            out["S32"] = s32
        else:
            out["codes"] = codes
            out["scales"] = scales
        if self.cap:
            out["U"], out["W"] = U, W
        if ref is not None:
            out["ref"] = ref
        return out

    def write_tiles(self, tiles: Sequence[int], codes=None, scales=None, U=None, W=None, ref=None, S32=None):
        """Encode host arrays (shapes as read_tiles returns) into the given tiles."""
        torch = _torch()
        torch.cuda.synchronize(self.device)
        host = self.buf.view(-1)
        for pos, t in enumerate(tiles):
            h = t % self.heads
            sec = self._sections[h]
            base = self.tile_offset(t // self.heads, h)
            parts = []
            if S32 is not None:
                parts.append((0, codec.encode_codes(S32[pos:pos + 1], 32)[0]))
            if codes is not None:
                parts.append((0, codec.encode_codes(codes[pos:pos + 1], sec["bits"])[0]))
            if scales is not None:
                parts.append((sec["scales"], codec.encode_scales(scales[pos:pos + 1], self.scale_f16)[0]))
            enc = codec.encode_e4m3_columns if self.pw else codec.encode_fp16_columns
            if U is not None:
                parts.append((sec["bypass_u"], enc(U[pos:pos + 1])[0]))
            if W is not None:
                parts.append((sec["bypass_w"], enc(W[pos:pos + 1])[0]))
            if ref is not None:
                parts.append((sec["ref"], codec.encode_codes(ref[pos:pos + 1], 32)[0]))
            for off, data in parts:
                src = torch.from_numpy(np.ascontiguousarray(data)).to(self.device)
                host[base + off: base + off + src.numel()].copy_(src)
        torch.cuda.synchronize(self.device)


from .diagnostics import ErrorAccounting  # noqa: E402
