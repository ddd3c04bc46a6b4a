"""Error accounting of the low-bit recurrence on the device.

Wraps rsq_decode_step_diag (include/rsq.h): the step advances the state as a
plain decode step does and also folds its rounding errors into per-tile
accumulators ("Preserving Updates in Low-Bit Recurrent State Quantization",
Fig. 1: per-step errors R and E_T = sum a_{tau:T} R_tau; Fig. 2: the
coherent gains g_T, g_T^lost, g_T^moved; Fig. 4: lost, moved and reversed
updates; Table 5: quartiles of |b| / step and the lost fraction).

The reductions below (sums of squares, sorting for quartiles) summarise the
buffers the kernel wrote; they are read-outs, not steps of the recurrence.
"""
import numpy as np

PLANES = ("E", "D", "E_lost", "D_lost", "E_moved", "D_moved")
COUNTS = ("updated", "lost", "moved", "reversed")


def _torch():
    import torch
    return torch


class ErrorAccounting:
    """Accumulators for one State. Zeroed at construction and by reset()."""

    def __init__(self, state, keep_ratio=True):
        torch = _torch()
        self.state = state
        T = state.batch * state.heads
        n = state.d_k * state.d_v
        dev = state.device
        self.acc = torch.zeros((T, 6, n), dtype=torch.float32, device=dev)
        self.counts = torch.zeros((T, 4), dtype=torch.int32, device=dev)
        self.ratio = torch.full((T, n), -1.0, dtype=torch.float32, device=dev) if keep_ratio else None

    def reset(self):
        self.acc.zero_()
        self.counts.zero_()
        if self.ratio is not None:
            self.ratio.fill_(-1.0)

    def step(self, q, k, v, alpha=None, beta=None, out=None, stream=None):
        """One decode step with accounting; returns o_t."""
        return self.state.decode_step_diag(q, k, v, alpha, beta, self.acc, self.counts,
                                           ratio=self.ratio, out=out, stream=stream)

    # ------------------------------------------------------------ read-outs
    def plane(self, name):
        """Accumulator plane as float32 numpy [tiles, d_k, d_v] (row-major)."""
        st = self.state
        T, dk, dv = st.batch * st.heads, st.d_k, st.d_v
        p = self.acc[:, PLANES.index(name)].cpu().numpy()
        return _unchunk(p, T, dk, dv)

    def ratios(self):
        """This step's |b| / step per element, float32 numpy [tiles, d_k, d_v]
        (-1 where the element had no update or no finite step)."""
        st = self.state
        T = st.batch * st.heads
        return _unchunk(self.ratio.cpu().numpy(), T, st.d_k, st.d_v)

    def count_table(self):
        """uint32 numpy [tiles, 4]: updated, lost, moved, reversed."""
        return self.counts.cpu().numpy().view(np.uint32)

    def gains(self):
        """Per-tile coherent gains (g, g_lost, g_moved) as float64 numpy [tiles, 3]:
        sum E^2 / sum D over each tile's elements."""
        a = self.acc.double()
        e = (a[:, 0::2] ** 2).sum(dim=2)
        d = a[:, 1::2].sum(dim=2)
        return (e / d).cpu().numpy()

    def ratio_quartiles(self):
        """(Q25, Q50, Q75) of this step's |b| / step over every updated
        element of every tile: the sorted values at index floor(p (n - 1))."""
        torch = _torch()
        v = self.ratio.reshape(-1)
        v = v[v >= 0]
        if v.numel() == 0:
            return (float("nan"),) * 3
        srt = torch.sort(v).values
        n = srt.numel()
        return tuple(float(srt[int(np.floor(p * (n - 1)))]) for p in (0.25, 0.5, 0.75))


def _unchunk(p, T, dk, dv):
    """fp32 chunk layout (chunk (rb, cb) at (cb * d_k/8 + rb) * 64, row r of
    the chunk at 8 r) -> [T, d_k, d_v]."""
    return p.reshape(T, dv // 8, dk // 8, 8, 8).transpose(0, 2, 3, 1, 4).reshape(T, dk, dv)
