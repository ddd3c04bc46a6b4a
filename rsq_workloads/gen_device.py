"""Seeded per-step inputs drawn on the device (torch's generator).

The same distributions as gen.step_inputs, drawn by torch on the GPU so that
long full-size runs (thousands of steps of a 16384-tile workload) need no
host-side generation. The stream differs from gen.step_inputs (numpy
draws): a comparison with the oracle that uses these inputs hands the oracle
the drawn values themselves (copied to the host), never a host re-draw.

  q, k   Gaussian, L2-normalised in fp32 (Mamba2: N(0,1)/sqrt(d_k)), then
         rounded to the workload's input dtype (bf16: torch's RNE)
  v      N(0, 1)
  GDN    alpha = exp(-softplus(N(-4, 1))), beta = sigmoid(N(0, 1)) per (b, h)
  Mamba2 alpha = exp(-dt e^a), dt ~ U(0.001, 0.1) per (b, h), a per head
  GLA    alpha = sigmoid(N(3, 1)) per key channel

Step t draws from a generator seeded with seed * 1_000_003 + t. Nothing here
computes any part of the recurrence or the quantizer.
"""
from typing import Dict, Optional

from .configs import Workload


def device_step_inputs(w: Workload, t: int, a_log=None, device="cuda", seed: Optional[int] = None) -> Dict:
    """Inputs of step t (t >= 1) as device tensors: q, k, v in the input dtype,
    alpha / beta fp32. `a_log` [heads] (Mamba2's a) is required for Mamba2."""
    import torch
    if t < 1:
        raise ValueError("steps are numbered from 1")
    s = (w.seed if seed is None else seed) * 1_000_003 + t
    g = torch.Generator(device=device)
    g.manual_seed(s)
    B, H, dk, dv = w.batch, w.heads, w.d_k, w.d_v
    f32 = torch.float32
    q = torch.randn((B, H, dk), generator=g, device=device, dtype=f32)
    k = torch.randn((B, H, dk), generator=g, device=device, dtype=f32)
    if w.model == "mamba2":
        q = q / dk ** 0.5
        k = k / dk ** 0.5
    else:
        q = q / q.norm(dim=-1, keepdim=True)
        k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn((B, H, dv), generator=g, device=device, dtype=f32)
    dt = torch.bfloat16 if w.in_dtype == "bf16" else f32
    out = {"q": q.to(dt).contiguous(), "k": k.to(dt).contiguous(), "v": v.to(dt).contiguous(),
           "alpha": None, "beta": None}
    if w.model == "gdn":
        x = torch.randn((B, H), generator=g, device=device, dtype=f32) - 4.0
        out["alpha"] = torch.exp(-torch.nn.functional.softplus(x)).contiguous()
        out["beta"] = torch.sigmoid(torch.randn((B, H), generator=g, device=device, dtype=f32)).contiguous()
    elif w.model == "mamba2":
        if a_log is None:
            raise ValueError("Mamba2 needs the per-head a")
        d = torch.rand((B, H), generator=g, device=device, dtype=f32) * 0.099 + 0.001
        a = torch.as_tensor(a_log, dtype=f32, device=device).exp()[None, :]
        out["alpha"] = torch.exp(-d * a).contiguous()
    elif w.model == "gla":
        z = torch.randn((B, H, dk), generator=g, device=device, dtype=f32) + 3.0
        out["alpha"] = torch.sigmoid(z).contiguous()
    return out
