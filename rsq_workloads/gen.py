"""Seeded per-step input generators.

Each step t >= 1 of workload w draws from numpy's default_rng([w.seed, t]);
per-head static parameters come from default_rng([w.seed, 0]). The draw order
within a step is q, k, v, then the gate draws, each a full [B, H, .] array in
C order. Normalisation and gate formulas are evaluated in float64 and rounded
once to float32; bf16 inputs are then rounded from float32 to nearest-even.
Both the oracle and the GPU path receive exactly these bits.

Nothing here computes any part of the recurrence or the quantizer.
"""
from dataclasses import dataclass
from typing import Dict, List, Optional
import numpy as np

from .configs import Workload


def bf16_round(x32: np.ndarray):
    """Round float32 to bfloat16, nearest-even. Returns (float32 values, uint16 bits)."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    vals = (r.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return vals, r


def _normalized_gaussian(rng, shape):
    g = rng.standard_normal(shape)
    return g / np.sqrt(np.sum(g * g, axis=-1, keepdims=True))


def _to_input(x64: np.ndarray, in_dtype: str):
    x32 = x64.astype(np.float32)
    if in_dtype == "bf16":
        return bf16_round(x32)
    return x32, None


def static_params(w: Workload) -> Dict[str, np.ndarray]:
    """Per-head parameters fixed for the whole run."""
    out: Dict[str, np.ndarray] = {}
    if w.model == "mamba2":
        rng = np.random.default_rng([w.seed, 0])
        out["a_log"] = rng.uniform(0.0, 2.0, size=w.heads)  # a ~ U(0, 2)
    if w.model == "retnet":
        out["gamma"] = np.full(w.heads, w.gamma, dtype=np.float32)
    if w.coherence > 0:
        # per-tile persistent key and value directions, from their own stream
        rng = np.random.default_rng([w.seed, 0, 1])
        B, H = w.batch, w.heads
        if w.model == "mamba2":
            out["k_bar"] = rng.standard_normal((B, H, w.d_k)) / np.sqrt(w.d_k)
        else:
            out["k_bar"] = _normalized_gaussian(rng, (B, H, w.d_k))
        out["v_bar"] = rng.standard_normal((B, H, w.d_v))
    return out


def step_inputs(w: Workload, t: int, static: Optional[Dict] = None) -> Dict[str, np.ndarray]:
    """Inputs of decode step t (t >= 1) for every tile.

    Returns float32 arrays q, k [B, H, d_k], v [B, H, d_v] (bf16-exact when
    in_dtype is bf16), their uint16 bf16 bit patterns under q_bits/k_bits/v_bits
    when applicable, alpha ([B, H] or [B, H, d_k] float32, absent for RetNet) and
    beta ([B, H] float32, GDN only).
    """
    if t < 1:
        raise ValueError("steps are numbered from 1")
    if static is None:
        static = static_params(w)
    B, H, dk, dv = w.batch, w.heads, w.d_k, w.d_v
    rng = np.random.default_rng([w.seed, t])
    out: Dict[str, np.ndarray] = {}
    if w.model == "mamba2":
        q64 = rng.standard_normal((B, H, dk)) / np.sqrt(dk)
        k64 = rng.standard_normal((B, H, dk)) / np.sqrt(dk)
    else:
        q64 = _normalized_gaussian(rng, (B, H, dk))
        k64 = _normalized_gaussian(rng, (B, H, dk))
    v64 = rng.standard_normal((B, H, dv))
    if w.coherence > 0:
        # mix the fresh draws with the tile's persistent directions:
        # x = rho x_bar + sqrt(1 - rho^2) x_t (keys renormalised where the
        # workload normalises them)
        rho = float(w.coherence)
        mix = np.sqrt(1.0 - rho * rho)
        k64 = rho * static["k_bar"] + mix * k64
        if w.model != "mamba2":
            k64 = k64 / np.sqrt(np.sum(k64 * k64, axis=-1, keepdims=True))
        v64 = rho * static["v_bar"] + mix * v64
    for name, x in (("q", q64), ("k", k64), ("v", v64)):
        vals, bits = _to_input(x, w.in_dtype)
        out[name] = vals
        if bits is not None:
            out[name + "_bits"] = bits
    if w.model == "gdn":
        x = rng.normal(-4.0, 1.0, size=(B, H))
        softplus = np.logaddexp(0.0, x)
        out["alpha"] = np.exp(-softplus).astype(np.float32)
        out["beta"] = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, H))))).astype(np.float32)
    elif w.model == "mamba2":
        dt = rng.uniform(0.001, 0.1, size=(B, H))
        out["alpha"] = np.exp(-dt * np.exp(static["a_log"])[None, :]).astype(np.float32)
    elif w.model == "gla":
        z = rng.normal(3.0, 1.0, size=(B, H, dk))
        out["alpha"] = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    return out


@dataclass
class InputPool:
    """P consecutive steps of inputs, generated once and then cycled.

    Step t (t >= 1) of a long run uses pool entry (t - 1) % P, which keeps
    input generation out of any timed region.
    """
    workload: Workload
    steps: List[Dict[str, np.ndarray]]

    @classmethod
    def build(cls, w: Workload, size: int, first_step: int = 1) -> "InputPool":
        static = static_params(w)
        return cls(w, [step_inputs(w, first_step + i, static) for i in range(size)])

    def __len__(self) -> int:
        return len(self.steps)

    def at(self, t: int) -> Dict[str, np.ndarray]:
        return self.steps[(t - 1) % len(self.steps)]
