"""The five workloads, as plain data.

Model names follow Table 1 of "Preserving Updates in Low-Bit Recurrent State
Quantization": RetNet (A = gamma I), Mamba2 (A = alpha_t I), GLA
(A = Diag(alpha_t)) and GDN, the Gated DeltaNet delta rule.

Field meanings
  model        'retnet' | 'mamba2' | 'gla' | 'gdn'
  batch, heads state tiles are (b, h) pairs, batch-major
  d_k, d_v     per-head state is d_k x d_v (A_t multiplies on the left)
  steps        decode horizon
  in_dtype     'f32' | 'bf16' for q, k, v
  bits         4, 6, 8 or 32 (32 = unquantized fp32 state); ignored when
               mixed_bits is set
  mixed_bits   None, or (n_int8_first_heads, n_int6, n_int4): per-head widths
               drawn from a seeded permutation (see head_bits_for)
  head_bits    None, or an explicit tuple of per-head widths (overrides bits
               and mixed_bits)
  group        scale group size along d_v
  scale_mode   'dynamic' | 'persistent' | 'yoked'
  scale_dtype  'f32' | 'f16' (storage dtype of the per-group step size)
  trigger      persistent scales grow when absmax > trigger * qmax * s
  bdr, bdr_eps Bounded Directional Rounding on/off and its error gate
  lrb_k, lrb_m low-rank bypass: k residual columns, merge every m steps
  lrb_eps      merge threshold epsilon_L (fraction of the step size)
  gamma        RetNet decay, one value for every head
  pw_window    Gated DeltaNet only: keep the last W pure writes as FP8 pairs
               beside the low-bit history (0 = off)
  hadamard     store the state after a Walsh-Hadamard rotation of each scale
               group (the INT4+Had baseline); no BDR, bypass or yoked scales
  coherence    rho in [0, 1): k_t and v_t mix a persistent per-tile direction
               (weight rho) with the fresh draw (weight sqrt(1 - rho^2));
               0 = independent steps
  seed         base seed; step t draws from default_rng([seed, t]), t >= 1,
               static per-head parameters from default_rng([seed, 0])
"""
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple
import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    model: str
    batch: int
    heads: int
    d_k: int
    d_v: int
    steps: int
    in_dtype: str
    bits: int
    group: int
    scale_mode: str
    scale_dtype: str
    mixed_bits: Optional[Tuple[int, int, int]] = None
    head_bits: Optional[Tuple[int, ...]] = None
    trigger: float = 1.0
    bdr: bool = False
    bdr_eps: float = 0.5
    lrb_k: int = 0
    lrb_m: int = 0
    lrb_eps: float = 0.5
    gamma: float = 0.97
    seed: int = 1000
    coherence: float = 0.0
    hadamard: bool = False
    pw_window: int = 0

    @property
    def tiles(self) -> int:
        return self.batch * self.heads

    @property
    def bypass(self) -> bool:
        return self.lrb_m > 0

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def head_bits_for(w: Workload) -> np.ndarray:
    """Per-head bit widths (int32 [heads]).

    An explicit w.head_bits is returned as it is. Uniform workloads give
    w.bits for every head. A mixed workload
    (n8, n6, n4) gives INT8 to the first n8 heads and splits the remaining
    heads by a seeded permutation: the first n6 entries of
    default_rng([seed, 0]).permutation(heads - n8) become INT6, the rest INT4.
    The same assignment holds for every batch row.
    """
    if w.head_bits is not None:
        assert len(w.head_bits) == w.heads
        return np.asarray(w.head_bits, dtype=np.int32)
    if w.mixed_bits is None:
        return np.full(w.heads, w.bits, dtype=np.int32)
    n8, n6, n4 = w.mixed_bits
    assert n8 + n6 + n4 == w.heads
    out = np.empty(w.heads, dtype=np.int32)
    out[:n8] = 8
    perm = np.random.default_rng([w.seed, 0]).permutation(w.heads - n8)
    rest = np.arange(n8, w.heads)
    out[rest[perm[:n6]]] = 6
    out[rest[perm[n6:]]] = 4
    return out


CONFIGS = [
    # 0: RetNet, one 64x64 head, INT4 group 64, dynamic fp32 scales.
    Workload(name="retnet_int4_g64_dyn_b1h1_64x64", model="retnet", batch=1,
             heads=1, d_k=64, d_v=64, steps=256, in_dtype="f32", bits=4,
             group=64, scale_mode="dynamic", scale_dtype="f32", gamma=0.97,
             seed=1000),
    # 1: Gated DeltaNet, INT4 group 32, persistent fp16 scales.
    Workload(name="gdn_int4_g32_persist_b64h16_128x128", model="gdn",
             batch=64, heads=16, d_k=128, d_v=128, steps=1024,
             in_dtype="bf16", bits=4, group=32, scale_mode="persistent",
             scale_dtype="f16", trigger=1.0, seed=1001),
    # 2: Mamba2, INT8 per row (group = d_v = 64), dynamic fp32 scales.
    Workload(name="mamba2_int8_row_dyn_b128h64_128x64", model="mamba2",
             batch=128, heads=64, d_k=128, d_v=64, steps=2048,
             in_dtype="bf16", bits=8, group=64, scale_mode="dynamic",
             scale_dtype="f32", seed=1002),
    # 3: GLA, INT4 group 32, dynamic fp16 scales, BDR, rank-4 bypass, m=16.
    Workload(name="gla_int4_g32_bdr_lrb4m16_b32h8_256x128", model="gla",
             batch=32, heads=8, d_k=256, d_v=128, steps=1024,
             in_dtype="bf16", bits=4, group=32, scale_mode="dynamic",
             scale_dtype="f16", bdr=True, bdr_eps=0.5, lrb_k=4, lrb_m=16,
             lrb_eps=0.5, seed=1003),
    # 4: Gated DeltaNet serving step, per-head INT8/INT6/INT4 (4/14/14).
    Workload(name="gdn_mixed864_g32_persist_b512h32_128x128", model="gdn",
             batch=512, heads=32, d_k=128, d_v=128, steps=4096,
             in_dtype="bf16", bits=4, mixed_bits=(4, 14, 14), group=32,
             scale_mode="persistent", scale_dtype="f16", trigger=1.0,
             seed=1004),
]
