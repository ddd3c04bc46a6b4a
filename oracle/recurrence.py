"""The recurrence, the quantizer, BDR, the bypass and its merge, written out.

TEST INFRASTRUCTURE (see the package docstring).

Sources (all on the page "Preserving Updates in Low-Bit Recurrent State
Quantization" unless noted):
  * Table 1: decay A_t and update B_t for RetNet, Mamba2, GLA, Gated DeltaNet.
  * Abstract: the state is requantized after every update; the Low-Rank
    Bypass (LRB) accumulates small updates in a low-rank buffer and merges its
    sufficiently large elements into the state periodically; Bounded
    Directional Rounding (BDR) rounds elements that moved opposite to their
    update toward the update instead.
  * Fig. 3: LRB writes into the quantized state every m steps.
  * Fig. 4: the three ways rounding distorts an update d (lost, moved,
    reversed) and the BDR correction.
  * Table 2 / Table 6: INT4 stored at 4.50 bits (group 32 with a 16-bit
    step size); LRB hyperparameters k, m, eps_L, eps_B.
  * Abstract of "When Dynamic Scaling Fails: A Scale-State Feedback Governs
    Recurrent-State Quantization in Linear-Attention and SSM LLMs": dynamic
    scaling, persistent scaling, and scales yoked to a full-precision
    reference.

Readings taken where the pages are silent (each is also listed in the design
notes of the repository):
  R1  The step is S_t = A_t S_{t-1} + B_t; S is d_k x d_v and A_t acts on the
      left (Diag(alpha_t) scales key rows).
  R2  Readout o_t = S_t^T q_t uses the updated state before requantization.
  R3  Symmetric step-size scale per group of g consecutive columns of one row:
      codes c in [-2^(b-1), 2^(b-1)-1], value c*s. Dynamic: s = absmax/qmax
      with qmax = 2^(b-1)-1. An all-zero group (or a scale that rounds to 0)
      stores s = 0 and codes 0.
  R4  Persistent: s grows to absmax/qmax only when absmax > trigger*qmax*s;
      it never shrinks.
  R5  Yoked: absmax is taken over a float32 reference state that follows the
      same recurrence without quantization.
  R6  Requantization rounds the exact product x * RN(1/s) to the nearest
      integer, ties to even, then clamps to the code range.
  R7  BDR: the update of element (i, j) has sign sigma = sign(k_i) sign(w_j)
      (sign(L_ij) at a merge). The element is reversed when sigma != 0 and
      the new value c*s lies strictly on the other side of the no-update value
      r (the decayed old value; the old value itself at a merge). A reversed
      element moves one code toward its update, c + sigma, when the new error
      |x - (c + sigma) s| stays within (0.5 + eps_B) s.
  R8  LRB: every update goes into the bypass as one fp16 column pair
      (U[:, n] = k, W[:, n] = w); between merges the quantized state only
      decays, and U decays with it: U <- fp16(Diag(a) U), the exact product
      rounded once to binary16. A merge builds
      L = U W^T, adds the elements with |L_ij| > eps_L * s_iG to the state,
      requantizes with BDR (sigma = sign(L_ij)), and keeps the best rank-k
      approximation of the rest as balanced fp16 factors; n becomes k.
  R9  The canonical fp32 chain (mode 'f32'):
        c1_iG = fl(a_i s_iG),  r_ij = fl(c_ij c1_iG)
        GDN:  u_j = pairwise sum over i of fl(k_i fl(c_ij s_iG)),
              w_j = fl(beta fl(v_j - fl(alpha u_j)))
        x_ij = fma(k_i, w_j, r_ij)
        s' from fl(m / qmax) (correctly rounded), then the storage dtype
        inv = RN(1/s'); y = x inv (exact); c = clamp(RNE(y))
      The readout o_t is compared with a tolerance, so its order is free.
  R10 Gated DeltaNet with a bypass: the state read by the retrieval is the
      stored state plus the bypass, S_{t-1} = s_hat + U W^T, so
      u = s_hat^T k + W (U^T k). U and W are the factors before this step's
      decay and append. In mode 'f32' each term keeps R9's rules:
        u~_j = pairwise sum over i of fl(k_i s_hat_ij)         (R9)
        z_c  = pairwise sum over i of fl(U_ic k_i)             (the same tree)
        b_j  = W_j0 z_0 + W_j1 z_1 + ... in column order, one fused
               multiply-add per column, from 0
        u_j  = fl(u~_j + b_j)
      then w_j = fl(beta fl(v_j - fl(alpha u_j))) as without a bypass. The
      whole update k w^T goes into the bypass (R8).
"""
from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Tuple
import numpy as np

from .fp import F32, F64, Arith, f16_round, f16_of_exact

FORGIVE = 1e-6   # decision-boundary window, in the units of each decision


def qrange(bits):
    """Code range [lo, hi] and qmax for b-bit symmetric codes (R3)."""
    bits = np.asarray(bits)
    lo = -(2 ** (bits - 1))
    hi = 2 ** (bits - 1) - 1
    return lo, hi, hi


@dataclass
class OState:
    """State of T tiles. Arrays are per tile, tiles batch-major.

    codes   int32 [T, d_k, d_v]     quantized tiles (zeros when bits == 32)
    scales  float32 [T, d_k, d_v/g] stored step sizes (exact in scale dtype)
    bits    int32 [T]               code width per tile, or 32 for fp32 state
    S32     float32 [T, d_k, d_v]   fp32 state (bits == 32 only)
    U, W    float32 [T, d_k, cap], [T, d_v, cap] fp16-exact bypass factors
    n       bypass columns in use
    ref     float32 [T, d_k, d_v]   yoked reference state
    t       steps taken
    flags   status bits (1 non-finite, 2 fp16 scale overflow, 4 clipped)
    """
    codes: np.ndarray
    scales: np.ndarray
    bits: np.ndarray
    S32: Optional[np.ndarray] = None
    U: Optional[np.ndarray] = None
    W: Optional[np.ndarray] = None
    n: int = 0
    ref: Optional[np.ndarray] = None
    t: int = 0
    flags: int = 0

    def copy(self) -> "OState":
        cp = lambda a: None if a is None else a.copy()
        return OState(self.codes.copy(), self.scales.copy(), self.bits.copy(),
                      cp(self.S32), cp(self.U), cp(self.W), self.n,
                      cp(self.ref), self.t, self.flags)

    def dequant(self) -> np.ndarray:
        """Dense float64 state: c*s (+ U W^T when a bypass is present)."""
        if self.S32 is not None:
            return self.S32.astype(np.float64)
        g = self.codes.shape[2] // self.scales.shape[2]
        s = np.repeat(self.scales.astype(np.float64), g, axis=2)
        S = self.codes.astype(np.float64) * s
        if self.U is not None and self.n > 0:
            S = S + np.einsum("tic,tjc->tij", self.U[:, :, :self.n].astype(np.float64),
                              self.W[:, :, :self.n].astype(np.float64))
        return S


NONFINITE, SCALE_OVERFLOW, CLIPPED = 1, 2, 4


def tile_bits(w, head_bits=None) -> np.ndarray:
    from rsq_workloads import head_bits_for
    hb = head_bits_for(w) if head_bits is None else np.asarray(head_bits, np.int32)
    return np.tile(hb, w.batch).astype(np.int32)


def zero_state(w, head_bits=None) -> OState:
    """Initial state (reading: codes 0, scales 0, empty bypass, zero reference)."""
    T, dk, dv = w.tiles, w.d_k, w.d_v
    bits = tile_bits(w, head_bits)
    st = OState(codes=np.zeros((T, dk, dv), np.int32),
                scales=np.zeros((T, dk, dv // w.group), np.float32), bits=bits)
    if np.all(bits == 32):
        st.S32 = np.zeros((T, dk, dv), np.float32)
    elif np.any(bits == 32):
        raise ValueError("fp32 and quantized tiles cannot be mixed")
    if w.lrb_m > 0:
        cap = w.lrb_k + w.lrb_m
        st.U = np.zeros((T, dk, cap), np.float32)
        st.W = np.zeros((T, dv, cap), np.float32)
    if w.scale_mode == "yoked":
        st.ref = np.zeros((T, dk, dv), np.float32)
    return st


def _flat(w, x):
    return None if x is None else np.asarray(x).reshape((w.tiles,) + np.asarray(x).shape[2:])


def decay_rows(w, inp, static=None) -> np.ndarray:
    """Per-row decay a_i of every tile, float32 [T, d_k] (Table 1, column A_t).

    RetNet gamma (per head), Mamba2 and GDN alpha_t (per tile), GLA alpha_t,i
    (per key channel).
    """
    T, dk = w.tiles, w.d_k
    if w.model == "retnet":
        gamma = (static or {}).get("gamma")
        if gamma is None:
            gamma = np.full(w.heads, w.gamma, np.float32)
        g = np.tile(np.asarray(gamma, np.float32), w.batch)
        return np.broadcast_to(g[:, None], (T, dk)).astype(np.float32)
    alpha = _flat(w, inp["alpha"]).astype(np.float32)
    if w.model == "gla":
        return alpha.reshape(T, dk)
    return np.broadcast_to(alpha.reshape(T, 1), (T, dk)).astype(np.float32)


def _to_storage(x, w, A: Arith):
    """Round a computed step size to the scale storage dtype."""
    if w.scale_dtype == "f16":
        with np.errstate(over="ignore"):
            return np.asarray(x).astype(np.float16).astype(np.float32)
    return np.asarray(x).astype(np.float32)


def scale_rule(m, s_old, qmax, w, A: Arith):
    """New stored step size per group (R3-R5). m, s_old: [T, d_k, ng]; qmax: [T,1,1].

    Returns (s_new float32, grew mask, threshold used by the persistent rule).
    """
    ratio = A.div(m, A.c(qmax))
    fresh = _to_storage(ratio, w, A)
    if w.scale_mode in ("dynamic", "yoked"):
        return fresh, np.ones(m.shape, bool), None
    thr = A.mul(A.mul(w.trigger, A.c(qmax)), s_old)
    grew = A.c(m) > thr
    return np.where(grew, fresh, s_old).astype(np.float32), grew, thr


def quantize_group_codes(x, s_full, bits_full, A: Arith):
    """RNE codes of x on the grid s_full (R6). Returns (codes, y, clipped mask).

    f32 mode: inv = RN(1/s) and y = x*inv exactly (a product of two float32 is
    exact in float64). f64 mode: y = x/s. s = 0 gives code 0.
    """
    lo, hi, _ = qrange(bits_full)
    zero = s_full == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        if A.name == "f32":
            inv = np.where(zero, np.float32(0), np.float32(1) / np.where(zero, 1, s_full).astype(np.float32))
            y = x.astype(np.float64) * inv.astype(np.float64)
        else:
            y = np.where(zero, 0.0, x.astype(np.float64) / np.where(zero, 1, s_full).astype(np.float64))
    rn = np.rint(y)
    clipped = np.isfinite(rn) & ((rn < lo) | (rn > hi))
    rn = np.where(np.isfinite(rn), rn, np.where(y > 0, hi, lo))
    c = np.clip(rn, lo, hi).astype(np.int32)
    return c, y, clipped


def bdr_apply(c, x, r, sigma, s_full, bits_full, eps, A: Arith):
    """Bounded Directional Rounding (R7). Returns (codes, reversed, corrected)."""
    lo, hi, _ = qrange(bits_full)
    val = A.mul(c.astype(A.dt), s_full)
    rev = (sigma != 0) & (s_full > 0) & (
        ((sigma > 0) & (val < A.c(r))) | ((sigma < 0) & (val > A.c(r))))
    cand = np.clip(c + sigma, lo, hi).astype(np.int32)
    err = np.abs(A.sub(x, A.mul(cand.astype(A.dt), s_full)))
    gate = err <= A.mul(A.add(0.5, eps), s_full)
    fix = rev & gate & (cand != c)
    return np.where(fix, cand, c).astype(np.int32), rev, fix


def _expand(a, g):
    return np.repeat(a, g, axis=2)


def _group_absmax(x, g):
    T, dk, dv = x.shape
    return np.max(np.abs(x.reshape(T, dk, dv // g, g)), axis=3)


def _fp16_midpoint_near(ratio32):
    """True where a float32 value lies within FORGIVE binary16 spacings of a binary16
    rounding midpoint (the storage rounding of a scale, measured like a code rounding:
    in units of the grid being rounded to)."""
    r = np.abs(ratio32.astype(np.float64))
    h16 = r.astype(np.float16)
    h = h16.astype(np.float64)
    nxt = np.nextafter(h16, np.float16(np.inf)).astype(np.float64)
    prv = np.nextafter(h16, np.float16(0)).astype(np.float64)
    with np.errstate(invalid="ignore"):
        near = ((np.abs(r - 0.5 * (h + nxt)) < FORGIVE * (nxt - h)) |
                (np.abs(r - 0.5 * (h + prv)) < FORGIVE * (h - prv)))
    return near & (r > 0) & np.isfinite(r) & np.isfinite(h)


def _requantize(st, w, x, r, sigma, A, xref=None):
    """Scale rule + RNE + optional BDR for the whole state. Returns (codes, scales, diag)."""
    g = w.group
    bits_full = st.bits[:, None, None]
    _, _, qmax = qrange(bits_full)
    m = _group_absmax(xref if xref is not None else x, g)
    s_new, grew, thr = scale_rule(m, st.scales, qmax, w, A)
    flags = 0
    if w.scale_dtype == "f16" and np.any(np.isinf(s_new)):
        flags |= SCALE_OVERFLOW
    s_full = _expand(s_new, g)
    c, y, clipped = quantize_group_codes(x, s_full, bits_full, A)
    c_rtn = c.copy()
    rev = fix = np.zeros(c.shape, bool)
    if w.bdr:
        c, rev, fix = bdr_apply(c, x, r, sigma, s_full, bits_full, w.bdr_eps, A)
    if np.any(clipped):
        flags |= CLIPPED
    # decision-boundary windows used by the parity harness
    frac = y - np.floor(y)
    near = np.abs(frac - 0.5) < FORGIVE
    gnear = np.zeros(m.shape, bool)
    if thr is not None:
        with np.errstate(invalid="ignore", divide="ignore"):
            gnear |= np.abs(m.astype(np.float64) - thr.astype(np.float64)) <= FORGIVE * np.abs(thr.astype(np.float64))
    if w.scale_dtype == "f16":
        ratio = A.div(m, A.c(qmax)).astype(np.float32)
        gnear |= _fp16_midpoint_near(ratio) & (grew if thr is not None else True)
    near |= _expand(gnear, g)
    diag = dict(y=y, m=m, grew=grew, thr=thr, s_new=s_new, c_rtn=c_rtn,
                reversed=rev, corrected=fix, clipped=clipped, near=near,
                group_near=gnear)
    return c, s_new, flags, diag


def _retrieval(w, A, k, shat_or_S):
    """Gated DeltaNet retrieval u_j = sum_i k_i S_ij (R9: pairwise over i)."""
    terms = A.mul(k[:, :, None], shat_or_S)
    return A.tree_sum(terms, axis=1)


def _bypass_retrieval(A, k, U, W):
    """The bypass's share of the Gated DeltaNet retrieval, b = W (U^T k) (R10).

    k [T, d_k]; U [T, d_k, n], W [T, d_v, n] (binary16 values). Returns b [T, d_v]:
    z_c = pairwise sum over rows of fl(U_ic k_i), then b_j accumulated over the
    columns in order with one fused multiply-add each.
    """
    z = A.tree_sum(A.mul(U, k[:, :, None]), axis=1)          # [T, n]
    b = A.c(np.zeros(W.shape[:2]))
    for c in range(U.shape[2]):
        b = A.c(A.fma(W[:, :, c], z[:, c][:, None], b))
    return b


def step(st: OState, inp: Dict, w, A: Arith = F32, static=None):
    """One decode step of every tile (Table 1 + R1-R9).

    inp holds q, k ([B, H, d_k]), v ([B, H, d_v]) as float32 values, and
    alpha / beta as the model needs. Returns (new state, o [T, d_v] float64,
    diag dict).
    """
    T, dk, dv, g = w.tiles, w.d_k, w.d_v, w.group
    q = A.c(_flat(w, inp["q"]))
    k = A.c(_flat(w, inp["k"]))
    v = A.c(_flat(w, inp["v"]))
    a = decay_rows(w, inp, static)                      # [T, dk]
    gdn = w.model == "gdn"
    if gdn:
        alpha = A.c(_flat(w, inp["alpha"])).reshape(T)
        beta = A.c(_flat(w, inp["beta"])).reshape(T)
    new = st.copy()
    new.t = st.t + 1
    diag: Dict = {}

    # ---- fp32 state (bits == 32): S_t = A_t S_{t-1} + B_t, no quantizer
    if st.S32 is not None:
        S = st.S32
        r = A.mul(a[:, :, None], S)
        if gdn:
            u = _retrieval(w, A, k, S)
            wv = A.mul(beta[:, None], A.sub(v, A.mul(alpha[:, None], u)))
        else:
            wv = v
        x = A.c(A.fma(k[:, :, None], wv[:, None, :], r))
        new.S32 = x
        o = np.einsum("ti,tij->tj", q.astype(np.float64), x.astype(np.float64))
        if not np.all(np.isfinite(x)):
            new.flags |= NONFINITE
        return new, o, dict(x=x, w=wv)

    codes_f = st.codes.astype(A.dt)
    s_full = _expand(st.scales, g)
    # 1. dequantize and decay: r = fl(c * fl(a * s))
    c1 = A.mul(a[:, :, None], st.scales)
    r = A.mul(codes_f, _expand(c1, g))
    # 2. retrieval (GDN): w = beta (v - alpha * S^T k)
    if gdn:
        shat = A.mul(codes_f, s_full)
        u = _retrieval(w, A, k, shat)
        if st.U is not None and st.n > 0:
            u = A.add(u, _bypass_retrieval(A, k, st.U[:, :, :st.n], st.W[:, :, :st.n]))
        wv = A.mul(beta[:, None], A.sub(v, A.mul(alpha[:, None], u)))
        diag["u"] = u
    else:
        wv = v
    diag["w"] = wv
    sigma = (np.sign(k)[:, :, None] * np.sign(wv)[:, None, :]).astype(np.int32)
    # 3. update
    if st.U is not None:
        cap = st.U.shape[2]
        if st.n >= cap:
            raise ValueError("bypass full: merge first")
        n = st.n
        # the exact product a_i U_ic (float32 x binary16 fits float64) rounded once to binary16
        new.U[:, :, :n] = f16_of_exact(a[:, :, None].astype(np.float64) * st.U[:, :, :n].astype(np.float64))
        new.U[:, :, n] = f16_round(k)
        new.W[:, :, n] = f16_round(wv)
        new.n = n + 1
        x = A.c(r)
        sigma = np.zeros_like(sigma)          # no update reaches the state (R8)
    else:
        x = A.c(A.fma(k[:, :, None], wv[:, None, :], r))
    if not np.all(np.isfinite(x)):
        new.flags |= NONFINITE
    # 4. readout from the pre-requantization state (R2)
    o = np.einsum("ti,tij->tj", q.astype(np.float64), x.astype(np.float64))
    if new.U is not None and new.n > 0:
        z = np.einsum("tic,ti->tc", new.U[:, :, :new.n].astype(np.float64), q.astype(np.float64))
        o = o + np.einsum("tjc,tc->tj", new.W[:, :, :new.n].astype(np.float64), z)
    # yoked reference: the same recurrence in fp32 without quantization (R5)
    xref = None
    if st.ref is not None:
        rr = A.mul(a[:, :, None], st.ref)
        if gdn:
            uref = _retrieval(w, A, k, st.ref)
            wref = A.mul(beta[:, None], A.sub(v, A.mul(alpha[:, None], uref)))
        else:
            wref = v
        xref = A.c(A.fma(k[:, :, None], wref[:, None, :], rr))
        new.ref = xref
    # 5-7. scale rule, requantization, BDR
    c, s_new, fl, qd = _requantize(st, w, x, r, sigma, A, xref)
    new.codes, new.scales = c, s_new
    new.flags |= fl
    diag.update(qd)
    diag["x"] = x
    diag["r"] = r
    diag["sigma"] = sigma
    return new, o, diag


def merge(st: OState, w, A: Arith = F32):
    """Low-Rank Bypass merge (R8), called after every m-th step.

    L = U W^T accumulated over bypass columns in index order
    (f32: L <- fl(L + fl(U_c W_c)), the fp16 products are exact in float32);
    M = |L| > fl(eps_L s); x = s_hat + L on M; requantize with BDR
    (sigma = sign(L) on M, reference r = s_hat); the residual L on not-M is
    replaced by its best rank-k approximation (SVD), stored as balanced fp16
    factors U_k S_k^(1/2), V_k S_k^(1/2) with each stored U column's
    largest-magnitude entry (the first one on ties) positive; n = k.
    Returns (new state, diag with L, M, R and the singular values of R).
    """
    if st.U is None:
        raise ValueError("no bypass")
    g, n, k = w.group, st.n, w.lrb_k
    T, dk, dv = st.codes.shape
    L = A.c(np.zeros((T, dk, dv)))
    for c in range(n):
        L = A.add(L, A.mul(st.U[:, :, c][:, :, None], st.W[:, :, c][:, None, :]))
    s_full = _expand(st.scales, g)
    shat = A.mul(st.codes.astype(A.dt), s_full)
    thr = A.mul(w.lrb_eps, s_full)
    M = np.abs(L) > thr
    x = A.c(np.where(M, A.add(shat, L), shat))
    sigma = (np.sign(L) * M).astype(np.int32)
    new = st.copy()
    c, s_new, fl, qd = _requantize(st, w, x, shat, sigma, A)
    # the merge-threshold window
    near_m = np.abs(np.abs(L.astype(np.float64)) - thr.astype(np.float64)) < FORGIVE * s_full
    qd["near"] = qd["near"] | near_m
    new.codes, new.scales = c, s_new
    new.flags |= fl
    if not np.all(np.isfinite(x)):
        new.flags |= NONFINITE
    R = np.where(M, 0.0, L.astype(np.float64))
    new.U[:] = 0
    new.W[:] = 0
    svals = np.zeros((T, min(dk, dv)))
    for ti in range(T):
        Uu, S, Vt = np.linalg.svd(R[ti], full_matrices=False)
        svals[ti] = S
        for j in range(min(k, S.size)):       # rank <= min(d_k, d_v): further columns stay 0
            uc = f16_round(Uu[:, j] * np.sqrt(S[j]))
            wc = f16_round(Vt[j, :] * np.sqrt(S[j]))
            # sign fixed on the stored column (binary16 rounding is odd-symmetric)
            if uc[np.argmax(np.abs(uc))] < 0:
                uc, wc = -uc, -wc
            new.U[ti, :, j] = uc
            new.W[ti, :, j] = wc
    new.n = k
    qd.update(L=L, M=M, R=R, svals=svals, x=x)
    return new, qd


def readout(st: OState, q, w) -> np.ndarray:
    """o = deq(S)^T q (+ W (U^T q)), float64 [T, d_v]; reads the state only."""
    qf = _flat(w, q).astype(np.float64)
    return np.einsum("ti,tij->tj", qf, st.dequant())
