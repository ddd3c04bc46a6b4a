"""Closed forms of the unquantized recurrence (float64).

TEST INFRASTRUCTURE (see the package docstring).

Unrolling S_t = A_t S_{t-1} + B_t (Table 1 of "Preserving Updates in Low-Bit
Recurrent State Quantization") from S_0 = 0:

  diagonal decays (RetNet, Mamba2, GLA), B_t = k_t v_t^T:
      S_t[i, j] = sum_tau ( prod_{s=tau+1..t} a_{s,i} ) k_{tau,i} v_{tau,j}

  Gated DeltaNet, where S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1}
  + beta_t k_t v_t^T (the delta-rule row of Table 1 expanded):
      S_t = sum_tau [ M_t M_{t-1} ... M_{tau+1} ] beta_tau k_tau v_tau^T,
      M_s = alpha_s (I - beta_s k_s k_s^T)

These sums are evaluated directly, never by running the recurrence, so they
pin the oracle's fp32-state path independently.
"""
import numpy as np


def unrolled_diag(a_seq, k_seq, v_seq):
    """S_t for diagonal decays. a_seq [t, d_k], k_seq [t, d_k], v_seq [t, d_v] (one tile)."""
    a = np.asarray(a_seq, np.float64)
    k = np.asarray(k_seq, np.float64)
    v = np.asarray(v_seq, np.float64)
    t = a.shape[0]
    S = np.zeros((k.shape[1], v.shape[1]))
    for tau in range(t):
        decay = np.prod(a[tau + 1:], axis=0) if tau + 1 < t else np.ones(k.shape[1])
        S += (decay * k[tau])[:, None] * v[tau][None, :]
    return S


def unrolled_gdn(alpha_seq, beta_seq, k_seq, v_seq):
    """S_t for the Gated DeltaNet rule as the ordered-product sum (one tile)."""
    al = np.asarray(alpha_seq, np.float64)
    be = np.asarray(beta_seq, np.float64)
    k = np.asarray(k_seq, np.float64)
    v = np.asarray(v_seq, np.float64)
    t, dk = k.shape
    S = np.zeros((dk, v.shape[1]))
    for tau in range(t):
        P = np.eye(dk)
        for s in range(tau + 1, t):
            Ms = al[s] * (np.eye(dk) - be[s] * np.outer(k[s], k[s]))
            P = Ms @ P
        S += P @ (be[tau] * np.outer(k[tau], v[tau]))
    return S


def readout(S, q):
    """o = S^T q."""
    return np.asarray(S, np.float64).T @ np.asarray(q, np.float64)
