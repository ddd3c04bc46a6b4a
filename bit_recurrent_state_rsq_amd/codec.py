"""Host-side reading and writing of the documented state-buffer layout.

The byte layout is the one include/rsq.h documents (8x8 chunks, two's
complement codes, group-major step sizes, fp16 bypass columns). This module
turns tile bytes into numpy arrays and back; it is used for checkpoints,
inspection and tests, never on the decode path.
"""
import numpy as np


def _sext(v, bits):
    v = v.astype(np.int32)
    return np.where(v >= (1 << (bits - 1)), v - (1 << bits), v)


def decode_codes(raw: np.ndarray, bits: int, d_k: int, d_v: int) -> np.ndarray:
    """raw: uint8 [T, d_k*d_v*bits/8] -> int32 codes [T, d_k, d_v] (float32 state for bits 32)."""
    T = raw.shape[0]
    nrb, ncb = d_k // 8, d_v // 8
    ch = raw.reshape(T, ncb, nrb, 8 * bits)
    if bits == 32:
        f = ch.view(np.float32).reshape(T, ncb, nrb, 8, 8)         # [cb, rb, r, c]
        return f.transpose(0, 2, 3, 1, 4).reshape(T, d_k, d_v)
    if bits == 8:
        v = ch.view(np.int8).reshape(T, ncb, nrb, 8, 8).astype(np.int32)
    elif bits == 4:
        b = ch.reshape(T, ncb, nrb, 8, 4)
        lo = _sext(b & 0xF, 4)
        hi = _sext(b >> 4, 4)
        v = np.concatenate([lo, hi], axis=-1)
    elif bits == 6:
        b = ch[..., :32].reshape(T, ncb, nrb, 8, 4)
        h = np.concatenate([_sext(b & 0xF, 4), _sext(b >> 4, 4)], axis=-1)     # [.., r, 8]
        cr = ch[..., 32:].reshape(T, ncb, nrb, 4, 4)                            # word p, byte c
        l_even = np.concatenate([cr & 3, (cr >> 2) & 3], axis=-1)               # row 2p, cols 0..7
        l_odd = np.concatenate([(cr >> 4) & 3, (cr >> 6) & 3], axis=-1)          # row 2p+1
        lo = np.stack([l_even, l_odd], axis=4).reshape(T, ncb, nrb, 8, 8).astype(np.int32)
        v = 4 * h + lo
    else:
        raise ValueError("bits %d" % bits)
    return v.transpose(0, 2, 3, 1, 4).reshape(T, d_k, d_v).astype(np.int32)


def encode_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """int32 codes [T, d_k, d_v] (float32 state for bits 32) -> uint8 [T, bytes]."""
    T, d_k, d_v = codes.shape
    nrb, ncb = d_k // 8, d_v // 8
    c = codes.reshape(T, nrb, 8, ncb, 8).transpose(0, 3, 1, 2, 4)   # [cb, rb, r, col]
    if bits == 32:
        return np.ascontiguousarray(c.astype(np.float32)).view(np.uint8).reshape(T, -1)
    lo_, hi_ = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    if np.any(codes < lo_) or np.any(codes > hi_):
        raise ValueError("codes out of range for %d bits" % bits)
    if bits == 8:
        return np.ascontiguousarray(c.astype(np.int8)).view(np.uint8).reshape(T, -1)
    if bits == 4:
        u = (c & 0xF).astype(np.uint8)
        b = u[..., :4] | (u[..., 4:] << 4)
        return np.ascontiguousarray(b).reshape(T, -1)
    if bits == 6:
        h = ((c >> 2) & 0xF).astype(np.uint8)
        l = (c & 3).astype(np.uint8)
        nib = h[..., :4] | (h[..., 4:] << 4)                         # [.., r, 4]
        le, lo = l[..., 0::2, :], l[..., 1::2, :]                    # rows 2p and 2p+1
        cr = le[..., :4] | (le[..., 4:] << 2) | (lo[..., :4] << 4) | (lo[..., 4:] << 6)
        out = np.concatenate([nib.reshape(T, ncb, nrb, 32), cr.reshape(T, ncb, nrb, 16)], axis=-1)
        return np.ascontiguousarray(out).reshape(T, -1)
    raise ValueError("bits %d" % bits)


def decode_scales(raw: np.ndarray, d_k: int, d_v: int, group: int, f16: bool) -> np.ndarray:
    """uint8 [T, bytes] -> float32 step sizes [T, d_k, d_v/group]."""
    T, ng = raw.shape[0], d_v // group
    n = ng * d_k
    v = raw[:, : n * (2 if f16 else 4)]
    a = v.view(np.float16 if f16 else np.float32).astype(np.float32).reshape(T, ng, d_k)
    return a.transpose(0, 2, 1).copy()


def encode_scales(s: np.ndarray, f16: bool) -> np.ndarray:
    T = s.shape[0]
    a = np.ascontiguousarray(s.transpose(0, 2, 1)).astype(np.float16 if f16 else np.float32)
    return a.view(np.uint8).reshape(T, -1)


def decode_fp16_columns(raw: np.ndarray, cap: int, dim: int) -> np.ndarray:
    """uint8 [T, cap*dim*2] -> float32 [T, dim, cap] (column c contiguous in storage)."""
    T = raw.shape[0]
    return raw[:, : cap * dim * 2].view(np.float16).astype(np.float32).reshape(T, cap, dim).transpose(0, 2, 1).copy()


def encode_fp16_columns(a: np.ndarray) -> np.ndarray:
    T = a.shape[0]
    return np.ascontiguousarray(a.transpose(0, 2, 1)).astype(np.float16).view(np.uint8).reshape(T, -1)


def _e4m3_table() -> np.ndarray:
    """float32 values of the 256 OCP E4M3 codes (bias 7, 3 mantissa bits,
    0x7F / 0xFF NaN)."""
    b = np.arange(256)
    e, m = (b >> 3) & 15, b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(b & 0x80, -mag, mag).astype(np.float32)


E4M3 = _e4m3_table()


def decode_e4m3_columns(raw: np.ndarray, cap: int, dim: int) -> np.ndarray:
    """uint8 [T, cap*dim] E4M3 -> float32 [T, dim, cap] (column c contiguous in storage)."""
    T = raw.shape[0]
    return E4M3[raw[:, : cap * dim].astype(np.int64)].reshape(T, cap, dim).transpose(0, 2, 1).copy()


def encode_e4m3_columns(a: np.ndarray) -> np.ndarray:
    """float32 [T, dim, cap] of values on the E4M3 grid -> uint8 [T, cap*dim]."""
    T = a.shape[0]
    x = np.ascontiguousarray(a.transpose(0, 2, 1)).reshape(T, -1).astype(np.float32)
    pos = E4M3[:127]
    mag = np.where(np.isnan(x), 0.0, np.abs(x))
    idx = np.searchsorted(pos, mag)
    if np.any(pos[np.minimum(idx, 126)] != mag):
        raise ValueError("values are not on the E4M3 grid")
    out = (idx | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), out)

