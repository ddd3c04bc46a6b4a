"""C ABI host-side tests: exports, validation, state size accounting and the
documented byte layout. No GPU is used: every call here returns before the
library touches the device."""
import ctypes
import os
import re

import numpy as np
import pytest

bitrsq = pytest.importorskip("bit_recurrent_state_rsq_amd")
from bit_recurrent_state_rsq_amd import _abi, codec, make_config, state_bytes  # noqa: E402
from bit_recurrent_state_rsq_amd._abi import lib  # noqa: E402

import oracle  # noqa: E402
from oracle import accounting as acc  # noqa: E402
from rsq_workloads import CONFIGS, head_bits_for  # noqa: E402
from bit_recurrent_state_rsq_amd import config_kwargs_from  # noqa: E402

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "rsq.h")


def test_every_declared_entry_point_is_exported():
    src = open(HEADER).read()
    names = set(re.findall(r"^\s*(?:rsq_status|const char\*|int32_t)\s+(rsq_\w+)\s*\(", src, re.M))
    assert names == set(_abi.EXPORTS)
    for n in names:
        assert hasattr(lib, n)
    assert lib.rsq_abi_version() == _abi.ABI_VERSION


def _status_of(**kw):
    cfg, keep = make_config(**kw)
    n = ctypes.c_size_t()
    return lib.rsq_state_bytes(ctypes.byref(cfg), ctypes.byref(n)), lib.rsq_last_error().decode()


GOOD = dict(model="gdn", batch=2, heads=4, d_k=128, d_v=128, group=32, bits=4,
            scale_mode="persistent", scale_dtype="f16", in_dtype="bf16")


@pytest.mark.parametrize("change,code", [
    (dict(group=24), _abi.RSQ_E_INVALID),
    (dict(group=64, d_v=96), _abi.RSQ_E_INVALID),
    (dict(bits=5), _abi.RSQ_E_INVALID),
    (dict(bits=2), _abi.RSQ_E_INVALID),
    (dict(d_k=100), _abi.RSQ_E_INVALID),
    (dict(batch=0), _abi.RSQ_E_INVALID),
    (dict(scale_mode=7), _abi.RSQ_E_INVALID),
    (dict(scale_dtype="bf16"), _abi.RSQ_E_INVALID),
    (dict(trigger=0.0), _abi.RSQ_E_INVALID),
    (dict(model="retnet"), _abi.RSQ_E_INVALID),                    # RetNet without gamma
    (dict(model="gla", gamma=[0.9] * 4), _abi.RSQ_E_INVALID),      # gamma for a non-RetNet model
    (dict(lrb_k=2, lrb_m=0), _abi.RSQ_E_INVALID),
    (dict(lrb_k=1, lrb_m=15, scale_mode="yoked"), _abi.RSQ_E_UNSUPPORTED),   # yoked scales with a bypass
    (dict(model="gla", lrb_k=20, lrb_m=20), _abi.RSQ_E_UNSUPPORTED),
    (dict(model="gla", lrb_k=1, lrb_m=3, scale_mode="yoked"), _abi.RSQ_E_UNSUPPORTED),
    (dict(d_k=96), _abi.RSQ_E_UNSUPPORTED),                        # not a multiple of 128 rows
    (dict(d_k=256, d_v=256), _abi.RSQ_E_UNSUPPORTED),              # more than 32768 elements
    (dict(bits=32, bdr=True), _abi.RSQ_E_INVALID),
    (dict(head_bits=[4, 6, 8, 32]), _abi.RSQ_E_INVALID),
    # the merge of a 1024 x 32 tile with 32 bypass columns needs more LDS than a CU has
    (dict(model="gla", d_k=1024, d_v=32, lrb_k=16, lrb_m=16), _abi.RSQ_E_UNSUPPORTED),
])
def test_invalid_configurations_are_rejected(change, code):
    kw = dict(GOOD)
    kw.update(change)
    got, msg = _status_of(**kw)
    assert got == code, msg
    assert msg and msg != "no error"


def test_delta_rule_with_a_bypass_is_accepted():
    """Gated DeltaNet with the low-rank bypass at Table 6's setting (k = 1, m = 15)."""
    got, msg = _status_of(**dict(GOOD, lrb_k=1, lrb_m=15, lrb_eps=0.5, bdr=True, bdr_eps=0.3))
    assert got == _abi.RSQ_OK, msg


def test_bad_abi_version():
    cfg, keep = make_config(**GOOD)
    cfg.abi_version = 99
    n = ctypes.c_size_t()
    assert lib.rsq_state_bytes(ctypes.byref(cfg), ctypes.byref(n)) == _abi.RSQ_E_INVALID
    assert "abi_version" in lib.rsq_last_error().decode()


def test_alloc_argument_errors_before_any_device_work():
    cfg, keep = make_config(**GOOD)
    n = ctypes.c_size_t()
    assert lib.rsq_state_bytes(ctypes.byref(cfg), ctypes.byref(n)) == 0
    h = ctypes.c_void_p()
    assert lib.rsq_state_alloc(ctypes.byref(cfg), None, n.value, 0, None, ctypes.byref(h)) == _abi.RSQ_E_INVALID
    assert lib.rsq_state_alloc(ctypes.byref(cfg), ctypes.c_void_p(0x1000010), n.value, 0, None,
                               ctypes.byref(h)) == _abi.RSQ_E_INVALID          # not 256-aligned
    assert lib.rsq_state_alloc(ctypes.byref(cfg), ctypes.c_void_p(0x1000000), n.value - 1, 0, None,
                               ctypes.byref(h)) == _abi.RSQ_E_BUFFER
    assert lib.rsq_state_alloc(ctypes.byref(cfg), ctypes.c_void_p(0x1000000), n.value, 5, None,
                               ctypes.byref(h)) == _abi.RSQ_E_INVALID
    assert h.value is None


def test_calls_on_a_null_state():
    P = ctypes.c_void_p
    assert lib.rsq_decode_step(None, P(16), P(16), P(16), None, None, P(16), None) == _abi.RSQ_E_INVALID
    assert lib.rsq_merge_bypass(None, None) == _abi.RSQ_E_INVALID
    assert lib.rsq_readout(None, P(16), P(16), None) == _abi.RSQ_E_INVALID
    f = ctypes.c_uint32()
    assert lib.rsq_get_status(None, ctypes.byref(f), None) == _abi.RSQ_E_INVALID
    assert lib.rsq_state_free(None) == 0


@pytest.mark.parametrize("ci", range(5))
def test_state_bytes_equal_the_storage_formula(ci):
    """rsq_state_bytes = header (256) + head table + sum of tile payloads (codes,
    step sizes, bypass), each section padded to 256 bytes; for these workloads
    no section needs padding."""
    w = CONFIGS[ci]
    hb = head_bits_for(w)
    kw = config_kwargs_from(w, head_bits=hb if w.mixed_bits else None)
    total = state_bytes(**kw)
    sb = 2 if w.scale_dtype == "f16" else 4
    cap = w.lrb_k + w.lrb_m if w.lrb_m else 0
    payload = w.batch * sum(acc.tile_payload_bytes(int(b), w.group, sb, w.d_k, w.d_v, cap) for b in hb)
    table = -(-(256 + 32 * w.heads) // 256) * 256
    assert total == table + payload
    # and the payload matches the per-element bits accounting
    avg_bits = payload * 8 / (w.tiles * w.d_k * w.d_v)
    if not cap and not w.mixed_bits:
        a, _ = acc.bits_per_element(w.bits, w.group, 8 * sb, w.d_k, w.d_v)
        assert avg_bits == a


# ------------------------------------------------------------------ byte layout

def _chunk_by_hand(codes8x8, bits):
    """Bytes of one 8x8 chunk written out from the layout description in rsq.h."""
    out = bytearray()
    if bits == 4:
        for r in range(8):
            for c in range(4):
                out.append(((codes8x8[r][c] & 0xF) | ((codes8x8[r][c + 4] & 0xF) << 4)) & 0xFF)
    elif bits == 8:
        for r in range(8):
            for c in range(8):
                out.append(codes8x8[r][c] & 0xFF)
    elif bits == 6:
        for r in range(8):
            for c in range(4):
                hi0, hi1 = (codes8x8[r][c] >> 2) & 0xF, (codes8x8[r][c + 4] >> 2) & 0xF
                out.append(hi0 | (hi1 << 4))
        for p in range(4):
            for c in range(4):
                lo = lambda r, cc: codes8x8[r][cc] & 3
                out.append(lo(2 * p, c) | (lo(2 * p, c + 4) << 2) | (lo(2 * p + 1, c) << 4) | (lo(2 * p + 1, c + 4) << 6))
    return bytes(out)


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_codec_matches_the_documented_chunk_layout(bits):
    rng = np.random.default_rng(bits)
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    dk, dv = 16, 24
    codes = rng.integers(lo, hi + 1, size=(3, dk, dv)).astype(np.int32)
    enc = codec.encode_codes(codes, bits)
    for t in range(3):
        for cb in range(dv // 8):
            for rb in range(dk // 8):
                off = (cb * (dk // 8) + rb) * 8 * bits
                want = _chunk_by_hand(codes[t, 8 * rb:8 * rb + 8, 8 * cb:8 * cb + 8].tolist(), bits)
                assert bytes(enc[t, off:off + 8 * bits]) == want
    assert np.array_equal(codec.decode_codes(enc, bits, dk, dv), codes)


def test_codec_roundtrips_fp32_scales_and_bypass():
    rng = np.random.default_rng(0)
    S = rng.standard_normal((2, 16, 32)).astype(np.float32)
    assert np.array_equal(codec.decode_codes(codec.encode_codes(S, 32), 32, 16, 32), S)
    for f16 in (True, False):
        s = np.abs(rng.standard_normal((2, 16, 4))).astype(np.float16 if f16 else np.float32).astype(np.float32)
        assert np.array_equal(codec.decode_scales(codec.encode_scales(s, f16), 16, 32, 8, f16), s)
    U = rng.standard_normal((2, 16, 5)).astype(np.float16).astype(np.float32)
    assert np.array_equal(codec.decode_fp16_columns(codec.encode_fp16_columns(U), 5, 16), U)


@pytest.mark.parametrize("change,code", [
    (dict(hadamard=True, bdr=True), _abi.RSQ_E_UNSUPPORTED),
    (dict(hadamard=True, scale_mode="yoked"), _abi.RSQ_E_UNSUPPORTED),
    (dict(hadamard=True, bits=32), _abi.RSQ_E_UNSUPPORTED),
    (dict(hadamard=True, model="gla", lrb_k=2, lrb_m=4), _abi.RSQ_E_UNSUPPORTED),
])
def test_hadamard_rejects_unsupported_combinations(change, code):
    kw = dict(GOOD, **change)
    st, msg = _status_of(**kw)
    assert st == code, msg
    assert "Hadamard" in msg


def test_hadamard_flag_changes_the_config_identity_only_when_set():
    ok, _ = _status_of(**dict(GOOD, hadamard=True))
    assert ok == _abi.RSQ_OK
    cfg, keep = make_config(**dict(GOOD, hadamard=False))
    assert cfg.hadamard == 0
    cfg, keep = make_config(**dict(GOOD, hadamard=True))
    assert cfg.hadamard == 1


@pytest.mark.parametrize("W", [1, 8, 16])
def test_state_bytes_with_a_pure_write_window(W):
    """The window adds W E4M3 pairs (d_k + d_v bytes each) per tile, its two
    sections (keys, values) each padded to 256 bytes."""
    w = CONFIGS[1].with_(pw_window=W)
    total = state_bytes(**config_kwargs_from(w))
    pad = lambda n: -(-n // 256) * 256
    payload = w.batch * w.heads * (acc.tile_payload_bytes(4, w.group, 2, w.d_k, w.d_v)
                                   + pad(W * w.d_k) + pad(W * w.d_v))
    if W * w.d_k % 256 == 0 and W * w.d_v % 256 == 0:
        assert payload == w.batch * w.heads * acc.tile_payload_bytes(4, w.group, 2, w.d_k, w.d_v, pw=W)
    table = -(-(256 + 32 * w.heads) // 256) * 256
    assert total == table + payload


@pytest.mark.parametrize("change,code", [
    (dict(pw_window=17), _abi.RSQ_E_INVALID),
    (dict(pw_window=-1), _abi.RSQ_E_INVALID),
    (dict(pw_window=4, model="gla"), _abi.RSQ_E_UNSUPPORTED),
    (dict(pw_window=4, bits=32), _abi.RSQ_E_UNSUPPORTED),
    (dict(pw_window=4, bdr=True), _abi.RSQ_E_UNSUPPORTED),
    (dict(pw_window=4, hadamard=True), _abi.RSQ_E_UNSUPPORTED),
    (dict(pw_window=4, scale_mode="yoked"), _abi.RSQ_E_UNSUPPORTED),
])
def test_pure_write_window_rejects_bad_configurations(change, code):
    st, msg = _status_of(**dict(GOOD, **change))
    assert st == code, msg


def test_e4m3_codec_matches_the_format():
    """Host E4M3 table (product codec) against the oracle's, and a round trip."""
    from oracle import window as ow
    v = ow.e4m3_values().astype(np.float32)
    fin = np.isfinite(v)
    assert np.array_equal(codec.E4M3[fin], v[fin]) and np.array_equal(np.isnan(codec.E4M3), ~fin)
    rng = np.random.default_rng(2)
    vals = ow.fp8_round(rng.standard_normal((3, 16, 5)) * 4)
    assert np.array_equal(codec.decode_e4m3_columns(codec.encode_e4m3_columns(vals), 5, 16), vals)
