"""ctypes view of the C ABI in include/rsq.h (librsq.so next to this file).

Argument marshalling only: every step of the decode path runs in the HIP
library. Importing this module fails loudly when the library has not been
built; there is no fallback implementation.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librsq.so")

ABI_VERSION = 3

RSQ_OK = 0
RSQ_E_INVALID = -1
RSQ_E_UNSUPPORTED = -2
RSQ_E_BUFFER = -3
RSQ_E_BYPASS_FULL = -4
RSQ_E_NO_BYPASS = -5
RSQ_E_HIP = -6
RSQ_E_ATTACH = -7

RETNET, MAMBA2, GLA, GDN = 0, 1, 2, 3
MODELS = {"retnet": RETNET, "mamba2": MAMBA2, "gla": GLA, "gdn": GDN}
SCALE_DYNAMIC, SCALE_PERSISTENT, SCALE_YOKED = 0, 1, 2
SCALE_MODES = {"dynamic": SCALE_DYNAMIC, "persistent": SCALE_PERSISTENT, "yoked": SCALE_YOKED}
F32, F16, BF16 = 0, 1, 2
DTYPES = {"f32": F32, "f16": F16, "bf16": BF16}
INIT_ZERO, ATTACH = 0, 1
F_NONFINITE, F_SCALE_OVERFLOW, F_CLIPPED = 1, 2, 4

EXPORTS = ["rsq_state_bytes", "rsq_state_alloc", "rsq_state_free", "rsq_state_layout",
           "rsq_tile_sections", "rsq_state_counters", "rsq_decode_step", "rsq_decode_step_timed",
           "rsq_decode_step_diag", "rsq_merge_bypass", "rsq_merge_bypass_timed",
           "rsq_readout", "rsq_get_status", "rsq_last_error", "rsq_abi_version", "rsq_allocate_head_bits"]


class Config(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_uint32),
        ("model", ctypes.c_int32), ("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
        ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("head_bits", ctypes.POINTER(ctypes.c_int32)),
        ("scale_mode", ctypes.c_int32), ("scale_dtype", ctypes.c_int32),
        ("persist_trigger", ctypes.c_float),
        ("bdr", ctypes.c_int32),
        ("bdr_eps", ctypes.c_float),
        ("lrb_k", ctypes.c_int32), ("lrb_m", ctypes.c_int32),
        ("lrb_eps", ctypes.c_float),
        ("gamma", ctypes.POINTER(ctypes.c_float)),
        ("in_dtype", ctypes.c_int32),
        ("hadamard", ctypes.c_int32),
        ("pw_window", ctypes.c_int32),
    ]


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("header", "status", "head_table", "tiles", "batch_stride", "tile_codes",
                 "tile_scales", "tile_bypass_u", "tile_bypass_w", "tile_ref", "total")]


class Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("rsq error %d: %s" % (code, msg))
        self.code = code


def _load():
    # PyTorch supplies device memory and streams, so the library must bind to the
    # HIP runtime PyTorch loaded: import it first, and librsq.so's libamdhip64
    # dependency then resolves (by soname) to that same runtime.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError("librsq.so is not built (expected at %s); run "
                          "`python bit_recurrent_state_rsq_amd/build.py`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    pcfg = ctypes.POINTER(Config)
    sig = {
        "rsq_state_bytes": (I32, [pcfg, ctypes.POINTER(SZ)]),
        "rsq_state_alloc": (I32, [pcfg, P, SZ, I32, P, ctypes.POINTER(P)]),
        "rsq_state_free": (I32, [P]),
        "rsq_state_layout": (I32, [P, ctypes.POINTER(Layout)]),
        "rsq_tile_sections": (I32, [P, I32] + [ctypes.POINTER(SZ)] * 6 + [ctypes.POINTER(I32)]),
        "rsq_state_counters": (I32, [P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(I32)]),
        "rsq_decode_step": (I32, [P, P, P, P, P, P, P, P]),
        "rsq_decode_step_timed": (I32, [P, P, P, P, P, P, P, P, P, P]),
        "rsq_decode_step_diag": (I32, [P, P, P, P, P, P, P, P, P, P, P]),
        "rsq_merge_bypass": (I32, [P, P]),
        "rsq_merge_bypass_timed": (I32, [P, P, P, P]),
        "rsq_readout": (I32, [P, P, P, P]),
        "rsq_get_status": (I32, [P, ctypes.POINTER(ctypes.c_uint32), P]),
        "rsq_last_error": (ctypes.c_char_p, []),
        "rsq_abi_version": (I32, []),
        "rsq_allocate_head_bits": (I32, [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float), I32,
                                         ctypes.c_float, ctypes.POINTER(I32)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if lib.rsq_abi_version() != ABI_VERSION:
        raise ImportError("librsq.so ABI %d, binding expects %d" % (lib.rsq_abi_version(), ABI_VERSION))
    return lib


lib = _load()


def check(code):
    if code != RSQ_OK:
        raise Error(code, lib.rsq_last_error().decode())
    return code
