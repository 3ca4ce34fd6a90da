"""ctypes view of libbitnet_mi355x.so (the C ABI declared in include/bitnet_mi355x.h).

Argument marshalling only: every step of the forward runs in the library's
HIP kernels. Loading fails loudly when the library has not been built; there
is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
import re
import threading

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libbitnet_mi355x.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG_DIR), "include", "bitnet_mi355x.h")

# bitnet_status
OK = 0
ERR_INVALID_ARG = 1
ERR_NOT_POW2 = 2
ERR_BAD_BITS = 3
ERR_ALIGN = 4
ERR_UNSUPPORTED = 5
ERR_HIP = 6
STATUS_NAMES = {OK: "OK", ERR_INVALID_ARG: "INVALID_ARG", ERR_NOT_POW2: "NOT_POW2",
                ERR_BAD_BITS: "BAD_BITS", ERR_ALIGN: "ALIGN", ERR_UNSUPPORTED: "UNSUPPORTED",
                ERR_HIP: "HIP"}

# bitnet_dtype
F32 = 0
BF16 = 1

_i64 = ctypes.c_int64
_int = ctypes.c_int
_size = ctypes.c_size_t
_ptr = ctypes.c_void_p

# name -> (restype, argtypes); mirrors the header one to one.
SIGNATURES = {
    "bitnet_abi_version": (_int, []),
    "bitnet_last_error": (ctypes.c_char_p, []),
    "bitnet_ternarize_workspace_bytes": (_size, [_i64, _i64]),
    "bitnet_ternarize_weights": (_int, [_ptr, _i64, _i64, _ptr, _ptr, _ptr, _size, _ptr]),
    "bitnet_pack_2bit": (_int, [_ptr, _i64, _i64, _ptr, _ptr]),
    "bitnet_forward_workspace_bytes": (_size, [_i64, _i64, _i64, _int, _int]),
    "bitnet_hbitlinear_forward": (_int, [_ptr, _int, _i64, _i64, _ptr, _i64, _ptr, _int, _int,
                                         _ptr, _ptr, _size, _ptr]),
    "bitnet_quantize_activations": (_int, [_ptr, _int, _i64, _i64, _int, _int, _ptr, _ptr, _ptr,
                                           _ptr]),
    "bitnet_hbitlinear_forward_stages": (_int, [_ptr, _int, _i64, _i64, _ptr, _i64, _ptr, _int,
                                                _int, _ptr, _ptr, _size, _int, _ptr]),
    "bitnet_ternary_gemm_i32": (_int, [_ptr, _i64, _i64, _ptr, _i64, _ptr, _ptr]),
    "bitnet_ternary_linear_dequant": (_int, [_ptr, _ptr, _ptr, _i64, _i64, _ptr, _i64, _ptr,
                                             _int, _ptr, _ptr]),
    "bitnet_forward_prologue_workspace_bytes": (_size, [_i64, _i64, _i64, _int, _int]),
    "bitnet_hbitlinear_forward_prologue": (_int, [_ptr, _ptr, _int, _i64, _i64, _int, _ptr,
                                                  ctypes.c_float, _ptr, _i64, _ptr, _int, _int,
                                                  _ptr, _ptr, _size, _ptr]),
    "bitnet_quantize_activations_prologue": (_int, [_ptr, _ptr, _int, _i64, _i64, _int, _ptr,
                                                    ctypes.c_float, _int, _int, _ptr, _ptr,
                                                    _ptr]),
    "bitnet_kv_quantize": (_int, [_ptr, _int, _i64, _i64, _i64, _int, _ptr, _ptr, _ptr]),
    "bitnet_kv_quantize_packed": (_int, [_ptr, _int, _i64, _i64, _i64, _int, _ptr, _ptr, _ptr,
                                         _ptr]),
    "bitnet_tl2_bytes": (_size, [_i64, _i64]),
    "bitnet_tl2_forward_workspace_bytes": (_size, [_i64, _i64]),
    "bitnet_hbitlinear_forward_tl2_batched": (_int, [_ptr, _int, _i64, _i64, _ptr, _i64, _ptr,
                                                     _int, _ptr, _ptr, _size, _ptr]),
    "bitnet_pack_tl2": (_int, [_ptr, _i64, _i64, _ptr, _ptr]),
    "bitnet_hbitlinear_forward_tl2": (_int, [_ptr, _int, _i64, _i64, _ptr, _i64, _ptr, _int, _ptr,
                                             _ptr]),
    "bitnet_backward_workspace_bytes": (_size, [_i64, _i64, _i64, _int, _int, _int]),
    "bitnet_hbitlinear_backward": (_int, [_ptr, _int, _i64, _i64, _ptr, _ptr, _i64, _ptr, _ptr,
                                          _int, _int, _ptr, _ptr, _ptr, _size, _ptr]),
    "bitnet_hbitlinear_forward_noalloc": (_int, [_ptr, _int, _i64, _i64, _ptr, _i64, _ptr, _int,
                                                 _int, _ptr, _ptr]),
    "bitnet_stream_read": (_int, [_ptr, _size, _ptr, _ptr]),
    "bitnet_test_fail_next_launch": (None, [_int]),
}

# bytes of the fixed scratch of bitnet_hbitlinear_forward_noalloc
NOALLOC_SCRATCH_BYTES = 64 << 20

# stages of bitnet_hbitlinear_forward_stages
STAGE_QUANTIZE = 1
STAGE_PRODUCT = 2

_lock = threading.Lock()
_lib = None


class BitNetError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        self.fn = fn
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{fn} failed with BITNET_ERR_{self.status_name}: {message}")


def header_declared_functions() -> list[str]:
    """Names of the functions include/bitnet_mi355x.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitnet_[a-z0-9_]+)\s*\(", text)))


def load() -> ctypes.CDLL:
    """Load the HIP library (no HIP call is made at load)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m bit_activation_linear_amd.build_lib). There is no fallback path.")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def call(name: str, *args) -> None:
    lib = load()
    status = getattr(lib, name)(*args)
    if status != OK:
        msg = lib.bitnet_last_error().decode(errors="replace")
        raise BitNetError(name, status, msg)
