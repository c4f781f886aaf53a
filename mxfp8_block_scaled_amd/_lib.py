"""ctypes view of libmxfp8.so (the C ABI declared in include/mxfp8.h)."""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmxfp8.so")

# name -> (restype, argtypes), in the order of include/mxfp8.h
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_INT = ctypes.c_int
SIGNATURES = {
    "mx_scale_bytes": (_I64, [_I64, _I64]),
    "mx_status_string": (ctypes.c_char_p, [_INT]),
    "mx_last_error": (ctypes.c_char_p, []),
    "mx_quantize_dim0": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "mx_quantize_dim1": (_INT, [_P, _I64, _I64, _I64, _I64, _P, _P, _P]),
    "mx_quantize_dim0_dim1": (_INT, [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "mx_quantize_ex": (_INT, [_P, _I64, _I64, _I64, _I64, _INT, _INT, _P, _P, _P, _P, _P]),
    "mx_quantize_weight_32x32": (_INT, [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "mx_grouped_mm_fwd": (_INT, [_P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _P, _INT, _P]),
    "mx_grouped_mm_dgrad": (_INT, [_P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _P, _INT, _P]),
    "mx_grouped_mm_wgrad": (_INT, [_P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _P, _INT, _P, _I64, _P]),
    "mx_grouped_mm_wgrad_noalloc": (_INT, [_P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _P, _INT, _P]),
    "mx_grouped_mm_wgrad_workspace_bytes": (_I64, [_I32, _I64, _I64, _I64, _INT]),
    "mx_dequantize": (_INT, [_P, _P, _I64, _I64, _I64, _INT, _P, _P]),
    "mx_scales_to_logical": (_INT, [_P, _I64, _I64, _P, _P]),
    "mx_transpose_bf16": (_INT, [_P, _I64, _I64, _I64, _I64, _P, _P]),
    "mx_grouped_mm_bf16_fwd": (_INT, [_P, _P, _P, _I32, _I64, _I64, _I64, _P, _INT, _P]),
    "mx_grouped_mm_bf16_dgrad": (_INT, [_P, _P, _P, _I32, _I64, _I64, _I64, _P, _INT, _P]),
    "mx_grouped_mm_bf16_wgrad": (_INT, [_P, _P, _P, _I32, _I64, _I64, _I64, _P, _INT, _P, _I64, _P]),
    "mx_padded_rows": (_I64, [_I64, _I32]),
    "mx_check_offs": (_INT, [_P, _I32, _I64, _I32, _P, _P]),
    "mx_probe_mfma": (_INT, [_I64, _P, _P]),
    "mx_probe_mfma_dot": (_INT, [_INT, _P, _P, _P, _P, _P, _P, _P]),
    "mx_pad_quantize_dim0_dim1": (_INT, [_P, _I64, _I64, _I64, _P, _I32, _I64, _P, _P, _P, _P, _P, _P]),
    "mx_pad_quantize_ex": (_INT, [_P, _I64, _I64, _I64, _P, _I32, _I64, _INT, _P, _P, _P, _P, _P, _P]),
    "mx_grouped_mm_fwd_padded": (_INT, [_P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64, _P, _INT, _P]),
    "mx_grouped_mm_dgrad_padded": (_INT, [_P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I64, _P, _INT, _P]),
    "mx_pad_token_groups": (_INT, [_P, _I64, _I64, _I64, _P, _I32, _P, _I64, _P, _P]),
    "mx_unpad_token_groups": (_INT, [_P, _I64, _I64, _I64, _P, _I32, _P, _I64, _I64, _INT, _P]),
}

MX_OUT_F32 = 0
MX_OUT_BF16 = 1

_lib = None


class MXError(RuntimeError):
    def __init__(self, status, name, message):
        self.status = status
        super().__init__(f"{name}: {message} (status {status})")


def load():
    """Load the library once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m mxfp8_block_scaled_amd.build` "
            "(hipcc --offload-arch=gfx950). There is no fallback implementation."
        )
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def call(name, *args):
    """Call an entry point that returns a status; raise MXError on failure."""
    lib = load()
    st = getattr(lib, name)(*args)
    if st != 0:
        status = lib.mx_status_string(st).decode()
        raise MXError(st, name, f"{status}: {lib.mx_last_error().decode()}")
    return st
