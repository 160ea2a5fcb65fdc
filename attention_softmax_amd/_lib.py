"""ctypes loader for libsms.so (the C ABI of include/sms.h).

torch is imported before the library is opened, so libsms.so binds to the HIP
runtime torch already loaded and torch's stream handles and device pointers are
valid inside it. There is no fallback: if the library is missing, every call
raises.
"""

import ctypes
import os
import threading

import torch  # noqa: F401  (must be loaded first; see module docstring)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsms.so")

# Mirrors of the enums in include/sms.h.
SMS_OK = 0
STATUS_NAMES = {0: "SMS_OK", 1: "SMS_ERR_NULL", 2: "SMS_ERR_SHAPE", 3: "SMS_ERR_STRIDE",
                4: "SMS_ERR_DTYPE", 5: "SMS_ERR_MASK_MODE", 6: "SMS_ERR_ALIGN", 7: "SMS_ERR_HIP",
                8: "SMS_ERR_CAUSAL", 9: "SMS_ERR_WORKSPACE"}
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}
MASK_MODES = {"none": 0, "sq_sk": 1, "b_sq_sk": 2, "b_1_sk": 3, "full": 4, "key_lengths": 5}
MASK_BOOL = 0x10
CAUSAL_CODES = {"none": 0, "top_left": 1, "bottom_right": 2}
EXPORTS = ("sms_forward", "sms_backward", "sms_forward_ws", "sms_backward_ws",
           "sms_forward_noalloc", "sms_noalloc_scratch_bytes",
           "sms_workspace_bytes", "sms_attention_forward", "sms_attention_backward",
           "sms_attention_workspace_bytes", "sms_max_sk", "sms_path",
           "sms_copy_reference", "sms_status_str", "sms_abi_version")
ABI_VERSION = 7

_lock = threading.Lock()
_lib = None


class SmsError(RuntimeError):
    """A non-OK status returned by libsms.so."""

    def __init__(self, fn, status, text):
        self.status = status
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)} ({text})")


def _declare(L):
    i64, vp, f32, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    strides = ctypes.POINTER(ctypes.c_int64)
    L.sms_forward.argtypes = [vp, strides, vp, i32, vp, strides, i32, i64, i64, i64, i64, f32,
                              i32, vp]
    L.sms_forward.restype = i32
    L.sms_backward.argtypes = [vp, strides, vp, strides, vp, strides, i32, i64, i64, i64, i64,
                               f32, i32, vp]
    L.sms_backward.restype = i32
    L.sms_forward_ws.argtypes = [vp, strides, vp, i32, vp, strides, i32, i64, i64, i64, i64, f32,
                                 i32, vp, i64, vp]
    L.sms_forward_ws.restype = i32
    L.sms_backward_ws.argtypes = [vp, strides, vp, strides, vp, strides, i32, i64, i64, i64, i64,
                                  f32, i32, vp, i64, vp]
    L.sms_backward_ws.restype = i32
    L.sms_forward_noalloc.argtypes = [vp, strides, vp, i32, vp, strides, i32, i64, i64, i64, i64,
                                      f32, i32, vp]
    L.sms_forward_noalloc.restype = i32
    L.sms_noalloc_scratch_bytes.argtypes = []
    L.sms_noalloc_scratch_bytes.restype = i64
    L.sms_attention_forward.argtypes = [vp, strides, vp, strides, vp, strides, vp, i32, vp,
                                        strides, vp, i32, i64, i64, i64, i64, i64, i64, f32, i32,
                                        vp]
    L.sms_attention_forward.restype = i32
    L.sms_attention_backward.argtypes = [vp, strides, vp, strides, vp, strides, vp, strides, vp,
                                         strides, vp, vp, i32, vp, strides, vp, strides, vp,
                                         strides, i32, i64, i64, i64, i64, i64, i64, f32, i32, vp,
                                         i64, vp]
    L.sms_attention_backward.restype = i32
    L.sms_attention_workspace_bytes.argtypes = [i64, i64, i64]
    L.sms_attention_workspace_bytes.restype = i64
    L.sms_workspace_bytes.argtypes = [i32, i64, i64, i64, i64, i32]
    L.sms_workspace_bytes.restype = i64
    L.sms_max_sk.argtypes = [i32]
    L.sms_max_sk.restype = i64
    L.sms_path.argtypes = [i32, i64, i32]
    L.sms_path.restype = i32
    L.sms_copy_reference.argtypes = [vp, vp, i64, vp]
    L.sms_copy_reference.restype = i32
    L.sms_status_str.argtypes = [i32]
    L.sms_status_str.restype = ctypes.c_char_p
    L.sms_abi_version.argtypes = []
    L.sms_abi_version.restype = i32


def lib():
    """The loaded library; raises if libsms.so has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"{LIB_PATH} is missing: build it with `python -m attention_softmax_amd.build`")
            L = ctypes.CDLL(LIB_PATH)
            _declare(L)
            if L.sms_abi_version() != ABI_VERSION:
                raise ImportError(f"libsms.so ABI {L.sms_abi_version()} != {ABI_VERSION}")
            _lib = L
    return _lib


def check(fn, status):
    if status != SMS_OK:
        raise SmsError(fn, status, lib().sms_status_str(status).decode())


def strides4(values):
    return (ctypes.c_int64 * 4)(*[int(v) for v in values])
