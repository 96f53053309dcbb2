"""ctypes binding of libtq.so (the C ABI declared in include/tq.h).

Argument marshalling only: every step of the method runs in the library's
HIP kernels.  If the shared library is missing this module raises at import
time; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

# torch ships its own HIP runtime.  Importing it first makes libtq.so bind to
# that same runtime (libtq's libamdhip64.so.7 dependency is then already
# loaded), so torch's device memory and stream handles are valid in libtq's
# calls; loading libtq.so first would bring in a second HIP runtime.
import torch  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
# TQ_LIBRARY may name another build of libtq.so (for A/B timing of build options)
LIB_PATH = os.environ.get("TQ_LIBRARY") or os.path.join(HERE, "libtq.so")

TQ_OK, TQ_ERR_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_WORKSPACE, TQ_ERR_HIP = 0, -1, -2, -3, -4
TQ_MODE_MSE, TQ_MODE_PROD, TQ_MODE_GROUPED, TQ_MODE_GROUPED_PROD = 0, 1, 2, 3
TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2
TQ_STREAM_READ_SINK = 65536
MODES = {"mse": TQ_MODE_MSE, "prod": TQ_MODE_PROD, "grouped": TQ_MODE_GROUPED, "grouped_prod": TQ_MODE_GROUPED_PROD}

EXPORTED = ["tq_build_codebook", "tq_encode_keys", "tq_encode_keys_batched", "tq_encode_values", "tq_append_kv", "tq_decode_attention",
            "tq_decode_attention_append", "tq_decode_attention_noalloc", "tq_decode_attention_paged_append", "tq_decode_attention_paged", "tq_dequantize_keys", "tq_dequantize_values", "tq_channel_moments",
            "tq_select_outlier_channels", "tq_status_string", "tq_idx_row_bytes", "tq_stream_read"]


class TqError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (fn, status_string(status), status))


class KeyConfig(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("mode", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("bits_outlier", ctypes.c_int32), ("bits_normal", ctypes.c_int32),
                ("d_outlier", ctypes.c_int32), ("seed", ctypes.c_uint64)]


class KeyBatch(ctypes.Structure):
    """tq_key_batch: one key set of tq_encode_keys_batched."""
    _fields_ = [("tables", ctypes.c_void_p), ("keys", ctypes.c_void_p), ("slots", ctypes.c_void_p),
                ("idx", ctypes.c_void_p), ("signs", ctypes.c_void_p), ("norm", ctypes.c_void_p),
                ("rnorm", ctypes.c_void_p)]


def key_config(d=128, mode="prod", bits=3, seed=42, bits_outlier=4, bits_normal=2, d_outlier=0) -> KeyConfig:
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    return KeyConfig(d, m, bits, bits_outlier, bits_normal, d_outlier, seed)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libtq.so is not built (run kv_cache_quantization_encode_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    CFG = ctypes.POINTER(KeyConfig)
    lib.tq_status_string.restype = ctypes.c_char_p
    lib.tq_status_string.argtypes = [I32]
    lib.tq_idx_row_bytes.restype = SZ
    lib.tq_idx_row_bytes.argtypes = [CFG]
    lib.tq_build_codebook.restype = I32
    lib.tq_build_codebook.argtypes = [CFG, P, ctypes.POINTER(SZ), ctypes.POINTER(ctypes.c_double)]
    lib.tq_encode_keys.restype = I32
    lib.tq_encode_keys.argtypes = [CFG, P, P, I32, I64, I64, P, I64, P, P, P, P, P]
    lib.tq_encode_values.restype = I32
    lib.tq_encode_values.argtypes = [I32, I32, I32, P, I32, I64, I64, P, I64, P, P, P, P]
    lib.tq_encode_keys_batched.restype = I32
    lib.tq_encode_keys_batched.argtypes = [CFG, ctypes.POINTER(KeyBatch), I32, I32, I64, I64, I64, P]
    lib.tq_append_kv.restype = I32
    lib.tq_append_kv.argtypes = [CFG, P, P, P, I32, I64, I64, I64, P, I64, P, P, P, P, I32, I32, P, P, P, P]
    lib.tq_decode_attention.restype = I32
    lib.tq_decode_attention.argtypes = [CFG, P, P, I32, I32, I32, I32, P, I32, P, P, P, P,
                                        I32, I32, P, P, P, ctypes.c_float, P, P, P, P,
                                        ctypes.POINTER(SZ), P]
    lib.tq_decode_attention_append.restype = I32
    lib.tq_decode_attention_append.argtypes = [CFG, P, P, I32, I32, I32, I32, P, I32, P, P, I32, P, P, P, P,
                                               I32, I32, P, P, P, ctypes.c_float, P, P, P, P,
                                               ctypes.POINTER(SZ), P]
    lib.tq_decode_attention_noalloc.restype = I32
    lib.tq_decode_attention_noalloc.argtypes = [CFG, P, P, I32, I32, I32, I32, P, I32, P, P, P, P,
                                                I32, I32, P, P, P, ctypes.c_float, P, P, P, P]
    lib.tq_decode_attention_paged.restype = I32
    lib.tq_decode_attention_paged.argtypes = [CFG, P, P, I32, I32, I32, I32, P, P, I32, I32, I32, P, P, P, P,
                                              I32, I32, P, P, P, ctypes.c_float, P, P, P, P,
                                              ctypes.POINTER(SZ), P]
    lib.tq_decode_attention_paged_append.restype = I32
    lib.tq_decode_attention_paged_append.argtypes = [CFG, P, P, I32, I32, I32, I32, P, P, I32, I32, I32, P, P, I32,
                                                     P, P, P, P, I32, I32, P, P, P, ctypes.c_float, P, P, P, P,
                                                     ctypes.POINTER(SZ), P]
    lib.tq_dequantize_keys.restype = I32
    lib.tq_dequantize_keys.argtypes = [CFG, P, I64, P, I64, P, P, P, P, P, I32, I64, P]
    lib.tq_dequantize_values.restype = I32
    lib.tq_dequantize_values.argtypes = [I32, I32, I32, I64, P, I64, P, P, P, P, I32, I64, P]
    lib.tq_channel_moments.restype = I32
    lib.tq_channel_moments.argtypes = [P, I32, I64, I64, I32, P, P, ctypes.POINTER(SZ), P]
    lib.tq_select_outlier_channels.restype = I32
    lib.tq_select_outlier_channels.argtypes = [P, I32, I64, I64, I32, I32, P, P, ctypes.POINTER(SZ), P]
    lib.tq_stream_read.restype = I32
    lib.tq_stream_read.argtypes = [P, SZ, P, P]
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.tq_status_string(int(status)).decode()


def check(fn: str, status: int):
    if status != TQ_OK:
        raise TqError(fn, status)
