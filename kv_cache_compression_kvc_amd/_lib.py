"""ctypes binding of include/kvc.h (argument marshalling only).

The library is loaded after ``torch`` so that it binds to the same HIP
runtime instance as torch (device pointers and stream handles are then
shared).  Loading fails loudly if the library has not been built or if a
second HIP runtime ends up mapped into the process; there is no fallback.
"""

import ctypes
import os

import torch  # noqa: F401  (must be imported before the HIP library loads)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkvc.so")
HOST_LIB_PATH = os.path.join(PKG, "libkvc_host.so")

KVC_OK = 0
STATUS = {
    0: "KVC_OK", -1: "KVC_EINVAL", -2: "KVC_ESHAPE", -3: "KVC_EBITS", -4: "KVC_EGROUP",
    -5: "KVC_EDTYPE", -6: "KVC_EALIGN", -7: "KVC_ENOSPC", -8: "KVC_EHIP", -9: "KVC_ERANGE",
}
DTYPE = {"bf16": 0, "fp16": 1}

# every function include/kvc.h declares
EXPORTS = [
    "kvc_abi_version", "kvc_strerror", "kvc_encoded_size", "kvc_sign_mask", "kvc_encode",
    "kvc_decode", "kvc_paged_layout", "kvc_encode_paged", "kvc_decode_paged",
    "kvc_debug_rotate", "kvc_unfused_workspace_size", "kvc_encode_unfused", "kvc_decode_unfused",
    "kvc_chunked_size", "kvc_encode_send", "kvc_receive_decode", "kvc_probe_copy",
    "kvc_encode_unfused_noalloc", "kvc_probe_stream", "kvc_paged_order", "kvc_encode_with",
    "kvc_decode_with", "kvc_encode_paged_with", "kvc_decode_paged_with", "kvc_probe_blocks",
    "kvc_probe_stream_runs",
]
TRANSFORM = {"auto": 0, "matrix": 1, "butterfly": 2}   # kvc_transform
NOALLOC_WORKSPACE_BYTES = 64 << 20   # KVC_NOALLOC_WORKSPACE_BYTES
HOST_EXPORTS = ["kvc_abi_version", "kvc_strerror", "kvc_encoded_size", "kvc_sign_mask",
                "kvc_paged_layout", "kvc_unfused_workspace_size", "kvc_chunked_size", "kvc_paged_order"]


class KvcDesc(ctypes.Structure):
    _fields_ = [
        ("layers", ctypes.c_int64),
        ("tokens", ctypes.c_int64),
        ("kv_heads", ctypes.c_int64),
        ("head_dim", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("bits_k", ctypes.c_int32),
        ("bits_v", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("seed", ctypes.c_uint64),
    ]


class KvcPaged(ctypes.Structure):
    _fields_ = [
        ("num_blocks", ctypes.c_int64),
        ("block_size", ctypes.c_int32),
        ("num_reqs", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("out_offsets", ctypes.c_void_p),
        ("err_flag", ctypes.c_void_p),
        ("order", ctypes.c_void_p),
        ("order_len", ctypes.c_int64),
    ]


class KvcPagedItem(ctypes.Structure):
    _fields_ = [
        ("block", ctypes.c_int32),
        ("block_index", ctypes.c_int32),
        ("req", ctypes.c_int32),
        ("len", ctypes.c_int32),
        ("offset", ctypes.c_int64),
        ("reserved", ctypes.c_int64),
    ]


class KvcLaunchOpts(ctypes.Structure):
    _fields_ = [
        ("transform", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("start_event", ctypes.c_void_p),
        ("stop_event", ctypes.c_void_p),
    ]


class KvcError(RuntimeError):
    def __init__(self, status, lib=None):
        text = lib.kvc_strerror(status).decode() if lib is not None else ""
        super().__init__("%s (%d): %s" % (STATUS.get(status, "?"), status, text))
        self.status = status


def _declare(lib, names):
    P = ctypes.POINTER
    sig = {
        "kvc_abi_version": (ctypes.c_int32, []),
        "kvc_strerror": (ctypes.c_char_p, [ctypes.c_int32]),
        "kvc_encoded_size": (ctypes.c_int32, [P(KvcDesc), ctypes.c_int64, P(ctypes.c_uint64),
                                              P(ctypes.c_uint64)]),
        "kvc_sign_mask": (ctypes.c_int32, [ctypes.c_uint64, ctypes.c_int64, P(ctypes.c_uint64)]),
        "kvc_encode": (ctypes.c_int32, [P(KvcDesc), ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_uint64, ctypes.c_void_p]),
        "kvc_decode": (ctypes.c_int32, [P(KvcDesc), ctypes.c_void_p, ctypes.c_uint64,
                                        ctypes.c_void_p, ctypes.c_void_p]),
        "kvc_encode_with": (ctypes.c_int32, [P(KvcDesc), ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_uint64, P(KvcLaunchOpts), ctypes.c_void_p]),
        "kvc_decode_with": (ctypes.c_int32, [P(KvcDesc), ctypes.c_void_p, ctypes.c_uint64,
                                             ctypes.c_void_p, P(KvcLaunchOpts), ctypes.c_void_p]),
        "kvc_encode_paged_with": (ctypes.c_int32, [P(KvcDesc), ctypes.c_void_p, P(KvcPaged), ctypes.c_void_p,
                                                   ctypes.c_uint64, P(KvcLaunchOpts), ctypes.c_void_p]),
        "kvc_decode_paged_with": (ctypes.c_int32, [P(KvcDesc), ctypes.c_void_p, ctypes.c_uint64, P(KvcPaged),
                                                   ctypes.c_void_p, P(KvcLaunchOpts), ctypes.c_void_p]),
        "kvc_paged_order": (ctypes.c_int32, [P(ctypes.c_int32), ctypes.c_int32, ctypes.c_int32, P(ctypes.c_int32),
                                             P(ctypes.c_int64), ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                                             P(ctypes.c_int64)]),
        "kvc_paged_layout": (ctypes.c_int32, [P(KvcDesc), P(ctypes.c_int32), ctypes.c_int32,
                                              P(ctypes.c_int64), P(ctypes.c_uint64)]),
        "kvc_encode_paged": (ctypes.c_int32, [P(KvcDesc), ctypes.c_void_p, P(KvcPaged),
                                              ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]),
        "kvc_decode_paged": (ctypes.c_int32, [P(KvcDesc), ctypes.c_void_p, ctypes.c_uint64,
                                              P(KvcPaged), ctypes.c_void_p, ctypes.c_void_p]),
        "kvc_debug_rotate": (ctypes.c_int32, [P(KvcDesc), ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p]),
        "kvc_unfused_workspace_size": (ctypes.c_int32, [P(KvcDesc), P(ctypes.c_uint64)]),
        "kvc_encode_unfused": (ctypes.c_int32, [P(KvcDesc), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                                ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]),
        "kvc_decode_unfused": (ctypes.c_int32, [P(KvcDesc), ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]),
        "kvc_encode_unfused_noalloc": (ctypes.c_int32, [P(KvcDesc), ctypes.c_void_p, ctypes.c_void_p,
                                                        ctypes.c_uint64, ctypes.c_void_p]),
        "kvc_chunked_size": (ctypes.c_int32, [P(KvcDesc), ctypes.c_int64, P(ctypes.c_uint64),
                                              P(ctypes.c_uint64)]),
        "kvc_encode_send": (ctypes.c_int32, [P(KvcDesc), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                             ctypes.c_int64, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                             ctypes.c_void_p]),
        "kvc_receive_decode": (ctypes.c_int32, [P(KvcDesc), ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                                ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_void_p]),
        "kvc_probe_stream": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint64,
                                              ctypes.c_int32, ctypes.c_void_p]),
        "kvc_probe_stream_runs": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                                   ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
        "kvc_probe_blocks": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p,
                                              ctypes.c_int64, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_void_p]),
        "kvc_probe_copy": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                            ctypes.c_void_p]),
    }
    for n in names:
        f = getattr(lib, n)
        f.restype, f.argtypes = sig[n]
    return lib


def _hip_runtimes():
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


_LIB = None
_HOST = None


def lib():
    """The HIP library (libkvc.so); raises if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libkvc.so is not built: run `python -m kv_cache_compression_kvc_amd.build`")
        _LIB = _declare(ctypes.CDLL(LIB_PATH), EXPORTS)
        runtimes = _hip_runtimes()
        if len(runtimes) > 1:
            raise ImportError("two HIP runtimes are mapped (%s); import torch first" % runtimes)
    return _LIB


def host_lib():
    """The host-only half (libkvc_host.so, built with g++)."""
    global _HOST
    if _HOST is None:
        if not os.path.exists(HOST_LIB_PATH):
            raise ImportError("libkvc_host.so is not built")
        _HOST = _declare(ctypes.CDLL(HOST_LIB_PATH), HOST_EXPORTS)
    return _HOST


def check(status):
    if status != KVC_OK:
        raise KvcError(status, _LIB or _HOST)
