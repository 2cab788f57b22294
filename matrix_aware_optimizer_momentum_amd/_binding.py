"""ctypes binding of libsm (include/sm.h).

Argument marshalling only: every step of the optimizer runs in the HIP
kernels of libsm.so.  PyTorch supplies device memory and the current HIP
stream.  There is no fallback: if the library is missing, lib() raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_DIR, "libsm.so")

SM_OK = 0
STATUS_NAMES = {0: "SM_OK", 1: "SM_ERR_ARG", 2: "SM_ERR_SHAPE", 3: "SM_ERR_DTYPE",
                4: "SM_ERR_WORKSPACE", 5: "SM_ERR_UNSUPPORTED", 6: "SM_ERR_HIP"}
F32, BF16 = 0, 1
SIGN_MUON, CACHE_MUON, LION_MUON = 0, 1, 2
UPDATE_VOTE, UPDATE_POLAR = 0, 1
MODE_TRIGGER, MODE_FORCE_FRESH, MODE_FORCE_REUSE = 0, 1, 2
ENC_BITS, ENC_INT8 = 0, 1
NS_NOALLOC_MAX_WS = 64 << 20   # SM_NS_NOALLOC_MAX_WS

KERNEL_KINDS = ["ema", "norm", "gemm_gram", "gemm_apply", "gemm_rr", "probe", "sign_pack",
                "vote_update", "lion", "polar_update", "misc", "spectral"]

# Every function the header declares, with its ctypes signature.
c_int, c_int32, c_int64, c_float, c_double = (ctypes.c_int, ctypes.c_int32, ctypes.c_int64,
                                             ctypes.c_float, ctypes.c_double)
c_void_p, c_size_t, c_char_p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_char_p


class NSParams(ctypes.Structure):
    _fields_ = [("iters", c_int32), ("a", c_float), ("b", c_float), ("c", c_float),
                ("eps", c_float)]


class Matrix(ctypes.Structure):
    _fields_ = [("m", c_int32), ("n", c_int32), ("w", c_void_p), ("mom", c_void_p),
                ("grad", c_void_p), ("q_cache", c_void_p), ("cache_state", c_void_p)]


class Config(ctypes.Structure):
    _fields_ = [("algo", c_int32), ("update", c_int32), ("M", c_int32), ("wdt", c_int32),
                ("mdt", c_int32), ("gdt", c_int32), ("lr", c_float), ("beta1", c_float),
                ("beta2", c_float), ("period", c_int32), ("ns", NSParams), ("gamma", c_float),
                ("cache_mode", c_int32), ("encoding", c_int32), ("vote_polar", c_int32)]


P = ctypes.POINTER
SIGNATURES = {
    "sm_status_string": (c_char_p, [c_int]),
    "sm_last_hip_error": (c_int, []),
    "sm_version": (c_int, []),
    "sm_ns_polar_ws": (c_int, [c_int, c_int, c_int, c_int, P(c_size_t)]),
    "sm_ns_polar": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int, P(NSParams),
                            c_void_p, c_size_t, c_void_p]),
    "sm_ns_polar_noalloc": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                    P(NSParams), c_void_p]),
    "sm_gram_ns_cached_ws": (c_int, [c_int, c_int, c_int, c_int, P(c_size_t)]),
    "sm_gram_ns_cached": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_int, c_int, c_int, c_int, c_int, P(NSParams), c_float,
                                  c_int, c_int64, c_void_p, c_size_t, c_void_p]),
    "sm_sign_pack": (c_int, [c_void_p, c_int, c_int64, c_void_p, c_void_p]),
    "sm_vote_update": (c_int, [c_void_p, c_int, c_int64, c_int64, c_void_p, c_int, c_float,
                               c_void_p, c_void_p]),
    "sm_sign_int8": (c_int, [c_void_p, c_int, c_int64, c_void_p, c_void_p]),
    "sm_vote_update_int8": (c_int, [c_void_p, c_int, c_int64, c_int64, c_void_p, c_int, c_float,
                                    c_void_p, c_void_p]),
    "sm_vote": (c_int, [c_void_p, c_int, c_int, c_int64, c_int64, c_void_p, c_int, c_void_p]),
    "sm_polar_update": (c_int, [c_void_p, c_int, c_void_p, c_int, c_int64, c_float, c_void_p]),
    "sm_spectral_norm_ws": (c_int, [c_int, c_int, c_int, P(c_size_t)]),
    "sm_spectral_norm": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_int,
                                 c_void_p, c_void_p, c_size_t, c_void_p]),
    "sm_step_ws": (c_int, [P(Config), P(Matrix), c_int, P(c_size_t)]),
    "sm_step": (c_int, [P(Config), P(Matrix), c_int, c_int64, c_void_p, c_size_t, c_void_p,
                        c_void_p]),
    "sm_step_graph": (c_int, [P(Config), P(Matrix), c_int, c_int64, c_void_p, c_size_t,
                              c_void_p, P(c_void_p)]),
    "sm_graph_launch": (c_int, [c_void_p, c_void_p]),
    "sm_graph_destroy": (c_int, [c_void_p]),
    "sm_profile_enable": (c_int, [c_int]),
    "sm_profile_reset": (c_int, []),
    "sm_profile_read": (c_int, [c_int, P(c_double), P(c_int64), P(c_double)]),
    "sm_profile_read_bytes": (c_int, [c_int, P(c_double)]),
    "sm_kernel_kind_name": (c_char_p, [c_int]),
    "sm_mfma_ceiling": (c_int, [c_int, c_int, c_int, c_void_p, c_size_t, c_void_p, c_void_p]),
}

_lib = None
_lock = threading.Lock()


class SmError(RuntimeError):
    def __init__(self, code: int, where: str, hip_code: int = 0):
        self.code = code
        self.where = where
        self.hip_code = hip_code
        msg = f"{where}: {STATUS_NAMES.get(code, code)}"
        if hip_code:
            msg += f" (hipError {hip_code})"
        super().__init__(msg)


def lib():
    """Load libsm.so once and declare its signatures; raise if it is missing."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                                   "(the HIP library is required; there is no fallback)")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
        return _lib


def check(code: int, where: str):
    if code != SM_OK:
        raise SmError(code, where, lib().sm_last_hip_error() if code == 6 else 0)
