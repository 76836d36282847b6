"""ctypes view of the C ABI declared in include/ea_attn.h.

Loads exact_attention_04_amd/libea_attn.so (built in-tree by
``exact_attention_04_amd.build``).  There is no fallback: if the library is
missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libea_attn.so")

EA_OK, EA_EINVAL, EA_EUNSUPPORTED, EA_EDEVICE, EA_EHIP, EA_ESCRATCH = 0, 1, 2, 3, 4, 5
EA_F16, EA_BF16, EA_FP8_E4M3, EA_F32 = 1, 2, 3, 4
EA_ABI_VERSION = 5

# Every symbol the header declares.
EXPORTS = ("ea_attn_fwd", "ea_attn_fwd_noalloc", "ea_attn_bwd", "ea_attn_plan", "ea_status_string",
           "ea_last_hip_error", "ea_abi_version")


class AttnArgs(ctypes.Structure):
    """Mirror of ``ea_attn_args``."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("q_descale", ctypes.c_float),
        ("k_descale", ctypes.c_float),
        ("v_descale", ctypes.c_float),
        ("batch", ctypes.c_int64),
        ("seqlen_q", ctypes.c_int64),
        ("seqlen_k", ctypes.c_int64),
        ("nheads_q", ctypes.c_int64),
        ("nheads_k", ctypes.c_int64),
        ("headdim", ctypes.c_int64),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("q_stride_b", ctypes.c_int64), ("q_stride_s", ctypes.c_int64), ("q_stride_h", ctypes.c_int64),
        ("k_stride_b", ctypes.c_int64), ("k_stride_s", ctypes.c_int64), ("k_stride_h", ctypes.c_int64),
        ("v_stride_b", ctypes.c_int64), ("v_stride_s", ctypes.c_int64), ("v_stride_h", ctypes.c_int64),
        ("o_stride_b", ctypes.c_int64), ("o_stride_s", ctypes.c_int64), ("o_stride_h", ctypes.c_int64),
        ("lse_stride_b", ctypes.c_int64), ("lse_stride_h", ctypes.c_int64),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_int64),
        ("pv_dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class BwdArgs(ctypes.Structure):
    """Mirror of ``ea_attn_bwd_args``."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("batch", ctypes.c_int64),
        ("seqlen", ctypes.c_int64),
        ("nheads_q", ctypes.c_int64),
        ("nheads_k", ctypes.c_int64),
        ("headdim", ctypes.c_int64),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("dout", ctypes.c_void_p),
        ("lse", ctypes.c_void_p), ("delta", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
    ] + [(f"{t}_stride_{a}", ctypes.c_int64) for t in ("q", "k", "v", "o", "do", "dq", "dk", "dv") for a in "bsh"] + [
        ("lse_stride_b", ctypes.c_int64), ("lse_stride_h", ctypes.c_int64),
        ("delta_stride_b", ctypes.c_int64), ("delta_stride_h", ctypes.c_int64),
    ]


class PlanInfo(ctypes.Structure):
    """Mirror of ``ea_attn_plan_info``."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("block_m", ctypes.c_int32),
        ("block_n", ctypes.c_int32),
        ("waves", ctypes.c_int32),
        ("lds_bytes", ctypes.c_int32),
        ("grid", ctypes.c_int64),
        ("kv_tiles", ctypes.c_int64),
        ("masked_tiles", ctypes.c_int64),
        ("kernel", ctypes.c_char * 64),
        ("workspace_bytes", ctypes.c_int64),
        ("splits", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


_lib = None
_lock = threading.Lock()


def bind(h: ctypes.CDLL) -> ctypes.CDLL:
    """Declare the argument and result types of the exported functions on a
    loaded library handle."""
    h.ea_attn_fwd.argtypes = [ctypes.POINTER(AttnArgs), ctypes.c_void_p]
    h.ea_attn_fwd.restype = ctypes.c_int
    h.ea_attn_fwd_noalloc.argtypes = [ctypes.POINTER(AttnArgs), ctypes.c_void_p]
    h.ea_attn_fwd_noalloc.restype = ctypes.c_int
    h.ea_attn_bwd.argtypes = [ctypes.POINTER(BwdArgs), ctypes.c_void_p]
    h.ea_attn_bwd.restype = ctypes.c_int
    h.ea_attn_plan.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(PlanInfo)]
    h.ea_attn_plan.restype = ctypes.c_int
    h.ea_status_string.argtypes = [ctypes.c_int]
    h.ea_status_string.restype = ctypes.c_char_p
    h.ea_last_hip_error.argtypes = []
    h.ea_last_hip_error.restype = ctypes.c_int
    h.ea_abi_version.argtypes = []
    h.ea_abi_version.restype = ctypes.c_uint32
    return h


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m exact_attention_04_amd.build` "
                    "(there is no non-HIP fallback)")
            h = bind(ctypes.CDLL(LIB_PATH))
            if h.ea_abi_version() != EA_ABI_VERSION:
                raise RuntimeError(f"{LIB_PATH}: ABI version {h.ea_abi_version()} != {EA_ABI_VERSION}")
            _lib = h
    return _lib


def status_string(code: int) -> str:
    return lib().ea_status_string(code).decode()


class AttnError(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, code: int, hip_error: int = 0):
        self.code = code
        self.hip_error = hip_error
        msg = f"ea_attn status {code}: {status_string(code)}"
        if code == EA_EHIP:
            msg += f" (hipError_t {hip_error})"
        super().__init__(msg)


class AttnArgumentError(AttnError, ValueError):
    """EA_EINVAL, EA_EUNSUPPORTED or EA_ESCRATCH."""


def check(code: int) -> None:
    if code == EA_OK:
        return
    if code in (EA_EINVAL, EA_EUNSUPPORTED, EA_ESCRATCH):
        raise AttnArgumentError(code)
    raise AttnError(code, lib().ea_last_hip_error() if code == EA_EHIP else 0)


def fwd(args: AttnArgs, stream: int) -> int:
    return lib().ea_attn_fwd(ctypes.byref(args), ctypes.c_void_p(stream))


def fwd_noalloc(args: AttnArgs, stream: int) -> int:
    """The allocation-free forward (library scratch; args.workspace must be NULL)."""
    return lib().ea_attn_fwd_noalloc(ctypes.byref(args), ctypes.c_void_p(stream))


def bwd(args: BwdArgs, stream: int) -> int:
    return lib().ea_attn_bwd(ctypes.byref(args), ctypes.c_void_p(stream))


def plan(args: AttnArgs) -> PlanInfo:
    info = PlanInfo()
    info.struct_size = ctypes.sizeof(PlanInfo)
    check(lib().ea_attn_plan(ctypes.byref(args), ctypes.byref(info)))
    return info
