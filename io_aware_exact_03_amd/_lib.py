"""ctypes binding of libfa.so (include/fa.h).  Argument marshalling only:
torch supplies device memory and the current stream; every step of the
computation runs in the library's HIP kernels.  There is no CPU fallback:
if the library is missing or fails to load, calls raise."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
STATUS = {0: "FA_OK", 1: "FA_ERR_ARG", 2: "FA_ERR_UNSUPPORTED", 3: "FA_ERR_ALIGN", 4: "FA_ERR_HIP", 5: "FA_ERR_SCRATCH"}
DECODE_SCRATCH_BYTES = 16 << 20  # FA_DECODE_SCRATCH_BYTES

# name -> (restype, argtypes), mirroring include/fa.h
_vp, _i, _f, _fp = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_void_p
_ip = ctypes.POINTER(ctypes.c_int)
SIGNATURES = {
    "fa_fwd": (_i, [_vp, _vp, _vp, _vp, _fp, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "fa_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _fp, _fp, _fp, _fp, _fp, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "fa_bwd_stage": (_i, [_i, _vp, _vp, _vp, _vp, _vp, _fp, _fp, _fp, _fp, _fp, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "fa_fwd_gqa": (_i, [_vp, _vp, _vp, _vp, _fp, _i, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "fa_fwd_chunk": (_i, [_vp, _vp, _vp, _vp, _fp, _i, _i, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "fa_bwd_gqa": (_i, [_vp, _vp, _vp, _vp, _vp, _fp, _fp, _fp, _fp, _fp, _i, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "fa_kv_head": (_i, [_i, _i, _i]),
    "fa_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _fp, _vp, ctypes.c_size_t, _i, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "fa_decode_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i, _i, _i]),
    "fa_decode_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _fp, _i, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "fa_decode_plan": (_i, [_i, _i, _i, _i, _i, _ip]),
    "fa_fwd_fp8": (_i, [_vp, _vp, _vp, _vp, _fp, _i, _i, _i, _i, _i, _f, _f, _f, _f, _i, _vp]),
    "fa_fwd_fa1": (_i, [_vp, _vp, _vp, _vp, _fp, _vp, ctypes.c_size_t, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "fa_fa1_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i, _i]),
    "fa_naive_fwd": (_i, [_vp, _vp, _vp, _vp, _fp, _vp, _vp, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "fa_naive_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i, _i]),
    "fa_strerror": (ctypes.c_char_p, [_i]),
    "fa_last_hip_error": (_i, []),
    "fa_causal_stages": (_i, [_i, _i, _i, _i, _ip, _ip]),
    "fa_fwd_tile": (_i, [_i, _i, _ip, _ip, _ip]),
    "fa_ceiling_mfma": (_i, [_vp, _vp, _i, _i, _i, _vp]),
    "fa_ceiling_copy": (_i, [_vp, _vp, ctypes.c_size_t, _vp]),
    "fa_ceiling_read": (_i, [_vp, ctypes.c_size_t, _vp, _vp]),
    "fa_ceiling_read_sink_bytes": (ctypes.c_size_t, []),
    "fa_ceiling_valu": (_i, [_i, _vp, _vp, _i, _vp]),
    "fa_ceiling_mix": (_i, [_i, _vp, _vp, _i, _i, _vp]),
}

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {STATUS.get(status, status)} ({load().fa_strerror(status).decode()})"
        if status == 4:
            msg += f", hipError_t={load().fa_last_hip_error()}"
        super().__init__(msg)


def load(path: str | None = None):
    """Load libfa.so once (raises OSError if it is not built).  The
    IO_AWARE_FA_LIB environment variable names another build of the same
    library (a tile variant) to load instead."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("IO_AWARE_FA_LIB") or LIB_PATH
    if not os.path.exists(p):
        raise OSError(f"{p} is not built; run io_aware_exact_03_amd.build or __graft_entry__.build()")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def check(status: int, where: str) -> None:
    if status != 0:
        raise FaError(status, where)
