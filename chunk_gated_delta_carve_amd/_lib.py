"""ctypes view of libcarve.so (the C ABI declared in include/carve.h)."""
from __future__ import annotations

import ctypes
import os

# CARVE_LIB_PATH may name another build of the same library (the host
# sanitizer build, build.py --sanitize); by default the in-tree libcarve.so.
LIB_PATH = os.environ.get("CARVE_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcarve.so")

CARVE_OK, CARVE_EINVAL, CARVE_EUNSUPPORTED, CARVE_EALIGN, CARVE_EWORKSPACE, CARVE_EHIP = range(6)
CARVE_F32, CARVE_BF16 = 0, 1
CARVE_DECAY_LOGITS = 1
CARVE_QK_L2NORM = 2
CARVE_DETACH_MEAN = 4
EXPORTED = ("carve_recurrent_ref_shapes", "carve_chunk_fwd", "carve_chunk_fwd_noalloc", "carve_chunk_bwd",
            "carve_recurrent_step", "carve_error_string")


class CarveConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "H", "T", "dk", "dv", "L", "rank", "dtype", "flags")]


class CarveShapes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("q", "k", "v", "g", "bx", "w", "ub_down", "ub_up", "o", "state", "mean",
                 "workspace_bytes", "bwd_workspace_bytes")]


class CarveError(RuntimeError):
    def __init__(self, code: int, text: str):
        super().__init__(f"carve status {code}: {text}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load libcarve.so once. Raises if the library has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m chunk_gated_delta_carve_amd.build`"
                " (there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        L.carve_recurrent_ref_shapes.argtypes = [ctypes.POINTER(CarveConfig), ctypes.POINTER(CarveShapes)]
        L.carve_recurrent_ref_shapes.restype = ctypes.c_int
        L.carve_chunk_fwd.argtypes = [ctypes.POINTER(CarveConfig)] + [vp] * 14 + [ctypes.c_size_t, vp]
        L.carve_chunk_fwd.restype = ctypes.c_int
        L.carve_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(CarveConfig)] + [vp] * 14
        L.carve_chunk_fwd_noalloc.restype = ctypes.c_int
        L.carve_chunk_bwd.argtypes = [ctypes.POINTER(CarveConfig)] + [vp] * 24 + [ctypes.c_size_t, vp]
        L.carve_chunk_bwd.restype = ctypes.c_int
        L.carve_recurrent_step.argtypes = [ctypes.POINTER(CarveConfig), ctypes.c_int32] + [vp] * 13
        L.carve_recurrent_step.restype = ctypes.c_int
        L.carve_error_string.argtypes = [ctypes.c_int]
        L.carve_error_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def error_string(code: int) -> str:
    return lib().carve_error_string(code).decode()


def check(code: int) -> None:
    if code != CARVE_OK:
        raise CarveError(code, error_string(code))


def ref_shapes(cfg: CarveConfig) -> CarveShapes:
    out = CarveShapes()
    check(lib().carve_recurrent_ref_shapes(ctypes.byref(cfg), ctypes.byref(out)))
    return out
