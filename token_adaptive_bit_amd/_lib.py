"""ctypes binding of libmbq.so (the C ABI declared in include/mbq.h).

Argument marshalling only: every step of the path runs in the library's HIP kernels.
PyTorch provides device memory and the current stream.  If the shared library is
missing the import of this module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmbq.so")

MBQ_F32, MBQ_BF16 = 0, 1
STATIC_SCRATCH_BYTES = 16 << 20      # MBQ_STATIC_SCRATCH_BYTES
ABI_VERSION = 3

STATUS = {0: "MBQ_OK", -1: "MBQ_ERR_ARG", -2: "MBQ_ERR_SHAPE", -3: "MBQ_ERR_RANGE",
          -4: "MBQ_ERR_WORKSPACE", -5: "MBQ_ERR_DEVICE", -6: "MBQ_ERR_UNSUPPORTED"}

EXPORTS = ("mbq_describe", "mbq_pack", "mbq_pack_rows", "mbq_pack_bitplane", "mbq_route", "mbq_regroup", "mbq_route_mlp_workspace",
           "mbq_route_mlp", "mbq_linear_workspace", "mbq_linear", "mbq_linear_static", "mbq_route_linear",
           "mbq_route_linear_workspace", "mbq_route_prepare_workspace", "mbq_route_prepare",
           "mbq_route_linear_prepared",
           "mbq_linear_lowrank_workspace",
           "mbq_linear_lowrank", "mbq_status_str", "mbq_abi_version")


class MbqDesc(ctypes.Structure):
    _fields_ = [("abi", ctypes.c_int32), ("n", ctypes.c_int32), ("k", ctypes.c_int32),
                ("group", ctypes.c_int32), ("slices", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("row_blocks", ctypes.c_int32), ("k_tiles", ctypes.c_int32),
                ("groups_padded", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("codes_bytes", ctypes.c_uint64), ("params_bytes", ctypes.c_uint64),
                ("params_offset", ctypes.c_uint64), ("slice_stride", ctypes.c_uint64),
                ("total_bytes", ctypes.c_uint64)]

    def as_dict(self) -> dict:
        return {f: getattr(self, f) for f, _ in self._fields_}


MBQ_PATH_AUTO, MBQ_PATH_GENERIC = 0, 1
MBQ_MUL_AUTO, MBQ_MUL_BF16, MBQ_MUL_FP8_FP4 = 0, 1, 2


class MbqOpts(ctypes.Structure):
    """Kernel and tiling choices of the routed linear (mbq_opts in include/mbq.h)."""
    _fields_ = [("path", ctypes.c_int32), ("decode_mul", ctypes.c_int32),
                ("prefill_slots", ctypes.c_int32), ("decode_launches", ctypes.c_int32)]


class MbqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_str(status)})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m token_adaptive_bit_amd.build`")
    # One HIP runtime per process: torch ships its own libamdhip64.so.7, and libmbq must
    # bind to that one (same SONAME) rather than load the system copy next to it, or the
    # two HSA runtimes fight over the device.  Importing torch first makes the dynamic
    # linker reuse torch's runtime for libmbq.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, U64, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_uint64, ctypes.c_void_p
    D = P(MbqDesc)
    lib.mbq_describe.argtypes = [I32, I32, I32, I32, D]
    lib.mbq_pack.argtypes = [D, VP, I32, VP, VP, VP]
    lib.mbq_pack_rows.argtypes = [D, I32, I32, VP, I32, VP, VP, VP]
    lib.mbq_pack_bitplane.argtypes = [D, VP, I32, VP, VP, VP]
    lib.mbq_route.argtypes = [I32, I32, I32, VP, I32, VP, VP, VP, VP, VP, VP]
    lib.mbq_regroup.argtypes = [I32, I32, VP, VP, VP, VP]
    lib.mbq_route_mlp_workspace.argtypes = [I32, I32, I32, P(ctypes.c_size_t)]
    lib.mbq_route_mlp.argtypes = [I32, I32, I32, I32, VP, I32, VP, VP, VP, VP, ctypes.c_double,
                                  VP, VP, VP, VP, VP, ctypes.c_size_t, VP]
    lib.mbq_linear_workspace.argtypes = [D, I32, I32, P(ctypes.c_size_t)]
    O = P(MbqOpts)
    lib.mbq_linear.argtypes = [D, VP, I32, VP, I32, VP, VP, VP, I32, VP, ctypes.c_size_t, O, VP]
    lib.mbq_route_linear_workspace.argtypes = [D, I32, I32, P(ctypes.c_size_t)]
    lib.mbq_route_prepare_workspace.argtypes = [D, I32, P(ctypes.c_size_t)]
    lib.mbq_route_prepare.argtypes = [D, I32, VP, VP, VP, ctypes.c_size_t, VP]
    lib.mbq_route_linear_prepared.argtypes = [D, VP, I32, VP, ctypes.c_size_t, VP, VP, VP, VP, VP, I32, VP]
    lib.mbq_linear_static.argtypes = [D, VP, I32, VP, I32, VP, VP, VP, I32, O, VP]
    lib.mbq_route_linear.argtypes = [D, VP, I32, VP, I32, VP, VP, VP, VP, VP, VP, I32, VP,
                                     ctypes.c_size_t, O, VP]
    lib.mbq_linear_lowrank_workspace.argtypes = [D, I32, I32, I32, P(ctypes.c_size_t)]
    lib.mbq_linear_lowrank.argtypes = [D, VP, I32, VP, I32, VP, VP, VP, VP, I32, VP, I32, VP,
                                       ctypes.c_size_t, O, VP]
    lib.mbq_status_str.argtypes = [I32]
    lib.mbq_status_str.restype = ctypes.c_char_p
    lib.mbq_abi_version.argtypes = []
    for name in EXPORTS:
        if name not in ("mbq_status_str",):
            getattr(lib, name).restype = I32
    if lib.mbq_abi_version() != ABI_VERSION:
        raise ImportError("libmbq ABI version mismatch")
    return lib


LIB = _load()


def _str(status: int) -> str:
    return LIB.mbq_status_str(status).decode()


def check(status: int, what: str) -> None:
    if status != 0:
        raise MbqError(status, what)


def describe(n: int, k: int, group: int, slices: int) -> MbqDesc:
    d = MbqDesc()
    check(LIB.mbq_describe(n, k, group, slices, ctypes.byref(d)), "mbq_describe")
    return d


def workspace_bytes(desc: MbqDesc, t: int, x_dtype: int) -> int:
    n = ctypes.c_size_t(0)
    check(LIB.mbq_linear_workspace(ctypes.byref(desc), t, x_dtype, ctypes.byref(n)),
          "mbq_linear_workspace")
    return int(n.value)


def route_linear_workspace_bytes(desc: MbqDesc, t: int, x_dtype: int) -> int:
    n = ctypes.c_size_t(0)
    check(LIB.mbq_route_linear_workspace(ctypes.byref(desc), t, x_dtype, ctypes.byref(n)),
          "mbq_route_linear_workspace")
    return int(n.value)


def route_mlp_workspace_bytes(t: int, k: int, hidden: int) -> int:
    n = ctypes.c_size_t(0)
    check(LIB.mbq_route_mlp_workspace(t, k, hidden, ctypes.byref(n)), "mbq_route_mlp_workspace")
    return int(n.value)


def lowrank_workspace_bytes(desc: MbqDesc, t: int, x_dtype: int, rank: int) -> int:
    n = ctypes.c_size_t(0)
    check(LIB.mbq_linear_lowrank_workspace(ctypes.byref(desc), t, x_dtype, rank, ctypes.byref(n)),
          "mbq_linear_lowrank_workspace")
    return int(n.value)
