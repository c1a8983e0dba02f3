"""ctypes view of the C ABI in include/moe.h (libmoe_mi355x.so).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_W_NATIVE, MOE_W_FP8_E4M3, MOE_W_MXFP4 = 0, 1, 2
MOE_A_NATIVE, MOE_A_MXFP8 = 0, 1
MOE_NUM_STAGES = 8
MOE_STATIC_SCRATCH_BYTES = 64 << 20
STAGE_NAMES = ["router", "scan", "permute", "gate_up", "down", "shared_gate_up", "shared_down", "combine"]
MOE_NUM_BSTAGES = 9
BSTAGE_NAMES = ["prep", "recompute", "down_bwd", "router_bwd", "dx_expert", "wgrad_down", "wgrad_gate_up",
                "shared", "dx"]
STATUS = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_UNSUPPORTED",
          4: "MOE_ERR_WORKSPACE", 5: "MOE_ERR_HIP"}


class MoeShape(C.Structure):
    _fields_ = [("T", C.c_int32), ("d", C.c_int32), ("d_e", C.c_int32), ("E", C.c_int32), ("k", C.c_int32),
                ("capacity", C.c_int32), ("renormalize", C.c_int32), ("d_e_shared", C.c_int32),
                ("dtype", C.c_int32), ("scoring", C.c_int32), ("n_group", C.c_int32), ("topk_group", C.c_int32),
                ("wfmt", C.c_int32), ("afmt", C.c_int32)]


class MoeWScales(C.Structure):
    """Scales of quantised expert weights (device pointers)."""
    _fields_ = [("gate", C.c_void_p), ("up", C.c_void_p), ("down", C.c_void_p)]


# every symbol include/moe.h declares, with its argument and result types
_P = C.c_void_p
SIGNATURES = {
    "moe_capacity": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_double, C.POINTER(C.c_int32)]),
    "moe_workspace_bytes": (C.c_int, [C.POINTER(MoeShape), C.POINTER(C.c_size_t)]),
    "moe_status_str": (C.c_char_p, [C.c_int]),
    "moe_route": (C.c_int, [C.POINTER(MoeShape), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "moe_permute": (C.c_int, [C.POINTER(MoeShape), _P, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P]),
    "moe_expert_ffn": (C.c_int, [C.POINTER(MoeShape), _P, _P, _P, _P, _P, C.POINTER(MoeWScales), _P, _P,
                                 C.c_size_t, _P]),
    "moe_combine": (C.c_int, [C.POINTER(MoeShape), _P, _P, _P, _P, _P, _P]),
    "moe_forward": (C.c_int, [C.POINTER(MoeShape)] + [_P] * 9 + [C.POINTER(MoeWScales)] * 2 + [_P] * 11
                    + [_P, C.c_size_t, _P, _P]),
    "moe_forward_noalloc": (C.c_int, [C.POINTER(MoeShape)] + [_P] * 9 + [C.POINTER(MoeWScales)] * 2 + [_P] * 11
                            + [_P, _P]),
    "moe_mxfp8_quantize": (C.c_int, [C.c_int32, C.c_int32, _P, _P, _P, _P]),
    "moe_backward_workspace_bytes": (C.c_int, [C.POINTER(MoeShape), C.POINTER(C.c_size_t)]),
    "moe_backward": (C.c_int, [C.POINTER(MoeShape)] + [_P] * 16 + [C.c_float] + [_P] * 10
                     + [_P, C.c_size_t, _P, _P]),
}

_lib = None


def lib() -> C.CDLL:
    """The loaded library (raises ImportError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'` "
                              "(or python sparse_mixture_experts_17_amd/build.py)")
        # torch's ROCm wheel carries its own HIP runtime (same soname): load torch first so
        # the library binds to that one runtime and torch's streams and pointers are valid.
        import torch  # noqa: F401
        l = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")


def check(fn: str, status: int) -> None:
    if status != 0:
        raise MoeError(fn, status)
