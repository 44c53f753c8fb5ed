"""ctypes view of the C ABI in include/moe.h (argument marshalling only).

The shared library libmoe_mi355x.so is built in-tree by
mixture_experts_layer_03_amd.build.  There is no fallback: if the library is
missing or cannot be loaded, every entry point raises.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

MOE_OK, MOE_EINVAL_CONFIG, MOE_EINVAL_ARG, MOE_EWORKSPACE, MOE_EUNSUPPORTED, MOE_EHIP = range(6)
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_EINVAL_CONFIG", 2: "MOE_EINVAL_ARG", 3: "MOE_EWORKSPACE",
                4: "MOE_EUNSUPPORTED", 5: "MOE_EHIP"}
DT_F32, DT_BF16, DT_U8_AFFINE, DT_U4_AFFINE = 0, 1, 2, 3
SCORE_SOFTMAX, SCORE_SIGMOID = 0, 1
PATH_AUTO, PATH_DECODE, PATH_PREFILL = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_NOALLOC_SCRATCH_BYTES
STAGES = {"router": 1, "topk": 2, "permute": 4, "up": 8, "down": 16, "shared_up": 32,
          "shared_down": 64, "combine": 128}


class moe_config(C.Structure):
    _fields_ = [
        ("hidden", C.c_int64), ("num_experts", C.c_int64), ("top_k", C.c_int64),
        ("moe_intermediate", C.c_int64), ("shared_intermediate", C.c_int64),
        ("n_group", C.c_int64), ("topk_group", C.c_int64),
        ("score_function", C.c_int32), ("norm_topk_prob", C.c_int32),
        ("use_expert_bias", C.c_int32), ("routed_scaling_factor", C.c_float),
        ("act_dtype", C.c_int32), ("router_dtype", C.c_int32), ("expert_dtype", C.c_int32),
        ("shared_dtype", C.c_int32), ("quant_group", C.c_int64), ("path", C.c_int32),
    ]


class moe_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "router", "router_bias", "expert_bias", "gate", "up", "down",
        "gate_scale", "gate_zero", "up_scale", "up_zero", "down_scale", "down_zero",
        "shared_gate", "shared_up", "shared_down")]


class MoEError(RuntimeError):
    """A C ABI call returned an error status."""

    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


_lib = None


def lib() -> C.CDLL:
    """The loaded shared library (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m mixture_experts_layer_03_amd.build`")
    L = C.CDLL(LIB_PATH)
    P, I64, SZ = C.c_void_p, C.c_int64, C.c_size_t
    cfgp = C.POINTER(moe_config)
    wp = C.POINTER(moe_weights)
    sigs = {
        "moe_config_default": [cfgp],
        "moe_validate_config": [cfgp],
        "moe_workspace_size": [cfgp, I64, C.POINTER(SZ)],
        "moe_select_path": [cfgp, I64, C.POINTER(C.c_int32)],
        "moe_route": [cfgp, I64, P, P, P, P, P, P, P, SZ, P],
        "moe_permute": [cfgp, I64, P, P, P, P, P, SZ, P],
        "moe_experts": [cfgp, I64, P, wp, P, P, P, P, SZ, P],
        "moe_forward": [cfgp, I64, P, wp, P, P, P, P, P, SZ, P],
        "moe_forward_noalloc": [cfgp, I64, P, wp, P, P, P, P, P],
        "moe_dense_workspace_size": [cfgp, I64, I64, C.POINTER(SZ)],
        "moe_dense_mlp": [cfgp, I64, I64, P, P, P, P, P, P, SZ, P],
    }
    for name, args in sigs.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = C.c_int
    L.moe_profile_enable.argtypes = [C.c_int32, C.c_int32]
    L.moe_profile_collect.argtypes = [C.c_int32, C.POINTER(C.c_float), C.POINTER(C.c_int32)]
    L.moe_profile_disable.argtypes = []
    L.moe_profile_reset.argtypes = []
    for n in ("moe_profile_enable", "moe_profile_collect", "moe_profile_disable", "moe_profile_reset"):
        getattr(L, n).restype = C.c_int
    L.moe_status_str.argtypes = [C.c_int]
    L.moe_status_str.restype = C.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = C.c_char_p
    L.moe_abi_version.argtypes = []
    L.moe_abi_version.restype = C.c_int32
    _lib = L
    return L


def check(status: int) -> None:
    if status != MOE_OK:
        raise MoEError(status, lib().moe_last_error().decode(errors="replace"))
