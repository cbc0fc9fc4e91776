"""ctypes view of libqmoe.so (the C ABI declared in include/qmoe.h)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqmoe.so")

QMOE_OK, QMOE_ERR_INVALID, QMOE_ERR_SHAPE, QMOE_ERR_DTYPE = 0, 1, 2, 3
QMOE_ERR_UNSUPPORTED, QMOE_ERR_UNBOUND, QMOE_ERR_DEVICE = 4, 5, 6
STATUS_NAMES = {0: "OK", 1: "INVALID", 2: "SHAPE", 3: "DTYPE", 4: "UNSUPPORTED", 5: "UNBOUND",
                6: "DEVICE"}

QMOE_F32, QMOE_BF16, QMOE_E8M0 = 0, 1, 2
QMOE_LAYOUT_ROWS, QMOE_LAYOUT_TILES = 0, 1
QMOE_FC1, QMOE_FC2, QMOE_FC3 = 1, 2, 3
QMOE_NOALLOC_SCRATCH_BYTES = 64 << 20
ACT = {"swiglu": 0, "identity": 1, "relu": 2, "silu": 3, "gelu": 4}


class QmoeParams(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int64), ("hidden_size", ctypes.c_int64),
                ("inter_size", ctypes.c_int64), ("num_experts", ctypes.c_int64),
                ("k", ctypes.c_int64), ("expert_weight_bits", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("swiglu_fusion", ctypes.c_int32),
                ("activation", ctypes.c_int32), ("normalize_routing_weights", ctypes.c_int32),
                ("swiglu_alpha", ctypes.c_float), ("swiglu_beta", ctypes.c_float),
                ("swiglu_limit", ctypes.c_float), ("act_dtype", ctypes.c_int32),
                ("scale_dtype", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("strict_blocks", ctypes.c_int32), ("weight_layout", ctypes.c_int32),
                ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("routed_scaling_factor", ctypes.c_float),
                ("e_score_correction_bias", ctypes.c_void_p),
                ("compute_mode", ctypes.c_int32), ("gelu_mode", ctypes.c_int32),
                ("expert_output_scale", ctypes.c_float),
                ("apply_router_weight_on_input", ctypes.c_int32),
                ("use_sparse_mixer", ctypes.c_int32), ("sparse_mixer_eps", ctypes.c_float)]


class QmoeWorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "topk_ids", "topk_w", "counts", "padded_offsets", "sorted_assign", "assign_pos",
        "tile_list", "num_tiles", "permute_scratch", "h", "y", "xq", "total")] + [
        ("fused_routing", ctypes.c_int32)] + [(n, ctypes.c_size_t) for n in (
        "xcodes", "xfactors", "hcodes", "hfactors", "xsum", "x16", "xlift", "h16", "hlift", "hpart")]


class QmoeStack(ctypes.Structure):
    _fields_ = [("weights", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("bias", ctypes.c_void_p)]


EXPORTS = ("qmoe_validate", "qmoe_tile_m", "qmoe_max_rows", "qmoe_max_tiles",
           "qmoe_permute_scratch_size", "qmoe_workspace_size", "qmoe_route", "qmoe_permute",
           "qmoe_grouped_gemm_fc1_swiglu", "qmoe_grouped_gemm_fc2", "qmoe_combine",
           "qmoe_forward", "qmoe_forward_noalloc", "qmoe_workspace_layout_of", "qmoe_packed_stack_size", "qmoe_pack_stack", "qmoe_linear_woq",
           "qmoe_quantize_act", "qmoe_time_next_gemm", "qmoe_last_error")

_lib = None


def load() -> ctypes.CDLL:
    """Loads the built HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python weight_only_quantized_softmax_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(QmoeParams)
    vp, sz, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64
    st = ctypes.c_int
    L.qmoe_validate.argtypes, L.qmoe_validate.restype = [P], st
    L.qmoe_tile_m.argtypes, L.qmoe_tile_m.restype = [P], ctypes.c_int32
    L.qmoe_max_rows.argtypes, L.qmoe_max_rows.restype = [P], i64
    L.qmoe_max_tiles.argtypes, L.qmoe_max_tiles.restype = [P], i64
    L.qmoe_permute_scratch_size.argtypes, L.qmoe_permute_scratch_size.restype = [P], sz
    L.qmoe_workspace_size.argtypes, L.qmoe_workspace_size.restype = [P], sz
    L.qmoe_route.argtypes, L.qmoe_route.restype = [P, vp, vp, vp, vp], st
    L.qmoe_permute.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.qmoe_permute.restype = st
    L.qmoe_grouped_gemm_fc1_swiglu.argtypes = [P, vp, vp, vp, vp, vp, QmoeStack, QmoeStack, vp,
                                               vp]
    L.qmoe_grouped_gemm_fc1_swiglu.restype = st
    L.qmoe_grouped_gemm_fc2.argtypes = [P, vp, vp, vp, QmoeStack, vp, vp]
    L.qmoe_grouped_gemm_fc2.restype = st
    L.qmoe_combine.argtypes, L.qmoe_combine.restype = [P, vp, vp, vp, vp, vp, vp], st
    L.qmoe_forward.argtypes = [P, vp, vp, QmoeStack, QmoeStack, QmoeStack, vp, vp, vp, sz, vp]
    L.qmoe_forward.restype = st
    L.qmoe_forward_noalloc.argtypes = [P, vp, vp, QmoeStack, QmoeStack, QmoeStack, vp, vp, vp]
    L.qmoe_forward_noalloc.restype = st
    L.qmoe_workspace_layout_of.argtypes = [P, ctypes.POINTER(QmoeWorkspaceLayout)]
    L.qmoe_workspace_layout_of.restype = st
    L.qmoe_packed_stack_size.argtypes = [P, ctypes.c_int32]
    L.qmoe_packed_stack_size.restype = sz
    L.qmoe_pack_stack.argtypes, L.qmoe_pack_stack.restype = [P, ctypes.c_int32, vp, vp, vp], st
    L.qmoe_linear_woq.argtypes = [P, vp, QmoeStack, vp, vp]
    L.qmoe_linear_woq.restype = st
    L.qmoe_quantize_act.argtypes = [P, vp, i64, i64, vp, vp]
    L.qmoe_quantize_act.restype = st
    L.qmoe_time_next_gemm.argtypes, L.qmoe_time_next_gemm.restype = [vp, vp], st
    L.qmoe_last_error.argtypes, L.qmoe_last_error.restype = [], ctypes.c_char_p
    _lib = L
    return L


class QmoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"qmoe {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


def check(status: int) -> None:
    if status != QMOE_OK:
        msg = load().qmoe_last_error().decode(errors="replace")
        raise QmoeError(status, msg)
