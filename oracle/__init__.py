"""TEST INFRASTRUCTURE ONLY: ctypes access to the plain fp64 CPU oracle.

Only ``tests/``, the smoke check and the bench's CPU-baseline leg may import this
package. It never touches the GPU library and the GPU library never touches it.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qmoe_oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")

F32, BF16, E8M0 = 0, 1, 2
_SDT = {"f32": F32, "bf16": BF16, "e8m0": E8M0}
ACTS = {"swiglu": 0, "identity": 1, "relu": 2, "silu": 3, "gelu": 4}


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (-O2, IEEE semantics, no fast-math)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-fopenmp", "-fPIC", "-shared",
                               "-fno-fast-math", SRC, "-o", tmp])
        os.replace(tmp, LIB)
    return LIB


class Params(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("I", ctypes.c_int64),
                ("E", ctypes.c_int64), ("k", ctypes.c_int64), ("bits", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("fusion", ctypes.c_int32),
                ("activation", ctypes.c_int32), ("normalize", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("scale_dtype", ctypes.c_int32),
                ("pad_", ctypes.c_int32), ("alpha", ctypes.c_double),
                ("beta", ctypes.c_double), ("limit", ctypes.c_double),
                ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("routed_scale", ctypes.c_double), ("score_bias", ctypes.c_void_p),
                ("int8_act", ctypes.c_int32), ("pad2_", ctypes.c_int32),
                ("gelu_mode", ctypes.c_int32), ("on_input", ctypes.c_int32),
                ("out_scale", ctypes.c_double), ("sparse_mixer", ctypes.c_int32),
                ("pad3_", ctypes.c_int32), ("mixer_eps", ctypes.c_double)]


class Stack(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("s", ctypes.c_void_p), ("b", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=False)
        L = ctypes.CDLL(LIB)
        P = ctypes.POINTER(Params)
        S = ctypes.POINTER(Stack)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_route.argtypes = [P, vp, vp, vp]
        L.oracle_permute.argtypes = [P, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_permute.restype = i64
        L.oracle_weight.argtypes = [P, S, i64, i64, i64, i64, i64]
        L.oracle_weight.restype = ctypes.c_double
        L.oracle_fc1_rows.argtypes = [P, S, S, vp, i64, vp, vp, vp, vp, i32]
        L.oracle_fc2_rows.argtypes = [P, S, vp, i64, vp, vp, vp, i32]
        L.oracle_combine.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.oracle_forward.argtypes = [P, S, S, S, vp, vp, vp, i64, vp, vp, vp, i32]
        L.oracle_round_bf16.argtypes = [vp, i64, vp]
        L.oracle_int8_round.argtypes = [P, vp, i64, i64, vp]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def params(cfg, T: int, score_bias: Optional[np.ndarray] = None) -> Params:
    """The oracle's parameter block; score_bias: the selection bias [E] in the activation
    dtype (the caller keeps the array alive during the call)."""
    lim = cfg.limit if (cfg.limit is not None and cfg.limit > 0) else math.inf
    return Params(T=T, H=cfg.H, I=cfg.I, E=cfg.E, k=cfg.k, bits=cfg.bits,
                  block_size=cfg.block_size, fusion=cfg.fusion,
                  activation=ACTS[cfg.activation], normalize=int(cfg.normalize),
                  act_dtype=F32 if cfg.act_dtype == "f32" else BF16,
                  scale_dtype=_SDT[cfg.scale_dtype], pad_=0,
                  alpha=cfg.alpha, beta=cfg.beta, limit=lim, n_group=cfg.n_group,
                  topk_group=cfg.topk_group, routed_scale=cfg.routed_scale,
                  score_bias=_ptr(score_bias), int8_act=int(cfg.int8),
                  gelu_mode=cfg.gelu_mode, on_input=int(cfg.on_input),
                  out_scale=cfg.out_scale, sparse_mixer=int(cfg.sparse_mixer),
                  mixer_eps=cfg.mixer_eps)


def _stack(w, s, b) -> Stack:
    return Stack(w=_ptr(w), s=_ptr(s), b=_ptr(b))


def stacks(inp):
    fc1 = _stack(inp.w1, inp.s1, inp.b1)
    fc2 = _stack(inp.w2, inp.s2, inp.b2) if inp.w2 is not None else Stack()
    fc3 = _stack(inp.w3, inp.s3, inp.b3) if inp.w3 is not None else Stack()
    return fc1, fc2, fc3


def route(cfg, logits: np.ndarray, score_bias: Optional[np.ndarray] = None):
    T = logits.shape[0]
    p = params(cfg, T, score_bias)
    ids = np.zeros((T, cfg.k), np.int32)
    w = np.zeros((T, cfg.k), np.float64)
    lib().oracle_route(ctypes.byref(p), _ptr(logits), _ptr(ids), _ptr(w))
    return ids, w


def max_rows(cfg, T: int, M: int) -> int:
    return T * cfg.k + min(cfg.E, T * cfg.k) * (M - 1)


def max_tiles(cfg, T: int, M: int) -> int:
    return (T * cfg.k) // M + min(cfg.E, T * cfg.k)


def permute(cfg, ids: np.ndarray, M: int):
    T = ids.shape[0]
    p = params(cfg, T)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    counts = np.zeros(cfg.E, np.int32)
    offs = np.zeros(cfg.E + 1, np.int32)
    sa = np.full(max_rows(cfg, T, M), -7, np.int32)
    pos = np.zeros(T * cfg.k, np.int32)
    tiles = np.zeros((max_tiles(cfg, T, M), 2), np.int32)
    nt = np.zeros(1, np.int32)
    P = lib().oracle_permute(ctypes.byref(p), M, _ptr(ids), _ptr(counts), _ptr(offs), _ptr(sa),
                             _ptr(pos), _ptr(tiles), _ptr(nt))
    return dict(counts=counts, padded_offsets=offs, sorted_assign=sa[:P], assign_pos=pos,
                tiles=tiles[: int(nt[0])], num_tiles=int(nt[0]), rows=int(P))


def weight(cfg, st: Stack, N: int, K: int, e: int, n: int, kk: int) -> float:
    p = params(cfg, 1)
    return lib().oracle_weight(ctypes.byref(p), ctypes.byref(st), N, K, e, n, kk)


def fc1_rows(cfg, inp, row_token, row_expert, nthreads: int = 0, row_w=None) -> np.ndarray:
    """fc1 + activation of the listed rows; row_w (optional): a factor per row on the input
    (the routing weight, when it goes to the expert's input)."""
    p = params(cfg, inp.x.shape[0])
    fc1, _, fc3 = stacks(inp)
    rt = np.ascontiguousarray(row_token, dtype=np.int32)
    re = np.ascontiguousarray(row_expert, dtype=np.int32)
    rw = None if row_w is None else np.ascontiguousarray(row_w, dtype=np.float64)
    h = np.zeros((len(rt), cfg.I), np.float64)
    lib().oracle_fc1_rows(ctypes.byref(p), ctypes.byref(fc1), ctypes.byref(fc3), _ptr(inp.x),
                          len(rt), _ptr(rt), _ptr(re), _ptr(rw), _ptr(h), nthreads)
    return h


def linear(cfg, inp, rows=None, nthreads: int = 0) -> np.ndarray:
    """A single-expert weight-only-quantized linear layer (CLIKA "QLinearWoQ" page, class
    description: y = x @ dequant(W)^T + bias, the activation as its fused epilogue): the fc1
    row evaluation with every row its own token and expert 0. rows: the x rows to evaluate
    (default all)."""
    assert cfg.E == 1 and cfg.k == 1 and cfg.activation != "swiglu"
    rt = np.arange(inp.x.shape[0]) if rows is None else np.asarray(rows)
    return fc1_rows(cfg, inp, rt, np.zeros(len(rt), np.int32), nthreads)


def fc2_rows(cfg, inp, h_in: np.ndarray, row_index, row_expert, nthreads: int = 0) -> np.ndarray:
    p = params(cfg, 1)
    _, fc2, _ = stacks(inp)
    ri = np.ascontiguousarray(row_index, dtype=np.int32)
    re = np.ascontiguousarray(row_expert, dtype=np.int32)
    y = np.zeros((len(ri), cfg.H), np.float64)
    lib().oracle_fc2_rows(ctypes.byref(p), ctypes.byref(fc2), _ptr(np.ascontiguousarray(h_in)),
                          len(ri), _ptr(ri), _ptr(re), _ptr(y), nthreads)
    return y


def combine(cfg, y: np.ndarray, assign_pos: np.ndarray, w: np.ndarray, shared=None):
    T = w.shape[0]
    p = params(cfg, T)
    y = np.ascontiguousarray(y, dtype=np.float32)
    pos = np.ascontiguousarray(assign_pos, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    out64 = np.zeros((T, cfg.H), np.float64)
    outr = np.zeros((T, cfg.H), np.float32 if cfg.act_dtype == "f32" else np.uint16)
    lib().oracle_combine(ctypes.byref(p), _ptr(y), _ptr(pos), _ptr(w), _ptr(shared),
                         _ptr(out64), _ptr(outr))
    return out64, outr


def forward(cfg, inp, sel=None, nthreads: int = 0):
    """Oracle forward for all tokens (sel=None) or the listed token indices."""
    T = inp.x.shape[0]
    p = params(cfg, T, inp.ebias)
    fc1, fc2, fc3 = stacks(inp)
    if sel is not None:
        sel = np.ascontiguousarray(sel, dtype=np.int64)
        n = len(sel)
    else:
        n = T
    out64 = np.zeros((n, cfg.H), np.float64)
    outr = np.zeros((n, cfg.H), np.float32 if cfg.act_dtype == "f32" else np.uint16)
    lib().oracle_forward(ctypes.byref(p), ctypes.byref(fc1), ctypes.byref(fc2), ctypes.byref(fc3),
                         _ptr(inp.x), _ptr(inp.logits), _ptr(inp.shared), n, _ptr(sel),
                         _ptr(out64), _ptr(outr), nthreads)
    return out64, outr


def int8_round(cfg, a: np.ndarray) -> np.ndarray:
    """The int8 activation tier's per-block rounding of the rows of a ([rows, cols], stored
    in the activation dtype); the result has a's dtype and shape."""
    a = np.ascontiguousarray(a)
    rows, cols = a.shape
    out = np.zeros_like(a)
    p = params(cfg, rows)
    lib().oracle_int8_round(ctypes.byref(p), _ptr(a), rows, cols, _ptr(out))
    return out


def round_bf16(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.zeros(v.shape, np.uint16)
    lib().oracle_round_bf16(_ptr(v), v.size, _ptr(out))
    return out
