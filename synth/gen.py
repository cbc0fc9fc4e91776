"""Seeded synthetic inputs for the weight-only-quantized MoE forward.

Both the GPU path's tests/bench and the CPU oracle take their inputs from here.
This module only draws random numbers and stores them in the element types of
the QMoE tensor contract (graiphic "QMoE" page, inputs list); it holds none of
the method's arithmetic.

Storage conventions (what the arrays hold):

* floating tensors in "bf16" are ``uint16`` arrays of bfloat16 bit patterns,
  tensors in "f32" are ``float32`` arrays;
* quantized stacks are ``uint8`` arrays ``[E, N, K // pack]`` of independent
  uniformly random bytes (every bit pattern of every field is equally likely).
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Optional

import numpy as np

from .configs import Config

TENSOR_IDS = {"x": 1, "logits": 2, "w1": 3, "s1": 4, "b1": 5, "w3": 6, "s3": 7,
              "b3": 8, "w2": 9, "s2": 10, "b2": 11, "shared": 12, "h": 13, "y": 14,
              "topk_w": 15, "topk_ids": 16, "ebias": 17}


def rng_for(cfg: Config, tensor: str, T: Optional[int] = None, seed: int = 0) -> np.random.Generator:
    key = [cfg.seed_base, zlib.crc32(cfg.name.encode()), TENSOR_IDS[tensor], -1 if T is None else T, seed]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([v & 0xFFFFFFFF for v in key])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Store float32 values as bfloat16 bit patterns, round-to-nearest-even."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def store(values_f64: np.ndarray, dtype: str) -> np.ndarray:
    """Values in a storage type: f32, bf16 bits (RNE), or e8m0 (scales only: the byte e of
    the power of two 2^(e - 127) nearest to the value in log2, e in [1, 254])."""
    if dtype == "e8m0":
        e = np.rint(np.log2(np.asarray(values_f64, dtype=np.float64))) + 127
        return np.clip(e, 1, 254).astype(np.uint8)
    v32 = np.asarray(values_f64, dtype=np.float32)
    if dtype == "f32":
        return v32
    if dtype == "bf16":
        return f32_to_bf16_bits(v32)
    raise ValueError(dtype)


def as_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """View stored values as float32 (exact for every storage type)."""
    if dtype == "e8m0":
        return np.ldexp(np.float32(1.0), np.asarray(a, dtype=np.int32) - 127).astype(np.float32)
    return bf16_bits_to_f32(a) if dtype == "bf16" else np.asarray(a, dtype=np.float32)


def random_bytes(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return np.frombuffer(rng.bytes(n), dtype=np.uint8).reshape(shape).copy()


@dataclasses.dataclass
class Inputs:
    cfg: Config
    T: int
    x: np.ndarray
    logits: np.ndarray
    w1: np.ndarray
    s1: np.ndarray
    b1: Optional[np.ndarray]
    w2: np.ndarray
    s2: np.ndarray
    b2: Optional[np.ndarray]
    w3: Optional[np.ndarray] = None
    s3: Optional[np.ndarray] = None
    b3: Optional[np.ndarray] = None
    shared: Optional[np.ndarray] = None
    ebias: Optional[np.ndarray] = None  # selection bias [E], activation dtype


def gen_weights(cfg: Config, which: str, N: int, K: int, seed: int = 0):
    """One quantized stack: (bytes [E,N,K/pack], scales, optional bias)."""
    w = random_bytes(rng_for(cfg, "w" + which, seed=seed), (cfg.E, N, K // cfg.pack))
    srng = rng_for(cfg, "s" + which, seed=seed)
    sshape = (cfg.E, N) if cfg.block_size == 0 else (cfg.E, N, cfg.nblocks(K))
    s = store(srng.uniform(cfg.scale_lo, cfg.scale_hi, size=sshape), cfg.scale_dtype)
    want_bias = {"1": cfg.fc1_bias, "3": cfg.fc1_bias, "2": cfg.fc2_bias}[which]
    b = None
    if want_bias:
        b = store(rng_for(cfg, "b" + which, seed=seed).normal(0.0, cfg.bias_sigma, size=(cfg.E, N)),
                  cfg.act_dtype)
    return w, s, b


def gen_activations(cfg: Config, T: int, seed: int = 0, shared: bool = False):
    x = store(rng_for(cfg, "x", T, seed).normal(0.0, cfg.x_sigma, size=(T, cfg.H)), cfg.act_dtype)
    lg = rng_for(cfg, "logits", T, seed).normal(0.0, cfg.logit_sigma, size=(T, cfg.E))
    if cfg.logit_skew:
        lg[:, 0] += cfg.logit_skew
    logits = store(lg, cfg.act_dtype)
    sh = None
    if shared:
        sh = store(rng_for(cfg, "shared", T, seed).normal(0.0, 1.0, size=(T, cfg.H)), cfg.act_dtype)
    return x, logits, sh


def gen_score_bias(cfg: Config, seed: int = 0) -> Optional[np.ndarray]:
    """The selection bias [E] of a config that has one (activation dtype), else None."""
    if not cfg.score_bias:
        return None
    return store(rng_for(cfg, "ebias", seed=seed).normal(0.0, cfg.ebias_sigma, size=cfg.E),
                 cfg.act_dtype)


def make_inputs(cfg: Config, T: int, seed: int = 0, shared: bool = False) -> Inputs:
    x, logits, sh = gen_activations(cfg, T, seed, shared)
    w1, s1, b1 = gen_weights(cfg, "1", cfg.n1, cfg.H, seed)
    w2, s2, b2 = gen_weights(cfg, "2", cfg.H, cfg.I, seed)
    w3 = s3 = b3 = None
    if cfg.has_fc3:
        w3, s3, b3 = gen_weights(cfg, "3", cfg.I, cfg.H, seed)
    return Inputs(cfg=cfg, T=T, x=x, logits=logits, w1=w1, s1=s1, b1=b1, w2=w2, s2=s2,
                  b2=b2, w3=w3, s3=s3, b3=b3, shared=sh, ebias=gen_score_bias(cfg, seed))


def make_linear_inputs(cfg: Config, T: int, seed: int = 0) -> Inputs:
    """Inputs of a single-expert linear layer (E = 1, k = 1): x [T, H] and the one weight
    stack [1, I, H/pack] with its scales and optional bias; no logits and no fc2 stack."""
    assert cfg.E == 1 and cfg.k == 1 and cfg.activation != "swiglu"
    x = store(rng_for(cfg, "x", T, seed).normal(0.0, cfg.x_sigma, size=(T, cfg.H)), cfg.act_dtype)
    w1, s1, b1 = gen_weights(cfg, "1", cfg.I, cfg.H, seed)
    return Inputs(cfg=cfg, T=T, x=x, logits=None, w1=w1, s1=s1, b1=b1, w2=None, s2=None, b2=None)


def gen_stage_h(cfg: Config, rows: int, seed: int = 0, sigma: float = 1.0) -> np.ndarray:
    """A synthetic fc2 input [rows, I] in the activation dtype."""
    return store(rng_for(cfg, "h", rows, seed).normal(0.0, sigma, size=(rows, cfg.I)), cfg.act_dtype)


def gen_stage_y(cfg: Config, rows: int, seed: int = 0) -> np.ndarray:
    """A synthetic per-assignment expert output [rows, H] in float32."""
    return rng_for(cfg, "y", rows, seed).normal(0.0, 1.0, size=(rows, cfg.H)).astype(np.float32)


def gen_topk_w(cfg: Config, T: int, seed: int = 0) -> np.ndarray:
    return rng_for(cfg, "topk_w", T, seed).uniform(0.0, 1.0, size=(T, cfg.k)).astype(np.float32)


def gen_topk_ids(cfg: Config, T: int, seed: int = 0, skew: float = 0.0) -> np.ndarray:
    """Distinct expert ids per token, drawn without replacement (optionally skewed)."""
    rng = rng_for(cfg, "topk_ids", T, seed)
    p = np.ones(cfg.E)
    if skew:
        p[0] += skew
    p = p / p.sum()
    out = np.empty((T, cfg.k), dtype=np.int32)
    for t in range(T):
        out[t] = rng.choice(cfg.E, size=cfg.k, replace=False, p=p)
    return out
