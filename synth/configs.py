"""Workload definitions for the weight-only-quantized MoE forward.

Pure data: shapes, flags and the value distributions of the synthetic inputs.
Nothing here computes any part of the method.

Field meanings follow the QMoE operator contract (graiphic "QMoE" page, inputs
and attributes) and the ClikaRT QMoEWoQ ``make``/``forward`` signatures:

* ``H`` hidden_size, ``I`` inter_size, ``E`` num_experts, ``k`` top-k.
* ``bits`` expert_weight_bits (4 or 8); ``block_size`` 0 = one scale per
  output row, else the K-block length of one scale.
* ``fusion`` swiglu_fusion: 0 separate fc1 (gate) and fc3 (up) stacks,
  1 fused gate/up rows interleaved, 2 fused gate rows then up rows.
* ``limit`` ``inf`` means no clamp.
* ``act_dtype``/``scale_dtype``: "f32" or "bf16".
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    T_points: Tuple[int, ...]
    H: int
    I: int
    E: int
    k: int
    normalize: bool
    fusion: int
    alpha: float
    beta: float
    limit: float
    bits: int
    block_size: int
    act_dtype: str
    scale_dtype: str
    fc1_bias: bool
    fc2_bias: bool
    activation: str = "swiglu"
    x_sigma: float = 1.0
    logit_sigma: float = 1.0
    logit_skew: float = 0.0          # added to expert 0's logit before rounding
    scale_lo: float = 0.005
    scale_hi: float = 0.02
    bias_sigma: float = 0.02
    seed_base: int = 20261203
    # routing variants (CLIKA "MoE" page routing kwargs; ClikaRT "QMoEWoQ" page selection
    # bias): grouped top-k, weight scaling, and a selection bias [E] ~ N(0, ebias_sigma)
    n_group: int = 0
    topk_group: int = 0
    routed_scale: float = 1.0
    score_bias: bool = False
    ebias_sigma: float = 0.5
    # the int8 activation tier (ClikaRT "QMoEWoQ" page, class description)
    int8: bool = False
    # the remaining routing kwargs and activations (CLIKA "MoE" page: gelu_mode,
    # apply_router_weight_on_input, expert_output_scale, sparse_mixer_eps; graiphic "QMoE"
    # page: activation_type gelu, use_sparse_mixer): gelu_mode 0 the exact gelu, 1 its tanh
    # approximation; on_input: the routing weight scales the expert's input; out_scale:
    # multiplies every expert's output; sparse_mixer: the two-pick sparse mixer routing
    gelu_mode: int = 0
    on_input: bool = False
    out_scale: float = 1.0
    sparse_mixer: bool = False
    mixer_eps: float = 0.01

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    @property
    def pack(self) -> int:
        return 8 // self.bits

    @property
    def n1(self) -> int:
        """Rows of the fc1 stack: 2*I when gate and up are fused, else I."""
        return 2 * self.I if (self.activation == "swiglu" and self.fusion != 0) else self.I

    @property
    def has_fc3(self) -> bool:
        return self.activation == "swiglu" and self.fusion == 0

    def nblocks(self, K: int) -> int:
        """Scales per row for a K-long row; a short last block is allowed."""
        return 0 if self.block_size == 0 else -(-K // self.block_size)


INF = math.inf

# c1: tiny fp32 case (correctness only).
C1 = Config(name="c1-tiny-fp32", T_points=(16,), H=128, I=256, E=8, k=2, normalize=True,
            fusion=2, alpha=1.0, beta=0.0, limit=INF, bits=4, block_size=32,
            act_dtype="f32", scale_dtype="f32", fc1_bias=False, fc2_bias=False)

# c2: decode-shaped int4 layer, interleaved gate/up, gpt-oss style clamp.
C2 = Config(name="c2-decode-int4", T_points=(1, 8, 64), H=2880, I=2880, E=32, k=4,
            normalize=True, fusion=1, alpha=1.702, beta=1.0, limit=7.0, bits=4,
            block_size=32, act_dtype="bf16", scale_dtype="bf16", fc1_bias=True,
            fc2_bias=True, logit_sigma=2.0)

# c3: prefill-shaped int4 layer, separate gate (fc1) and up (fc3) stacks,
# per-row scales, expert 0 receives about 40% of the assignments.
C3 = Config(name="c3-prefill-int4", T_points=(4096,), H=4096, I=14336, E=8, k=2,
            normalize=True, fusion=0, alpha=1.0, beta=0.0, limit=INF, bits=4,
            block_size=0, act_dtype="bf16", scale_dtype="bf16", fc1_bias=False,
            fc2_bias=False, logit_skew=1.70)

# c4: many small experts, int8 weights, K=2880 with 128-blocks (ragged last block).
C4 = Config(name="c4-many-expert-int8", T_points=(512,), H=2880, I=2880, E=128, k=4,
            normalize=False, fusion=2, alpha=1.0, beta=0.0, limit=7.0, bits=8,
            block_size=128, act_dtype="bf16", scale_dtype="f32", fc1_bias=False,
            fc2_bias=False, scale_lo=0.005 / 16, scale_hi=0.02 / 16)

# c5: block-size / bit-width sweep (bits and block_size are overridden per point).
C5 = Config(name="c5-sweep", T_points=(1, 256, 4096), H=2048, I=1408, E=64, k=6,
            normalize=True, fusion=2, alpha=1.0, beta=0.0, limit=INF, bits=4,
            block_size=32, act_dtype="bf16", scale_dtype="bf16", fc1_bias=True,
            fc2_bias=False, scale_lo=0.002, scale_hi=0.05)

# Single-expert linear layers (QLinearWoQ): one quantized weight [I, H] (out_features I,
# in_features H), the layer shapes of the MoE workloads above read as dense layers.
# lin-decode: c2's fused gate/up projection (2880 -> 5760), 4-bit, bs 32, bias, SiLU.
LIN_DECODE = Config(name="lin-decode-int4", T_points=(1, 64), H=2880, I=5760, E=1, k=1,
                    normalize=False, fusion=0, alpha=1.0, beta=0.0, limit=INF, bits=4,
                    block_size=32, act_dtype="bf16", scale_dtype="bf16", fc1_bias=True,
                    fc2_bias=False, activation="silu")
# lin-prefill: c3's gate projection (4096 -> 14336), 4-bit per-row scales, no bias.
LIN_PREFILL = Config(name="lin-prefill-int4", T_points=(4096,), H=4096, I=14336, E=1, k=1,
                     normalize=False, fusion=0, alpha=1.0, beta=0.0, limit=INF, bits=4,
                     block_size=0, act_dtype="bf16", scale_dtype="bf16", fc1_bias=False,
                     fc2_bias=False, activation="identity")
LINEAR = {"lin-decode": LIN_DECODE, "lin-prefill": LIN_PREFILL}

# MX FP4 weights (E2M1 codes, one E8M0 scale per 32 k: the gpt-oss checkpoint format the
# ClikaRT QMoEWoQ page names), on the c2 decode layer and the c5 sweep shape. Scales are
# the powers of two nearest to U(scale_lo, scale_hi) in log2 (2^-8 .. 2^-6 here).
C2_MX = C2.with_(name="c2-decode-mxfp4", scale_dtype="e8m0")
C5_MX = C5.with_(name="c5-sweep-mxfp4", bits=4, block_size=32, scale_dtype="e8m0")
MX = {"c2-mx": C2_MX, "c5-mx": C5_MX}

# Routing variants on the c5 shape (64 experts in 8 groups of 8, 4 groups kept, k = 6, a
# selection bias and a weight scale of 2.5) and on c2 (a selection bias only).
C5_ROUTED = C5.with_(name="c5-grouped-biased", n_group=8, topk_group=4, routed_scale=2.5,
                     score_bias=True)
C2_BIASED = C2.with_(name="c2-biased", score_bias=True)
# the int8 activation tier on the decode, prefill and many-expert shapes
C2_INT8 = C2.with_(name="c2-decode-int4-a8", int8=True)
C4_INT8 = C4.with_(name="c4-many-expert-int8-a8", int8=True)
C5_INT8 = C5.with_(name="c5-sweep-a8", int8=True)
C2_MX_INT8 = C2_MX.with_(name="c2-decode-mxfp4-a8", int8=True)

C5_BITS = (4, 8)
C5_BLOCKS = (16, 32, 64, 128)

ALL = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5}


def c5_point(bits: int, block_size: int) -> Config:
    return C5.with_(bits=bits, block_size=block_size,
                    name=f"c5-sweep-b{bits}-bs{block_size}")


def tiny(**kw) -> Config:
    """A small config for unit tests; every field may be overridden."""
    base = Config(name="tiny", T_points=(5,), H=64, I=32, E=4, k=2, normalize=True,
                  fusion=2, alpha=1.0, beta=0.0, limit=INF, bits=4, block_size=16,
                  act_dtype="f32", scale_dtype="f32", fc1_bias=False, fc2_bias=False)
    return base.with_(**kw)
