"""The int8 activation tier on the GPU (ClikaRT "QMoEWoQ" page, class description: on the
int8 block tier the activation is quantised to int8 per block ahead of the dot product).

* the rounding itself (qmoe_quantize_act) bit for bit against the oracle's, both dtypes,
  ragged last blocks, in place and out of place;
* the forward with compute_mode int8 against the oracle's int8 forward on the decode,
  prefill, many-expert and MX FP4 shapes, at the bf16 tolerance.

With fp32 activations the forward refuses the tier (QMOE_ERR_UNSUPPORTED, checked on the
host): the codes of h are decided from h, and an fp32 h that differs from the oracle's fp64
h in its last bit (summation order) can move one code by a step, which is worth more than
the fp32 tolerance. The rounding itself is checked in both dtypes.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_softmax_amd as qm
from synth import configs
from synth.gen import store
from tests.gpu_helpers import dev, host, params_for
from tests.test_gpu_parity import check_forward, say

pytestmark = pytest.mark.gpu


def _rows(rng, rows, cols, bs):
    nb = -(-cols // bs)
    mag = 2.0 ** rng.integers(-12, 12, (rows, nb))
    v = rng.normal(0, 1, (rows, cols)) * np.repeat(mag, bs, axis=1)[:, :cols]
    if rows > 0:
        v[0, :min(cols, bs)] = 0.0
    if rows > 1:
        w = min(cols, bs)
        v[1, 0] = 127.0 * 2.0 ** -3
        v[1, 1:w] = (rng.integers(-126, 126, w - 1) + 0.5) * 2.0 ** -3
    if rows > 2:
        v[2, 0] = 127.5 * 2.0 ** -3
    return v


@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols,bs", [(1, 2880, 32), (64, 2880, 128), (300, 2048, 16),
                                          (7, 80, 32), (5, 200, 64), (3, 81, 16),
                                          (0, 64, 32)])
@pytest.mark.parametrize("inplace", [False, True])
def test_quantize_act_bit_exact(act, rows, cols, bs, inplace):
    say("quantize", act, rows, cols, bs, "inplace" if inplace else "")
    rng = np.random.default_rng(rows * 7 + cols + bs)
    # the rounding reads block_size and the activation dtype of the parameter block; its
    # other shapes only need to be valid ones
    cfg = configs.tiny(act_dtype=act, block_size=bs)
    v = store(_rows(rng, rows, cols, bs), act)
    p = params_for(cfg, max(rows, 1))
    x = dev(v, act)
    out = x if inplace else torch.empty_like(x)
    qm.qmoe_quantize_act(p, x, out)
    torch.cuda.synchronize()
    want = oracle.int8_round(cfg, v) if rows else v
    assert np.array_equal(host(out), want)


def test_quantize_act_rejects_per_row_scales():
    cfg = configs.tiny(act_dtype="bf16", block_size=0, H=64)
    p = params_for(cfg, 4)
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(qm.QmoeError):
        qm.qmoe_quantize_act(p, x, x)


@pytest.mark.parametrize("T", [1, 8, 64])
@pytest.mark.parametrize("layout", ["rows", "tiles"])
def test_forward_int8_c2_decode(T, layout):
    check_forward(configs.C2_INT8, T, shared=(T == 8), layout=layout)


def test_forward_int8_c4_many_experts_ragged_blocks():
    check_forward(configs.C4_INT8, 512, sample=16, layout="tiles")


@pytest.mark.parametrize("bits,bs", [(4, 32), (8, 128), (4, 16)])
@pytest.mark.parametrize("T", [256, 4096])
def test_forward_int8_c5(T, bits, bs):
    check_forward(configs.c5_point(bits, bs).with_(int8=True), T, sample=6, layout="tiles")


@pytest.mark.parametrize("T", [1, 64])
def test_forward_int8_mxfp4_c2(T):
    check_forward(configs.C2_MX_INT8, T, layout="tiles")


@pytest.mark.parametrize("T", [16, 256])
def test_forward_int8_with_routing_variants(T):
    # grouped top-k, selection bias and weight scaling together with the int8 tier
    check_forward(configs.C5_ROUTED.with_(int8=True), T, sample=6, layout="tiles")


@pytest.mark.parametrize("bits,bs", [(4, 32), (8, 64)])
def test_forward_int8_rows_layout_prefill(bits, bs):
    # the weights as given (rows layout) through the 128-row kernels
    check_forward(configs.c5_point(bits, bs).with_(int8=True), 4096, sample=6, layout="rows")


def test_forward_int8_unfused_gate_up():
    # separate gate (fc1) and up (fc3) stacks, per-block scales of 64, 32-row tiles
    cfg = configs.tiny(E=8, k=2, act_dtype="bf16", scale_dtype="bf16", H=256, I=128,
                       fusion=0, bits=4, block_size=64, fc1_bias=True, fc2_bias=True,
                       limit=7.0, int8=True)
    check_forward(cfg, 300, layout="tiles")


# The int8 dot on the int8 matrix cores (prefill-sized tiles, tiled layout, integer codes,
# blocks of 64 and 128, H and I multiples of 64): 4- and 8-bit codes, both block lengths, K
# an odd multiple of 64 for 4-bit codes (the second half of the last 128-k step is past K),
# a ragged last block of 64 (c4's 2880 with blocks of 128), fused and separate gate/up.
I8_DOT_CASES = {
    "c5-b4-bs64-T4096": (configs.c5_point(4, 64).with_(int8=True), 4096),
    "c5-b4-bs128-T4096": (configs.c5_point(4, 128).with_(int8=True), 4096),
    "c5-b8-bs64-T4096": (configs.c5_point(8, 64).with_(int8=True), 4096),
    "c5-b8-bs128-T4096": (configs.c5_point(8, 128).with_(int8=True), 4096),
    "c2-b4-bs64-K2880-T1024": (configs.C2_INT8.with_(block_size=64), 1024),
    "c4-b8-bs128-ragged-T2048": (configs.C4_INT8, 2048),
    "separate-gate-up-b4-bs64": (configs.tiny(E=4, k=2, act_dtype="bf16", scale_dtype="bf16",
                                              H=2048, I=1536, fusion=0, bits=4, block_size=64,
                                              fc1_bias=True, fc2_bias=True, int8=True), 4096),
}


@pytest.mark.parametrize("name", sorted(I8_DOT_CASES))
def test_forward_int8_dot(name):
    cfg, T = I8_DOT_CASES[name]
    p = params_for(cfg, T, layout="tiles")
    assert qm.qmoe_tile_m(p) == 128
    assert qm.qmoe_workspace_layout_of(p).xcodes != 0  # the int8 matrix-core path is taken
    check_forward(cfg, T, sample=24, layout="tiles")
