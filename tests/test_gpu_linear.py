"""The single-expert linear layer qmoe_linear_woq (QLinearWoQ) against the oracle, element
by element: every tile height (16, 32 and 128 rows, by the token count), both weight
layouts, 4- and 8-bit weights with per-row and block scales (a short last block
included), each plain activation, fp32 and bf16 activations, and the two full-size layer
shapes on sampled rows."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_softmax_amd as qm
from synth import configs, gen
from tests.gpu_helpers import check_output, dev, host_f64

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qm._lib.load()
    torch.cuda.init()


def lin_params(cfg, T, layout="rows", tile_m=0):
    return qm.linear_params(T, cfg.H, cfg.I, expert_weight_bits=cfg.bits,
                            block_size=cfg.block_size, activation=cfg.activation,
                            act_dtype=cfg.act_dtype, scale_dtype=cfg.scale_dtype,
                            tile_m=tile_m, weight_layout=layout, gelu_mode=cfg.gelu_mode)


def run_linear(cfg, inp, layout, tile_m=0):
    T = inp.x.shape[0]
    p = lin_params(cfg, T, layout, tile_m)
    w = dev(inp.w1)
    if layout == "tiles":
        w = qm.pack_stack(p, "fc1", w)
    stack = (w, dev(inp.s1, cfg.scale_dtype),
             dev(inp.b1, cfg.act_dtype) if inp.b1 is not None else None)
    y = qm.linear_woq(p, dev(inp.x, cfg.act_dtype), stack)
    torch.cuda.synchronize()
    return host_f64(y, cfg.act_dtype), qm.qmoe_tile_m(p)


def check(cfg, T, layout, sample=None, tile_m=0):
    inp = gen.make_linear_inputs(cfg, T)
    got, M = run_linear(cfg, inp, layout, tile_m)
    print("linear", cfg.name, layout, "T", T, "K", cfg.H, "N", cfg.I, "M", M, flush=True)
    assert got.shape == (T, cfg.I)
    rows = np.arange(T)
    if sample is not None and sample < T:
        rng = np.random.default_rng(T + 5)
        rows = np.unique(np.concatenate([[0, T - 1], rng.choice(T, size=sample - 2, replace=False)]))
    ref = oracle.linear(cfg, inp, rows=rows, nthreads=NTHREADS)
    # the layer's output is the result: max |err| against the unrounded fp64 oracle, relative
    # to its RMS, at the activation dtype's bound (the bf16 rounding floor and the error
    # beyond it are printed beside it)
    print("  " + check_output(got[rows], ref, cfg.act_dtype), flush=True)
    return M


SMALL = {
    "b4-bs32-silu-bias": configs.tiny(E=1, k=1, fusion=0, activation="silu", bits=4, block_size=32,
                                      H=544, I=352, fc1_bias=True, act_dtype="bf16",
                                      scale_dtype="bf16"),
    "b4-bs64-shortblock-identity": configs.tiny(E=1, k=1, fusion=0, activation="identity", bits=4,
                                                block_size=64, H=544, I=224, act_dtype="bf16",
                                                scale_dtype="bf16"),
    "b8-perrow-relu-f32scale": configs.tiny(E=1, k=1, fusion=0, activation="relu", bits=8,
                                            block_size=0, H=448, I=192, fc1_bias=True,
                                            act_dtype="bf16", scale_dtype="f32"),
    "b8-bs16-silu": configs.tiny(E=1, k=1, fusion=0, activation="silu", bits=8, block_size=16,
                                 H=512, I=160, act_dtype="bf16", scale_dtype="bf16"),
    "b4-perrow-relu": configs.tiny(E=1, k=1, fusion=0, activation="relu", bits=4, block_size=0,
                                   H=384, I=256, fc1_bias=True, act_dtype="bf16",
                                   scale_dtype="bf16"),
}
# (tokens, tile_m): the library's 16- and 32-row choices and the 128-row kernels asked
# for explicitly (the library keeps them for large grids), each with a ragged last tile
TOKENS = ((5, 0), (37, 0), (300, 128))


@pytest.mark.parametrize("layout", ["rows", "tiles"])
@pytest.mark.parametrize("T,tile_m", TOKENS)
@pytest.mark.parametrize("name", sorted(SMALL))
def test_linear_matches_oracle(name, T, tile_m, layout):
    M = check(SMALL[name], T, layout, tile_m=tile_m)
    assert M == {5: 16, 37: 32, 300: 128}[T]


@pytest.mark.parametrize("T", [1, 16, 70])
def test_linear_fp32_activations(T):
    cfg = configs.tiny(E=1, k=1, fusion=0, activation="silu", bits=4, block_size=32, H=128,
                       I=96, fc1_bias=True)
    check(cfg, T, "rows")


@pytest.mark.parametrize("T", configs.LIN_DECODE.T_points)
@pytest.mark.parametrize("layout", ["rows", "tiles"])
def test_linear_decode_full_size(T, layout):
    check(configs.LIN_DECODE, T, layout, sample=8)


def test_linear_prefill_full_size_sampled():
    check(configs.LIN_PREFILL, 4096, "tiles", sample=6)


def test_linear_3d_input_and_no_padding_rows():
    cfg = SMALL["b4-bs32-silu-bias"]
    inp = gen.make_linear_inputs(cfg, 37)
    p = lin_params(cfg, 37)
    x = dev(inp.x, "bf16").view(1, 37, cfg.H)
    stack = (dev(inp.w1), dev(inp.s1, "bf16"), dev(inp.b1, "bf16"))
    # y gets exactly T rows: a guard row after it must stay untouched
    buf = torch.full((38, cfg.I), 3.0, dtype=torch.bfloat16, device="cuda")
    qm.qmoe_linear_woq(p, x.view(37, cfg.H), stack, buf[:37])
    y3 = qm.linear_woq(p, x, stack)
    torch.cuda.synchronize()
    assert y3.shape == (1, 37, cfg.I)
    assert torch.equal(y3.view(37, cfg.I).view(torch.int16), buf[:37].view(torch.int16))
    assert torch.all(buf[37] == 3.0)
