"""The packing entry point on the GPU: qmoe_pack_stack writes, byte for byte, what the
reference packer (tests/tiled_ref.py, from the layout description in include/qmoe.h)
produces, for every stack kind, both bit widths, and row and K counts that leave partial
tiles. The GEMMs that read the tiled layout are checked against the oracle with the other
parity tests (layout "tiles")."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import weight_only_quantized_softmax_amd as qm
from tests import tiled_ref as tr
from tests.gpu_helpers import dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qm._lib.load()
    torch.cuda.init()


PACK_CASES = [
    # (bits, which, swiglu_fusion, activation, H, I, E)
    (4, "fc1", 1, "swiglu", 2880, 2880, 2),   # decode shape: K = 22.5 tiles
    (4, "fc1", 2, "swiglu", 160, 40, 3),      # rows per stream not a multiple of 16
    (4, "fc1", 0, "swiglu", 224, 48, 2),
    (4, "fc3", 0, "swiglu", 224, 48, 2),
    (4, "fc2", 0, "swiglu", 96, 352, 3),
    (8, "fc1", 1, "swiglu", 704, 352, 2),     # K = 11 tiles of 64
    (8, "fc1", 2, "swiglu", 96, 80, 2),
    (8, "fc2", 0, "swiglu", 80, 96, 3),       # 80 rows: 5 blocks; K = 1.5 tiles
    (8, "fc1", 0, "relu", 128, 96, 2),
]


@pytest.mark.parametrize("bits,which,fusion,act,H,I,E", PACK_CASES)
def test_pack_matches_reference(bits, which, fusion, act, H, I, E):
    # fp32 activations admit every multiple of the packing factor as H and I (the bf16
    # path wants multiples of 32); the packing itself does not depend on the activations
    p = qm.make_params(4, H, I, E, 1, expert_weight_bits=bits, block_size=0,
                       swiglu_fusion=fusion, activation=act, act_dtype="f32", scale_dtype="f32")
    K, N, S, R, _ = tr.stack_geometry(which, H, I, bits, fusion, swiglu=act == "swiglu")
    rng = np.random.default_rng(bits * 100 + H + I)
    w = rng.integers(0, 256, size=(E, N, K * bits // 8), dtype=np.uint8)
    print("pack", bits, which, fusion, act, H, I, E, flush=True)
    got = host(qm.pack_stack(p, which, dev(w)))
    torch.cuda.synchronize()
    want = tr.pack(w, which, H, I, bits, fusion, swiglu=act == "swiglu")
    assert got.shape == want.shape
    assert np.array_equal(got, want)


@pytest.mark.parametrize("which,fusion,H,I,E", [("fc1", 1, 2880, 2880, 2), ("fc1", 2, 160, 64, 3),
                                               ("fc2", 0, 96, 352, 2)])
def test_pack_mxfp4_keeps_code_order(which, fusion, H, I, E):
    # MX FP4 (E8M0 scales): element i of a word in nibble i, the order of the scaled FP4
    # conversions; the params may name either layout (the packing reads only the shapes)
    p = qm.make_params(4, H, I, E, 1, expert_weight_bits=4, block_size=32, swiglu_fusion=fusion,
                       act_dtype="bf16", scale_dtype="e8m0", weight_layout="rows")
    K, N, S, R, _ = tr.stack_geometry(which, H, I, 4, fusion)
    rng = np.random.default_rng(H + I + E)
    w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    print("pack mxfp4", which, fusion, H, I, E, flush=True)
    got = host(qm.pack_stack(p, which, dev(w)))
    torch.cuda.synchronize()
    want = tr.pack(w, which, H, I, 4, fusion, natural=True)
    assert np.array_equal(got, want)
