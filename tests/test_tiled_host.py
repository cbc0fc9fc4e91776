"""The tiled weight layout without a GPU: the reference packer against hand-worked bytes
of the layout description in include/qmoe.h, its inverse, the library's size query, and
the packing entry point's host-side checks."""
from __future__ import annotations

import numpy as np
import pytest

import weight_only_quantized_softmax_amd as qm
from weight_only_quantized_softmax_amd import _lib
from tests import tiled_ref as tr


def _rows4(codes):
    """[E, N, K] four-bit codes -> rows layout, element 2j in the low nibble."""
    return (codes[:, :, 0::2] | (codes[:, :, 1::2] << 4)).astype(np.uint8)


def test_worked_example_4bit_nibble_order():
    # one row of K = 128 four-bit codes c[k] = k mod 16 (fc2 stack: H rows, K = I)
    H, I = 16, 128
    codes = np.zeros((1, H, I), np.uint8)
    codes[0, 0] = np.arange(I) % 16
    pk = tr.pack(_rows4(codes), "fc2", H, I, 4, 0).reshape(64, 16)  # one tile
    # lane 0 (row 0, q = 0), word 0: k = 0..7 in nibbles (0, 2, 4, 6, 1, 3, 5, 7) -> 0x75316420
    assert pk[0, 0:4].tolist() == [0x20, 0x64, 0x31, 0x75]
    # lane 16 (row 0, q = 1): word 0 holds k = 8..15, word 1 k = 40..47 (also 8..15 mod 16)
    assert pk[16, 0:4].tolist() == [0xA8, 0xEC, 0xB9, 0xFD]
    assert pk[16, 4:8].tolist() == [0xA8, 0xEC, 0xB9, 0xFD]
    # word 3 of lane 48 (q = 3): k = 96 + 24 .. 127 -> codes 8..15
    assert pk[48, 12:16].tolist() == [0xA8, 0xEC, 0xB9, 0xFD]
    # lanes of rows 1..15 hold zero codes
    assert not pk[1:16].any() and not pk[17:32].any()


def test_worked_example_8bit_and_padding():
    # fc2 stack, 8-bit, K = 80 (one full tile of 64 and a ragged one), 20 rows (two row blocks)
    H, I = 20, 80
    codes = (np.arange(H * I, dtype=np.int64).reshape(1, H, I) % 251).astype(np.uint8)
    pk = tr.pack(codes.copy(), "fc2", H, I, 8, 0).reshape(1, 1, 2, 2, 64, 16)
    # tile (b=0, t=0), lane 16*q + n: bytes 8j + i = element 32j + 8q + i of row n
    for n, q, j in [(0, 0, 0), (5, 3, 1), (15, 2, 0)]:
        assert pk[0, 0, 0, 0, 16 * q + n, 8 * j:8 * j + 8].tolist() == \
            codes[0, n, 32 * j + 8 * q:32 * j + 8 * q + 8].tolist()
    # tile t = 1 covers k 64..127: only k < 80 (q = 0, 1 of j = 0) carry codes
    assert pk[0, 0, 0, 1, 16 * 1 + 2, 0:8].tolist() == codes[0, 2, 72:80].tolist()
    assert not pk[0, 0, 0, 1, 32:, :].any() and not pk[0, 0, 0, 1, :, 8:].any()
    # row block 1 holds rows 16..19; lanes of rows 20..31 are zero
    assert pk[0, 0, 1, 0, 3, 0:8].tolist() == codes[0, 19, 0:8].tolist()
    assert not pk[0, 0, 1, :, 4:16].any()


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("which,fusion,H,I", [("fc1", 1, 160, 48), ("fc1", 2, 96, 40),
                                              ("fc1", 0, 200, 24), ("fc3", 0, 200, 24),
                                              ("fc2", 0, 96, 72)])
def test_reference_pack_unpack_roundtrip(bits, which, fusion, H, I):
    rng = np.random.default_rng(bits * 7 + H)
    K, N, S, R, _ = tr.stack_geometry(which, H, I, bits, fusion)
    w = rng.integers(0, 256, size=(3, N, K * bits // 8), dtype=np.uint8)
    pk = tr.pack(w, which, H, I, bits, fusion)
    ssk = 128 if bits == 4 else 64
    assert pk.size == 3 * S * (-(-R // 16)) * (-(-K // ssk)) * 1024
    assert np.array_equal(tr.unpack(pk, 3, which, H, I, bits, fusion), tr.codes_of(w, K, bits))


def _params(**kw):
    base = dict(num_tokens=64, hidden_size=2880, inter_size=1408, num_experts=32, k=4,
                expert_weight_bits=4, block_size=32, swiglu_fusion=1)
    base.update(kw)
    T = base.pop("num_tokens")
    H, I, E, k = (base.pop(n) for n in ("hidden_size", "inter_size", "num_experts", "k"))
    return qm.make_params(T, H, I, E, k, **base)


@pytest.mark.parametrize("bits,fusion,act", [(4, 1, "swiglu"), (8, 2, "swiglu"),
                                             (4, 0, "swiglu"), (8, 0, "relu")])
def test_packed_stack_size(bits, fusion, act):
    p = _params(expert_weight_bits=bits, swiglu_fusion=fusion, activation=act)
    E, H, I = 32, 2880, 1408
    for which in ("fc1", "fc2", "fc3"):
        K, N, S, R, _ = tr.stack_geometry(which, H, I, bits, fusion, swiglu=act == "swiglu")
        ssk = 128 if bits == 4 else 64
        want = E * S * (-(-R // 16)) * (-(-K // ssk)) * 1024
        if which == "fc3" and not (act == "swiglu" and fusion == 0):
            want = 0
        assert qm.qmoe_packed_stack_size(p, which) == want, which


def test_pack_stack_host_checks():
    lib = _lib.load()
    p = _params()
    fake = 1 << 40  # never dereferenced: every call below fails before any device work
    assert lib.qmoe_pack_stack(p, 9, fake, fake + (1 << 32), None) == _lib.QMOE_ERR_INVALID
    assert lib.qmoe_pack_stack(p, _lib.QMOE_FC3, fake, fake + (1 << 32), None) == _lib.QMOE_ERR_INVALID
    assert lib.qmoe_pack_stack(p, _lib.QMOE_FC1, None, fake, None) == _lib.QMOE_ERR_UNBOUND
    assert lib.qmoe_pack_stack(p, _lib.QMOE_FC1, fake, None, None) == _lib.QMOE_ERR_UNBOUND
    assert lib.qmoe_pack_stack(p, _lib.QMOE_FC1, fake, fake + (1 << 32) + 16, None) == \
        _lib.QMOE_ERR_INVALID  # not 256-byte aligned
    assert lib.qmoe_pack_stack(p, _lib.QMOE_FC1, fake, fake + 256, None) == \
        _lib.QMOE_ERR_INVALID  # overlaps the source
    assert b"overlaps" in lib.qmoe_last_error()


def test_layout_validation():
    assert _lib.load().qmoe_validate(_params(weight_layout="tiles")) == _lib.QMOE_OK
    bad = _params()
    bad.weight_layout = 7
    assert _lib.load().qmoe_validate(bad) == _lib.QMOE_ERR_INVALID
    f32 = _params(weight_layout="tiles", act_dtype="f32", scale_dtype="f32",
                  hidden_size=128, inter_size=64)
    assert _lib.load().qmoe_validate(f32) == _lib.QMOE_ERR_UNSUPPORTED


def test_natural_order_roundtrip_and_differs():
    # the MX FP4 tile order (nibble i = element i) unpacks back to the same codes and, for
    # a word of distinct codes, differs from the decode order
    rng = np.random.default_rng(5)
    w = rng.integers(0, 256, size=(2, 64, 80), dtype=np.uint8)  # fc2 of H=64, I=160
    nat = tr.pack(w, "fc2", 64, 160, 4, 0, natural=True)
    dec = tr.pack(w, "fc2", 64, 160, 4, 0)
    assert not np.array_equal(nat, dec)
    back = tr.unpack(nat, 2, "fc2", 64, 160, 4, 0, natural=True)
    assert np.array_equal(back, tr.codes_of(w, 160, 4))
    # lane 0, word 0 of the first tile: row 0's elements 0..7 in nibbles 0..7, i.e. the
    # row's first four bytes unchanged
    assert np.array_equal(nat[:4], w[0, 0, :4])
