"""The C ABI library without a GPU: it loads, exports every declared entry point, and
rejects bad parameters and unbound pointers on the host before any device work."""
from __future__ import annotations

import ctypes
import math
import os
import re

import pytest

import weight_only_quantized_softmax_amd as qm
from weight_only_quantized_softmax_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmoe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmoe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libqmoe.so is not built (run __graft_entry__.build())")
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(_lib.EXPORTS) == set(names)


def good(**kw):
    base = dict(num_tokens=64, hidden_size=2880, inter_size=2880, num_experts=32, k=4,
                expert_weight_bits=4, block_size=32, swiglu_fusion=1, swiglu_alpha=1.702,
                swiglu_beta=1.0, swiglu_limit=7.0)
    base.update(kw)
    T = base.pop("num_tokens")
    H, I, E, k = (base.pop(n) for n in ("hidden_size", "inter_size", "num_experts", "k"))
    return qm.make_params(T, H, I, E, k, **base)


def status(p):
    return _lib.load().qmoe_validate(p)


def test_good_params_validate(lib):
    assert status(good()) == _lib.QMOE_OK
    assert lib.qmoe_last_error() == b""
    assert qm.qmoe_workspace_size(good()) > 0


BAD = [
    (dict(k=0), _lib.QMOE_ERR_INVALID),
    (dict(k=33, num_experts=64), _lib.QMOE_ERR_UNSUPPORTED),
    (dict(k=5, num_experts=4), _lib.QMOE_ERR_INVALID),
    (dict(num_experts=0), _lib.QMOE_ERR_UNSUPPORTED),
    (dict(num_experts=513), _lib.QMOE_ERR_UNSUPPORTED),
    (dict(expert_weight_bits=0), _lib.QMOE_ERR_INVALID),
    (dict(expert_weight_bits=2), _lib.QMOE_ERR_INVALID),
    (dict(block_size=24), _lib.QMOE_ERR_INVALID),
    (dict(block_size=8), _lib.QMOE_ERR_INVALID),
    (dict(block_size=1024), _lib.QMOE_ERR_UNSUPPORTED),
    (dict(swiglu_fusion=3), _lib.QMOE_ERR_INVALID),
    (dict(activation="identity", swiglu_fusion=1), _lib.QMOE_ERR_INVALID),
    (dict(num_tokens=-1), _lib.QMOE_ERR_INVALID),
    (dict(hidden_size=2881), _lib.QMOE_ERR_SHAPE),
    (dict(hidden_size=2880 + 16), _lib.QMOE_ERR_UNSUPPORTED),  # bf16 path needs K % 32
    (dict(block_size=128, strict_blocks=True), _lib.QMOE_ERR_SHAPE),  # 2880 % 128 != 0
    (dict(tile_m=8), _lib.QMOE_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("kw,want", BAD, ids=[str(k) for k, _ in BAD])
def test_bad_params_rejected(lib, kw, want):
    p = good(**kw)
    assert status(p) == want
    assert lib.qmoe_last_error() != b""
    assert lib.qmoe_workspace_size(p) == 0


def test_ragged_block_accepted_without_strict(lib):
    assert status(good(block_size=128)) == _lib.QMOE_OK


def test_bad_dtype_enum(lib):
    p = good()
    p.act_dtype = 7
    assert status(p) == _lib.QMOE_ERR_DTYPE
    p = good()
    p.scale_dtype = -1
    assert status(p) == _lib.QMOE_ERR_DTYPE


def test_f32_tile_fits_lds(lib):
    p = good(act_dtype="f32", hidden_size=128, inter_size=256, block_size=32)
    assert status(p) == _lib.QMOE_OK
    assert lib.qmoe_tile_m(p) == 16
    p = good(act_dtype="f32", hidden_size=4096, inter_size=4096, block_size=32)
    assert lib.qmoe_tile_m(p) == 2
    assert status(good(act_dtype="f32", hidden_size=4096, inter_size=4096, tile_m=16)) == \
        _lib.QMOE_ERR_UNSUPPORTED


def test_default_tile_heights(lib):
    # 128 rows from 64 expected rows per expert, 32 from 12, else 16 (bf16 activations)
    from synth import configs
    from tests.gpu_helpers import params_for

    c2, c3, c4 = configs.C2, configs.C3, configs.C4
    c5 = configs.c5_point(4, 32)
    for cfg, T, want in [(c2, 1, 16), (c2, 64, 16), (c3, 4096, 128), (c4, 512, 32),
                         (c5, 1, 16), (c5, 256, 32), (c5, 4096, 128)]:
        assert lib.qmoe_tile_m(params_for(cfg, T)) == want, (cfg.name, T)
    assert status(good(tile_m=32)) == _lib.QMOE_OK
    assert status(good(tile_m=64)) == _lib.QMOE_ERR_UNSUPPORTED


def test_max_rows_and_tiles(lib):
    p = good(num_tokens=64)  # T*k = 256, M = 16, E = 32
    assert lib.qmoe_tile_m(p) == 16
    assert lib.qmoe_max_tiles(p) == 256 // 16 + 32
    assert lib.qmoe_max_rows(p) == (256 // 16 + 32) * 16
    p = good(num_tokens=1)
    assert lib.qmoe_max_tiles(p) == 0 + 4


# Null pointers are rejected before any launch (no GPU is touched on these paths).
def test_unbound_pointers(lib):
    p = good()
    V = ctypes.c_void_p
    assert lib.qmoe_route(p, None, V(16), V(16), None) == _lib.QMOE_ERR_UNBOUND
    assert b"router_logits" in lib.qmoe_last_error()
    assert lib.qmoe_combine(p, V(16), None, V(16), None, V(16), None) == _lib.QMOE_ERR_UNBOUND
    st = _lib.QmoeStack(weights=16, scales=None, bias=None)
    full = _lib.QmoeStack(weights=16, scales=16, bias=None)
    assert lib.qmoe_grouped_gemm_fc2(p, V(16), V(16), V(16), st, V(16), None) == \
        _lib.QMOE_ERR_UNBOUND
    assert b"fc2.scales" in lib.qmoe_last_error()
    # separate gate/up stacks need fc3
    p0 = good(swiglu_fusion=0)
    assert lib.qmoe_grouped_gemm_fc1_swiglu(p0, V(16), V(16), V(16), V(16), None, full,
                                            _lib.QmoeStack(), V(16), None) == \
        _lib.QMOE_ERR_UNBOUND
    assert b"fc3" in lib.qmoe_last_error()
    assert lib.qmoe_forward(p, V(16), V(16), full, full, _lib.QmoeStack(), None, V(16), None, 0,
                            None) == _lib.QMOE_ERR_UNBOUND
    assert b"workspace" in lib.qmoe_last_error()


def test_workspace_checks(lib):
    p = good()
    V = ctypes.c_void_p
    full = _lib.QmoeStack(weights=16, scales=16, bias=None)
    need = lib.qmoe_workspace_size(p)
    assert lib.qmoe_forward(p, V(16), V(16), full, full, _lib.QmoeStack(), None, V(16), V(256),
                            need - 1, None) == _lib.QMOE_ERR_INVALID
    assert lib.qmoe_forward(p, V(16), V(16), full, full, _lib.QmoeStack(), None, V(16), V(300),
                            need, None) == _lib.QMOE_ERR_INVALID
    assert b"aligned" in lib.qmoe_last_error()


def test_permute_scratch(lib):
    small = good(num_tokens=64)
    assert lib.qmoe_permute_scratch_size(small) == 0
    big = good(num_tokens=4096, num_experts=64, k=6)
    need = lib.qmoe_permute_scratch_size(big)
    assert need > 0
    V = ctypes.c_void_p
    args = [V(16)] * 7
    assert lib.qmoe_permute(big, *args, None, 0, None) == _lib.QMOE_ERR_UNBOUND
    assert lib.qmoe_permute(big, *args, V(16), need - 1, None) == _lib.QMOE_ERR_INVALID


def test_zero_tokens_is_a_no_op(lib):
    p = good(num_tokens=0)
    assert status(p) == _lib.QMOE_OK
    V = ctypes.c_void_p
    # nothing is dereferenced or launched for T = 0, even with NULL buffers
    assert lib.qmoe_route(p, None, None, None, None) == _lib.QMOE_OK
    assert lib.qmoe_forward(p, None, None, _lib.QmoeStack(), _lib.QmoeStack(), _lib.QmoeStack(),
                            None, None, None, 0, None) == _lib.QMOE_OK


def test_infinite_limit_and_defaults_marshal(lib):
    p = good(swiglu_limit=math.inf)
    assert math.isinf(p.swiglu_limit)
    assert status(p) == _lib.QMOE_OK


def test_every_gpu_parity_case_passes_validation(lib):
    """Each parameter block the GPU parity tests build is accepted by the host checks, so
    that a GPU run never starts a case the library would refuse."""
    import itertools

    from synth import configs
    from tests import test_gpu_parity as t
    from tests.gpu_helpers import params_for

    bad = []
    cases = [(cfg, T, 0, "rows", "route " + n) for n, (cfg, T) in t.ROUTE_CASES.items()]
    cases += [t.stage_cfg(n, m) + (m, lay, "stage " + n) for n, m, lay in t.STAGE_CASES]
    for c in (configs.C1, configs.C2, configs.C3, configs.C4):
        cases += [(c, T, 0, "rows", "forward") for T in c.T_points]
    for c in (configs.C2, configs.C3, configs.C4):
        cases += [(c, T, 0, "tiles", "forward") for T in c.T_points]
    for b, bs in itertools.product(configs.C5_BITS, configs.C5_BLOCKS):
        cases += [(configs.c5_point(b, bs), T, 0, lay, "c5") for T in configs.C5.T_points
                  for lay in ("rows", "tiles")]
    # the variants: MX FP4, routing options, the int8 tier
    for c in (configs.C2_MX, configs.C5_MX, configs.C2_BIASED, configs.C5_ROUTED,
              configs.C2_INT8, configs.C4_INT8, configs.C5_INT8, configs.C2_MX_INT8,
              configs.C5_ROUTED.with_(int8=True)):
        cases += [(c, T, 0, "tiles", "variant") for T in c.T_points]
    cases += [(configs.c5_point(b, bs).with_(int8=True), 4096, 0, "rows", "int8 rows")
              for b, bs in ((4, 32), (8, 64))]
    cases += [(cfg, T, 0, "tiles", "full-size stages " + n) for n, (cfg, T) in t.FULL_STAGE_CASES.items()]
    for E, k, T, _ in t.FUSED_ROUTING_CASES + t.FUSED_ROUTING_EDGES:
        cases.append((configs.tiny(E=E, k=k, act_dtype="bf16", scale_dtype="bf16", H=64, I=64,
                                   bits=4, block_size=32, fusion=1), T, 0, "rows", "fused"))
    from tests import test_gpu_int8 as i8
    for n, (cfg, T) in i8.I8_DOT_CASES.items():
        cases.append((cfg, T, 0, "tiles", "int8 dot " + n))
        p8 = params_for(cfg, T, layout="tiles")
        if lib.qmoe_tile_m(p8) != 128:
            bad.append(("int8 dot case is not prefill-sized", n))
    from tests import test_gpu_variants as v
    cases += [(cfg, 300 if m == 128 else 40, m, lay, "variant stage " + n)
              for n, cfg in v.STAGE_VARIANTS.items() for m in (16, 32, 128)
              for lay in ("rows", "tiles")]
    cases += [(v._mixer(E, eps, act), 257, 0, "rows", "mixer")
              for E, eps, act in ((8, 0.01, "bf16"), (64, 0.2, "f32"), (300, 0.01, "bf16"))]
    for cfg, T, m, lay, what in cases:
        if lib.qmoe_validate(params_for(cfg, T, tile_m=m, layout=lay)) != 0:
            bad.append((what, cfg.name, T, m, lay, lib.qmoe_last_error()))
    assert not bad


def test_linear_woq_host_checks(lib):
    """qmoe_linear_woq: one expert, k = 1, no SwiGLU; NULL buffers are unbound; zero rows
    enqueue nothing (no device is touched on these paths)."""
    lp = qm.linear_params(8, 256, 128, block_size=32, activation="silu")
    S = _lib.QmoeStack
    full = S(weights=1 << 20, scales=1 << 20, bias=None)
    assert lib.qmoe_linear_woq(lp, None, full, 1 << 20, None) == _lib.QMOE_ERR_UNBOUND
    assert lib.qmoe_linear_woq(lp, 1 << 20, S(), 1 << 20, None) == _lib.QMOE_ERR_UNBOUND
    assert lib.qmoe_linear_woq(lp, 1 << 20, full, None, None) == _lib.QMOE_ERR_UNBOUND
    moe = qm.make_params(8, 256, 128, 4, 2, block_size=32, activation="silu")
    assert lib.qmoe_linear_woq(moe, 1 << 20, full, 1 << 20, None) == _lib.QMOE_ERR_INVALID
    sw = qm.make_params(8, 256, 128, 1, 1, block_size=32, activation="swiglu")
    assert lib.qmoe_linear_woq(sw, 1 << 20, full, 1 << 20, None) == _lib.QMOE_ERR_INVALID
    empty = qm.linear_params(0, 256, 128, block_size=32)
    assert lib.qmoe_linear_woq(empty, None, S(), None, None) == _lib.QMOE_OK
    # one expert: 128-row tiles only where their grid is large (32 tiles x 32 column blocks)
    assert lib.qmoe_tile_m(qm.linear_params(4096, 4096, 14336)) == 128
    assert lib.qmoe_tile_m(qm.linear_params(64, 2880, 5760)) == 32
    assert lib.qmoe_tile_m(qm.linear_params(300, 256, 128)) == 32
    assert lib.qmoe_tile_m(qm.linear_params(37, 256, 128)) == 32
    assert lib.qmoe_tile_m(qm.linear_params(5, 256, 128)) == 16


def test_mxfp4_params(lib):
    """E8M0 scales select MX FP4 weights: 4-bit, blocks of 32, bf16 activations, tiled
    layout; the packing accepts the parameters whatever their layout."""
    mx = dict(scale_dtype="e8m0", block_size=32, weight_layout="tiles")
    assert status(good(**mx)) == _lib.QMOE_OK
    assert status(good(**dict(mx, expert_weight_bits=8))) == _lib.QMOE_ERR_INVALID
    assert status(good(**dict(mx, block_size=16))) == _lib.QMOE_ERR_INVALID
    assert status(good(**dict(mx, block_size=0))) == _lib.QMOE_ERR_INVALID
    assert status(good(**dict(mx, weight_layout="rows"))) == _lib.QMOE_ERR_UNSUPPORTED
    assert status(good(**dict(mx, act_dtype="f32"))) == _lib.QMOE_ERR_UNSUPPORTED
    rows = good(**dict(mx, weight_layout="rows"))
    tiles = good(**mx)
    assert lib.qmoe_packed_stack_size(rows, _lib.QMOE_FC1) == lib.qmoe_packed_stack_size(tiles, _lib.QMOE_FC1) > 0
    p = good(**mx)
    p.scale_dtype = 3
    assert status(p) == _lib.QMOE_ERR_DTYPE


def test_variant_params(lib):
    """gelu takes gelu_mode 0 or 1; the sparse mixer picks k = 2 without renormalisation,
    grouping or selection bias, with a finite eps >= 0; the weight on the input is refused
    with the int8 tier and in the linear layer; the output scale must be finite (no device
    is touched on these paths)."""
    assert status(good(activation="gelu", swiglu_fusion=0)) == _lib.QMOE_OK
    assert status(good(activation="gelu", swiglu_fusion=0, gelu_mode=2)) == _lib.QMOE_ERR_INVALID
    assert status(good(activation="gelu", swiglu_fusion=1)) == _lib.QMOE_ERR_INVALID
    mix = dict(k=2, normalize_routing_weights=False, use_sparse_mixer=True, sparse_mixer_eps=0.01)
    assert status(good(**mix)) == _lib.QMOE_OK
    assert status(good(**dict(mix, k=3))) == _lib.QMOE_ERR_INVALID
    assert status(good(**dict(mix, normalize_routing_weights=True))) == _lib.QMOE_ERR_INVALID
    assert status(good(**dict(mix, sparse_mixer_eps=-1.0))) == _lib.QMOE_ERR_INVALID
    assert status(good(**dict(mix, sparse_mixer_eps=math.inf))) == _lib.QMOE_ERR_INVALID
    assert status(good(**dict(mix, n_group=2, topk_group=1))) == _lib.QMOE_ERR_INVALID
    assert status(good(apply_router_weight_on_input=True)) == _lib.QMOE_OK
    assert status(good(apply_router_weight_on_input=True,
                       compute_mode="int8")) == _lib.QMOE_ERR_UNSUPPORTED
    assert status(good(expert_output_scale=math.nan)) == _lib.QMOE_ERR_INVALID
    lp = qm.linear_params(8, 256, 128, block_size=32, activation="gelu")
    assert status(lp) == _lib.QMOE_OK
    full = _lib.QmoeStack(weights=1 << 20, scales=1 << 20, bias=None)
    lp.apply_router_weight_on_input = 1
    assert lib.qmoe_linear_woq(lp, 1 << 20, full, 1 << 20, None) == _lib.QMOE_ERR_INVALID
    # the fc1 entry point needs the routing weights when they go to the input
    V = ctypes.c_void_p
    p = good(apply_router_weight_on_input=True)
    assert lib.qmoe_grouped_gemm_fc1_swiglu(p, V(16), V(16), V(16), V(16), None, full,
                                            _lib.QmoeStack(), V(16), None) == \
        _lib.QMOE_ERR_UNBOUND
    assert b"topk_w" in lib.qmoe_last_error()


def test_int8_tier_params(lib):
    """compute_mode int8 needs per-block scales; unknown modes are rejected; the workspace
    grows by the rounded copy of x; qmoe_quantize_act checks its shape and needs
    block_size > 0 (no device is touched on these paths)."""
    assert status(good(compute_mode="int8")) == _lib.QMOE_OK
    assert status(good(compute_mode="int8", block_size=0)) == _lib.QMOE_ERR_INVALID
    # fp32 activations keep the float path (the rounding entry point takes both dtypes)
    assert status(good(compute_mode="int8", act_dtype="f32")) == _lib.QMOE_ERR_UNSUPPORTED
    assert lib.qmoe_quantize_act(good(act_dtype="f32"), 1 << 20, 0, 64, 1 << 20,
                                 None) == _lib.QMOE_OK
    p = good()
    p.compute_mode = 2
    assert status(p) == _lib.QMOE_ERR_INVALID
    f, q = good(), good(compute_mode="int8")
    xbytes = q.num_tokens * q.hidden_size * 2
    assert lib.qmoe_workspace_size(q) >= lib.qmoe_workspace_size(f) + xbytes
    assert lib.qmoe_quantize_act(good(), 1 << 20, 0, 64, 1 << 20, None) == _lib.QMOE_OK
    assert lib.qmoe_quantize_act(good(), 1 << 20, 4, 0, 1 << 20, None) == _lib.QMOE_ERR_SHAPE
    assert lib.qmoe_quantize_act(good(), None, 4, 64, 1 << 20, None) == _lib.QMOE_ERR_UNBOUND
    assert lib.qmoe_quantize_act(good(block_size=0), 1 << 20, 4, 64, 1 << 20,
                                 None) == _lib.QMOE_ERR_INVALID
