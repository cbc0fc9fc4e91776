"""The remaining routing and activation options on the GPU against the oracle (CLIKA "MoE"
page, routing kwargs gelu_mode, apply_router_weight_on_input, expert_output_scale,
sparse_mixer_eps; graiphic "QMoE" page, activation_type gelu and use_sparse_mixer):

* the sparse mixer's routing bit for bit (ids) and its weights within 2e-6, with logits
  crafted around its threshold, on the row-per-token and wave-per-token paths;
* gelu (both forms), the routing weight on the input and the expert output scale through
  the fc1 stage at every tile height and both weight layouts, through the combine, and
  through whole forwards on the decode, mid and prefill shapes (the forward's own routing
  and grouping read back and compared bit for bit, as in test_gpu_parity).
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_softmax_amd as qm
from synth import configs, gen
from tests.gpu_helpers import (DeviceInputs, check_output, dev, host, host_f64, max_excess_err,
                               params_for)
from tests.test_gpu_parity import check_forward, oracle_layout, run_route, say

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qm._lib.load()
    torch.cuda.init()


# --------------------------------------------------------------------------- sparse mixer

def _mixer(E, eps, act="bf16", **kw):
    return configs.tiny(E=E, k=2, sparse_mixer=True, mixer_eps=eps, normalize=False,
                        act_dtype=act, **kw)


def _near_threshold_logits(rng, T, E, eps, act):
    """Logits whose neighbours trail the top ones by ratios around 2 eps, so that the drop
    decisions fall on both sides of the threshold; plus ties and zeros."""
    base = rng.normal(0, 1.0, (T, E))
    top = np.argmax(base, axis=1)
    for t in range(T):
        m = base[t, top[t]]
        for e in rng.choice(E, size=min(E, 6), replace=False):
            r = 2 * eps * rng.uniform(0.5, 1.5)
            base[t, e] = m - r * max(abs(m), 1e-3)
    base[0, :] = 0.0
    base[1, : E // 2] = 1.0
    return gen.store(base, act)


@pytest.mark.parametrize("E,eps,act", [(8, 0.01, "bf16"), (64, 0.01, "f32"), (64, 0.2, "bf16"),
                                       (130, 0.05, "f32"), (300, 0.01, "bf16")])
def test_sparse_mixer_route_matches_oracle(E, eps, act):
    cfg = _mixer(E, eps, act)
    say("mixer route", E, eps, act)
    rng = np.random.default_rng(E)
    lg = _near_threshold_logits(rng, 257, E, eps, act)
    ids, w = run_route(cfg, lg, 257)
    rids, rw = oracle.route(cfg, lg)
    assert np.array_equal(ids, rids)
    assert np.max(np.abs(w - rw)) < 2e-6
    kept = np.mean(rw[:, 0] < 0.999999)
    say(f"  tokens whose first pick keeps a neighbour: {kept:.2f}")
    assert 0.05 < kept  # the threshold was exercised


@pytest.mark.parametrize("T", [1, 8, 64, 300])
def test_forward_sparse_mixer_decode_shape(T):
    # c2's layer with the mixer's two picks (the one-kernel routing up to 64 tokens)
    cfg = configs.C2.with_(name="c2-sparse-mixer", k=2, normalize=False, sparse_mixer=True,
                           mixer_eps=0.01, logit_sigma=0.05)
    check_forward(cfg, T, sample=16 if T > 64 else None, layout="tiles")


# --------------------------------------------------------------------------- stages

STAGE_VARIANTS = {
    "gelu-erf-b4-bs32-bias": configs.tiny(activation="gelu", gelu_mode=0, fusion=0,
                                          act_dtype="bf16", scale_dtype="bf16", H=512, I=256,
                                          E=8, block_size=32, fc1_bias=True),
    "gelu-tanh-b8-perrow": configs.tiny(activation="gelu", gelu_mode=1, fusion=0, bits=8,
                                        act_dtype="bf16", scale_dtype="bf16", H=384, I=256,
                                        E=8, block_size=0),
    "on-input-interleaved-bs32-clamp": configs.C2.with_(H=512, I=256, E=8, on_input=True),
    "on-input-separate-perrow": configs.C3.with_(H=512, I=384, E=4, logit_skew=0.0,
                                                 on_input=True),
    "on-input-gelu-b4-bs64": configs.tiny(activation="gelu", fusion=0, on_input=True,
                                          act_dtype="bf16", scale_dtype="bf16", H=544, I=224,
                                          E=8, block_size=64, fc1_bias=True),
    "on-input-concat-b8-bs128-f32scale": configs.C4.with_(H=704, I=352, E=8, on_input=True),
}


@pytest.mark.parametrize("tile_m", [16, 32, 128])
@pytest.mark.parametrize("layout", ["rows", "tiles"])
@pytest.mark.parametrize("name", sorted(STAGE_VARIANTS))
def test_fc1_stage_variants(name, layout, tile_m):
    cfg = STAGE_VARIANTS[name]
    T = 300 if tile_m == 128 else 40
    inp = gen.make_inputs(cfg, T)
    p = params_for(cfg, T, tile_m=tile_m, layout=layout)
    M = qm.qmoe_tile_m(p)
    assert M == tile_m
    say("fc1 variant", name, layout, "M", M)
    ids, perm, sa, erow = oracle_layout(cfg, T, M)
    d = DeviceInputs(inp)
    if layout == "tiles":
        d = d.tiled(p)
    rows = qm.qmoe_max_rows(p)
    sa_pad = np.full(rows, -1, np.int32)
    sa_pad[:len(sa)] = sa
    tl = np.zeros((qm.qmoe_max_tiles(p), 2), np.int32)
    tl[:perm["num_tiles"]] = perm["tiles"]
    # routing weights of the assignments (read only when the weight goes to the input)
    w = gen.gen_topk_w(cfg, T)
    h = torch.full((rows, cfg.I), 7.0, dtype=torch.bfloat16, device="cuda")
    qm.qmoe_grouped_gemm_fc1_swiglu(p, d.x, dev(sa_pad), dev(tl),
                                    dev(np.array([perm["num_tiles"]], np.int32)), d.fc1, d.fc3, h,
                                    topk_w=dev(np.ascontiguousarray(w, np.float32)))
    torch.cuda.synchronize()
    got = host_f64(h, "bf16")
    real = np.where(sa >= 0)[0]
    rw = w.reshape(-1)[sa[real]].astype(np.float64) if cfg.on_input else None
    ref = oracle.fc1_rows(cfg, inp, sa[real] // cfg.k, erow[real], nthreads=NTHREADS, row_w=rw)
    ex = max_excess_err(got[real], ref)
    say(f"  fc1 error beyond the bf16 rounding of h / rms {ex:.3e}")
    assert ex <= 2e-2
    pads = np.where(sa < 0)[0]
    assert np.all(got[pads] == 0.0)


@pytest.mark.parametrize("on_input,scale", [(True, 1.0), (False, 0.625), (True, -1.5)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_combine_stage_variants(on_input, scale, dtype):
    c = configs.tiny(E=16, k=4, H=1024, I=64, act_dtype=dtype, block_size=32,
                     scale_dtype="bf16", on_input=on_input, out_scale=scale)
    T = 33
    p = params_for(c, T)
    ids = gen.gen_topk_ids(c, T)
    perm = oracle.permute(c, ids, qm.qmoe_tile_m(p))
    y = gen.gen_stage_y(c, perm["rows"])
    w = gen.gen_topk_w(c, T)
    sh = gen.gen_activations(c, T, shared=True)[2]
    out = torch.empty((T, c.H), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                      device="cuda")
    qm.qmoe_combine(p, dev(y), dev(perm["assign_pos"]), dev(w), dev(sh, dtype), out)
    torch.cuda.synchronize()
    ref64, _ = oracle.combine(c, y, perm["assign_pos"], w, sh)
    say("  " + check_output(host_f64(out, dtype), ref64, dtype))


# --------------------------------------------------------------------------- forwards

@pytest.mark.parametrize("T", [1, 8, 64])
def test_forward_on_input_decode(T):
    cfg = configs.C2.with_(name="c2-weight-on-input", on_input=True, out_scale=0.75)
    check_forward(cfg, T, layout="tiles")


@pytest.mark.parametrize("T,layout", [(256, "tiles"), (4096, "tiles"), (4096, "rows")])
def test_forward_gelu_c5_shape(T, layout):
    for mode in (0, 1):
        cfg = configs.c5_point(4, 32).with_(name=f"c5-gelu{mode}", activation="gelu", fusion=0,
                                            gelu_mode=mode)
        check_forward(cfg, T, sample=16, layout=layout)


@pytest.mark.parametrize("T", [1, 64])
def test_forward_gelu_decode(T):
    cfg = configs.c5_point(8, 64).with_(name="c5-gelu-tanh-b8", activation="gelu", fusion=0,
                                        gelu_mode=1)
    check_forward(cfg, T, layout="tiles")


def test_forward_on_input_prefill_perrow():
    # the 128-row per-row-scale kernel with the weight on the input and an output scale
    cfg = configs.C3.with_(name="c3-small-on-input", H=1024, I=1536, E=4, on_input=True,
                           out_scale=1.25)
    check_forward(cfg, 2048, sample=16, layout="tiles")


def test_forward_on_input_prefill_blocks():
    cfg = configs.c5_point(4, 64).with_(name="c5-on-input", on_input=True)
    check_forward(cfg, 4096, sample=16, layout="tiles")


def test_forward_variants_fp32_activations():
    # fp32 activations (the VALU kernel): gelu, the weight on the input, an output scale
    for cfg in (configs.C1.with_(name="c1-gelu-on-input", activation="gelu", fusion=0,
                                 on_input=True, out_scale=0.5),
                configs.C1.with_(name="c1-swiglu-on-input", on_input=True),
                _mixer(8, 0.02, "f32", H=128, I=64)):
        check_forward(cfg, 16)


def test_linear_gelu():
    for mode in (0, 1):
        cfg = configs.tiny(E=1, k=1, fusion=0, activation="gelu", gelu_mode=mode, bits=4,
                           block_size=32, H=544, I=352, fc1_bias=True, act_dtype="bf16",
                           scale_dtype="bf16")
        inp = gen.make_linear_inputs(cfg, 37)
        p = qm.linear_params(37, cfg.H, cfg.I, block_size=32, activation="gelu", gelu_mode=mode,
                             weight_layout="tiles")
        w = qm.pack_stack(p, "fc1", dev(inp.w1))
        y = qm.linear_woq(p, dev(inp.x, "bf16"), (w, dev(inp.s1, "bf16"), dev(inp.b1, "bf16")))
        torch.cuda.synchronize()
        ref = oracle.linear(cfg, inp, nthreads=NTHREADS)
        say("  linear gelu", mode, check_output(host_f64(y, "bf16"), ref, "bf16"))
