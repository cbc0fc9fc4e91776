"""Pins for the CPU oracle: it is checked here against things other than itself.

* an independent dense brute-force reference (tests/bruteforce.py) on tiny inputs,
* closed forms (zero-point weights, integer-exact products, uniform and one-hot logits),
* library routines (scipy softmax, torch bfloat16 rounding, torch silu, numpy stable sort),
* layout equivalences that a wrong nibble order, gate/up swap or scale index would break,
* the hand-worked examples in tests/golden/.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import softmax

import oracle
from synth import configs, gen
from synth.gen import as_f32, store
from tests import bruteforce

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rms(a):
    return float(np.sqrt(np.mean(np.square(a))))


# --------------------------------------------------------------------------- brute force

BRUTE_CASES = {
    "f32-concat-b4-bs16": configs.tiny(),
    "bf16-interleaved-b8-bs32-bias-clamp": configs.tiny(
        act_dtype="bf16", scale_dtype="bf16", fusion=1, bits=8, block_size=32, fc1_bias=True,
        fc2_bias=True, alpha=1.702, beta=1.0, limit=7.0, scale_lo=0.02, scale_hi=0.06),
    "bf16-separate-fc3-perrow-bias": configs.tiny(
        act_dtype="bf16", scale_dtype="bf16", fusion=0, block_size=0, fc1_bias=True,
        fc2_bias=True, E=5, k=3),
    "f32-ragged-bs32-K80": configs.tiny(H=80, I=48, block_size=32, limit=2.0,
                                        scale_lo=0.05, scale_hi=0.1),
    "f32-identity": configs.tiny(activation="identity", fusion=0, fc2_bias=True),
    "f32-relu": configs.tiny(activation="relu", fusion=0, fc1_bias=True),
    "bf16-silu-b8": configs.tiny(activation="silu", fusion=0, bits=8, act_dtype="bf16"),
    "f32-no-renorm-E6k3": configs.tiny(normalize=False, E=6, k=3, logit_sigma=2.0),
    "bf16-fscale-b8-bs64": configs.tiny(act_dtype="bf16", scale_dtype="f32", bits=8,
                                        block_size=64, H=128, I=64),
    "bf16-grouped-biased-scaled": configs.tiny(act_dtype="bf16", scale_dtype="bf16", E=16, k=3,
                                               n_group=4, topk_group=2, score_bias=True,
                                               routed_scale=2.5, fusion=1, fc1_bias=True),
    "f32-grouped-norenorm": configs.tiny(E=12, k=2, n_group=3, topk_group=1, normalize=False,
                                         logit_sigma=2.0),
    "bf16-mxfp4-interleaved-bias": configs.tiny(act_dtype="bf16", scale_dtype="e8m0", bits=4,
                                                block_size=32, H=96, I=64, fusion=1,
                                                fc1_bias=True, fc2_bias=True, limit=7.0,
                                                scale_lo=0.01, scale_hi=0.2),
    "bf16-int8-interleaved-bs32-bias": configs.tiny(
        act_dtype="bf16", scale_dtype="bf16", fusion=1, bits=4, block_size=32, fc1_bias=True,
        fc2_bias=True, limit=7.0, int8=True),
    "f32-int8-ragged-bs32-K80": configs.tiny(H=80, I=48, block_size=32, limit=2.0,
                                             scale_lo=0.05, scale_hi=0.1, int8=True),
    "bf16-int8-mxfp4-separate": configs.tiny(act_dtype="bf16", scale_dtype="e8m0", bits=4,
                                             block_size=32, H=96, I=64, fusion=0,
                                             scale_lo=0.01, scale_hi=0.2, int8=True),
    # gelu (both forms), the routing weight on the input, the expert output scale
    "f32-gelu-exact-bias": configs.tiny(activation="gelu", fusion=0, gelu_mode=0, fc1_bias=True,
                                        fc2_bias=True),
    "bf16-gelu-tanh-b8": configs.tiny(activation="gelu", fusion=0, gelu_mode=1, bits=8,
                                      act_dtype="bf16", scale_dtype="bf16"),
    "f32-on-input-interleaved-bias-clamp": configs.tiny(on_input=True, fusion=1, fc1_bias=True,
                                                        fc2_bias=True, limit=3.0, E=5, k=3),
    "bf16-on-input-separate-out-scale": configs.tiny(act_dtype="bf16", scale_dtype="bf16",
                                                     fusion=0, on_input=True, out_scale=0.75,
                                                     fc2_bias=True, fc1_bias=True),
    "f32-out-scale-norenorm-gelu": configs.tiny(out_scale=2.0, normalize=False, fc2_bias=True,
                                                activation="gelu", fusion=0, E=6, k=3),
}


@pytest.mark.parametrize("name", sorted(BRUTE_CASES))
def test_oracle_matches_bruteforce(name):
    cfg = BRUTE_CASES[name]
    inp = gen.make_inputs(cfg, 7, shared=(name.startswith("bf16-separate")))
    ref = bruteforce.forward(cfg, inp)
    out64, _ = oracle.forward(cfg, inp)
    assert np.max(np.abs(out64 - ref)) <= 1e-11 * max(rms(ref), 1e-30)


def test_bruteforce_clamp_case_actually_clamps():
    # The clamp case must exercise the limit, or it pins nothing about it.
    cfg = BRUTE_CASES["bf16-interleaved-b8-bs32-bias-clamp"]
    inp = gen.make_inputs(cfg, 7)
    x = as_f32(inp.x, "bf16").astype(np.float64)
    W1 = bruteforce.dequant_dense(inp.w1, inp.s1, cfg, cfg.n1, cfg.H)
    z = np.einsum("th,enh->etn", x, W1)
    assert (z > 7).mean() > 0.05 and (z < -7).mean() > 0.05


# --------------------------------------------------------------------------- routing

def test_route_matches_subset_bruteforce_with_many_ties():
    cfg = configs.tiny(E=7, k=3, act_dtype="bf16")
    rng = np.random.default_rng(5)
    # values from a small set so exact ties are frequent, including -0 and +0
    vals = np.array([-1.0, -0.0, 0.0, 0.5, 1.0, 2.0], np.float32)
    lg = store(vals[rng.integers(0, len(vals), size=(300, cfg.E))], "bf16")
    ids, w = oracle.route(cfg, lg)
    lf = as_f32(lg, "bf16").astype(np.float64)
    ties = 0
    for t in range(lf.shape[0]):
        assert sorted(ids[t].tolist()) == bruteforce.select(cfg, lf[t])
        # slot order: descending logit, ascending index among equals
        assert all((lf[t, ids[t, j]] > lf[t, ids[t, j + 1]]) or
                   (lf[t, ids[t, j]] == lf[t, ids[t, j + 1]] and ids[t, j] < ids[t, j + 1])
                   for j in range(cfg.k - 1))
        kth = lf[t, ids[t, -1]]
        ties += int(np.sum(lf[t] == kth) > np.sum(lf[t, ids[t]] == kth))
    assert ties > 30  # the boundary tie rule was exercised


@pytest.mark.parametrize("n_group,topk_group,k,bias", [(4, 2, 3, True), (8, 3, 5, False),
                                                       (2, 1, 4, True)])
def test_grouped_biased_route_matches_subset_bruteforce_with_ties(n_group, topk_group, k, bias):
    # logits and biases on a coarse grid, so that selection keys, group scores and their
    # fp32 sums tie often; the brute force enumerates group sets and expert subsets
    E = 16
    cfg = configs.tiny(E=E, k=k, n_group=n_group, topk_group=topk_group, score_bias=bias,
                       routed_scale=1.5, act_dtype="f32")
    rng = np.random.default_rng(n_group * 10 + k)
    lg = (rng.integers(-3, 4, size=(40, E)) * 0.25).astype(np.float32)
    eb = (rng.integers(-2, 3, size=E) * 0.25).astype(np.float32) if bias else None
    ids, w = oracle.route(cfg, lg, eb)
    G = bruteforce.gates(cfg, lg.astype(np.float64), eb)
    for t in range(40):
        assert sorted(ids[t].tolist()) == sorted(np.nonzero(G[t])[0].tolist()), t
        assert np.allclose(w[t], G[t, ids[t]], rtol=1e-13)
    # the slots hold the chosen experts by descending key, equal keys in index order
    keys = lg if eb is None else lg + eb
    for t in range(40):
        kk = keys[t, ids[t]]
        assert all(kk[j] > kk[j + 1] or (kk[j] == kk[j + 1] and ids[t, j] < ids[t, j + 1])
                   for j in range(k - 1))


def test_route_uniform_logits_pick_lowest_indices():
    for normalize, expect in ((True, 1 / 3), (False, 1 / 8)):
        cfg = configs.tiny(E=8, k=3, normalize=normalize)
        lg = np.full((4, 8), 0.25, np.float32)
        ids, w = oracle.route(cfg, lg)
        assert (ids == np.array([0, 1, 2])).all()
        assert np.allclose(w, expect, rtol=0, atol=1e-15)


def test_route_negative_zero_equals_positive_zero():
    cfg = configs.tiny(E=4, k=2, act_dtype="bf16")
    lg = store(np.array([[-0.0, 0.0, -0.0, -1.0]], np.float32), "bf16")
    assert lg[0, 0] == 0x8000  # the stored pattern really is -0
    ids, _ = oracle.route(cfg, lg)
    assert ids.tolist() == [[0, 1]]


def test_route_one_hot():
    cfg = configs.tiny(E=6, k=1)
    lg = np.zeros((6, 6), np.float32)
    lg[np.arange(6), np.arange(6)[::-1]] = 30.0
    ids, w = oracle.route(cfg, lg)
    assert ids[:, 0].tolist() == [5, 4, 3, 2, 1, 0]
    assert np.all(w == 1.0)  # renormalised single weight is exactly one


def test_route_weights_are_scipy_softmax():
    cfg = configs.tiny(E=9, k=9, normalize=False, act_dtype="bf16")
    lg = store(np.random.default_rng(1).normal(0, 3, size=(50, 9)), "bf16")
    ids, w = oracle.route(cfg, lg)
    p = softmax(as_f32(lg, "bf16").astype(np.float64), axis=1)
    assert np.allclose(np.take_along_axis(p, ids, 1), w, rtol=1e-13, atol=0)


def test_route_renormalised_weights_sum_to_one():
    cfg = configs.tiny(E=32, k=4, act_dtype="bf16")
    lg = store(np.random.default_rng(2).normal(0, 2, size=(200, 32)), "bf16")
    _, w = oracle.route(cfg, lg)
    assert np.max(np.abs(w.sum(1) - 1.0)) < 1e-15
    assert np.all(np.diff(w, axis=1) <= 0)  # larger logit, larger weight


# --------------------------------------------------------------------------- permutation

@pytest.mark.parametrize("M", [1, 4, 16, 128])
def test_permute_is_stable_sort_padded(M):
    cfg = configs.tiny(E=10, k=3)
    ids = gen.gen_topk_ids(cfg, 57, skew=4.0)
    perm = oracle.permute(cfg, ids, M)
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")  # library stable sort
    counts = np.bincount(flat, minlength=cfg.E)
    assert (perm["counts"] == counts).all() and counts.sum() == flat.size
    offs = perm["padded_offsets"]
    assert offs[0] == 0 and np.all(offs % M == 0)
    assert np.all(np.diff(offs) == -(-counts // M) * M)
    sa = perm["sorted_assign"]
    real = sa[sa >= 0]
    assert (real == order).all()
    for e in range(cfg.E):
        seg = sa[offs[e]:offs[e + 1]]
        assert (seg[:counts[e]] >= 0).all() and (seg[counts[e]:] == -1).all()
        assert np.all(np.diff(seg[:counts[e]]) > 0)
    pos = perm["assign_pos"]
    assert (sa[pos] == np.arange(flat.size)).all()  # unpermute(permute) = identity
    tiles = perm["tiles"]
    assert tiles[:, 1].sum() == flat.size
    for t, (e, valid) in enumerate(tiles):
        row0 = t * M
        assert offs[e] <= row0 < offs[e + 1]
        assert valid == min(M, counts[e] - (row0 - offs[e]))
    assert perm["num_tiles"] <= oracle.max_tiles(cfg, 57, M)
    assert perm["rows"] <= oracle.max_rows(cfg, 57, M)


# --------------------------------------------------------------------------- closed forms

def _zero_point_weights(inp, cfg):
    fill = 0x88 if cfg.bits == 4 else 0x80
    for name in ("w1", "w2", "w3"):
        a = getattr(inp, name)
        if a is not None:
            a[...] = fill


@pytest.mark.parametrize("bits", [4, 8])
def test_zero_point_weights_give_bias_combination(bits):
    cfg = configs.tiny(bits=bits, fc1_bias=True, fc2_bias=True, E=6, k=3, act_dtype="bf16",
                       scale_dtype="bf16")
    inp = gen.make_inputs(cfg, 9, shared=True)
    _zero_point_weights(inp, cfg)
    out64, _ = oracle.forward(cfg, inp)
    lg = as_f32(inp.logits, "bf16").astype(np.float64)
    p = softmax(lg, axis=1)
    order = np.argsort(-lg, axis=1, kind="stable")[:, :cfg.k]
    w = np.take_along_axis(p, order, 1)
    w = w / w.sum(1, keepdims=True)
    b2 = as_f32(inp.b2, "bf16").astype(np.float64)
    expect = np.einsum("tj,tjh->th", w, b2[order]) + as_f32(inp.shared, "bf16")
    assert np.max(np.abs(out64 - expect)) < 1e-14


@pytest.mark.parametrize("bits,fusion", [(4, 0), (8, 0)])
def test_identity_unit_scales_is_integer_matmul(bits, fusion):
    # k=1 with renormalisation gives weight exactly 1; unit scales and small integer
    # inputs make every product and sum an exact integer.
    cfg = configs.tiny(bits=bits, fusion=fusion, activation="identity", k=1, E=3, H=64, I=32,
                       block_size=16)
    inp = gen.make_inputs(cfg, 6)
    inp.x[...] = np.random.default_rng(3).integers(-3, 4, size=inp.x.shape).astype(np.float32)
    inp.s1[...] = 1.0
    inp.s2[...] = 1.0
    out64, outr = oracle.forward(cfg, inp)
    ids, w = oracle.route(cfg, inp.logits)
    assert np.all(w == 1.0)
    q1 = bruteforce.dequant_dense(inp.w1, inp.s1, cfg, cfg.I, cfg.H).astype(np.int64)
    q2 = bruteforce.dequant_dense(inp.w2, inp.s2, cfg, cfg.H, cfg.I).astype(np.int64)
    xi = inp.x.astype(np.int64)
    expect = np.stack([(xi[t] @ q1[ids[t, 0]].T) @ q2[ids[t, 0]].T for t in range(6)])
    assert np.array_equal(out64, expect.astype(np.float64))
    assert np.array_equal(outr, expect.astype(np.float32))


def test_linearity_identity_no_bias():
    cfg = configs.tiny(activation="identity", fusion=0)
    inp = gen.make_inputs(cfg, 5)
    a, _ = oracle.forward(cfg, inp)
    inp.x *= np.float32(4.0)  # exact scaling by a power of two
    b, _ = oracle.forward(cfg, inp)
    assert np.allclose(b, 4.0 * a, rtol=1e-13, atol=1e-300)


def test_single_expert_is_dequant_ffn():
    # E = 1, k = 1: the block is one weight-only-quantized FFN (QLinearWoQ composition).
    cfg = configs.tiny(E=1, k=1, fusion=1, fc1_bias=True, fc2_bias=True)
    inp = gen.make_inputs(cfg, 4)
    out64, _ = oracle.forward(cfg, inp)
    W1 = torch.from_numpy(bruteforce.dequant_dense(inp.w1, inp.s1, cfg, cfg.n1, cfg.H)[0])
    W2 = torch.from_numpy(bruteforce.dequant_dense(inp.w2, inp.s2, cfg, cfg.H, cfg.I)[0])
    x = torch.from_numpy(inp.x.astype(np.float64))
    z = torch.nn.functional.linear(x, W1, torch.from_numpy(inp.b1[0].astype(np.float64)))
    h = torch.nn.functional.silu(z[:, 0::2]) * z[:, 1::2]
    y = torch.nn.functional.linear(h, W2, torch.from_numpy(inp.b2[0].astype(np.float64)))
    assert np.allclose(out64, y.numpy(), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("bits,bs,act,sdt", [(4, 32, "silu", "bf16"), (8, 0, "relu", "f32"),
                                              (4, 0, "identity", "f32"), (8, 64, "silu", "bf16")])
def test_linear_is_dense_dequant_matmul(bits, bs, act, sdt):
    # QLinearWoQ: y = act(x @ dequant(W)^T + b), against torch's linear and activation on
    # the independently dequantised weight; K = 80 gives a short last block for bs 32 and 64
    cfg = configs.tiny(E=1, k=1, fusion=0, activation=act, bits=bits, block_size=bs, H=80,
                       I=24, fc1_bias=True, act_dtype="bf16", scale_dtype=sdt)
    inp = gen.make_linear_inputs(cfg, 7)
    got = oracle.linear(cfg, inp)
    W = torch.from_numpy(bruteforce.dequant_dense(inp.w1, inp.s1, cfg, cfg.I, cfg.H)[0])
    x = torch.from_numpy(as_f32(inp.x, "bf16").astype(np.float64))
    b = torch.from_numpy(as_f32(inp.b1[0], "bf16").astype(np.float64))
    z = torch.nn.functional.linear(x, W, b)
    ref = {"silu": torch.nn.functional.silu, "relu": torch.relu, "identity": lambda v: v}[act](z)
    assert np.allclose(got, ref.numpy(), rtol=1e-12, atol=1e-13)
    # a row subset evaluates the same rows
    assert np.array_equal(oracle.linear(cfg, inp, rows=[6, 2]), got[[6, 2]])


def test_mxfp4_weights_are_e2m1_times_power_of_two():
    # every E2M1 code under three E8M0 scale bytes: the oracle's dequant against the
    # format's bit fields (bruteforce.e2m1_bits) and torch's own E8M0 conversion; spot
    # values 0, 0.5, 6 and the negative zero
    cfg = configs.tiny(E=1, k=1, fusion=0, activation="identity", act_dtype="bf16",
                       scale_dtype="e8m0", bits=4, block_size=32, H=96, I=16)
    codes = np.arange(96) % 16
    w = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    w = np.broadcast_to(w, (1, 16, 48)).copy()
    ebytes = np.array([127, 120, 131], np.uint8)
    s = np.broadcast_to(ebytes, (1, 16, 3)).copy()
    st = oracle.Stack(w=w.ctypes.data, s=s.ctypes.data, b=None)
    got = np.array([oracle.weight(cfg, st, 16, 96, 0, 5, k) for k in range(96)])
    scale = torch.from_numpy(ebytes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    want = bruteforce.e2m1_bits(codes) * np.repeat(scale, 32)
    assert np.array_equal(got, want)
    assert got[0] == 0.0 and got[1] == 0.5 and got[7] == 6.0 and got[15] == -6.0
    assert got[8] == 0.0 and math.copysign(1.0, got[8]) == -1.0
    assert np.all(np.abs(got[:8]) == np.abs(got[8:16]))


def test_swiglu_clamp_reading():
    # Only the gate is clamped from above; the up value is clamped on both sides.
    cfg = configs.tiny(fusion=2, bits=8, block_size=0, H=16, I=16, E=1, k=1, alpha=1.702,
                       beta=1.0, limit=7.0)
    inp = gen.make_inputs(cfg, 1)
    inp.x[...] = 0
    inp.x[0, 0] = 1.0
    inp.w1[...] = 0x80
    g = np.array([10, -10, 3, -3, 0.5, 20, -20, 7] * 2, np.float64)
    u = np.array([10, -10, -10, 10, 2, 0, 1, -7.5] * 2, np.float64)
    inp.s1[...] = 0.5
    inp.w1[0, :16, 0] = (128 + 2 * g).astype(np.uint8)
    inp.w1[0, 16:, 0] = (128 + 2 * u).astype(np.uint8)
    h = oracle.fc1_rows(cfg, inp, [0], [0])[0]
    gp = np.minimum(g, 7.0)
    up = np.clip(u, -7.0, 7.0)
    sig = 1.0 / (1.0 + np.exp(-1.702 * gp))
    assert np.allclose(h, gp * sig * (up + 1.0), rtol=1e-15, atol=0)
    # standard SwiGLU (alpha 1, beta 0, no limit) is silu(g) * u
    cfg2 = cfg.with_(alpha=1.0, beta=0.0, limit=math.inf)
    h2 = oracle.fc1_rows(cfg2, inp, [0], [0])[0]
    ref = (torch.nn.functional.silu(torch.tensor(g)) * torch.tensor(u)).numpy()
    assert np.allclose(h2, ref, rtol=1e-15, atol=1e-300)


# --------------------------------------------------------------------------- layout equivalences

def _fwd(cfg, inp):
    return oracle.forward(cfg, inp)[0]


def test_interleaved_equals_concatenated():
    cfg = configs.tiny(fusion=1, fc1_bias=True, act_dtype="bf16", scale_dtype="bf16")
    inp = gen.make_inputs(cfg, 6)
    a = _fwd(cfg, inp)
    I = cfg.I
    perm = np.concatenate([np.arange(0, 2 * I, 2), np.arange(1, 2 * I, 2)])
    inp.w1, inp.s1, inp.b1 = inp.w1[:, perm].copy(), inp.s1[:, perm].copy(), inp.b1[:, perm].copy()
    b = _fwd(cfg.with_(fusion=2), inp)
    assert np.array_equal(a, b)


def test_fused_equals_separate_stacks():
    cfg = configs.tiny(fusion=2, fc1_bias=True, block_size=0)
    inp = gen.make_inputs(cfg, 6)
    a = _fwd(cfg, inp)
    I = cfg.I
    inp.w3, inp.s3, inp.b3 = inp.w1[:, I:].copy(), inp.s1[:, I:].copy(), inp.b1[:, I:].copy()
    inp.w1, inp.s1, inp.b1 = inp.w1[:, :I].copy(), inp.s1[:, :I].copy(), inp.b1[:, :I].copy()
    b = _fwd(cfg.with_(fusion=0), inp)
    assert np.array_equal(a, b)


def test_4bit_equals_8bit_shifted_by_120():
    cfg4 = configs.tiny(bits=4, block_size=16)
    inp = gen.make_inputs(cfg4, 6)
    a = _fwd(cfg4, inp)

    def widen(w):
        lo, hi = (w & 0xF), (w >> 4)
        return (np.stack([lo, hi], -1).reshape(w.shape[0], w.shape[1], -1) + 120).astype(np.uint8)

    inp.w1, inp.w2 = widen(inp.w1), widen(inp.w2)
    b = _fwd(cfg4.with_(bits=8), inp)
    assert np.array_equal(a, b)


def test_per_row_equals_constant_blocks():
    cfg = configs.tiny(block_size=0, act_dtype="bf16", scale_dtype="bf16")
    inp = gen.make_inputs(cfg, 6)
    a = _fwd(cfg, inp)
    cb = cfg.with_(block_size=16)
    inp.s1 = np.repeat(inp.s1[:, :, None], cb.nblocks(cfg.H), 2).copy()
    inp.s2 = np.repeat(inp.s2[:, :, None], cb.nblocks(cfg.I), 2).copy()
    b = _fwd(cb, inp)
    assert np.array_equal(a, b)


def test_ragged_128_equals_64_with_pairs():
    # K = 192 with block 128: the last block holds 64 elements.
    cfg = configs.tiny(H=192, I=320, block_size=128, bits=8)
    inp = gen.make_inputs(cfg, 5)
    assert inp.s1.shape[2] == 2 and inp.s2.shape[2] == 3
    a = _fwd(cfg, inp)
    c64 = cfg.with_(block_size=64)
    inp.s1 = np.repeat(inp.s1, 2, axis=2)[:, :, :3].copy()
    inp.s2 = np.repeat(inp.s2, 2, axis=2)[:, :, :5].copy()
    b = _fwd(c64, inp)
    assert np.array_equal(a, b)


def test_token_permutation_equivariance():
    cfg = configs.tiny(act_dtype="bf16", E=6, k=2)
    inp = gen.make_inputs(cfg, 9)
    a = _fwd(cfg, inp)
    perm = np.random.default_rng(0).permutation(9)
    inp.x, inp.logits = inp.x[perm].copy(), inp.logits[perm].copy()
    b = _fwd(cfg, inp)
    assert np.array_equal(a[perm], b)


def test_token_subset_equals_full():
    cfg = configs.tiny(E=5, k=2)
    inp = gen.make_inputs(cfg, 11)
    full = _fwd(cfg, inp)
    sel = np.array([10, 3, 3, 0])
    part, _ = oracle.forward(cfg, inp, sel=sel)
    assert np.array_equal(part, full[sel])


# --------------------------------------------------------------------------- stage functions

def test_stage_functions_compose_to_forward():
    cfg = configs.tiny(E=5, k=2, fc1_bias=True, fc2_bias=True)
    inp = gen.make_inputs(cfg, 8)
    ids, w = oracle.route(cfg, inp.logits)
    perm = oracle.permute(cfg, ids, 4)
    rows = np.where(perm["sorted_assign"] >= 0)[0]
    a = perm["sorted_assign"][rows]
    expert = np.repeat(np.arange(cfg.E), np.diff(perm["padded_offsets"]))[rows]
    h = oracle.fc1_rows(cfg, inp, a // cfg.k, expert)
    y = oracle.fc2_rows(cfg, inp, h.astype(np.float32), np.arange(len(rows)), expert)
    Y = np.zeros((perm["rows"], cfg.H), np.float32)
    Y[rows] = y
    out64, _ = oracle.combine(cfg, Y, perm["assign_pos"], w.astype(np.float32))
    ref = _fwd(cfg, inp)
    # only the f32 storage of h, y and w separates the two
    assert np.max(np.abs(out64 - ref)) < 1e-5 * rms(ref)


# --------------------------------------------------------------------------- int8 tier

def _int8_rows(rng, rows, cols, bs):
    """Rows whose blocks span many magnitudes, with exact ties and block maxima that sit
    on the 127 * 2^e boundaries."""
    nb = -(-cols // bs)
    mag = 2.0 ** rng.integers(-20, 20, (rows, nb))
    v = rng.normal(0, 1, (rows, cols)) * np.repeat(mag, bs, axis=1)[:, :cols]
    v[0, :min(cols, bs)] = 0.0                 # an all-zero block
    # row 1: exact ties (n + 1/2) * 2^-3 under a block maximum of 127 * 2^-3
    if rows > 1:
        v[1, 0] = 127.0 * 2.0 ** -3          # the largest that keeps e = -3
        v[1, 1:min(cols, bs)] = (rng.integers(-126, 126, min(cols, bs) - 1) + 0.5) * 2.0 ** -3
    if rows > 2:
        v[2, 0] = 127.5 * 2.0 ** -3          # just too large: e = -2
    return v


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("bs,cols", [(32, 96), (32, 80), (16, 16), (64, 200), (128, 130)])
def test_int8_round_matches_scale_search(act, bs, cols):
    rng = np.random.default_rng(bs * 1000 + cols)
    cfg = configs.tiny(act_dtype=act, block_size=bs, H=cols)
    v = store(_int8_rows(rng, 9, cols, bs), act)
    got = as_f32(oracle.int8_round(cfg, v), act).astype(np.float64)
    want = bruteforce.int8_round(as_f32(v, act).astype(np.float64), bs)
    assert np.array_equal(got, want)


def test_int8_round_properties():
    rng = np.random.default_rng(3)
    bs, cols = 32, 100
    cfg = configs.tiny(act_dtype="f32", block_size=bs, H=cols)
    v = store(_int8_rows(rng, 40, cols, bs), "f32")
    out = oracle.int8_round(cfg, v)
    # idempotent: a rounded row is its own rounding
    assert np.array_equal(oracle.int8_round(cfg, out), out)
    x = v.astype(np.float64)
    q = out.astype(np.float64)
    for r in range(x.shape[0]):
        for b0 in range(0, cols, bs):
            blk, qb = x[r, b0:b0 + bs], q[r, b0:b0 + bs]
            a = np.max(np.abs(blk))
            if a == 0:
                assert not qb.any()
                continue
            # the scale: the power of two that makes the largest code land in [64, 127]
            e = math.frexp(np.max(np.abs(qb)))[1] - 7
            codes = qb / 2.0 ** e
            assert np.array_equal(codes, np.round(codes))
            assert 64 <= np.max(np.abs(codes)) <= 127
            # the error of each element is at most half a code step
            assert np.max(np.abs(qb - blk)) <= 2.0 ** (e - 1)


def test_int8_round_by_hand():
    # one block of three: max 1.0 -> e = -6 (127/64 >= 1 > 127/128): codes 64, -32 and
    # 0.3 * 64 = 19.2 -> 19; a second block of two: max 3.0 -> e = -5 (127/32 >= 3 > 127/64),
    # codes 2.5 * 32 = 80 and 3 * 32 = 96 exactly
    cfg = configs.tiny(act_dtype="f32", block_size=3, H=5)
    v = np.array([[1.0, -0.5, 0.3, 2.5, -3.0]], np.float32)
    got = oracle.int8_round(cfg, v)[0].astype(np.float64)
    assert got.tolist() == [1.0, -0.5, 19 / 64, 2.5, -3.0]
    # a tie: 2.5 * 2^-6 is half way between codes 2 and 3 under max 1.0; ties to even -> 2
    v = np.array([[1.0, 2.5 / 64, 3.5 / 64]], np.float32)
    got = oracle.int8_round(configs.tiny(act_dtype="f32", block_size=3, H=3), v)[0]
    assert got.astype(np.float64).tolist() == [1.0, 2 / 64, 4 / 64]


def test_int8_forward_differs_from_float_forward():
    # the tier changes the result (it is not silently off), by about the size int8 codes allow
    cfg = configs.tiny(act_dtype="f32", block_size=16, fusion=2)
    inp = gen.make_inputs(cfg, 5)
    f, _ = oracle.forward(cfg, inp)
    q, _ = oracle.forward(cfg.with_(int8=True), inp)
    d = rms(q - f) / rms(f)
    assert 1e-4 < d < 5e-2


# --------------------------------------------------------------------------- rounding

def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.normal(0, 1, 20000), rng.normal(0, 1e30, 200), rng.normal(0, 1e-38, 200),
        np.array([0.0, -0.0, 1.0, -2.5, 3.3895313892515355e38, 1e-45, -1e-40]),
    ]).astype(np.float32)
    # include exact ties: float32 values with the low 16 bits equal to 0x8000
    ties = (rng.integers(0x3F000000, 0x40000000, 500, dtype=np.uint32) & 0xFFFF0000) | 0x8000
    v = np.concatenate([v, ties.view(np.float32)])
    ours = oracle.round_bf16(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_round_bf16_is_single_rounding_from_double():
    # 1 + 2^-8 is exactly half way between bf16 neighbours 1 and 1 + 2^-7: ties to even.
    # Slightly above the half-way point must round up even though the float32
    # nearest to it is the half-way point itself.
    v = np.array([1 + 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, 1 + 3 * 2.0 ** -8], np.float64)
    out = oracle.round_bf16(v)
    assert out.tolist() == [0x3F80, 0x3F81, 0x3F82]


# --------------------------------------------------------------------------- golden, by hand

def test_golden_hand_examples():
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 2
    for case in cases:
        c = case["config"]
        cfg = configs.tiny(**c)
        T = case["T"]
        inp = gen.make_inputs(cfg, T)
        inp.x[...] = np.asarray(case["x"], np.float32)
        inp.logits[...] = np.asarray(case["logits"], np.float32)
        inp.w1[...] = case["w1_fill"]
        for e, n, byte, val in case["w1_set"]:
            inp.w1[e, n, byte] = val
        inp.s1[...] = np.asarray(case["s1"], np.float32).reshape(inp.s1.shape)
        inp.w2[...] = case["w2_fill"]
        for e, n, byte, val in case["w2_set"]:
            inp.w2[e, n, byte] = val
        inp.s2[...] = case["s2_fill"]
        out64, _ = oracle.forward(cfg, inp)
        assert np.allclose(out64, np.asarray(case["expect"]), rtol=1e-15, atol=1e-15), case["name"]


# --------------------------------------------------------------------------- gelu

@pytest.mark.parametrize("mode,approx", [(0, "none"), (1, "tanh")])
def test_gelu_matches_torch_and_scipy(mode, approx):
    """The single-expert layer with gelu (E = 1, k = 1: out = fc2(gelu(fc1(x)))) against torch's
    gelu on the dense dequantised weights; the exact form also against scipy's normal CDF;
    and the odd identity gelu(z) - gelu(-z) = z that both forms satisfy."""
    from scipy.special import ndtr
    cfg = configs.tiny(E=1, k=1, activation="gelu", fusion=0, gelu_mode=mode, fc1_bias=True,
                       H=64, I=48, scale_lo=0.05, scale_hi=0.2)
    inp = gen.make_inputs(cfg, 9)
    x = as_f32(inp.x, "f32").astype(np.float64)
    W1 = bruteforce.dequant_dense(inp.w1, inp.s1, cfg, cfg.I, cfg.H)[0]
    z = x @ W1.T + as_f32(inp.b1, "f32").astype(np.float64)[0]
    h_torch = torch.nn.functional.gelu(torch.from_numpy(z), approximate=approx).numpy()
    rows = oracle.fc1_rows(cfg, inp, np.arange(9), np.zeros(9, np.int32))
    assert np.max(np.abs(rows - h_torch)) <= 1e-12 * max(np.max(np.abs(h_torch)), 1.0)
    assert np.max(np.abs(z)) > 2.0  # the tails are exercised
    if mode == 0:
        assert np.max(np.abs(rows - z * ndtr(z))) <= 1e-12 * np.max(np.abs(z))
    # odd identity: h(z) - h(-z) = z, through the linear layer with x and -x
    neg = gen.make_inputs(cfg, 9)
    neg.x[...] = (-as_f32(inp.x, "f32")).astype(np.float32)
    neg.b1[...] = (-as_f32(inp.b1, "f32")).astype(np.float32)
    hn = oracle.fc1_rows(cfg, neg, np.arange(9), np.zeros(9, np.int32))
    assert np.max(np.abs((rows - hn) - z)) <= 1e-12 * np.max(np.abs(z))


# --------------------------------------------------------------------------- weights on input

def test_weight_on_input_is_linear_for_identity_experts():
    """With identity activation and no biases each expert is linear, so the routing weight may
    go to the input or to the output with the same result (closed form of linearity)."""
    base = configs.tiny(activation="identity", fusion=0, E=6, k=3, logit_sigma=2.0)
    inp = gen.make_inputs(base, 11)
    a, _ = oracle.forward(base, inp)
    b, _ = oracle.forward(base.with_(on_input=True), inp)
    assert np.max(np.abs(a - b)) <= 1e-12 * rms(a)


def test_weight_on_input_with_k1_renorm_is_the_plain_forward():
    """k = 1 with renormalisation gives weight 1: on the input or the output, the same."""
    base = configs.tiny(k=1, fusion=1, fc1_bias=True, fc2_bias=True, limit=2.0)
    inp = gen.make_inputs(base, 7)
    a, _ = oracle.forward(base, inp)
    b, _ = oracle.forward(base.with_(on_input=True), inp)
    assert np.array_equal(a, b)


def test_expert_output_scale_scales_the_routed_part():
    base = configs.tiny(fusion=2, fc2_bias=True, E=5, k=2)
    inp = gen.make_inputs(base, 6, shared=True)
    a, _ = oracle.forward(base, inp)
    b, _ = oracle.forward(base.with_(out_scale=-0.375), inp)
    sh = as_f32(inp.shared, "f32").astype(np.float64)
    assert np.max(np.abs((b - sh) - (-0.375) * (a - sh))) <= 1e-12 * rms(a)
    c, _ = oracle.forward(base.with_(out_scale=0.0), inp)  # 0 means 1
    assert np.array_equal(a, c)


# --------------------------------------------------------------------------- sparse mixer

def _mixer_cfg(E, eps, **kw):
    return configs.tiny(E=E, k=2, sparse_mixer=True, mixer_eps=eps, normalize=False, **kw)


def test_sparse_mixer_hand_examples():
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        cases = json.load(f)["mixer_cases"]
    assert len(cases) >= 5
    for case in cases:
        lg = np.asarray(case["logits"], np.float32)
        cfg = _mixer_cfg(lg.shape[1], case["eps"])
        ids, w = oracle.route(cfg, lg)
        assert ids.tolist() == case["ids"], case["name"]
        assert np.allclose(w, np.asarray(case["w"]), rtol=1e-14, atol=0), case["name"]


def test_sparse_mixer_limits():
    """eps beyond every ratio keeps every expert: the picks' weights are plain softmaxes
    (scipy), the second over the experts other than the first; eps = 0 with distinct
    logits keeps only the pick itself: weights 1. The picks are the two largest logits
    (numpy's stable argsort)."""
    rng = np.random.default_rng(11)
    lg = rng.normal(0, 1.5, (50, 9)).astype(np.float32)
    l64 = lg.astype(np.float64)
    order = np.argsort(-l64, axis=1, kind="stable")[:, :2]
    ids, w = oracle.route(_mixer_cfg(9, 1e30), lg)
    assert np.array_equal(ids, order)
    for t in range(lg.shape[0]):
        e1, e2 = order[t]
        assert abs(w[t, 0] - softmax(l64[t])[e1]) < 1e-14
        rest = np.delete(l64[t], e1)
        assert abs(w[t, 1] - softmax(rest)[e2 - (e2 > e1)]) < 1e-14
    ids0, w0 = oracle.route(_mixer_cfg(9, 0.0), lg)
    assert np.array_equal(ids0, order) and np.all(w0 == 1.0)
    ids2, w2 = oracle.route(_mixer_cfg(9, 0.0, routed_scale=2.5), lg)
    assert np.all(w2 == 2.5)


def test_sparse_mixer_forward_composes_with_its_routing():
    """The forward with the mixer mixes the dense expert outputs (brute force) under the
    mixer's routing weights, whose values are pinned above."""
    cfg = _mixer_cfg(6, 0.05, fusion=1, fc1_bias=True, fc2_bias=True, logit_sigma=0.3)
    inp = gen.make_inputs(cfg, 9)
    ids, w = oracle.route(cfg, inp.logits)
    G = np.zeros((9, cfg.E))
    for t in range(9):
        G[t, ids[t]] = w[t]
    assert np.mean(w[:, 0] < 0.999) > 0.3  # the threshold keeps neighbours for many tokens
    ref = bruteforce.forward(cfg, inp, mixer_gates=G)
    out64, _ = oracle.forward(cfg, inp)
    assert np.max(np.abs(out64 - ref)) <= 1e-11 * rms(ref)
