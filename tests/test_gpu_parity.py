"""Parity of the HIP path with the CPU oracle, stage by stage and end to end.

Every input is seeded and synthetic (synth/). Routing indices and the grouping are
compared bit for bit; floating outputs within the stated tolerance: max |err| <=
1e-4 * RMS for fp32 activations and 2e-2 * RMS for bf16 activations, measured against
the oracle's fp64 value before rounding. At full workload sizes the routing and grouping
of all tokens are compared, and outputs on a sample of tokens the oracle evaluates one by
one.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_softmax_amd as qm
from synth import configs, gen
from synth.gen import as_f32, store
from tests.gpu_helpers import (TOL, DeviceInputs, check_output, dev, host, host_f64,
                               max_excess_err, max_rel_err, params_for, rms)

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qm._lib.load()  # the HIP library must be present wherever a GPU is
    torch.cuda.init()


def say(*a):
    print(*a, flush=True)


# --------------------------------------------------------------------------- route

def run_route(cfg, logits_np, T, ebias_np=None):
    eb = dev(ebias_np, cfg.act_dtype) if ebias_np is not None else None
    p = params_for(cfg, T, ebias=eb)
    lg = dev(logits_np, cfg.act_dtype)
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    qm.qmoe_route(p, lg, ids, w)
    torch.cuda.synchronize()
    return host(ids), host(w)


ROUTE_CASES = {
    "c1": (configs.C1, 16), "c2-T64": (configs.C2, 64), "c3-T4096": (configs.C3, 4096),
    "c4-T512": (configs.C4, 512), "c5-T4096": (configs.C5, 4096),
    "E512-k8": (configs.tiny(E=512, k=8, act_dtype="bf16", logit_sigma=0.5), 300),
    "E130-k32": (configs.tiny(E=130, k=32, act_dtype="f32", normalize=False), 100),
    "E1-k1": (configs.tiny(E=1, k=1, act_dtype="bf16"), 7),
    # routing variants: selection bias, grouped top-k, weight scaling
    "c5-grouped-biased-T256": (configs.C5_ROUTED, 256),
    "c2-biased-T64": (configs.C2_BIASED, 64),
    "E256-g8-k8-biased-bf16": (configs.tiny(E=256, k=8, n_group=8, topk_group=4, score_bias=True,
                                            routed_scale=2.5, act_dtype="bf16"), 200),
    "E32-g4-top1-f32-norenorm": (configs.tiny(E=32, k=4, n_group=4, topk_group=1,
                                              normalize=False, act_dtype="f32"), 100),
    "E96-g16-biased-f32": (configs.tiny(E=96, k=6, n_group=16, topk_group=3, score_bias=True,
                                        act_dtype="f32", routed_scale=0.5), 64),
}


@pytest.mark.parametrize("name", sorted(ROUTE_CASES))
def test_route_matches_oracle(name):
    cfg, T = ROUTE_CASES[name]
    say("route", name, cfg.E, cfg.k, T)
    _, logits, _ = gen.gen_activations(cfg, T)
    eb = gen.gen_score_bias(cfg)
    ids, w = run_route(cfg, logits, T, eb)
    rids, rw = oracle.route(cfg, logits, eb)
    assert np.array_equal(ids, rids)
    assert np.max(np.abs(w - rw)) < 2e-6


@pytest.mark.parametrize("E,k", [(8, 2), (64, 6), (130, 4)])
def test_route_ties_and_signed_zero(E, k):
    cfg = configs.tiny(E=E, k=k, act_dtype="bf16")
    rng = np.random.default_rng(E)
    vals = np.array([-0.0, 0.0, 0.0, -1.5, 1.0, 1.0, 2.0], np.float32)
    logits = store(vals[rng.integers(0, len(vals), size=(257, E))], "bf16")
    logits[0, :] = 0x8000  # all -0: experts 0..k-1
    logits[1, :] = store(np.full(E, 0.25, np.float32), "bf16")
    ids, w = run_route(cfg, logits, 257)
    rids, rw = oracle.route(cfg, logits)
    assert np.array_equal(ids, rids)
    assert ids[0].tolist() == list(range(k)) and ids[1].tolist() == list(range(k))
    assert np.max(np.abs(w - rw)) < 2e-6


# --------------------------------------------------------------------------- permute

def run_permute(cfg, ids_np, T):
    p = params_for(cfg, T)
    M = qm.qmoe_tile_m(p)
    rows, tiles = qm.qmoe_max_rows(p), qm.qmoe_max_tiles(p)
    i32 = dict(dtype=torch.int32, device="cuda")
    ids = dev(np.ascontiguousarray(ids_np, np.int32))
    counts = torch.full((cfg.E,), -5, **i32)
    offs = torch.full((cfg.E + 1,), -5, **i32)
    sa = torch.full((rows,), -5, **i32)
    pos = torch.full((T * cfg.k,), -5, **i32)
    tl = torch.full((tiles, 2), -5, **i32)
    nt = torch.full((1,), -5, **i32)
    scratch = torch.empty(max(qm.qmoe_permute_scratch_size(p), 4), dtype=torch.uint8, device="cuda")
    qm.qmoe_permute(p, ids, counts, offs, sa, pos, tl, nt, scratch)
    torch.cuda.synchronize()
    return M, dict(counts=host(counts), padded_offsets=host(offs), sorted_assign=host(sa),
                   assign_pos=host(pos), tiles=host(tl), num_tiles=int(host(nt)[0]))


PERMUTE_CASES = [
    # (E, k, T, skew): fused one-block path and multi-block path (T*k > 4096)
    (32, 4, 1, 0.0), (32, 4, 8, 0.0), (32, 4, 64, 0.0), (128, 4, 512, 0.0), (8, 2, 4096, 6.0),
    (64, 6, 4096, 0.0), (64, 6, 256, 0.0), (1, 1, 5000, 0.0), (7, 3, 3000, 50.0), (512, 8, 700, 0.0),
]


@pytest.mark.parametrize("E,k,T,skew", PERMUTE_CASES)
def test_permute_matches_oracle(E, k, T, skew):
    cfg = configs.tiny(E=E, k=k, act_dtype="bf16", H=64, I=64)
    say("permute", E, k, T, skew)
    ids = gen.gen_topk_ids(cfg, T, skew=skew)
    M, got = run_permute(cfg, ids, T)
    ref = oracle.permute(cfg, ids, M)
    P, nt = ref["rows"], ref["num_tiles"]
    assert np.array_equal(got["counts"], ref["counts"])
    assert np.array_equal(got["padded_offsets"], ref["padded_offsets"])
    assert np.array_equal(got["sorted_assign"][:P], ref["sorted_assign"])
    assert np.all(got["sorted_assign"][P:] == -5)  # rows past the layout are untouched
    assert np.array_equal(got["assign_pos"], ref["assign_pos"])
    assert got["num_tiles"] == nt
    assert np.array_equal(got["tiles"][:nt], ref["tiles"])


# --------------------------------------------------------------------------- fc1 / fc2 stages

def oracle_layout(cfg, T, M, seed=0):
    ids = gen.gen_topk_ids(cfg, T, seed=seed, skew=2.0)
    perm = oracle.permute(cfg, ids, M)
    sa = perm["sorted_assign"]
    expert_of_row = np.repeat(np.arange(cfg.E), np.diff(perm["padded_offsets"]))
    return ids, perm, sa, expert_of_row


STAGE_CFGS = {
    "c1": configs.C1,
    "c2-interleaved-b4-bs32-bias-clamp": configs.C2.with_(H=512, I=256, E=8),
    "c3-separate-perrow": configs.C3.with_(H=1024, I=768, E=4, logit_skew=0.0),
    "c4-b8-bs128-ragged-f32scale": configs.C4.with_(H=704, I=352, E=8),
    "c5-b4-bs16": configs.c5_point(4, 16).with_(H=512, I=256, E=8),
    "c5-b8-bs32": configs.c5_point(8, 32).with_(H=512, I=256, E=8),
    "c5-b4-bs64": configs.c5_point(4, 64).with_(H=512, I=256, E=8),
    "c5-b8-bs128": configs.c5_point(8, 128).with_(H=512, I=256, E=8),
    "identity-b4-bs32": configs.tiny(activation="identity", fusion=0, act_dtype="bf16",
                                     scale_dtype="bf16", H=256, I=128, block_size=32,
                                     fc1_bias=True, fc2_bias=True),
    "relu-b8-perrow": configs.tiny(activation="relu", fusion=0, act_dtype="bf16", bits=8,
                                   block_size=0, H=256, I=128),
    "silu-f32": configs.tiny(activation="silu", fusion=0, H=128, I=64, fc1_bias=True),
    "b4-bs256-interleaved": configs.tiny(fusion=1, act_dtype="bf16", scale_dtype="bf16",
                                         block_size=256, H=768, I=160, fc1_bias=True),
    "b8-bs512-shortblock": configs.tiny(fusion=2, bits=8, act_dtype="bf16", scale_dtype="bf16",
                                        block_size=512, H=1152, I=544, E=4),
    "f32-interleaved-b8-bias": configs.tiny(fusion=1, bits=8, H=96, I=80, block_size=32,
                                            fc1_bias=True, fc2_bias=True, limit=3.0),
    # MX FP4 (E2M1 codes, E8M0 scales per 32 k; tiled layout only)
    "mxfp4-interleaved-bias-clamp": configs.C2_MX.with_(H=512, I=288, E=8),
    "mxfp4-separate-silu": configs.tiny(activation="silu", fusion=0, act_dtype="bf16",
                                        scale_dtype="e8m0", bits=4, block_size=32, H=352,
                                        I=160, fc1_bias=True, scale_lo=0.01, scale_hi=0.1),
}


# 128-row tiles (the prefill-sized kernel): every scale layout and bit width, each gate/up
# arrangement and the plain activations, K not a multiple of the kernel's K step (128 for
# 4-bit, 64 for 8-bit), a short last scale block, and T large enough that experts fill
# several tiles with a ragged last one.
TILE128_CFGS = {
    "c2-interleaved-b4-bs32-bias-clamp": configs.C2.with_(H=544, I=352, E=4),
    "c3-separate-perrow-raggedK": configs.C3.with_(H=800, I=416, E=4, logit_skew=0.0),
    "c4-b8-bs128-ragged-f32scale": configs.C4.with_(H=704, I=352, E=4),
    "c5-b4-bs16": configs.c5_point(4, 16).with_(H=512, I=288, E=8),
    "c5-b4-bs64-shortblock": configs.c5_point(4, 64).with_(H=544, I=224, E=8),
    "c5-b4-bs128": configs.c5_point(4, 128).with_(H=512, I=256, E=8),
    "c5-b8-bs16": configs.c5_point(8, 16).with_(H=512, I=256, E=8),
    "c5-b8-bs32": configs.c5_point(8, 32).with_(H=480, I=224, E=8),
    "c5-b8-bs64": configs.c5_point(8, 64).with_(H=512, I=256, E=8),
    "b4-bs256-interleaved": configs.tiny(fusion=1, act_dtype="bf16", scale_dtype="bf16",
                                         block_size=256, H=768, I=160, E=4, fc1_bias=True),
    "b8-bs256-shortblock": configs.tiny(fusion=2, bits=8, act_dtype="bf16", scale_dtype="f32",
                                        block_size=256, H=640, I=416, E=4),
    "relu-b8-perrow": configs.tiny(activation="relu", fusion=0, act_dtype="bf16", bits=8,
                                   block_size=0, H=352, I=160, E=4),
    # per-row scales with K a whole number of K steps (128 k for 4-bit, 64 k for 8-bit):
    # odd and even step counts, partial column blocks, every gate/up arrangement
    "c3-separate-perrow-oddsteps": configs.C3.with_(H=384, I=256, E=4, logit_skew=0.0),
    "perrow-b4-interleaved-bias": configs.tiny(fusion=1, act_dtype="bf16", scale_dtype="bf16",
                                               block_size=0, H=512, I=384, E=4, fc1_bias=True,
                                               fc2_bias=True, limit=7.0, alpha=1.702, beta=1.0),
    "perrow-b8-concat-f32scale": configs.tiny(fusion=2, bits=8, act_dtype="bf16",
                                              scale_dtype="f32", block_size=0, H=448, I=192, E=4,
                                              fc1_bias=True),
    "perrow-b4-silu": configs.tiny(activation="silu", fusion=0, act_dtype="bf16",
                                   scale_dtype="bf16", block_size=0, H=256, I=128, E=4),
    "identity-b4-perrow-bias": configs.tiny(activation="identity", fusion=0, act_dtype="bf16",
                                            scale_dtype="bf16", block_size=0, H=256, I=192,
                                            E=4, fc1_bias=True, fc2_bias=True),
    "mxfp4-concat-raggedK": configs.C5_MX.with_(H=544, I=224, E=8),
}

# every case in the rows layout at the library's tile height; the bf16 cases at both
# weight-streaming tile heights (16 rows, and 32 rows of two MFMA row blocks) and in both
# weight layouts (the tiled one from qmoe_pack_stack); the 128-row cases in both layouts
_BF16_STAGE = [n for n in sorted(STAGE_CFGS) if STAGE_CFGS[n].act_dtype == "bf16"]


def _layouts(cfg):
    """MX FP4 weights run in the tiled layout only."""
    return ("tiles",) if cfg.scale_dtype == "e8m0" else ("rows", "tiles")


STAGE_CASES = ([(n, 0, "rows") for n in sorted(STAGE_CFGS) if "rows" in _layouts(STAGE_CFGS[n])] +
               [(n, m, lay) for n in _BF16_STAGE for m in (16, 32)
                for lay in _layouts(STAGE_CFGS[n])] +
               [(n, 128, lay) for n in sorted(TILE128_CFGS) for lay in _layouts(TILE128_CFGS[n])])


def stage_cfg(name, tile_m):
    """The config and token count of a stage case."""
    if tile_m == 128:
        return TILE128_CFGS[name], 300
    return STAGE_CFGS[name], 40


def _stage_inputs(name, tile_m, layout):
    cfg, T = stage_cfg(name, tile_m)
    assert cfg.H % 32 == 0 or cfg.act_dtype == "f32"
    inp = gen.make_inputs(cfg, T)
    p = params_for(cfg, T, tile_m=tile_m, layout=layout)
    M = qm.qmoe_tile_m(p)
    assert tile_m == 0 or M == tile_m
    return cfg, T, inp, p, M


def _device(inp, p):
    d = DeviceInputs(inp)
    return d.tiled(p) if p.weight_layout == qm.QMOE_LAYOUT_TILES else d


@pytest.mark.parametrize("name,tile_m,layout", STAGE_CASES)
def test_fc1_stage(name, tile_m, layout):
    cfg, T, inp, p, M = _stage_inputs(name, tile_m, layout)
    say("fc1", name, layout, cfg.H, cfg.I, cfg.E, "T", T, "M", M)
    ids, perm, sa, erow = oracle_layout(cfg, T, M)
    d = _device(inp, p)
    rows = qm.qmoe_max_rows(p)
    sa_pad = np.full(rows, -1, np.int32)
    sa_pad[:len(sa)] = sa
    tl = np.zeros((qm.qmoe_max_tiles(p), 2), np.int32)
    tl[:perm["num_tiles"]] = perm["tiles"]
    tdt = torch.bfloat16 if cfg.act_dtype == "bf16" else torch.float32
    h = torch.full((rows, cfg.I), 7.0, dtype=tdt, device="cuda")
    qm.qmoe_grouped_gemm_fc1_swiglu(p, d.x, dev(sa_pad), dev(tl),
                                    dev(np.array([perm["num_tiles"]], np.int32)), d.fc1, d.fc3, h)
    torch.cuda.synchronize()
    got = host_f64(h, cfg.act_dtype)
    real = np.where(sa >= 0)[0]
    ref = oracle.fc1_rows(cfg, inp, sa[real] // cfg.k, erow[real], nthreads=NTHREADS)
    err = max_rel_err(got[real], ref)
    if cfg.act_dtype == "bf16":
        # h is stored in bfloat16: the bound applies to the error beyond that rounding
        ex = max_excess_err(got[real], ref)
        say(f"  fc1 max err / rms {err:.3e}, beyond bf16 storage {ex:.3e}")
        assert ex <= TOL["bf16"]
    else:
        say(f"  fc1 max err / rms {err:.3e}")
        assert err <= TOL["f32"]
    pads = np.where(sa < 0)[0]
    assert np.all(got[pads] == 0.0)


@pytest.mark.parametrize("name,tile_m,layout", STAGE_CASES)
def test_fc2_stage(name, tile_m, layout):
    cfg, T, inp, p, M = _stage_inputs(name, tile_m, layout)
    say("fc2", name, layout, "T", T, "M", M)
    ids, perm, sa, erow = oracle_layout(cfg, T, M, seed=1)
    rows = qm.qmoe_max_rows(p)
    hin = gen.gen_stage_h(cfg, rows, sigma=3.0)
    hin[sa.size:] = 0
    hin[:sa.size][sa < 0] = 0  # padding rows hold zeros, as fc1 writes them
    d = _device(inp, p)
    tl = np.zeros((qm.qmoe_max_tiles(p), 2), np.int32)
    tl[:perm["num_tiles"]] = perm["tiles"]
    y = torch.full((rows, cfg.H), 7.0, dtype=torch.float32, device="cuda")
    qm.qmoe_grouped_gemm_fc2(p, dev(hin, cfg.act_dtype), dev(tl),
                             dev(np.array([perm["num_tiles"]], np.int32)), d.fc2, y)
    torch.cuda.synchronize()
    got = host(y).astype(np.float64)
    real = np.where(sa >= 0)[0]
    ref = oracle.fc2_rows(cfg, inp, hin, real, erow[real], nthreads=NTHREADS)
    err = max_rel_err(got[real], ref)
    say("  fc2 max err / rms", err)
    # y stays fp32 on both paths; the products of bf16 inputs are exact, so it is far
    # inside the bf16 bound
    assert err <= (1e-4 if cfg.act_dtype == "f32" else 1e-3)
    # rows of tiles past the padded layout are never written
    P = int(perm["padded_offsets"][-1])
    assert np.all(got[P:] == 7.0)


# Full-size grids in the launch configuration the bench times (the library's tile height
# for the shapes, tiled weights), with the grouping of the workload's own routing: the first
# and the last valid row of EVERY tile are compared with the oracle, so that every work item
# of the grid (the XCD-banded order of the 128-row kernels included, with its last partial
# band) is checked. fc2 takes a synthetic h (never the GPU's fc1 output).
FULL_STAGE_CASES = {
    "c3-prefill-T4096": (configs.C3, 4096),
    "c4-many-expert-T512": (configs.C4, 512),
    "c5-b4-bs16-T4096": (configs.c5_point(4, 16), 4096),
    "c5-b4-bs32-T4096": (configs.c5_point(4, 32), 4096),
    "c5-b8-bs128-T4096": (configs.c5_point(8, 128), 4096),
    "c5-b4-bs64-T256": (configs.c5_point(4, 64), 256),
    "c5-mxfp4-T4096": (configs.C5_MX, 4096),
}


def _tile_ends(perm, M):
    """Padded row indices of the first and last valid row of every tile."""
    rows = []
    for i, (_, v) in enumerate(perm["tiles"][:perm["num_tiles"]]):
        rows += [i * M, i * M + int(v) - 1]
    return np.unique(np.array(rows, np.int64))


@pytest.mark.parametrize("name", sorted(FULL_STAGE_CASES))
def test_full_size_stages_every_tile(name):
    cfg, T = FULL_STAGE_CASES[name]
    inp = gen.make_inputs(cfg, T)
    p = params_for(cfg, T, layout="tiles")
    M = qm.qmoe_tile_m(p)
    ids_o, _ = oracle.route(cfg, inp.logits, inp.ebias)
    perm = oracle.permute(cfg, ids_o, M)
    sa = perm["sorted_assign"]
    erow = np.repeat(np.arange(cfg.E), np.diff(perm["padded_offsets"]))
    chk = _tile_ends(perm, M)
    say(f"full-size {name}: T={T} M={M} tiles={perm['num_tiles']} rows checked={chk.size}")
    d = DeviceInputs(inp).tiled(p)
    rows = qm.qmoe_max_rows(p)
    sa_pad = np.full(rows, -1, np.int32)
    sa_pad[:len(sa)] = sa
    tl = np.zeros((qm.qmoe_max_tiles(p), 2), np.int32)
    tl[:perm["num_tiles"]] = perm["tiles"]
    ntd = dev(np.array([perm["num_tiles"]], np.int32))
    tld = dev(tl)
    # fc1 + activation
    h = torch.full((rows, cfg.I), 7.0, dtype=torch.bfloat16, device="cuda")
    qm.qmoe_grouped_gemm_fc1_swiglu(p, d.x, dev(sa_pad), tld, ntd, d.fc1, d.fc3, h)
    torch.cuda.synchronize()
    got = host_f64(h[torch.from_numpy(chk).cuda()], "bf16")
    ref = oracle.fc1_rows(cfg, inp, sa[chk] // cfg.k, erow[chk], nthreads=NTHREADS)
    # h is an intermediate held in bfloat16: rounding it costs up to half a bf16 spacing of
    # each value by itself (the floor printed, large where SwiGLU's tail is heavy), so the
    # bound applies to the error beyond that rounding
    err = max_rel_err(got, ref)
    floor = max_rel_err(as_f32(oracle.round_bf16(ref), "bf16").astype(np.float64), ref)
    ex = max_excess_err(got, ref)
    say(f"  fc1 max|err|/rms {err:.3e} (bf16 rounding floor {floor:.3e}); beyond the rounding "
        f"{ex:.3e} (tolerance {TOL['bf16']:.0e})")
    assert ex <= TOL["bf16"]
    pads = np.where(sa < 0)[0]
    if pads.size:
        hp = host_f64(h[torch.from_numpy(pads[:4096].astype(np.int64)).cuda()], "bf16")
        assert np.all(hp == 0.0)  # padding rows are written as zeros
    del h
    # fc2
    hin = gen.gen_stage_h(cfg, rows, sigma=3.0)
    hin[sa.size:] = 0
    hin[:sa.size][sa < 0] = 0
    y = torch.full((rows, cfg.H), 7.0, dtype=torch.float32, device="cuda")
    qm.qmoe_grouped_gemm_fc2(p, dev(hin, "bf16"), tld, ntd, d.fc2, y)
    torch.cuda.synchronize()
    goty = host(y[torch.from_numpy(chk).cuda()]).astype(np.float64)
    refy = oracle.fc2_rows(cfg, inp, hin, chk, erow[chk], nthreads=NTHREADS)
    erry = max_rel_err(goty, refy)
    say(f"  fc2 max|err|/rms {erry:.3e} (tolerance 1e-3: fp32 y from exact bf16 products)")
    assert erry <= 1e-3
    P = int(perm["padded_offsets"][-1])
    if P < rows:
        assert np.all(host(y[P:]) == 7.0)  # rows past the padded layout are never written


# --------------------------------------------------------------------------- combine

@pytest.mark.parametrize("dtype,H,shared", [("bf16", 2880, False), ("bf16", 2048, True),
                                             ("f32", 1442, True), ("f32", 128, False)])
def test_combine_stage(dtype, H, shared):
    c = configs.tiny(E=16, k=4, H=H, I=64, act_dtype=dtype, block_size=32, scale_dtype="bf16")
    T = 33
    p = params_for(c, T)
    ids = gen.gen_topk_ids(c, T)
    perm = oracle.permute(c, ids, qm.qmoe_tile_m(p))
    y = gen.gen_stage_y(c, perm["rows"])
    w = gen.gen_topk_w(c, T)
    sh = gen.gen_activations(c, T, shared=True)[2] if shared else None
    out = torch.empty((T, H), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                      device="cuda")
    qm.qmoe_combine(p, dev(y), dev(perm["assign_pos"]), dev(w),
                    dev(sh, dtype) if sh is not None else None, out)
    torch.cuda.synchronize()
    ref64, _ = oracle.combine(c, y, perm["assign_pos"], w, sh)
    assert max_rel_err(host_f64(out, dtype), ref64) <= TOL[dtype]


def test_combine_rounds_to_nearest_even():
    # k = 1 with weight 1: the output is the bf16 rounding of y itself.
    c = configs.tiny(E=2, k=1, H=4096, act_dtype="bf16", block_size=32, scale_dtype="bf16")
    T = 8
    rng = np.random.default_rng(3)
    bits = rng.integers(0x3F000000, 0x40000000, size=(T, c.H), dtype=np.uint32)
    bits[:, ::2] = (bits[:, ::2] & 0xFFFF0000) | 0x8000  # exact ties
    y = bits.view(np.float32)
    p = params_for(c, T)
    out = torch.empty((T, c.H), dtype=torch.bfloat16, device="cuda")
    qm.qmoe_combine(p, dev(y), dev(np.arange(T, dtype=np.int32)), dev(np.ones((T, 1), np.float32)),
                    None, out)
    torch.cuda.synchronize()
    ref = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(host(out), ref)


# --------------------------------------------------------------------------- end to end

def forward_gpu(cfg, inp, d=None, reshape3d=False, layout="rows", workspace=None):
    T = inp.x.shape[0]
    base = d if d is not None else DeviceInputs(inp)
    p = params_for(cfg, T, layout=layout, ebias=base.ebias)
    if d is None:
        d = base.tiled(p) if p.weight_layout == qm.QMOE_LAYOUT_TILES else base
    x = d.x.view(1, T, cfg.H) if reshape3d else d.x
    sh = d.shared.view(1, T, cfg.H) if (reshape3d and d.shared is not None) else d.shared
    out = qm.forward(p, x, d.logits, d.fc1, d.fc2, d.fc3, sh, workspace=workspace)
    torch.cuda.synchronize()
    return out.reshape(T, cfg.H), d


def workspace_routing(p, ws, T, E, k):
    """The routing and grouping that qmoe_forward left in its workspace (ws: uint8 tensor)."""
    lay = qm.qmoe_workspace_layout_of(p)
    wb = host(ws)

    def piece(off, n, dt=np.int32):
        return wb[off:off + n * np.dtype(dt).itemsize].view(dt).copy()

    A = T * k
    rows, tiles = qm.qmoe_max_rows(p), qm.qmoe_max_tiles(p)
    got = dict(fused=int(lay.fused_routing), topk_w=piece(lay.topk_w, A, np.float32).reshape(T, k),
               counts=piece(lay.counts, E), padded_offsets=piece(lay.padded_offsets, E + 1),
               sorted_assign=piece(lay.sorted_assign, rows), assign_pos=piece(lay.assign_pos, A),
               tiles=piece(lay.tile_list, 2 * tiles).reshape(tiles, 2),
               num_tiles=int(piece(lay.num_tiles, 1)[0]))
    if not got["fused"]:
        got["topk_ids"] = piece(lay.topk_ids, A).reshape(T, k)
    return got


def check_grouping(got, ids_o, w_o, perm_o, E):
    """The forward's own routing and grouping against the oracle's, bit for bit (weights
    within 2e-6). The expert of each assignment follows from the grouping alone (the rows of
    expert e hold its assignments), so the fused path's ids are checked through it."""
    P, nt = perm_o["rows"], perm_o["num_tiles"]
    assert np.array_equal(got["counts"], perm_o["counts"])
    assert np.array_equal(got["padded_offsets"], perm_o["padded_offsets"])
    assert np.array_equal(got["sorted_assign"][:P], perm_o["sorted_assign"])
    assert np.array_equal(got["assign_pos"], perm_o["assign_pos"])
    assert got["num_tiles"] == nt
    assert np.array_equal(got["tiles"][:nt], perm_o["tiles"])
    ids_from_rows = np.full(ids_o.size, -1, np.int64)
    offs, cnt = got["padded_offsets"], got["counts"]
    for e in range(E):
        ids_from_rows[got["sorted_assign"][offs[e]:offs[e] + cnt[e]]] = e
    assert np.array_equal(ids_from_rows.reshape(ids_o.shape), ids_o)
    if "topk_ids" in got:
        assert np.array_equal(got["topk_ids"], ids_o)
    assert np.max(np.abs(got["topk_w"] - w_o)) < 2e-6


def check_forward(cfg, T, sample=None, shared=False, seed=0, layout="rows", expect_fused=None):
    say("forward", cfg.name, layout, "T", T, "bits", cfg.bits, "bs", cfg.block_size)
    inp = gen.make_inputs(cfg, T, seed=seed, shared=shared)
    p = params_for(cfg, T, layout=layout)
    ws = torch.full((max(qm.qmoe_workspace_size(p), 256),), 0xA5, dtype=torch.uint8, device="cuda")
    out, d = forward_gpu(cfg, inp, layout=layout, workspace=ws)
    got = host_f64(out, cfg.act_dtype)
    # the forward's own routing and grouping of every token (read back from its
    # workspace), bit for bit
    ids_o, w_o = oracle.route(cfg, inp.logits, inp.ebias)
    M = qm.qmoe_tile_m(p)
    perm_o = oracle.permute(cfg, ids_o, M)
    grp = workspace_routing(p, ws, T, cfg.E, cfg.k)
    say(f"  grouping bit-exact ({'one-kernel' if grp['fused'] else 'two-kernel'} routing, "
        f"M={M}, {perm_o['num_tiles']} tiles)")
    check_grouping(grp, ids_o, w_o, perm_o, cfg.E)
    if expect_fused is not None:
        assert bool(grp["fused"]) == expect_fused
    # outputs
    if sample is None or sample >= T:
        sel = np.arange(T)
    else:
        rng = np.random.default_rng(seed + 17)
        sel = np.unique(np.concatenate([[0, T - 1], rng.choice(T, size=sample - 2, replace=False)]))
    ref64, _ = oracle.forward(cfg, inp, sel=sel, nthreads=NTHREADS)
    say("  " + check_output(got[sel], ref64, cfg.act_dtype))
    return out, d, inp


def test_forward_c1_tiny_fp32():
    check_forward(configs.C1, 16)


@pytest.mark.parametrize("T", [1, 8, 64])
def test_forward_c2_decode(T):
    check_forward(configs.C2, T, shared=(T == 8))


def test_forward_c3_prefill_sampled():
    check_forward(configs.C3, 4096, sample=48)


def test_forward_c4_many_experts_sampled():
    check_forward(configs.C4, 512, sample=64)


# The forward forms each token's row sum once for the 128-row per-row-scale fc1 kernel on
# tiled weights (the zero point's correction). These layers (sized so that the library
# picks 128-row tiles itself) take that path with each fusion, both bit widths, biases, a
# plain activation and the weight on the input, with H not a multiple of the K step (a
# ragged last step).
ROWSUM_CASES = {
    "b4-separate": dict(),
    "b4-interleaved-clamp-bias": dict(fusion=1, alpha=1.702, beta=1.0, limit=7.0, fc1_bias=True),
    "b8-concatenated": dict(fusion=2, bits=8, scale_lo=0.005 / 16, scale_hi=0.02 / 16),
    "b4-gelu-tanh": dict(activation="gelu", gelu_mode=1),
    "b4-weight-on-input-f32scale": dict(on_input=True, scale_dtype="f32"),
}


@pytest.mark.parametrize("name", sorted(ROWSUM_CASES))
def test_forward_rowsum_path(name):
    cfg = configs.C3.with_(name=f"rowsum-{name}", H=1056, I=1024, E=4, k=2, **ROWSUM_CASES[name])
    T = 4096
    p = params_for(cfg, T, layout="tiles")
    assert qm.qmoe_tile_m(p) == 128
    assert qm.qmoe_workspace_layout_of(p).xsum != 0  # the per-token row sums are formed
    check_forward(cfg, T, sample=96, layout="tiles")


@pytest.mark.parametrize("bits", configs.C5_BITS)
@pytest.mark.parametrize("bs", configs.C5_BLOCKS)
@pytest.mark.parametrize("T", configs.C5.T_points)
def test_forward_c5_sweep(T, bs, bits):
    check_forward(configs.c5_point(bits, bs), T, sample=24)


# the tiled weight layout end to end: every workload
@pytest.mark.parametrize("T", [1, 8, 64])
def test_forward_tiled_c2_decode(T):
    check_forward(configs.C2, T, shared=(T == 8), layout="tiles")


def test_forward_tiled_c3_prefill_sampled():
    check_forward(configs.C3, 4096, sample=48, layout="tiles")


def test_forward_tiled_c4_many_experts_sampled():
    check_forward(configs.C4, 512, sample=64, layout="tiles")


@pytest.mark.parametrize("bits", configs.C5_BITS)
@pytest.mark.parametrize("bs", configs.C5_BLOCKS)
@pytest.mark.parametrize("T", [256, 4096])
def test_forward_tiled_c5_sweep(T, bs, bits):
    check_forward(configs.c5_point(bits, bs), T, sample=24, layout="tiles")


@pytest.mark.parametrize("T", [8, 64])
def test_forward_routing_variants_c2_biased(T):
    # a selection bias on c2 (T = 8 takes the one-kernel routing and grouping)
    check_forward(configs.C2_BIASED, T, layout="tiles")


@pytest.mark.parametrize("T", [16, 256])
def test_forward_routing_variants_c5_grouped(T):
    # grouped top-k, selection bias and weight scaling on the c5 shape
    check_forward(configs.C5_ROUTED, T, sample=6, layout="tiles")


@pytest.mark.parametrize("T", [1, 8, 64])
def test_forward_mxfp4_c2_decode(T):
    check_forward(configs.C2_MX, T, layout="tiles")


@pytest.mark.parametrize("T", [1, 256, 4096])
def test_forward_mxfp4_c5_sampled(T):
    check_forward(configs.C5_MX, T, sample=24, layout="tiles")


def test_forward_deterministic_and_3d_input():
    cfg = configs.C2
    inp = gen.make_inputs(cfg, 64, shared=True)
    a, d = forward_gpu(cfg, inp)
    b, _ = forward_gpu(cfg, inp, d)
    c, _ = forward_gpu(cfg, inp, d, reshape3d=True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_forward_edge_cases():
    # one expert, k = E, every token on one expert, T = 1
    for cfg, T in [(configs.tiny(E=1, k=1, act_dtype="bf16", H=128, I=64, fc2_bias=True), 37),
                   (configs.tiny(E=4, k=4, act_dtype="bf16", H=128, I=64, normalize=False), 20),
                   (configs.tiny(E=6, k=2, act_dtype="bf16", H=64, I=96, logit_skew=40.0), 50),
                   (configs.tiny(E=3, k=2, act_dtype="f32", H=64, I=32), 1)]:
        check_forward(cfg, T)


def test_forward_zero_tokens():
    cfg = configs.C2
    p = params_for(cfg, 0)
    x = torch.empty((0, cfg.H), dtype=torch.bfloat16, device="cuda")
    lg = torch.empty((0, cfg.E), dtype=torch.bfloat16, device="cuda")
    w = torch.empty(16, dtype=torch.uint8, device="cuda")
    out = qm.forward(p, x, lg, (w, w, None), (w, w, None))
    assert out.shape == (0, cfg.H)


FUSED_ROUTING_CASES = [
    (8, 2, 64, None), (64, 4, 17, None), (64, 6, 64, "bias"), (200, 8, 40, None),
    (256, 4, 64, "groups"), (512, 4, 16, None), (512, 8, 17, None), (384, 2, 16, "bias")]


# both sides of the one-kernel routing's token limits (64 at c2's 32 experts, 16 above 256)
FUSED_ROUTING_EDGES = [
    (32, 4, 1, None), (32, 4, 8, None), (32, 4, 16, None), (32, 4, 17, None), (32, 4, 65, None),
    (257, 4, 16, None), (300, 6, 17, "bias")]


@pytest.mark.parametrize("E,k,T,variant", FUSED_ROUTING_CASES + FUSED_ROUTING_EDGES)
def test_forward_fused_routing_sizes(E, k, T, variant):
    # qmoe_forward routes and groups in one kernel up to 64 tokens (16 above 256 experts,
    # one token a wave): both sides of those edges, routing variants included
    kw = dict(E=E, k=k, T=T, variant=variant)
    say("fused routing", kw)
    extra = {}
    if variant == "bias":
        extra = dict(score_bias=True)
    elif variant == "groups":
        extra = dict(n_group=8, topk_group=3, score_bias=True, routed_scale=2.0)
    cfg = configs.tiny(E=E, k=k, act_dtype="bf16", scale_dtype="bf16", H=64, I=64, bits=4,
                       block_size=32, logit_sigma=2.0, fusion=1, **extra)
    # one kernel routes and groups up to 64 tokens (a 16-lane row per token: E <= 256, k <= 16),
    # or 16 tokens (a wave per token)
    fused = T <= (64 if (E <= 256 and k <= 16) else 16)
    check_forward(cfg, T, expect_fused=fused)
