"""The fp16 block-scale path of qmoe_forward (4-bit codes, bf16 block scales, 128-row tiles,
tiled weights): x and h lifted into fp16 by a power of two per row, each weight
(q - 8) * scale exact in one fp16 operand.

Checked here, on the forward's own workspace:
- the fp16 rows of x, bit for bit against the lifting written out on the host (the power of
  two that puts each row's largest magnitude in [2^14, 2^15), then nearest fp16);
- h (fc1 + activation) and y (fc2) at the first and last valid row of every tile, element by
  element against the oracle's fc1_rows and fc2_rows (fc2 on the oracle's own h, rounded to
  bf16 as the method stores it);
- the output on sampled tokens against the oracle's forward;
- tokens and experts whose magnitudes sit far outside fp16's range (activations up to
  2^+-20, scales up to 2^24 and down to 2^-30 times the usual, blocks 2^20 apart within a
  row), which only pass if the lifts are applied and divided out exactly.
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
from tests.gpu_helpers import (TOL, DeviceInputs, check_output, host, host_f64, max_excess_err,
                               max_rel_err, params_for)

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qm._lib.load()
    torch.cuda.init()


def say(*a):
    print(*a, flush=True)


def lifted_f16(x_bf16_bits: np.ndarray):
    """Each row times 2^e (e puts the row's largest magnitude in [2^14, 2^15); 0 for a zero
    row), rounded to the nearest fp16: (fp16 bits, e)."""
    x = as_f32(x_bf16_bits, "bf16").astype(np.float64)
    m = np.max(np.abs(x), axis=1)
    e = np.zeros(len(m), np.int64)
    nz = m > 0
    e[nz] = 14 - np.floor(np.log2(m[nz])).astype(np.int64)
    return np.ldexp(x, e[:, None]).astype(np.float16).view(np.uint16), e


def tile_ends(perm, M):
    """First and last valid row of every tile."""
    rows = []
    for i, (_, v) in enumerate(perm["tiles"]):
        rows += [i * M, i * M + int(v) - 1]
    return np.unique(np.asarray(rows, np.int64))


def run_case(cfg, T, sample, extreme=False, tile_m=0):
    say("h16 forward", cfg.name, "T", T, "bs", cfg.block_size, "fusion", cfg.fusion,
        "extreme" if extreme else "")
    inp = gen.make_inputs(cfg, T)
    if extreme:
        # tokens 0 and 3 lifted up by 2^20 and 2^12, 1 and 4 down by 2^-20 and 2^-12, 2 all
        # zero; every scale of expert 0's fc1 (and fc3) up by 2^24 (its products would
        # overflow fp16 unlifted) and of its fc2 down by 2^-30, expert 1 the other way round
        # (2^-16, 2^24), and in every row of expert 2 the first block up by 2^20 against the
        # row's other blocks. Whole rows and experts move together, so no single element
        # dominates an output row.
        x = as_f32(inp.x, "bf16").astype(np.float64)
        for t, p2 in ((0, 20), (1, -20), (3, 12), (4, -12)):
            x[t] = np.ldexp(x[t], p2)
        x[2] = 0.0
        inp.x = store(x, "bf16")
        for name, e0, e1 in (("s1", 24, -16), ("s3", 24, -16), ("s2", -30, 24)):
            s = getattr(inp, name)
            if s is None:
                continue
            v = as_f32(s, "bf16").astype(np.float64)
            v[0] = np.ldexp(v[0], e0)
            v[1] = np.ldexp(v[1], e1)
            v[2, :, 0] = np.ldexp(v[2, :, 0], 20)
            setattr(inp, name, store(v, "bf16"))
    p = params_for(cfg, T, layout="tiles", tile_m=tile_m)
    M = p.tile_m or qm.qmoe_tile_m(p)
    assert M == 128
    lay = qm.qmoe_workspace_layout_of(p)
    assert lay.x16 != 0 and lay.h16 != 0, "the fp16 path is not taken for this layer"
    ws = torch.full((qm.qmoe_workspace_size(p),), 0xA5, dtype=torch.uint8, device="cuda")
    d = DeviceInputs(inp).tiled(p)
    out = qm.forward(p, d.x, d.logits, d.fc1, d.fc2, d.fc3, d.shared, workspace=ws)
    torch.cuda.synchronize()

    # x in fp16, bit for bit
    x16 = host(ws[lay.x16:lay.x16 + T * cfg.H * 2].view(torch.int16)).view(np.uint16).reshape(T, cfg.H)
    xl = host(ws[lay.xlift:lay.xlift + T * 4].view(torch.int32))
    want16, want_e = lifted_f16(inp.x)
    assert np.array_equal(xl, want_e), "row lifts of x"
    assert np.array_equal(x16, want16), "fp16 rows of x"

    ids_o, w_o = oracle.route(cfg, inp.logits, inp.ebias)
    perm = oracle.permute(cfg, ids_o, M)
    sa = perm["sorted_assign"]
    erow = np.repeat(np.arange(cfg.E), np.diff(perm["padded_offsets"]))
    chk = tile_ends(perm, M)
    if extreme:
        # and every row of the lifted tokens
        chk = np.unique(np.concatenate([chk, perm["assign_pos"][:5 * cfg.k]]))
    rows = qm.qmoe_max_rows(p)
    say(f"  tiles={perm['num_tiles']} rows checked={chk.size}")
    chk_d = torch.from_numpy(chk).cuda()

    # h at every tile's ends
    h = ws[lay.h:lay.h + rows * cfg.I * 2].view(torch.bfloat16).view(rows, cfg.I)
    got_h = host_f64(h[chk_d], "bf16")
    # with the routing weight on the input, each row's weight scales its fc1 sums
    row_w = w_o.reshape(-1)[sa[chk]].astype(np.float64) if cfg.on_input else None
    ref_h = oracle.fc1_rows(cfg, inp, sa[chk] // cfg.k, erow[chk], nthreads=NTHREADS, row_w=row_w)
    if extreme:
        # row by row, each against its own RMS (rows differ by up to 2^100)
        err = max(max_rel_err(g[None], r[None]) for g, r in zip(got_h, ref_h) if np.any(r))
        ex = max(max_excess_err(g[None], r[None]) for g, r in zip(got_h, ref_h) if np.any(r))
    else:
        err = max_rel_err(got_h, ref_h)
        ex = max_excess_err(got_h, ref_h)
    say(f"  h: max|err|/rms {err:.3e}; beyond the bf16 rounding {ex:.3e} (tolerance {TOL['bf16']:.0e})")
    assert ex <= TOL["bf16"]

    # y at the same rows, against fc2 of the oracle's own h
    hin = np.zeros((rows, cfg.I), np.uint16)
    hin[chk] = oracle.round_bf16(ref_h)
    y = ws[lay.y:lay.y + rows * cfg.H * 4].view(torch.float32).view(rows, cfg.H)
    got_y = host(y[chk_d]).astype(np.float64)
    ref_y = oracle.fc2_rows(cfg, inp, hin, chk, erow[chk], nthreads=NTHREADS)
    if extreme:
        erry = max(max_rel_err(g[None], r[None]) for g, r in zip(got_y, ref_y) if np.any(r))
    else:
        erry = max_rel_err(got_y, ref_y)
    say(f"  y: max|err|/rms {erry:.3e} (tolerance {TOL['bf16']:.0e}; h rounded on each side)")
    assert erry <= TOL["bf16"]

    # the output on sampled tokens (the extreme tokens among them)
    rng = np.random.default_rng(17)
    sel = np.unique(np.concatenate([np.arange(6), [T - 1], rng.choice(T, size=sample, replace=False)]))
    got = host_f64(out, "bf16")
    ref64, _ = oracle.forward(cfg, inp, sel=sel, nthreads=NTHREADS)
    if extreme:
        # each token against its own RMS
        for i, t in enumerate(sel):
            r = ref64[i]
            if not np.any(r):
                assert not np.any(got[t]), f"token {t}: zero row"
                continue
            say(f"  token {t}: " + check_output(got[t][None], r[None], "bf16"))
    else:
        say("  " + check_output(got[sel], ref64, "bf16"))


H16_CASES = {
    # the sweep's 4-bit points at full size
    "c5-b4-bs16-T4096": (configs.c5_point(4, 16), 4096),
    "c5-b4-bs32-T4096": (configs.c5_point(4, 32), 4096),
    "c5-b4-bs64-T4096": (configs.c5_point(4, 64), 4096),
    "c5-b4-bs128-T4096": (configs.c5_point(4, 128), 4096),
}

# smaller layers, on 128-row tiles by request: each fusion, biases, a plain activation, the
# weight on the input, K not a multiple of the 128-wide step
SMALL = dict(H=1056, I=992, E=4, k=2, bits=4, scale_dtype="bf16", scale_lo=0.002, scale_hi=0.05)
H16_SMALL = {
    "separate-bs32": dict(fusion=0, block_size=32),
    "interleaved-clamp-bias-bs16": dict(fusion=1, alpha=1.702, beta=1.0, limit=7.0, fc1_bias=True,
                                        fc2_bias=True, block_size=16),
    "concatenated-bs64": dict(fusion=2, block_size=64),
    "gelu-bs128": dict(activation="gelu", fusion=0, block_size=128),
    # the weight on the input with the clamped, interleaved SwiGLU: an unclamped one gives
    # this layer a heavy-tailed output whose bf16 rounding alone takes 1.7e-2 of the bound
    "weight-on-input-bs32": dict(on_input=True, block_size=32, fusion=1, alpha=1.702, beta=1.0,
                                 limit=7.0),
}


@pytest.mark.parametrize("name", sorted(H16_CASES))
def test_h16_forward_every_tile(name):
    cfg, T = H16_CASES[name]
    run_case(cfg, T, sample=24)


@pytest.mark.parametrize("name", sorted(H16_SMALL))
def test_h16_forward_small_layers(name):
    cfg = configs.C5.with_(name=f"h16-{name}", **SMALL, **H16_SMALL[name])
    run_case(cfg, 4096, sample=32, tile_m=128)


@pytest.mark.parametrize("fusion", [0, 2])
def test_h16_forward_extreme_magnitudes(fusion):
    cfg = configs.C5.with_(name=f"h16-extreme-f{fusion}", **SMALL, fusion=fusion, block_size=32)
    run_case(cfg, 4096, sample=8, extreme=True, tile_m=128)
