"""An independent dense reference for tiny inputs, used to pin the oracle.

It is built differently from the oracle on purpose:
* every expert's weights are dequantised at once with numpy bit operations;
* the expert set of a token is found by enumerating all C(E, k) subsets and
  keeping the one with the largest logit sum (ties: the lexicographically
  smallest index set), which equals "top-k, ties to the lower index";
* every expert's FFN is evaluated for every token and mixed through a dense
  [T, E] gate matrix; no grouping or permutation is involved;
* the sigmoid comes from scipy;
* the int8 activation tier's scale is found by trying every power of two in turn;
* gelu comes from torch (both of its forms), in float64;
* with the routing weight on the input, each expert's fc1 output is scaled by the dense
  gate weight (linearity) and the outputs are mixed through the 0/1 selection matrix.

Sources for what is computed: CLIKA "MoE" page (top-k routing per token, gated
FFN, routing-weighted sum of the expert outputs); CLIKA "QLinearWoQ" page
(y = x·dequant(W)ᵀ + b); graiphic "QMoE" page (tensor shapes,
swiglu_fusion, block_size, expert_weight_bits, activation parameters).
"""
from __future__ import annotations

import itertools

import numpy as np
import torch
from scipy.special import expit

from synth.gen import as_f32


def e2m1_bits(q: np.ndarray) -> np.ndarray:
    """E2M1 values from their bit fields (OCP MX FP4): sign bit 3, exponent bits 2..1 with
    bias 1, mantissa bit 0; exponent 0 is subnormal (0.5 * mantissa)."""
    sign = np.where((q >> 3) & 1, -1.0, 1.0)
    ex = (q >> 1) & 3
    m = (q & 1).astype(np.float64)
    mag = np.where(ex == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, ex - 1))
    return sign * mag


def dequant_dense(w: np.ndarray, s: np.ndarray, cfg, N: int, K: int) -> np.ndarray:
    E = w.shape[0]
    if cfg.bits == 4:
        lo = (w & 0x0F).astype(np.int64)
        hi = (w >> 4).astype(np.int64)
        q = np.stack([lo, hi], axis=-1).reshape(E, N, K)
    else:
        q = w.astype(np.int64)
    if cfg.scale_dtype == "e8m0":
        # MX FP4: no zero point, a power-of-two scale per block of 32
        scale = np.ldexp(1.0, np.repeat(s.astype(np.int64) - 127, cfg.block_size, axis=2)[:, :, :K])
        return e2m1_bits(q) * scale
    sf = as_f32(s, cfg.scale_dtype).astype(np.float64)
    if cfg.block_size == 0:
        scale = np.broadcast_to(sf[:, :, None], (E, N, K))
    else:
        scale = np.repeat(sf, cfg.block_size, axis=2)[:, :, :K]
    return (q - (1 << (cfg.bits - 1))).astype(np.float64) * scale


def _best_subset(values: np.ndarray, candidates, size: int):
    """The size-subset of candidates with the largest sum of values; ties: the
    lexicographically smallest (itertools yields them in that order)."""
    best, best_sum = None, None
    for subset in itertools.combinations(candidates, size):
        s = float(sum(values[list(subset)]))
        if best_sum is None or s > best_sum:
            best, best_sum = subset, s
    return list(best)


def select(cfg, keys_row: np.ndarray):
    """Experts of one token by subset enumeration. Grouped top-k: the topk_group groups
    whose largest keys have the largest sum, then the k experts of those groups whose keys
    have the largest sum."""
    cand = list(range(cfg.E))
    if cfg.n_group > 1:
        gsize = cfg.E // cfg.n_group
        gmax = keys_row.reshape(cfg.n_group, gsize).max(axis=1)
        groups = _best_subset(gmax, range(cfg.n_group), cfg.topk_group)
        cand = [e for g in sorted(groups) for e in range(g * gsize, (g + 1) * gsize)]
    return _best_subset(keys_row, cand, cfg.k)


def gates(cfg, logits: np.ndarray, ebias=None) -> np.ndarray:
    """Dense [T, E] routing weights (zero for unselected experts). ebias: the selection
    bias, added to the float32 logits in float32 for the choice only."""
    T = logits.shape[0]
    G = np.zeros((T, cfg.E))
    for t in range(T):
        row = logits[t]
        keys = row if ebias is None else (row.astype(np.float32) + ebias.astype(np.float32)).astype(np.float64)
        chosen = select(cfg, keys)
        p = np.exp(row - row.max())
        p = p / p.sum()
        wsel = p[chosen]
        if cfg.normalize:
            wsel = wsel / wsel.sum()
        G[t, chosen] = wsel * cfg.routed_scale
    return G


def int8_round(v: np.ndarray, bs: int) -> np.ndarray:
    """The int8 activation tier on the last axis by search: for each run of bs elements,
    try every scale 2^e from e = -300 up and keep the first with max|x| <= 127 * 2^e, then
    numpy's half-to-even rounding of x / 2^e."""
    v = np.asarray(v, np.float64)
    out = np.empty_like(v)
    flat, res = v.reshape(-1, v.shape[-1]), out.reshape(-1, v.shape[-1])
    for r in range(flat.shape[0]):
        for b0 in range(0, flat.shape[1], bs):
            blk = flat[r, b0:b0 + bs]
            a = np.max(np.abs(blk))
            e = 0
            if a > 0:
                e = next(c for c in range(-300, 300) if a <= 127.0 * 2.0 ** c)
            res[r, b0:b0 + bs] = np.round(blk / 2.0 ** e) * 2.0 ** e
    return out


def round_act(v: np.ndarray, act_dtype: str) -> np.ndarray:
    """Single rounding of doubles to the activation dtype: float32 by numpy's cast; bf16 by
    rounding the significand to 8 bits, half to even (normal values)."""
    if act_dtype == "f32":
        return v.astype(np.float32).astype(np.float64)
    _, ex = np.frexp(v)
    q = np.ldexp(1.0, ex - 8)
    return np.round(v / q) * q


def _act_pair(cfg, g, u):
    L = cfg.limit
    g = np.minimum(g, L)
    u = np.clip(u, -L, L)
    return g * expit(cfg.alpha * g) * (u + cfg.beta)


def forward(cfg, inp, mixer_gates=None) -> np.ndarray:
    """The dense forward. mixer_gates: the [T, E] routing weights to mix with instead of the
    subset search (the sparse mixer's routing is pinned on its own)."""
    x = as_f32(inp.x, cfg.act_dtype).astype(np.float64)
    lg = as_f32(inp.logits, cfg.act_dtype).astype(np.float64)
    E, H, I = cfg.E, cfg.H, cfg.I
    W1 = dequant_dense(inp.w1, inp.s1, cfg, cfg.n1, H)
    W2 = dequant_dense(inp.w2, inp.s2, cfg, H, I)

    def bias(b):
        return 0.0 if b is None else as_f32(b, cfg.act_dtype).astype(np.float64)

    if cfg.int8:
        x = int8_round(x, cfg.block_size)
    eb = None if inp.ebias is None else as_f32(inp.ebias, cfg.act_dtype)
    G = gates(cfg, lg, eb) if mixer_gates is None else mixer_gates
    # the routing weight on the input: expert e sees G[t, e] * x_t, and x -> x W^T is linear
    gin = G.T[:, :, None] if cfg.on_input else 1.0
    z1 = gin * np.einsum("th,enh->etn", x, W1) + (0.0 if inp.b1 is None else bias(inp.b1)[:, None, :])
    if cfg.activation == "swiglu":
        if cfg.fusion == 1:
            g, u = z1[:, :, 0::2], z1[:, :, 1::2]
        elif cfg.fusion == 2:
            g, u = z1[:, :, :I], z1[:, :, I:]
        else:
            W3 = dequant_dense(inp.w3, inp.s3, cfg, I, H)
            z3 = gin * np.einsum("th,enh->etn", x, W3) + (0.0 if inp.b3 is None else bias(inp.b3)[:, None, :])
            g, u = z1, z3
        h = _act_pair(cfg, g, u)
    elif cfg.activation == "identity":
        h = z1
    elif cfg.activation == "relu":
        h = np.maximum(z1, 0.0)
    elif cfg.activation == "silu":
        h = z1 * expit(z1)
    elif cfg.activation == "gelu":
        h = torch.nn.functional.gelu(torch.from_numpy(z1),
                                     approximate="tanh" if cfg.gelu_mode else "none").numpy()
    else:
        raise ValueError(cfg.activation)
    if cfg.int8:
        h = int8_round(round_act(h, cfg.act_dtype), cfg.block_size)
    y = np.einsum("eti,ehi->eth", h, W2) + (0.0 if inp.b2 is None else bias(inp.b2)[:, None, :])
    y = y * (cfg.out_scale if cfg.out_scale != 0 else 1.0)
    mix = (G != 0).astype(np.float64) if cfg.on_input else G
    out = np.einsum("te,eth->th", mix, y)
    if inp.shared is not None:
        out = out + as_f32(inp.shared, cfg.act_dtype).astype(np.float64)
    return out
