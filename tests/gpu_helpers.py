"""Host-side helpers for the GPU tests: moving synthetic inputs to the device and
building the library's parameter block from a workload definition."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import weight_only_quantized_softmax_amd as qm
from synth.gen import as_f32


def dev(a: np.ndarray, dtype: str = None) -> torch.Tensor:
    """numpy array -> device tensor; uint16 arrays holding bf16 bits become bfloat16."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if dtype == "bf16" or (dtype is None and a.dtype == np.uint16):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def host_f64(t: torch.Tensor, dtype: str) -> np.ndarray:
    return as_f32(host(t), dtype).astype(np.float64)


def params_for(cfg, T: int, tile_m: int = 0, strict: bool = False, layout: str = "rows",
               ebias=None):
    """ebias: the device selection bias [E] (required when the config has one)."""
    if cfg.scale_dtype == "e8m0":
        layout = "tiles"  # MX FP4 weights run in the tiled layout only
    return qm.make_params(T, cfg.H, cfg.I, cfg.E, cfg.k, expert_weight_bits=cfg.bits,
                          block_size=cfg.block_size, swiglu_fusion=cfg.fusion,
                          activation=cfg.activation, normalize_routing_weights=cfg.normalize,
                          swiglu_alpha=cfg.alpha, swiglu_beta=cfg.beta, swiglu_limit=cfg.limit,
                          act_dtype=cfg.act_dtype, scale_dtype=cfg.scale_dtype, tile_m=tile_m,
                          strict_blocks=strict, weight_layout=layout, n_group=cfg.n_group,
                          topk_group=cfg.topk_group, routed_scaling_factor=cfg.routed_scale,
                          e_score_correction_bias=ebias,
                          compute_mode="int8" if cfg.int8 else "float")


class DeviceInputs:
    """Device copies of a synth.gen.Inputs bundle."""

    def __init__(self, inp):
        cfg = inp.cfg
        a, s = cfg.act_dtype, cfg.scale_dtype
        self.x = dev(inp.x, a)
        self.logits = dev(inp.logits, a)
        self.fc1 = (dev(inp.w1), dev(inp.s1, s), dev(inp.b1, a) if inp.b1 is not None else None)
        self.fc2 = (dev(inp.w2), dev(inp.s2, s), dev(inp.b2, a) if inp.b2 is not None else None)
        self.fc3 = None
        if inp.w3 is not None:
            self.fc3 = (dev(inp.w3), dev(inp.s3, s), dev(inp.b3, a) if inp.b3 is not None else None)
        self.shared = dev(inp.shared, a) if inp.shared is not None else None
        self.ebias = dev(inp.ebias, a) if inp.ebias is not None else None

    def tiled(self, p):
        """A copy whose weight stacks are in the tiled layout (qmoe_pack_stack), scales and
        biases shared."""
        t = object.__new__(DeviceInputs)
        t.__dict__.update(self.__dict__)
        for name in ("fc1", "fc2", "fc3"):
            st = getattr(self, name)
            if st is not None:
                setattr(t, name, (qm.pack_stack(p, name, st[0]),) + tuple(st[1:]))
        torch.cuda.synchronize()
        return t


def rms(a) -> float:
    return float(np.sqrt(np.mean(np.square(np.asarray(a, dtype=np.float64)))))


def max_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / RMS(ref)."""
    r = rms(ref)
    return float(np.max(np.abs(got - ref)) / (r if r > 0 else 1.0))


# Tolerances stated for the path: fp32 activations 1e-4 * RMS, bf16 activations 2e-2 * RMS.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def half_ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Half the bfloat16 spacing at each value: the most that rounding to bf16 can move it."""
    _, e = np.frexp(np.abs(np.asarray(v, dtype=np.float64)))
    return np.ldexp(1.0, e - 9)


def max_excess_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max(|got - ref| - half a bf16 spacing of ref, 0) / RMS(ref): the error beyond what
    storing the result in bfloat16 costs by itself."""
    r = rms(ref)
    ex = np.maximum(np.abs(got - ref) - half_ulp_bf16(ref), 0.0)
    return float(np.max(ex) / (r if r > 0 else 1.0))


def check_output(got: np.ndarray, ref: np.ndarray, dtype: str) -> str:
    """The output bound: max |got - ref| <= TOL[dtype] * RMS(ref), against the unrounded fp64
    reference. A bf16 output cannot be closer to the exact value than its own rounding; where
    that floor alone (half a bf16 spacing of the largest values, relative to the RMS) reaches
    the bound -- heavy-tailed outputs whose largest value exceeds about 10 RMS -- the bound
    applies to the error beyond half a bf16 spacing of each value instead. Returns a line
    with the error, the floor and the rule applied; raises AssertionError on a breach."""
    err = max_rel_err(got, ref)
    if dtype != "bf16":
        assert err <= TOL[dtype], f"max|err|/rms {err:.3e} > {TOL[dtype]:.0e}"
        return f"max|err|/rms = {err:.3e} (tolerance {TOL[dtype]:.0e})"
    floor = max_rel_err(as_f32(oracle.round_bf16(ref), "bf16").astype(np.float64), ref)
    ex = max_excess_err(got, ref)
    msg = (f"max|err|/rms = {err:.3e} (tolerance {TOL['bf16']:.0e}; bf16 rounding floor "
           f"{floor:.3e}; beyond the rounding {ex:.3e})")
    if floor < TOL["bf16"]:
        assert err <= TOL["bf16"], msg
        return msg
    assert ex <= TOL["bf16"], msg
    return msg + " [floor reaches the bound: graded beyond the rounding]"

