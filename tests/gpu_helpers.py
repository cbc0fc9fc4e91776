"""Host-side helpers for the GPU tests: moving synthetic inputs to the device and
building the library's parameter block from a workload definition."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from synth.device import DeviceInputs, dev, host, params_for  # noqa: F401 (re-exported)
from synth.gen import as_f32


def host_f64(t: torch.Tensor, dtype: str) -> np.ndarray:
    return as_f32(host(t), dtype).astype(np.float64)


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

