"""The output bound the GPU tests apply (tests/gpu_helpers.check_output), checked on the
host: a correctly rounded bf16 output passes, an output off by more than the bound fails,
and heavy-tailed outputs whose own rounding reaches the bound are graded beyond it."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from synth.gen import as_f32
from tests.gpu_helpers import check_output


def _bf16(v):
    return as_f32(oracle.round_bf16(v), "bf16").astype(np.float64)


def test_rounded_output_passes_and_offset_fails():
    rng = np.random.default_rng(0)
    ref = rng.normal(0, 1, 4096)
    check_output(_bf16(ref), ref, "bf16")
    bad = _bf16(ref)
    bad[17] += 0.03 * np.sqrt(np.mean(ref ** 2))
    with pytest.raises(AssertionError):
        check_output(bad, ref, "bf16")
    check_output(ref.astype(np.float32).astype(np.float64), ref, "f32")
    with pytest.raises(AssertionError):
        check_output(ref + 2e-4, ref, "f32")


def test_heavy_tail_graded_beyond_rounding():
    rng = np.random.default_rng(1)
    ref = rng.normal(0, 1, 4096)
    ref[5] = 40.0  # half a bf16 spacing at 40 is 0.0625, over 2e-2 of the RMS
    msg = check_output(_bf16(ref), ref, "bf16")
    assert "beyond the rounding" in msg
    bad = _bf16(ref)
    bad[9] += 0.05  # a real error elsewhere still fails
    with pytest.raises(AssertionError):
        check_output(bad, ref, "bf16")
