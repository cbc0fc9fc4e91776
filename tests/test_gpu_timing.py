"""The measurement hook qmoe_time_next_gemm: the next grouped-GEMM launch records its own
start and end on the caller's HIP events, changes nothing in the results, and the hook
clears itself after that one launch."""
from __future__ import annotations

import pytest
import torch

import weight_only_quantized_softmax_amd as qm
from synth import configs, gen
from tests.gpu_helpers import DeviceInputs, params_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qm._lib.load()
    torch.cuda.init()


def _events(n):
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    return ev


@pytest.mark.parametrize("layout", ["rows", "tiles"])
def test_time_next_gemm_times_one_kernel(layout):
    cfg, T = configs.C2, 8
    print("timing hook", cfg.name, layout, "T", T, flush=True)
    inp = gen.make_inputs(cfg, T)
    p = params_for(cfg, T, layout=layout)
    d = DeviceInputs(inp)
    if layout == "tiles":
        d = d.tiled(p)
    ref = qm.forward(p, d.x, d.logits, d.fc1, d.fc2, d.fc3)
    torch.cuda.synchronize()

    k0, k1, f0, f1 = _events(4)
    f0.record()
    qm.qmoe_time_next_gemm(k0, k1)
    out = qm.forward(p, d.x, d.logits, d.fc1, d.fc2, d.fc3)
    f1.record()
    torch.cuda.synchronize()
    kernel_ms = k0.elapsed_time(k1)
    forward_ms = f0.elapsed_time(f1)
    print(f"  fc1 kernel {kernel_ms * 1e3:.1f} us inside a forward of {forward_ms * 1e3:.1f} us",
          flush=True)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert 0.0 < kernel_ms < forward_ms

    # the hook was used up by that launch: later launches leave the events alone
    out2 = qm.forward(p, d.x, d.logits, d.fc1, d.fc2, d.fc3)
    torch.cuda.synchronize()
    assert k0.elapsed_time(k1) == kernel_ms
    assert torch.equal(out2.view(torch.int16), ref.view(torch.int16))


def test_time_next_gemm_clear():
    k0, k1 = _events(2)
    qm.qmoe_time_next_gemm(k0, k1)
    qm.qmoe_time_next_gemm(None, None)
    cfg, T = configs.C2, 1
    inp = gen.make_inputs(cfg, T)
    p = params_for(cfg, T)
    d = DeviceInputs(inp)
    before = k0.elapsed_time(k1)
    qm.forward(p, d.x, d.logits, d.fc1, d.fc2, d.fc3)
    torch.cuda.synchronize()
    assert k0.elapsed_time(k1) == before
