"""qmoe_forward_noalloc (the forward whose intermediates live in the library's fixed device
array, for callers that cannot allocate) against qmoe_forward with a workspace, through the
C ABI: two calls in a row, the second with a smaller batch, each bit-identical to the
workspace forward and within the output bound of the oracle; and the size limit refused on
the host before anything is enqueued."""
from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_softmax_amd as qm
from weight_only_quantized_softmax_amd import _lib
from synth import configs, gen
from tests.gpu_helpers import DeviceInputs, check_output, host, host_f64, params_for

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qm._lib.load()
    torch.cuda.init()


def _forward_both(cfg, T, layout, seed):
    inp = gen.make_inputs(cfg, T, seed=seed, shared=True)
    base = DeviceInputs(inp)
    p = params_for(cfg, T, layout=layout, ebias=base.ebias)
    d = base.tiled(p) if layout == "tiles" else base
    assert qm.qmoe_workspace_size(p) <= qm.QMOE_NOALLOC_SCRATCH_BYTES
    lib = qm._lib.load()
    sid = torch.cuda.current_stream().cuda_stream
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    st = [qm._stack(s, n) for s, n in ((d.fc1, "fc1"), (d.fc2, "fc2"), (d.fc3, "fc3"))]
    out_na = torch.full((T, cfg.H), 3.0, dtype=torch.bfloat16, device="cuda")
    status = lib.qmoe_forward_noalloc(p, ptr(d.x), ptr(d.logits), st[0], st[1], st[2],
                                      ptr(d.shared), ptr(out_na), sid)
    assert status == _lib.QMOE_OK, lib.qmoe_last_error()
    ws = qm.alloc_workspace(p)
    out_ws = torch.full((T, cfg.H), 5.0, dtype=torch.bfloat16, device="cuda")
    status = lib.qmoe_forward(p, ptr(d.x), ptr(d.logits), st[0], st[1], st[2], ptr(d.shared),
                              ptr(out_ws), ptr(ws), ctypes.c_size_t(ws.numel()), sid)
    assert status == _lib.QMOE_OK, lib.qmoe_last_error()
    torch.cuda.synchronize()
    return inp, out_na, out_ws


@pytest.mark.parametrize("layout", ["tiles", "rows"])
def test_noalloc_matches_workspace_forward_twice(layout):
    # a large call, then a smaller one: the second must not see the first's leftovers
    for T, seed in ((64, 3), (8, 4)):
        print(f"noalloc c2 T={T} {layout}", flush=True)
        inp, out_na, out_ws = _forward_both(configs.C2, T, layout, seed)
        assert np.array_equal(host(out_na), host(out_ws))
        ref64, _ = oracle.forward(configs.C2, inp, nthreads=NTHREADS)
        print("  " + check_output(host_f64(out_na, "bf16"), ref64, "bf16"), flush=True)


def test_noalloc_refuses_shapes_beyond_its_array():
    p = params_for(configs.C3, 4096, layout="tiles")
    assert qm.qmoe_workspace_size(p) > qm.QMOE_NOALLOC_SCRATCH_BYTES
    lib = qm._lib.load()
    S = _lib.QmoeStack
    full = S(weights=1 << 20, scales=1 << 20, bias=None)
    # refused on the host: nothing is dereferenced or launched
    status = lib.qmoe_forward_noalloc(p, 1 << 20, 1 << 20, full, full, full, None, 1 << 20,
                                      None)
    assert status == _lib.QMOE_ERR_UNSUPPORTED
    assert b"qmoe_workspace_size" in lib.qmoe_last_error()
