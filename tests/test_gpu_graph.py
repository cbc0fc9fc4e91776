"""qmoe_forward captured in a HIP graph: every replay equals the eager forward bit for bit.

The forward enqueues only kernel launches on the caller's stream (no synchronisation, no
memset, no allocation), so it can be captured; the bench replays such graphs. Each replay
is separated by the program's own eager work and synchronisations and checked against the
eager result, with the graph's inputs changed in place between replays."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import weight_only_quantized_softmax_amd as qm
from synth import configs, gen
from synth.device import DeviceInputs, dev, host, params_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qm._lib.load()
    torch.cuda.init()


@pytest.mark.parametrize("cfg,T", [(configs.C2, 64), (configs.C2, 1), (configs.C2_BIASED, 8),
                                   (configs.c5_point(4, 32), 256), (configs.C2_INT8, 64)],
                         ids=["c2-T64", "c2-T1", "c2-biased-T8", "c5-b4-bs32-T256", "c2-int8-T64"])
def test_forward_graph_replays_match_eager(cfg, T):
    print("graph", cfg.name, T, flush=True)
    inp = gen.make_inputs(cfg, T, shared=True)
    base = DeviceInputs(inp)
    p = params_for(cfg, T, layout="tiles", ebias=base.ebias)
    d = base.tiled(p)
    ws = qm.alloc_workspace(p)
    x = d.x.clone()
    lg = d.logits.clone()
    out_g = torch.empty_like(x)

    def eager():
        return qm.forward(p, x, lg, d.fc1, d.fc2, d.fc3, d.shared)

    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        qm.qmoe_forward(p, x, lg, d.fc1, d.fc2, d.fc3, d.shared, out_g, ws,
                        torch.cuda.current_stream())
    torch.cuda.synchronize()
    other = gen.make_inputs(cfg, T, seed=5)
    for r in range(4):
        if r == 2:  # new inputs, written in place into the captured buffers
            x.copy_(dev(other.x, cfg.act_dtype))
            lg.copy_(dev(other.logits, cfg.act_dtype))
        want = eager()
        torch.cuda.synchronize()
        out_g.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out_g), host(want)), f"replay {r}"
