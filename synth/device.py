"""Device copies of the synthetic inputs and the library's parameter block for a workload.

Shared by the GPU tests and the bench. Moves arrays to the device and fills the C ABI's
parameter block from a workload definition (synth.configs); no part of the method is
computed here.
"""
from __future__ import annotations

import numpy as np
import torch

import weight_only_quantized_softmax_amd as qm


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


def params_for(cfg, T: int, tile_m: int = 0, strict: bool = False, layout: str = "rows",
               ebias=None):
    """The parameter block of workload cfg at T tokens. ebias: the device selection bias [E]
    (required when the config has one)."""
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
                          compute_mode="int8" if cfg.int8 else "float", gelu_mode=cfg.gelu_mode,
                          expert_output_scale=cfg.out_scale,
                          apply_router_weight_on_input=cfg.on_input,
                          use_sparse_mixer=cfg.sparse_mixer,
                          sparse_mixer_eps=cfg.mixer_eps if cfg.sparse_mixer else 0.0)


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
