"""Python binding of the MI355X weight-only-quantized MoE library (libqmoe.so).

Argument marshalling only: every step runs in the library's HIP kernels. PyTorch is used
for device memory and the current stream. The entry points carry the C ABI's names
(include/qmoe.h); ``forward`` is a convenience wrapper in the shape of the QMoEWoQ
forward (x, router_logits, shared_output) -> out (ClikaRT "QMoEWoQ" page, forward).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import (ACT, QMOE_BF16, QMOE_E8M0, QMOE_ERR_DTYPE, QMOE_ERR_INVALID, QMOE_ERR_SHAPE,
                   QMOE_ERR_UNBOUND, QMOE_F32, QMOE_FC1, QMOE_FC2, QMOE_FC3, QMOE_LAYOUT_ROWS,
                   QMOE_NOALLOC_SCRATCH_BYTES,
                   QMOE_LAYOUT_TILES, QmoeError, QmoeParams, QmoeStack, QmoeWorkspaceLayout,
                   check, load)

__all__ = ["make_params", "qmoe_validate", "qmoe_tile_m", "qmoe_max_rows", "qmoe_max_tiles",
           "qmoe_permute_scratch_size", "qmoe_workspace_size", "qmoe_route", "qmoe_permute",
           "qmoe_grouped_gemm_fc1_swiglu", "qmoe_grouped_gemm_fc2", "qmoe_combine",
           "qmoe_forward", "qmoe_forward_noalloc", "qmoe_workspace_layout_of", "qmoe_packed_stack_size", "qmoe_pack_stack", "pack_stack",
           "qmoe_time_next_gemm", "qmoe_linear_woq", "qmoe_quantize_act", "linear_params", "linear_woq", "forward",
           "QmoeError", "QmoeParams"]

_DT = {"f32": QMOE_F32, "bf16": QMOE_BF16, "e8m0": QMOE_E8M0}
_LAYOUT = {"rows": QMOE_LAYOUT_ROWS, "tiles": QMOE_LAYOUT_TILES}
_WHICH = {"fc1": QMOE_FC1, "fc2": QMOE_FC2, "fc3": QMOE_FC3}
_COMPUTE = {"float": 0, "int8": 1}
_TORCH_DT = {QMOE_F32: torch.float32, QMOE_BF16: torch.bfloat16}

Stack = Optional[Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]]


def make_params(num_tokens: int, hidden_size: int, inter_size: int, num_experts: int, k: int, *,
                expert_weight_bits: int = 4, block_size: int = 0, swiglu_fusion: int = 0,
                activation: str = "swiglu", normalize_routing_weights: bool = True,
                swiglu_alpha: float = 1.0, swiglu_beta: float = 0.0,
                swiglu_limit: float = math.inf, act_dtype: str = "bf16",
                scale_dtype: str = "bf16", tile_m: int = 0,
                strict_blocks: bool = False, weight_layout: str = "rows", n_group: int = 0,
                topk_group: int = 0, routed_scaling_factor: float = 1.0,
                e_score_correction_bias: Optional[torch.Tensor] = None,
                compute_mode: str = "float", gelu_mode: int = 0,
                expert_output_scale: float = 1.0, apply_router_weight_on_input: bool = False,
                use_sparse_mixer: bool = False, sparse_mixer_eps: float = 0.0) -> QmoeParams:
    """The parameter block. e_score_correction_bias: a device tensor [E] in the activation
    dtype (the block keeps its address, so the tensor must outlive the calls)."""
    bias = None if e_score_correction_bias is None else _ptr(e_score_correction_bias,
                                                            "e_score_correction_bias")
    return QmoeParams(num_tokens=num_tokens, hidden_size=hidden_size, inter_size=inter_size,
                      num_experts=num_experts, k=k, expert_weight_bits=expert_weight_bits,
                      block_size=block_size, swiglu_fusion=swiglu_fusion,
                      activation=ACT[activation],
                      normalize_routing_weights=int(bool(normalize_routing_weights)),
                      swiglu_alpha=swiglu_alpha, swiglu_beta=swiglu_beta,
                      swiglu_limit=swiglu_limit, act_dtype=_DT[act_dtype],
                      scale_dtype=_DT[scale_dtype], tile_m=tile_m,
                      strict_blocks=int(bool(strict_blocks)),
                      weight_layout=_LAYOUT[weight_layout], n_group=n_group,
                      topk_group=topk_group, routed_scaling_factor=routed_scaling_factor,
                      e_score_correction_bias=bias, compute_mode=_COMPUTE[compute_mode],
                      gelu_mode=gelu_mode, expert_output_scale=expert_output_scale,
                      apply_router_weight_on_input=int(bool(apply_router_weight_on_input)),
                      use_sparse_mixer=int(bool(use_sparse_mixer)),
                      sparse_mixer_eps=sparse_mixer_eps)


def _ptr(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise QmoeError(QMOE_ERR_UNBOUND, f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise QmoeError(QMOE_ERR_SHAPE, f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _stack(st: Stack, name: str) -> QmoeStack:
    if st is None:
        return QmoeStack()
    w, s, b = (tuple(st) + (None,))[:3]
    return QmoeStack(weights=_ptr(w, name + ".weights"), scales=_ptr(s, name + ".scales"),
                     bias=_ptr(b, name + ".bias"))


def _expect(t: torch.Tensor, shape: Sequence[int], dtype: torch.dtype, name: str) -> None:
    if tuple(t.shape) != tuple(shape):
        raise QmoeError(QMOE_ERR_SHAPE, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise QmoeError(QMOE_ERR_DTYPE, f"{name} has dtype {t.dtype}, expected {dtype}")


def qmoe_validate(p: QmoeParams) -> None:
    check(load().qmoe_validate(p))


def qmoe_tile_m(p: QmoeParams) -> int:
    return int(load().qmoe_tile_m(p))


def qmoe_max_rows(p: QmoeParams) -> int:
    return int(load().qmoe_max_rows(p))


def qmoe_max_tiles(p: QmoeParams) -> int:
    return int(load().qmoe_max_tiles(p))


def qmoe_permute_scratch_size(p: QmoeParams) -> int:
    return int(load().qmoe_permute_scratch_size(p))


def qmoe_workspace_size(p: QmoeParams) -> int:
    n = int(load().qmoe_workspace_size(p))
    if n == 0:
        check(load().qmoe_validate(p))
    return n


def qmoe_forward_noalloc(p, input, router_logits, fc1: Stack, fc2: Stack, fc3: Stack,
                         shared_output, output, stream=None) -> None:
    """qmoe_forward with the library's fixed intermediate array instead of a workspace."""
    check(load().qmoe_forward_noalloc(p, _ptr(input, "input"),
                                      _ptr(router_logits, "router_logits"), _stack(fc1, "fc1"),
                                      _stack(fc2, "fc2"), _stack(fc3, "fc3"),
                                      _ptr(shared_output, "shared_output"),
                                      _ptr(output, "output"), _stream(stream)))


def qmoe_workspace_layout_of(p: QmoeParams) -> QmoeWorkspaceLayout:
    """Byte offsets of qmoe_forward's intermediates inside its workspace."""
    out = QmoeWorkspaceLayout()
    check(load().qmoe_workspace_layout_of(p, out))
    return out


def qmoe_route(p, router_logits, topk_ids, topk_w, stream=None) -> None:
    check(load().qmoe_route(p, _ptr(router_logits, "router_logits"), _ptr(topk_ids, "topk_ids"),
                            _ptr(topk_w, "topk_w"), _stream(stream)))


def qmoe_permute(p, topk_ids, counts, padded_offsets, sorted_assign, assign_pos, tile_list,
                 num_tiles, scratch=None, stream=None) -> None:
    nbytes = 0 if scratch is None else scratch.numel() * scratch.element_size()
    check(load().qmoe_permute(p, _ptr(topk_ids, "topk_ids"), _ptr(counts, "counts"),
                              _ptr(padded_offsets, "padded_offsets"),
                              _ptr(sorted_assign, "sorted_assign"), _ptr(assign_pos, "assign_pos"),
                              _ptr(tile_list, "tile_list"), _ptr(num_tiles, "num_tiles"),
                              _ptr(scratch, "scratch"), nbytes, _stream(stream)))


def qmoe_grouped_gemm_fc1_swiglu(p, x, sorted_assign, tile_list, num_tiles, fc1: Stack,
                                 fc3: Stack, h, stream=None, topk_w=None) -> None:
    """topk_w: the routing weights [T, k], read with apply_router_weight_on_input only."""
    check(load().qmoe_grouped_gemm_fc1_swiglu(
        p, _ptr(x, "x"), _ptr(sorted_assign, "sorted_assign"), _ptr(tile_list, "tile_list"),
        _ptr(num_tiles, "num_tiles"), _ptr(topk_w, "topk_w"), _stack(fc1, "fc1"),
        _stack(fc3, "fc3"), _ptr(h, "h"), _stream(stream)))


def qmoe_grouped_gemm_fc2(p, h, tile_list, num_tiles, fc2: Stack, y, stream=None) -> None:
    check(load().qmoe_grouped_gemm_fc2(p, _ptr(h, "h"), _ptr(tile_list, "tile_list"),
                                       _ptr(num_tiles, "num_tiles"), _stack(fc2, "fc2"),
                                       _ptr(y, "y"), _stream(stream)))


def qmoe_combine(p, y, assign_pos, topk_w, shared_output, output, stream=None) -> None:
    check(load().qmoe_combine(p, _ptr(y, "y"), _ptr(assign_pos, "assign_pos"),
                              _ptr(topk_w, "topk_w"), _ptr(shared_output, "shared_output"),
                              _ptr(output, "output"), _stream(stream)))


def qmoe_forward(p, input, router_logits, fc1: Stack, fc2: Stack, fc3: Stack, shared_output,
                 output, workspace, stream=None) -> None:
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(load().qmoe_forward(p, _ptr(input, "input"), _ptr(router_logits, "router_logits"),
                              _stack(fc1, "fc1"), _stack(fc2, "fc2"), _stack(fc3, "fc3"),
                              _ptr(shared_output, "shared_output"), _ptr(output, "output"),
                              _ptr(workspace, "workspace"), nbytes, _stream(stream)))


def qmoe_packed_stack_size(p: QmoeParams, which: str) -> int:
    return int(load().qmoe_packed_stack_size(p, _WHICH[which]))


def qmoe_pack_stack(p: QmoeParams, which: str, weights, packed, stream=None) -> None:
    check(load().qmoe_pack_stack(p, _WHICH[which], _ptr(weights, "weights"),
                                 _ptr(packed, "packed"), _stream(stream)))


def pack_stack(p: QmoeParams, which: str, weights: torch.Tensor, stream=None) -> torch.Tensor:
    """The tiled form of a rows-layout weight stack, in a new uint8 device tensor."""
    n = qmoe_packed_stack_size(p, which)
    if n == 0:
        check(load().qmoe_validate(p))
        raise QmoeError(QMOE_ERR_INVALID, f"stack {which} does not exist for these parameters")
    packed = torch.empty(n, dtype=torch.uint8, device=weights.device)
    qmoe_pack_stack(p, which, weights, packed, stream)
    return packed


def linear_params(num_tokens: int, in_features: int, out_features: int, *,
                  expert_weight_bits: int = 4, block_size: int = 0, activation: str = "identity",
                  act_dtype: str = "bf16", scale_dtype: str = "bf16", tile_m: int = 0,
                  strict_blocks: bool = False, weight_layout: str = "rows",
                  gelu_mode: int = 0) -> QmoeParams:
    """The parameter block of a QLinearWoQ layer: one expert, k = 1."""
    return make_params(num_tokens, in_features, out_features, 1, 1,
                       expert_weight_bits=expert_weight_bits, block_size=block_size,
                       activation=activation, normalize_routing_weights=False,
                       act_dtype=act_dtype, scale_dtype=scale_dtype, tile_m=tile_m,
                       strict_blocks=strict_blocks, weight_layout=weight_layout,
                       gelu_mode=gelu_mode)


def qmoe_linear_woq(p: QmoeParams, x, w: Stack, y, stream=None) -> None:
    check(load().qmoe_linear_woq(p, _ptr(x, "x"), _stack(w, "weight"), _ptr(y, "y"),
                                 _stream(stream)))


def linear_woq(p: QmoeParams, x: torch.Tensor, w: Stack, stream=None) -> torch.Tensor:
    """y = act(x @ dequant(W)^T + b) for x [*, in_features] (the QLinearWoQ forward)."""
    K, N = p.hidden_size, p.inter_size
    x2 = x.reshape(-1, K)
    if x2.shape[0] != p.num_tokens:
        raise QmoeError(QMOE_ERR_SHAPE, f"x holds {x2.shape[0]} rows, params say {p.num_tokens}")
    _expect(x2, (p.num_tokens, K), _TORCH_DT[p.act_dtype], "x")
    y = torch.empty(tuple(x.shape[:-1]) + (N,), dtype=x.dtype, device=x.device)
    qmoe_linear_woq(p, x2, w, y.view(-1, N), stream)
    return y


def qmoe_quantize_act(p: QmoeParams, x: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """The int8 activation tier's per-block rounding of the rows of x into out ([rows, cols])."""
    if x.dim() != 2 or tuple(out.shape) != tuple(x.shape) or out.dtype != x.dtype:
        raise QmoeError(QMOE_ERR_SHAPE, "qmoe_quantize_act: x and out must be [rows, cols] alike")
    rows, cols = x.shape
    check(load().qmoe_quantize_act(p, _ptr(x, "in"), rows, cols, _ptr(out, "out"), _stream(stream)))


def qmoe_time_next_gemm(start: Optional[torch.cuda.Event], stop: Optional[torch.cuda.Event]) -> None:
    """The calling thread's next grouped-GEMM launch records its own start and end on these
    events (each already recorded once, so that it exists)."""
    ev = lambda e: None if e is None else e.cuda_event  # noqa: E731
    check(load().qmoe_time_next_gemm(ev(start), ev(stop)))


def alloc_workspace(p: QmoeParams, device="cuda") -> torch.Tensor:
    return torch.empty(max(qmoe_workspace_size(p), 256), dtype=torch.uint8, device=device)


def forward(p: QmoeParams, x: torch.Tensor, router_logits: torch.Tensor, fc1: Stack, fc2: Stack,
            fc3: Stack = None, shared_output: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out = QMoE(x, router_logits) (+ shared_output); x is [T, H] or [B, S, H]."""
    H = p.hidden_size
    dt = _TORCH_DT[p.act_dtype]
    x2 = x.reshape(-1, H)
    if x2.shape[0] != p.num_tokens:
        raise QmoeError(QMOE_ERR_SHAPE, f"x holds {x2.shape[0]} tokens, params say {p.num_tokens}")
    _expect(x2, (p.num_tokens, H), dt, "x")
    _expect(router_logits.reshape(-1, p.num_experts), (p.num_tokens, p.num_experts), dt,
            "router_logits")
    if shared_output is not None:
        _expect(shared_output, tuple(x.shape), dt, "shared_output")
    out = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_workspace(p, x.device)
    qmoe_forward(p, x2, router_logits.reshape(-1, p.num_experts), fc1, fc2, fc3,
                 None if shared_output is None else shared_output.reshape(-1, H),
                 out.view(-1, H), workspace, stream)
    return out
