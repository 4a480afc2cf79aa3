"""Deferred MoE finalize for torch callers: the caller side of the fused op.

The contract (vLLM pull request #62174, Overview and Details): a decode MoE
layer may leave its top-k reduction open and hand the next layer a MoEOutput
that holds the unfinalized routed part (the GEMM2 rows, the permutation map
and the routing weights) plus the shared-expert output. The next layer's input
norm then finalizes it, adds the residual and normalises in one kernel. A layer
defers only when the fused kernel will run for the shape; otherwise it
finalizes as before. Releasing the deferred buffers, once the fused kernel has
been enqueued, is the consuming layer's job.

Here:
  * ``UnfinalizedMoEOutput`` / ``MoEOutput`` carry the deferred tensors;
  * ``defer_moe_finalize(T, H, K)`` is the producer's check (the library's
    path query, a host function: no GPU work, safe during graph capture);
  * ``fused_add_rmsnorm(hidden, residual, gamma, eps)`` is the consumer norm:
    a deferred MoEOutput goes to the fused finalize kernel, a plain tensor
    (attention / dense MLP output) to the dense residual add + RMSNorm kernel;
  * both kernels are registered as torch ops, with C++ kernels, that write
    into caller-provided outputs, so torch sees their effects (torch.compile
    traces them) and HIP graph capture records them:
    ``mfr::moe_finalize_rmsnorm`` and ``mfr::residual_add_rmsnorm``
    write a separate residual_out; ``mfr::moe_finalize_rmsnorm_`` and
    ``mfr::residual_add_rmsnorm_`` update the residual stream in place (it is
    then the one mutated argument, never passed twice); the ``_fp8`` forms of
    all four write the normed state as per-token FP8 codes and scales, the
    activation format of an FP8 projection.
Every step of the arithmetic runs in the HIP library; nothing here computes.
"""
import os
from dataclasses import dataclass
from typing import Optional, Tuple, Union

import torch

from . import binding
from . import build as _build

# The ops' schemas and kernels are C++ (csrc/mfr_torch_ops.cpp, built next to
# the HIP library it calls): an eager call through torch.ops then costs the
# dispatcher and the launch, not a Python layer. The kernels refuse tensors
# off the GPU.
if not os.path.exists(_build.OPS_LIB):
    raise ImportError(f"{_build.OPS_LIB} is not built; run top_finalize_residual_amd/build.py first")
torch.ops.load_library(_build.OPS_LIB)

_OP_NAMES = ("moe_finalize_rmsnorm", "moe_finalize_rmsnorm_", "moe_finalize_rmsnorm_fp8",
             "moe_finalize_rmsnorm_fp8_", "residual_add_rmsnorm", "residual_add_rmsnorm_",
             "residual_add_rmsnorm_fp8", "residual_add_rmsnorm_fp8_")


def _no_output(*args):
    """Fake-tensor kernel of every op: they write into their arguments and
    return nothing."""
    return None


for _name in _OP_NAMES:
    torch.library.register_fake(f"mfr::{_name}")(_no_output)
_OP = {name: getattr(torch.ops.mfr, name).default for name in _OP_NAMES}


@dataclass
class UnfinalizedMoEOutput:
    """The routed part of a MoE layer whose top-k reduction is still open.

    expert_out: [R, H] bf16 GEMM2 output rows; perm_idx: [T, K] int32 row of
    each (token, slot), negative = masked; topk_w: [T, K] fp32 routing weights;
    scale: routed scaling factor (1.0 when the router folded it into topk_w).
    """
    expert_out: torch.Tensor
    perm_idx: torch.Tensor
    topk_w: torch.Tensor
    scale: float = 1.0

    @property
    def num_tokens(self) -> int:
        return int(self.perm_idx.shape[0])

    @property
    def hidden_size(self) -> int:
        return int(self.expert_out.shape[1])

    @property
    def top_k(self) -> int:
        return int(self.perm_idx.shape[1])


@dataclass
class MoEOutput:
    """A MoE layer's output handed to the next layer's norm: the routed part
    (deferred, or already a [T, H] tensor) and the shared-expert output."""
    routed: Union[UnfinalizedMoEOutput, torch.Tensor]
    shared: torch.Tensor

    @property
    def deferred(self) -> bool:
        return isinstance(self.routed, UnfinalizedMoEOutput)


def defer_moe_finalize(num_tokens: int, hidden_size: int, top_k: int) -> bool:
    """True if the fused finalize accepts this shape, so a producer may leave
    its top-k reduction open. Host-only; no GPU work."""
    return binding.moe_finalize_rmsnorm_path(num_tokens, hidden_size, top_k) != binding.PATH_UNSUPPORTED


def _residual_out(ref: torch.Tensor, residual: torch.Tensor, residual_out, in_place):
    """The separate output for the new residual stream, or None for an
    in-place update of `residual`."""
    if residual_out is residual:
        return None
    if in_place:
        if residual_out is not None:
            raise ValueError("in_place=True writes the residual stream itself; pass no residual_out")
        return None
    return torch.empty_like(ref) if residual_out is None else residual_out


def _routed(hidden: "MoEOutput"):
    """(rows, perm_idx, weights, scale) of a MoEOutput's routed part."""
    if hidden.deferred:
        r = hidden.routed
        return r.expert_out, r.perm_idx, r.topk_w, float(r.scale)
    # An already finalized routed part goes through the same kernel as a single
    # routed row per token (weight 1, scale 1), which keeps the one-rounding
    # contract for routed + shared + residual.
    rows = hidden.routed
    T = rows.shape[0]
    idx = torch.arange(T, dtype=torch.int32, device=rows.device).unsqueeze(1)
    w = torch.ones((T, 1), dtype=torch.float32, device=rows.device)
    return rows, idx, w, 1.0


# (routed part, FP8 output, in place) -> op name (and its kernel above)
_OPS = {
    (True, False, False): "moe_finalize_rmsnorm",
    (True, False, True): "moe_finalize_rmsnorm_",
    (True, True, False): "moe_finalize_rmsnorm_fp8",
    (True, True, True): "moe_finalize_rmsnorm_fp8_",
    (False, False, False): "residual_add_rmsnorm",
    (False, False, True): "residual_add_rmsnorm_",
    (False, True, False): "residual_add_rmsnorm_fp8",
    (False, True, True): "residual_add_rmsnorm_fp8_",
}


def fused_add_rmsnorm(hidden: Union[MoEOutput, torch.Tensor], residual: torch.Tensor,
                      gamma: torch.Tensor, eps: float, *, in_place: bool = False,
                      residual_out: Optional[torch.Tensor] = None,
                      normed_out: Optional[torch.Tensor] = None, fp8: bool = False,
                      normed_fp8: Optional[torch.Tensor] = None,
                      fp8_scale: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, ...]:
    """The consumer norm of the next layer.

    hidden: a MoEOutput (deferred or finalized routed part plus shared output)
    or a plain [T, H] bf16 tensor (a dense layer's output).
    Returns (new residual stream, normed hidden state), both [T, H] bf16.
    in_place: write the new residual stream into `residual` itself (also
    implied by passing residual_out=residual).
    fp8: produce the normed hidden state as dynamic per-token FP8 for an FP8
    projection instead: returns (new residual stream, normed_fp8 [T, H]
    float8_e4m3fn, fp8_scale [T] float32), where a token's normed row is
    about normed_fp8 times its scale. normed_fp8 and fp8_scale may be given.
    A deferred routed part goes through the checked kernel, told the rows of
    its expert_out, so an out-of-range index is masked rather than read.
    """
    if fp8 and normed_out is not None:
        raise ValueError("fp8=True writes normed_fp8 and fp8_scale, not normed_out")
    if not fp8 and (normed_fp8 is not None or fp8_scale is not None):
        raise ValueError("normed_fp8 and fp8_scale are the outputs of fp8=True")
    moe = isinstance(hidden, MoEOutput)
    ref = hidden.shared if moe else hidden
    r_out = _residual_out(ref, residual, residual_out, in_place)
    if fp8:
        T, H = ref.shape
        if normed_fp8 is None:
            normed_fp8 = torch.empty((T, H), dtype=torch.float8_e4m3fn, device=ref.device)
        if fp8_scale is None:
            fp8_scale = torch.empty((T,), dtype=torch.float32, device=ref.device)
        outs = (normed_fp8, fp8_scale)
    else:
        outs = (torch.empty_like(ref) if normed_out is None else normed_out,)
    if moe:
        rows, idx, w, scale = _routed(hidden)
        args = (rows, idx, w, hidden.shared, residual, gamma, float(eps), scale)
    else:
        args = (hidden, residual, gamma, float(eps))
    op = _OP[_OPS[(moe, fp8, r_out is None)]]
    if r_out is None:
        op(*args, *outs)
        return (residual,) + outs
    op(*args, r_out, *outs)
    return (r_out,) + outs
