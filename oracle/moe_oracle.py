"""Plain fp64 CPU oracle for the grouped (mixture-of-experts) LoRA SwiGLU MLP.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
link this module: only the tests and the bench's CPU baseline leg use it. It
shares no code with the HIP library.

What it computes
----------------
The MoE form of the fused LoRA MLP that "Unsloth 深度分析报告" (section
创新之处, the grouped GEMM over experts) speeds up: E experts, each a LoRA
SwiGLU MLP with its own frozen weights and its own adapters, applied to the
token rows routed to it. The rows arrive grouped by expert (the routing,
top-k choice and the weighted combine of the expert outputs are the model's
steps around this one and are not part of it): rows offsets[e] ..
offsets[e+1]-1 of x belong to expert e, and

    y[offsets[e]:offsets[e+1]] = MLP_e(x[offsets[e]:offsets[e+1]])

with MLP_e the fused LoRA MLP of the MLP oracle under expert e's tensors.
The backward gives dx row by row the same way and, per expert, the six
adapter gradients summed over that expert's rows only (zero for an expert
that got no rows). Per-expert tensors are stacked along a leading axis E.
All arithmetic is numpy float64.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from . import lora_mlp_oracle as mlp


def expert_inputs(inp: Dict[str, np.ndarray], e: int, offsets: Sequence[int]) -> Dict[str, np.ndarray]:
    """Expert e's rows of x, dy and its slices of the stacked tensors."""
    lo, hi = int(offsets[e]), int(offsets[e + 1])
    d = {k: inp[k][e] for k in mlp.WEIGHT_KEYS}
    d["x"] = inp["x"][lo:hi]
    if "dy" in inp:
        d["dy"] = inp["dy"][lo:hi]
    return d


def forward_backward(inp: Dict[str, np.ndarray], offsets: Sequence[int], s: float,
                     row_chunk: Optional[int] = None) -> Dict[str, np.ndarray]:
    """y, dx [T, H] and the stacked adapter gradients [E, ...] for grouped rows."""
    E = len(offsets) - 1
    T, H = inp["x"].shape
    if int(offsets[0]) != 0 or int(offsets[-1]) != T or np.any(np.diff(np.asarray(offsets)) < 0):
        raise ValueError("offsets must rise from 0 to the number of rows")
    y = np.zeros((T, H))
    dx = np.zeros((T, H))
    grads = {k: np.zeros((E,) + inp[k.replace("d", "", 1)].shape[1:]) for k in mlp.ADAPTER_KEYS}
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue  # no rows: empty sums
        out = mlp.forward_backward(expert_inputs(inp, e, offsets), s, row_chunk=row_chunk)
        y[lo:hi] = out["y"]
        dx[lo:hi] = out["dx"]
        for k in mlp.ADAPTER_KEYS:
            grads[k][e] = out[k]
    res = {"y": y, "dx": dx}
    res.update(grads)
    return res


def flops(offsets: Sequence[int], H: int, I: int, r: int) -> int:
    """Useful FLOPs: the dense MLP's count over all routed rows."""
    return mlp.flops(int(offsets[-1]), H, I, r)
