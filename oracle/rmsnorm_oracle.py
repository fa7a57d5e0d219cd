"""Plain fp64 CPU oracle for the RMSNorm in front of the fused LoRA MLP.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
link this module: only the tests and the bench's CPU baseline leg use it. It
shares no code with the HIP library.

What it computes
----------------
RMSNorm is the step before the MLP in the Llama / Qwen decoder blocks the
pages train, and one of the hand-written forward+backward kernels of
"Unsloth 深度分析报告" (section 关键设计决策, the six kernels of the training
path). "Unsloth支持哪些模型？主流LLM兼容性一览" (section 4.2, Qwen's RMSNorm)
adds that the backward reuses the statistics the forward already computed
instead of recomputing them; the same page's model table (section 2.6)
gives eps = 1e-5 for one model family. The pages do not write the formula
out; this is the standard root-mean-square normalisation of a token row of
width H, with a frozen per-feature weight gamma:

    rstd_t  = (mean_h x_th^2 + eps)^(-1/2)
    xn_th   = x_th * rstd_t * gamma_h

and the gradient of <g, xn> for an upstream g (xhat = x * rstd):

    dx_th = rstd_t * (gamma_h g_th - xhat_th * mean_h(gamma_h g_th xhat_th))

gamma is frozen like the base weights (LoRA trains only the adapters), so
no d(gamma). The backward takes the forward's rstd as an input, which is the
pages' reuse of the forward statistics. The composition with the MLP
(``norm_mlp_forward_backward``) feeds xn to the MLP oracle and the MLP's dx
through the norm's backward. All arithmetic is numpy float64.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from . import lora_mlp_oracle as mlp


def forward(x: np.ndarray, gamma: np.ndarray, eps: float):
    """(xn, rstd) for rows x [T, H] and weight gamma [H]."""
    ms = np.mean(x * x, axis=1)                  # mean square of each row
    rstd = 1.0 / np.sqrt(ms + eps)
    xn = x * rstd[:, None] * gamma[None, :]
    return xn, rstd


def backward(x: np.ndarray, gamma: np.ndarray, rstd: np.ndarray, g: np.ndarray) -> np.ndarray:
    """dx for upstream g [T, H], with the forward's rstd (not recomputed)."""
    xhat = x * rstd[:, None]
    gg = g * gamma[None, :]                      # gradient w.r.t. xhat
    c = np.mean(gg * xhat, axis=1)               # the part along xhat
    return rstd[:, None] * (gg - xhat * c[:, None])


def norm_mlp_forward_backward(inp: Dict[str, np.ndarray], gamma: np.ndarray, eps: float, s: float,
                              row_chunk: Optional[int] = None) -> Dict[str, np.ndarray]:
    """y = MLP(RMSNorm(x)) and the gradients for dy: dx through the norm,
    the six adapter gradients as for the plain MLP, plus xn and rstd."""
    xn, rstd = forward(inp["x"], gamma, eps)
    inner = dict(inp)
    inner["x"] = xn
    out = mlp.forward_backward(inner, s, row_chunk=row_chunk)
    out["dxn"] = out["dx"]
    out["dx"] = backward(inp["x"], gamma, rstd, out["dxn"])
    out["xn"] = xn
    out["rstd"] = rstd
    return out


def bruteforce(x, gamma, eps: float, g):
    """Scalar loops over one small case: xn, rstd and dx from the chain rule
    written per element (d xn_j / d x_k), independent of the vector forms."""
    T, H = x.shape
    xn = np.zeros((T, H))
    rstd = np.zeros(T)
    dx = np.zeros((T, H))
    for t in range(T):
        ss = 0.0
        for h in range(H):
            ss += float(x[t, h]) ** 2
        r = (ss / H + eps) ** -0.5
        rstd[t] = r
        for h in range(H):
            xn[t, h] = float(x[t, h]) * r * float(gamma[h])
        # d r / d x_k = -r^3 x_k / H ;  d xn_j / d x_k = gamma_j (delta_jk r + x_j dr/dx_k)
        for k in range(H):
            drk = -(r ** 3) * float(x[t, k]) / H
            acc = 0.0
            for j in range(H):
                dj = float(gamma[j]) * ((r if j == k else 0.0) + float(x[t, j]) * drk)
                acc += float(g[t, j]) * dj
            dx[t, k] = acc
    return xn, rstd, dx
