"""Plain fp64 CPU oracle for the fused LoRA linear (one projection).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
link this module: only the tests and the bench's CPU baseline leg use it. It
shares no code with the HIP library.

What it computes
----------------
The "matmul + LoRA" fusion of "Unsloth 深度分析报告" (section 创新之处), one
projection of the model (a q, k, v or o projection, or one MLP projection)
with its adapter:

    y = x W^T + s (x A^T) B^T          W [out, in] frozen, A [r, in], B [out, r]

and the gradient of <dY, y>: dx = dY W + s (dY B) A, dA = s (dY B)^T x,
dB = s dY^T (x A^T). No dW (the base weight is frozen). The same readings
as the MLP oracle: s = alpha / r, PEFT factor shapes, no bias, no dropout.
All arithmetic is numpy float64.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np


def forward_backward(inp: Dict[str, np.ndarray], s: float,
                     row_chunk: Optional[int] = None) -> Dict[str, np.ndarray]:
    """y, dx, da, db for fp64 arrays x, w, a, b, dy (rows in optional chunks;
    the rows are independent, the adapter gradients are summed over chunks)."""
    x, w, a, b, dy = inp["x"], inp["w"], inp["a"], inp["b"], inp["dy"]
    T = x.shape[0]
    row_chunk = T if not row_chunk else row_chunk
    y = np.empty((T, w.shape[0]))
    dx = np.empty_like(x)
    da = np.zeros_like(a)
    db = np.zeros_like(b)
    for t0 in range(0, T, row_chunk):
        sl = slice(t0, min(T, t0 + row_chunk))
        p = x[sl] @ a.T                          # [t, r]
        y[sl] = x[sl] @ w.T + s * (p @ b.T)
        q = dy[sl] @ b                           # [t, r]
        dx[sl] = dy[sl] @ w + s * (q @ a)
        da += s * (q.T @ x[sl])
        db += s * (dy[sl].T @ p)
    return {"y": y, "dx": dx, "da": da, "db": db}


def merged_reference(x, w, a, b, s: float, dy) -> Dict[str, np.ndarray]:
    """Route through the merged weight W' = W + s B A ("Unsloth 还是 AirLLM？",
    section 组合玩法): y = x W'^T, and the dense gradient dW' = dY^T x gives
    dA = s B^T dW', dB = s dW' A^T by the chain rule through W'. Shares
    nothing with :func:`forward_backward`."""
    wm = w + s * (b @ a)
    dwm = dy.T @ x
    return {"y": x @ wm.T, "dx": dy @ wm, "da": s * (b.T @ dwm), "db": s * (dwm @ a.T)}


def bruteforce(x, w, a, b, s: float, dy) -> Dict[str, np.ndarray]:
    """The same quantities by explicit scalar loops (tiny shapes only)."""
    T, n_in = x.shape
    n_out, r = b.shape
    y = np.zeros((T, n_out))
    p = np.zeros((T, r))
    for t in range(T):
        for k in range(r):
            acc = 0.0
            for i in range(n_in):
                acc += x[t, i] * a[k, i]
            p[t, k] = acc
        for o in range(n_out):
            acc = 0.0
            for i in range(n_in):
                acc += x[t, i] * w[o, i]
            lo = 0.0
            for k in range(r):
                lo += p[t, k] * b[o, k]
            y[t, o] = acc + s * lo
    q = np.zeros((T, r))
    dx = np.zeros((T, n_in))
    for t in range(T):
        for k in range(r):
            acc = 0.0
            for o in range(n_out):
                acc += dy[t, o] * b[o, k]
            q[t, k] = acc
        for i in range(n_in):
            acc = 0.0
            for o in range(n_out):
                acc += dy[t, o] * w[o, i]
            lo = 0.0
            for k in range(r):
                lo += q[t, k] * a[k, i]
            dx[t, i] = acc + s * lo
    da = np.zeros((r, n_in))
    db = np.zeros((n_out, r))
    for k in range(r):
        for i in range(n_in):
            acc = 0.0
            for t in range(T):
                acc += q[t, k] * x[t, i]
            da[k, i] = s * acc
        for o in range(n_out):
            acc = 0.0
            for t in range(T):
                acc += dy[t, o] * p[t, k]
            db[o, k] = s * acc
    return {"y": y, "dx": dx, "da": da, "db": db}


def flops(T: int, n_in: int, n_out: int, r: int) -> int:
    """Algorithmic FLOPs of forward + backward (2mnk per product, real rank):
    2 T in out + 2 T r (in + out) forward; 2 T out in + 2 T out r (dY B) +
    2 T r in ((dY B) A) + 2 r T in (dA) + 2 out T r (dB) backward."""
    return 4 * T * n_in * n_out + 6 * T * r * (n_in + n_out)
