"""Plain fp64 CPU oracle for the LoRA SwiGLU MLP forward and backward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
link this module: only the tests, the smoke check and the bench's CPU
baseline leg use it. It shares no code with the HIP library.

What it computes
----------------
The fused LoRA MLP of "Unsloth 深度分析报告" (nightvoyager.top), section
"核心价值提炼 / 创新之处": one SwiGLU MLP whose gate, up and down projections
each carry a LoRA adapter, with a forward and a hand-derived backward fused
into one autograd unit. The pages say the fused path loses no accuracy
("Unsloth 还是 AirLLM？一个炼丹，一个硬跑", section "核心原理（为什么它快）" /
"Why it is fast"), so the oracle is the plain, unfused composition:

    proj(v; W, A, B) = v W^T + s (v A^T) B^T            (nn.Linear [out, in])
    G = proj(X; Wg, Ag, Bg)       U = proj(X; Wu, Au, Bu)
    Z = SiLU(G) * U               SiLU(g) = g * sigmoid(g)
    Y = proj(Z; Wd, Ad, Bd)

and its gradient for a loss whose gradient with respect to Y is dY. Base
weights are frozen (the same page, section "创新之处", and the AirLLM
training note of the first page: only adapters train), so there is no dW.

Readings where the pages are silent (each is listed in the design notes):
  * s = alpha / r; A is [r, in], B is [out, r]; no bias; no dropout.
  * what backward "recomputes": the result is the same function either way.
  * 4-bit weights: two's-complement nibbles, even element in the low nibble,
    64-element blocks along ``in``, w = bf16_rne(q * scale) with the product
    exact in fp32.

All arithmetic is numpy float64 (BLAS matmul as a step). Inputs are the exact
values handed to the GPU, upcast without loss.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

ADAPTER_KEYS = ("da_gate", "db_gate", "da_up", "db_up", "da_down", "db_down")
WEIGHT_KEYS = ("w_gate", "w_up", "w_down", "a_gate", "b_gate", "a_up", "b_up",
               "a_down", "b_down")


# ---------------------------------------------------------------------------
# activation

def sigmoid(g: np.ndarray) -> np.ndarray:
    """Logistic sigmoid, evaluated without overflow for either sign."""
    g = np.asarray(g, dtype=np.float64)
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-g[pos]))
    e = np.exp(g[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def silu(g: np.ndarray) -> np.ndarray:
    return g * sigmoid(g)


# ---------------------------------------------------------------------------
# forward / backward (the plain composition and its chain rule)

def forward(x, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up, a_down, b_down,
            s: float) -> Dict[str, np.ndarray]:
    """Forward of the LoRA SwiGLU MLP. Returns Y and the intermediates."""
    p_gate = x @ a_gate.T                       # [T, r]
    p_up = x @ a_up.T
    g = x @ w_gate.T + s * (p_gate @ b_gate.T)  # [T, I]
    u = x @ w_up.T + s * (p_up @ b_up.T)
    sg = sigmoid(g)
    z = g * sg * u
    p_down = z @ a_down.T                       # [T, r]
    y = z @ w_down.T + s * (p_down @ b_down.T)  # [T, H]
    return {"y": y, "g": g, "u": u, "sig": sg, "z": z,
            "p_gate": p_gate, "p_up": p_up, "p_down": p_down}


def backward(dy, x, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up, a_down,
             b_down, s: float, fwd: Optional[Dict[str, np.ndarray]] = None
             ) -> Dict[str, np.ndarray]:
    """Gradients of <dY, Y> with respect to X and the six adapter factors."""
    if fwd is None:
        fwd = forward(x, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up,
                      a_down, b_down, s)
    g, u, sg, z = fwd["g"], fwd["u"], fwd["sig"], fwd["z"]
    # down projection
    q_down = dy @ b_down                        # [T, r]
    db_down = s * (dy.T @ fwd["p_down"])        # [H, r]
    da_down = s * (q_down.T @ z)                # [r, I]
    dz = dy @ w_down + s * (q_down @ a_down)    # [T, I]
    # SwiGLU: d/dg [g sig(g)] = sig (1 + g (1 - sig))
    dg = dz * u * sg * (1.0 + g * (1.0 - sg))
    du = dz * (g * sg)
    # gate / up projections
    q_gate = dg @ b_gate                        # [T, r]
    q_up = du @ b_up
    db_gate = s * (dg.T @ fwd["p_gate"])        # [I, r]
    db_up = s * (du.T @ fwd["p_up"])
    da_gate = s * (q_gate.T @ x)                # [r, H]
    da_up = s * (q_up.T @ x)
    dx = dg @ w_gate + du @ w_up + s * (q_gate @ a_gate + q_up @ a_up)
    return {"dx": dx, "da_gate": da_gate, "db_gate": db_gate, "da_up": da_up,
            "db_up": db_up, "da_down": da_down, "db_down": db_down}


def forward_backward(inp: Dict[str, np.ndarray], s: float,
                     row_chunk: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Forward and backward over all rows, optionally in row chunks.

    ``inp`` holds fp64 arrays under the names x, dy and WEIGHT_KEYS. With
    ``row_chunk`` the token rows are processed in chunks and the adapter
    gradients summed over chunks (rows are independent in this MLP, so
    this is the same function, only with a bounded working set).
    """
    x, dy = inp["x"], inp["dy"]
    w = [inp[k] for k in WEIGHT_KEYS]
    T = x.shape[0]
    row_chunk = T if not row_chunk else row_chunk
    y = np.empty((T, inp["w_down"].shape[0]))
    dx = np.empty_like(x)
    acc = None
    for t0 in range(0, T, row_chunk):
        sl = slice(t0, min(T, t0 + row_chunk))
        f = forward(x[sl], *w, s)
        b = backward(dy[sl], x[sl], *w, s, fwd=f)
        y[sl] = f["y"]
        dx[sl] = b["dx"]
        if acc is None:
            acc = {k: b[k].copy() for k in ADAPTER_KEYS}
        else:
            for k in ADAPTER_KEYS:
                acc[k] += b[k]
    out = {"y": y, "dx": dx}
    out.update(acc)
    return out


def base_mlp_rows(x, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up, a_down,
                  b_down, s: float, dy=None) -> Dict[str, np.ndarray]:
    """Y (and dX if dY is given) for a subset of rows: the row-local outputs.

    The same function as :func:`forward`/:func:`backward`; provided so a test
    can check sampled rows of a full-size run without the whole token batch.
    """
    f = forward(x, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up, a_down,
                b_down, s)
    out = {"y": f["y"]}
    if dy is not None:
        out["dx"] = backward(dy, x, w_gate, w_up, w_down, a_gate, b_gate, a_up,
                             b_up, a_down, b_down, s, fwd=f)["dx"]
    return out


# ---------------------------------------------------------------------------
# independent second route: merged weights (pin for forward and backward)

def merged_reference(x, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up,
                     a_down, b_down, s: float, dy) -> Dict[str, np.ndarray]:
    """Route through merged weights W' = W + s B A.

    Merging an adapter into its base ("Unsloth 还是 AirLLM？", section
    "组合玩法" / "The combo") gives a plain SwiGLU MLP with the same output.
    Its dense weight gradients dW' then give the adapter gradients by the
    chain rule through W' = W + s B A:  dA = s B^T dW',  dB = s dW' A^T.
    Nothing here is shared with :func:`backward`.
    """
    wg = w_gate + s * (b_gate @ a_gate)
    wu = w_up + s * (b_up @ a_up)
    wd = w_down + s * (b_down @ a_down)
    g = x @ wg.T
    u = x @ wu.T
    sg = 1.0 / (1.0 + np.exp(-g))
    act = g * sg
    z = act * u
    y = z @ wd.T
    dz = dy @ wd
    dact = dz * u
    du = dz * act
    dg = dact * (sg + act * (1.0 - sg))          # d(g sig)/dg = sig + g sig (1 - sig)
    dwd = dy.T @ z
    dwg = dg.T @ x
    dwu = du.T @ x
    dx = dg @ wg + du @ wu
    return {"y": y, "dx": dx,
            "da_gate": s * (b_gate.T @ dwg), "db_gate": s * (dwg @ a_gate.T),
            "da_up": s * (b_up.T @ dwu), "db_up": s * (dwu @ a_up.T),
            "da_down": s * (b_down.T @ dwd), "db_down": s * (dwd @ a_down.T)}


# ---------------------------------------------------------------------------
# brute force: scalar loops, no matmul, no autograd (tiny shapes only)

def bruteforce(x, w_gate, w_up, w_down, a_gate, b_gate, a_up, b_up, a_down,
               b_down, s: float, dy) -> Dict[str, np.ndarray]:
    """Same quantities as :func:`forward_backward`, by explicit scalar loops."""
    X = np.asarray(x).tolist()
    DY = np.asarray(dy).tolist()
    Wg, Wu, Wd = (np.asarray(m).tolist() for m in (w_gate, w_up, w_down))
    Ag, Bg, Au, Bu, Ad, Bd = (np.asarray(m).tolist()
                              for m in (a_gate, b_gate, a_up, b_up, a_down, b_down))
    T, H = len(X), len(X[0])
    I, r = len(Wg), len(Ag)

    def sig(v):
        return 1.0 / (1.0 + math.exp(-v)) if v >= 0 else math.exp(v) / (1.0 + math.exp(v))

    Y = [[0.0] * H for _ in range(T)]
    DX = [[0.0] * H for _ in range(T)]
    dAg = [[0.0] * H for _ in range(r)]
    dAu = [[0.0] * H for _ in range(r)]
    dBg = [[0.0] * r for _ in range(I)]
    dBu = [[0.0] * r for _ in range(I)]
    dAd = [[0.0] * I for _ in range(r)]
    dBd = [[0.0] * r for _ in range(H)]
    for t in range(T):
        pg = [sum(X[t][h] * Ag[k][h] for h in range(H)) for k in range(r)]
        pu = [sum(X[t][h] * Au[k][h] for h in range(H)) for k in range(r)]
        G = [sum(X[t][h] * Wg[i][h] for h in range(H)) + s * sum(pg[k] * Bg[i][k] for k in range(r))
             for i in range(I)]
        U = [sum(X[t][h] * Wu[i][h] for h in range(H)) + s * sum(pu[k] * Bu[i][k] for k in range(r))
             for i in range(I)]
        S = [sig(G[i]) for i in range(I)]
        Z = [G[i] * S[i] * U[i] for i in range(I)]
        pd = [sum(Z[i] * Ad[k][i] for i in range(I)) for k in range(r)]
        for h in range(H):
            Y[t][h] = sum(Z[i] * Wd[h][i] for i in range(I)) + s * sum(pd[k] * Bd[h][k] for k in range(r))
        # backward, one token at a time; adapter grads accumulate over tokens
        qd = [sum(DY[t][h] * Bd[h][k] for h in range(H)) for k in range(r)]
        for h in range(H):
            for k in range(r):
                dBd[h][k] += s * DY[t][h] * pd[k]
        for k in range(r):
            for i in range(I):
                dAd[k][i] += s * qd[k] * Z[i]
        dZ = [sum(DY[t][h] * Wd[h][i] for h in range(H)) + s * sum(qd[k] * Ad[k][i] for k in range(r))
              for i in range(I)]
        dG = [dZ[i] * U[i] * S[i] * (1.0 + G[i] * (1.0 - S[i])) for i in range(I)]
        dU = [dZ[i] * G[i] * S[i] for i in range(I)]
        qg = [sum(dG[i] * Bg[i][k] for i in range(I)) for k in range(r)]
        qu = [sum(dU[i] * Bu[i][k] for i in range(I)) for k in range(r)]
        for i in range(I):
            for k in range(r):
                dBg[i][k] += s * dG[i] * pg[k]
                dBu[i][k] += s * dU[i] * pu[k]
        for k in range(r):
            for h in range(H):
                dAg[k][h] += s * qg[k] * X[t][h]
                dAu[k][h] += s * qu[k] * X[t][h]
        for h in range(H):
            DX[t][h] = (sum(dG[i] * Wg[i][h] + dU[i] * Wu[i][h] for i in range(I))
                        + s * sum(qg[k] * Ag[k][h] + qu[k] * Au[k][h] for k in range(r)))
    A = np.asarray
    return {"y": A(Y), "dx": A(DX), "da_gate": A(dAg), "db_gate": A(dBg),
            "da_up": A(dAu), "db_up": A(dBu), "da_down": A(dAd), "db_down": A(dBd)}


# ---------------------------------------------------------------------------
# 4-bit block weights

def bf16_round(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits and fp32's exponent range; below 2^-126 the
    quantum is fixed at 2^-133. Written from that definition with frexp and
    round-half-even, independent of any bit-level trick.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                      # v = m 2^e, 0.5 <= |m| < 1
    qexp = np.maximum(e - 8, -133)
    r = np.rint(np.ldexp(v, -qexp))         # exact scaling, then half-to-even
    out = np.ldexp(r, qexp)
    out = np.where(v == 0, v, out)          # keep the sign of zero
    big = np.abs(out) > 3.3895313892515355e38
    out = np.where(big, np.copysign(np.inf, v), out)
    return out


def unpack_int4(packed: np.ndarray, inn: int) -> np.ndarray:
    """Signed codes [out, in] from bytes [out, in/2] (even element = low nibble)."""
    b = np.asarray(packed, dtype=np.uint8)
    lo = (b & 0x0F).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    q = np.empty((b.shape[0], inn), dtype=np.int16)
    q[:, 0::2] = lo
    q[:, 1::2] = hi
    q[q >= 8] -= 16                           # two's complement nibble
    return q


def dequant_int4(packed: np.ndarray, scales: np.ndarray, inn: int,
                 block: int = 64) -> np.ndarray:
    """fp64 values of bf16_rne(q * scale), one fp16 scale per ``block`` codes."""
    q = unpack_int4(packed, inn).astype(np.float64)
    sc = np.asarray(scales, dtype=np.float16).astype(np.float64)
    sc = np.repeat(sc, block, axis=1)
    return bf16_round(q * sc)                 # q*scale is exact in fp64 and fp32


def dequant_int4_bits(packed: np.ndarray, scales: np.ndarray, inn: int,
                      block: int = 64) -> np.ndarray:
    """Raw bf16 bit patterns of :func:`dequant_int4` (for a bitwise compare)."""
    v = dequant_int4(packed, scales, inn, block)
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# algorithmic cost (for reporting, not for checking)

def flops(T: int, H: int, I: int, r: int) -> int:
    """Matmul FLOPs of one forward plus backward (2mnk per product).

    Forward: three base products 6THI and the adapter products 6Tr(H+I).
    Backward: dZ and dX through W_gate, W_up: 6THI; adapter terms 12Tr(H+I).
    """
    return 12 * T * H * I + 18 * T * r * (H + I)
