"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle, compare.

The HIP path is reached only through the C ABI (lora_swiglu_mlp_amd.mlp ->
abi -> liblora_mlp.so); the oracle is the fp64 numpy code under oracle/.
Both get the same seeded inputs from lora_swiglu_mlp_amd.inputs.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle
from lora_swiglu_mlp_amd import inputs as inp_mod

OUT_KEYS = ("y", "dx", "da_gate", "db_gate", "da_up", "db_up", "da_down", "db_down")
# max|gpu - ref| / max|ref| per output tensor
TOL = {"f32": 1e-4, "bf16": 2e-2}


def oracle_inputs(inp: dict, wl) -> dict:
    d = {}
    for k, v in inp.items():
        if k.endswith("_scales"):
            continue
        if wl.wfmt == "int4_b64" and k in ("w_gate", "w_up", "w_down", "w"):
            inn = wl.inter if k == "w_down" else wl.hidden  # the linear's w is [out, in = hidden]
            d[k] = oracle.dequant_int4(v, inp[k + "_scales"], inn)
        else:
            d[k] = inp_mod.to_f64(v, wl.dtype)
    return d


def run_hip(inp: dict, wl, flags: int = 0, device="cuda"):
    """Forward + backward on the GPU; returns fp64 numpy outputs and the model."""
    import torch
    from lora_swiglu_mlp_amd import mlp
    m, x, dy = mlp.from_inputs(inp, wl, device, flags)
    y, saved = m.forward(x)
    g = m.backward(dy, x, saved)
    torch.cuda.synchronize()
    out = {"y": y}
    out.update(g)
    return {k: v.float().cpu().numpy().astype(np.float64) for k, v in out.items()}, m


def run_hip_norm(inp: dict, wl, eps: float, flags: int = 0, device="cuda"):
    """RMSNorm then the MLP, forward + backward on the GPU (inp holds "gamma")."""
    import torch
    from lora_swiglu_mlp_amd import mlp
    m, x, dy = mlp.from_inputs(inp, wl, device, flags, norm_eps=eps)
    y, saved = m.forward(x)
    g = m.backward(dy, x, saved)
    torch.cuda.synchronize()
    out = {"y": y}
    out.update(g)
    return {k: v.float().cpu().numpy().astype(np.float64) for k, v in out.items()}, m


def norm_oracle(inp: dict, wl, eps: float, row_chunk: int = 2048) -> dict:
    """The fp64 oracle of RMSNorm then the MLP on the same stored inputs."""
    d = oracle_inputs(inp, wl)
    gamma = d.pop("gamma")
    return oracle.rmsnorm.norm_mlp_forward_backward(d, gamma, eps, wl.scale, row_chunk=row_chunk)


def run_hip_moe(inp: dict, offsets, wl, flags: int = 0, device="cuda"):
    """Grouped (MoE) forward + backward on the GPU; fp64 numpy outputs."""
    import torch
    from lora_swiglu_mlp_amd import mlp
    m, x, dy = mlp.moe_from_inputs(inp, offsets, wl, device, flags)
    y, saved = m.forward(x)
    g = m.backward(dy, x, saved)
    torch.cuda.synchronize()
    out = {"y": y}
    out.update(g)
    return {k: v.float().cpu().numpy().astype(np.float64) for k, v in out.items()}, m


def moe_oracle_inputs(inp: dict, wl) -> dict:
    """fp64 copies of stacked MoE inputs (4-bit weights decoded expert by expert)."""
    d = {}
    for k, v in inp.items():
        if k.endswith("_scales"):
            continue
        if wl.wfmt == "int4_b64" and k in ("w_gate", "w_up", "w_down"):
            inn = wl.inter if k == "w_down" else wl.hidden
            d[k] = np.stack([oracle.dequant_int4(v[e], inp[k + "_scales"][e], inn) for e in range(v.shape[0])])
        else:
            d[k] = inp_mod.to_f64(v, wl.dtype)
    return d


def relerr(got: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den


LIN_KEYS = ("y", "dx", "da", "db")


def run_hip_linear(inp: dict, wl, flags: int = 0, device="cuda"):
    """Fused LoRA linear forward + backward on the GPU; fp64 numpy outputs."""
    import torch
    from lora_swiglu_mlp_amd import mlp
    m, x, dy = mlp.linear_from_inputs(inp, wl, device, flags)
    y, saved = m.forward(x)
    g = m.backward(dy, x, saved)
    torch.cuda.synchronize()
    out = {"y": y}
    out.update(g)
    return {k: v.float().cpu().numpy().astype(np.float64) for k, v in out.items()}, m


def compare(got: dict, ref: dict, tol: float, label: str = "") -> dict:
    keys = OUT_KEYS if "da_gate" in ref else LIN_KEYS
    errs = {k: relerr(got[k], ref[k]) for k in keys if k in ref}
    print(f"[parity] {label} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    sys.stdout.flush()
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{label}: over tolerance {tol}: {bad}"
    return errs
