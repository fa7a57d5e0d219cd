"""Seeded synthetic inputs for the LoRA SwiGLU MLP.

This module draws the tensors that both the HIP path and the CPU checker
consume. It holds none of the method's arithmetic: it only draws random
numbers, rounds them to the storage dtype and packs 4-bit codes into bytes.

Workloads are synthetic stand-ins for the model shapes the pages name
(Llama-3-8B, Qwen2-7B and TinyLlama in "Unsloth支持哪些模型？主流LLM兼容性一览",
sections 2.1, 2.2 and 2.6; 32K packed rows from the same page's section 5).

Storage conventions (all row-major, nn.Linear ``[out, in]``):
  x, dy            [T, H]
  w_gate, w_up     [I, H]    (dense)  or packed int4 [I, H/2] u8 + fp16 scales [I, H/64]
  w_down           [H, I]    (dense)  or packed int4 [H, I/2] u8 + fp16 scales [H, I/64]
  a_gate, a_up     [r, H]    b_gate, b_up [I, r]
  a_down           [r, I]    b_down       [H, r]
bf16 tensors are numpy ``uint16`` arrays holding the raw bf16 bit patterns;
fp32 tensors are ``float32`` arrays.
"""
from __future__ import annotations

import dataclasses
from typing import Dict

import numpy as np

QBLOCK = 64  # elements per 4-bit quantisation block along the ``in`` axis


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tokens: int
    hidden: int
    inter: int
    rank: int
    alpha: float
    dtype: str            # "f32" or "bf16"
    wfmt: str = "dense"   # "dense" or "int4_b64"
    x_std: float = 1.0
    w_std: float = 0.02
    b_std: float = 0.01
    dy_std: float = 1.0
    qscale_std: float = 0.003
    seed: int = 0
    experts: int = 0      # grouped (MoE) workloads: number of experts
    top_k: int = 0        # ... and experts per token (routed rows = tokens * top_k)

    @property
    def scale(self) -> float:
        return self.alpha / self.rank

    @property
    def a_std(self) -> float:
        return 1.0 / self.rank

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    # tiny fp32 case the CPU checker finishes in well under a second
    "tiny_fp32": Workload("tiny_fp32", 256, 128, 344, 8, 16.0, "f32",
                          x_std=0.02, w_std=0.02),
    # Llama-3-8B MLP, batch 2 x seq 2048
    "llama3_8b": Workload("llama3_8b", 4096, 4096, 14336, 16, 16.0, "bf16"),
    # Qwen2-7B MLP, batch 4 x seq 2048
    "qwen2_7b": Workload("qwen2_7b", 8192, 3584, 18944, 64, 128.0, "bf16"),
    # TinyLlama-sized MLP over 32768 padding-free packed rows
    "tinyllama_long": Workload("tinyllama_long", 32768, 2048, 5632, 32, 32.0, "bf16"),
    # Llama-3-8B MLP with frozen weights held as 4-bit codes in 64-element blocks
    "llama3_8b_int4": Workload("llama3_8b_int4", 4096, 4096, 14336, 16, 16.0, "bf16",
                               wfmt="int4_b64"),
}


# ---------------------------------------------------------------------------
# storage conversions (no method arithmetic)

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 values of a stored tensor (bf16 bits or fp32)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Pack signed 4-bit codes ``q`` [out, in] (values in [-8, 7]) into bytes.

    Element k of a row goes to byte k//2: even k in the low nibble, odd k in
    the high nibble, each as a two's-complement nibble.
    """
    q = np.asarray(q, dtype=np.int16)
    assert q.ndim == 2 and q.shape[1] % 2 == 0
    assert q.min() >= -8 and q.max() <= 7
    nib = (q & 0xF).astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << np.uint8(4))).astype(np.uint8)


# ---------------------------------------------------------------------------
# draws

def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    raise ValueError(dtype)


def _draw_int4(rng: np.random.Generator, out: int, inn: int, qscale_std: float):
    if inn % QBLOCK:
        raise ValueError(f"int4 weights need in % {QBLOCK} == 0, got {inn}")
    q = rng.integers(-8, 8, size=(out, inn), dtype=np.int16)
    scales = np.abs(_normal(rng, (out, inn // QBLOCK), qscale_std)).astype(np.float16)
    return pack_int4(q), scales


def make_inputs(wl: Workload, seed: int | None = None, with_dy: bool = True) -> dict:
    """Draw one workload's tensors in a fixed order from ``default_rng(seed)``.

    Order: x, W_gate, W_up, W_down, A_gate, B_gate, A_up, B_up, A_down,
    B_down, dY. For int4 weights each W draw is its codes then its scales.
    """
    seed = wl.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    T, H, I, r, dt = wl.tokens, wl.hidden, wl.inter, wl.rank, wl.dtype
    if wl.wfmt not in ("dense", "int4_b64"):
        raise ValueError(wl.wfmt)
    if wl.wfmt == "int4_b64" and dt != "bf16":
        raise ValueError("int4 weights are defined for the bf16 workload only")
    out = {"x": _store(_normal(rng, (T, H), wl.x_std), dt)}
    for name, (o, i) in (("w_gate", (I, H)), ("w_up", (I, H)), ("w_down", (H, I))):
        if wl.wfmt == "dense":
            out[name] = _store(_normal(rng, (o, i), wl.w_std), dt)
        else:
            q, s = _draw_int4(rng, o, i, wl.qscale_std)
            out[name] = q
            out[name + "_scales"] = s
    out["a_gate"] = _store(_normal(rng, (r, H), wl.a_std), dt)
    out["b_gate"] = _store(_normal(rng, (I, r), wl.b_std), dt)
    out["a_up"] = _store(_normal(rng, (r, H), wl.a_std), dt)
    out["b_up"] = _store(_normal(rng, (I, r), wl.b_std), dt)
    out["a_down"] = _store(_normal(rng, (r, I), wl.a_std), dt)
    out["b_down"] = _store(_normal(rng, (H, r), wl.b_std), dt)
    if with_dy:
        out["dy"] = _store(_normal(rng, (T, H), wl.dy_std), dt)
    return out


# RMSNorm in front of the MLP (the same workloads with the norm switched on):
# eps as the pages' model table gives it for one family (1e-5, which is also
# Llama-3's), the weight drawn from its own seeded stream so the MLP's draws
# are unchanged.
NORM_EPS = 1e-5


def make_norm_gamma(wl: Workload, seed: int | None = None) -> np.ndarray:
    """RMSNorm weight [H] in the workload's storage, uniform in [0.5, 1.5)."""
    seed = wl.seed if seed is None else seed
    rng = np.random.default_rng([seed, 7])
    return _store((0.5 + rng.random(wl.hidden, dtype=np.float32)).astype(np.float32), wl.dtype)


# Fused LoRA linear workloads: ``hidden`` is the input width, ``inter`` the
# output width (the single projections of the same models; same draws).
LINEAR_WORKLOADS: Dict[str, Workload] = {
    "linear_tiny_fp32": Workload("linear_tiny_fp32", 256, 128, 344, 8, 16.0, "f32", x_std=0.02, w_std=0.02),
    # Llama-3-8B attention q / o projection (4096 -> 4096), batch 2 x seq 2048
    "linear_llama3_qo": Workload("linear_llama3_qo", 4096, 4096, 4096, 16, 16.0, "bf16"),
    # Llama-3-8B k / v projection with 8 key-value heads (4096 -> 1024)
    "linear_llama3_kv": Workload("linear_llama3_kv", 4096, 4096, 1024, 16, 16.0, "bf16"),
    # one Llama-3-8B MLP projection (4096 -> 14336) as a plain LoRA linear
    "linear_llama3_up": Workload("linear_llama3_up", 4096, 4096, 14336, 16, 16.0, "bf16"),
    "linear_llama3_up_int4": Workload("linear_llama3_up_int4", 4096, 4096, 14336, 16, 16.0, "bf16",
                                      wfmt="int4_b64"),
}


def make_linear_inputs(wl: Workload, seed: int | None = None, with_dy: bool = True) -> dict:
    """Draw one linear workload's tensors in a fixed order from
    ``default_rng(seed)``: x [T, in], W [out, in] (int4: codes then scales),
    A [r, in], B [out, r], dY [T, out]."""
    seed = wl.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    T, n_in, n_out, r, dt = wl.tokens, wl.hidden, wl.inter, wl.rank, wl.dtype
    if wl.wfmt not in ("dense", "int4_b64"):
        raise ValueError(wl.wfmt)
    if wl.wfmt == "int4_b64" and dt != "bf16":
        raise ValueError("int4 weights are defined for bf16 only")
    out = {"x": _store(_normal(rng, (T, n_in), wl.x_std), dt)}
    if wl.wfmt == "dense":
        out["w"] = _store(_normal(rng, (n_out, n_in), wl.w_std), dt)
    else:
        out["w"], out["w_scales"] = _draw_int4(rng, n_out, n_in, wl.qscale_std)
    out["a"] = _store(_normal(rng, (r, n_in), wl.a_std), dt)
    out["b"] = _store(_normal(rng, (n_out, r), wl.b_std), dt)
    if with_dy:
        out["dy"] = _store(_normal(rng, (T, n_out), wl.dy_std), dt)
    return out


# Grouped (MoE) workloads: ``tokens`` tokens each routed to ``top_k`` of
# ``experts`` experts, every expert a LoRA SwiGLU MLP of width ``inter``.
# The shapes are the public MoE MLP shapes of model families the pages name
# (Mistral's 8-expert top-2 Mixtral-8x7B; Qwen's 128-expert top-8 30B-A3B).
MOE_WORKLOADS: Dict[str, Workload] = {
    "moe_tiny_fp32": Workload("moe_tiny_fp32", 96, 128, 344, 8, 16.0, "f32", x_std=0.02, w_std=0.02,
                              experts=4, top_k=2),
    "moe_mixtral": Workload("moe_mixtral", 4096, 4096, 14336, 16, 16.0, "bf16", experts=8, top_k=2),
    "moe_qwen3": Workload("moe_qwen3", 4096, 2048, 768, 16, 16.0, "bf16", experts=128, top_k=8),
}


def route_counts(rng: np.random.Generator, tokens: int, experts: int, top_k: int):
    """Synthetic router: logits N(0, 1) plus a per-expert popularity bias
    N(0, 0.5); each token takes its top_k experts. Returns, per routed row in
    expert-grouped order, the token it came from, and the expert offsets."""
    bias = _normal(rng, (experts,), 0.5)
    logits = _normal(rng, (tokens, experts), 1.0) + bias[None, :]
    choice = np.argsort(-logits, axis=1, kind="stable")[:, :top_k]     # [tokens, top_k]
    expert = choice.reshape(-1)
    token = np.repeat(np.arange(tokens), top_k)
    order = np.argsort(expert, kind="stable")
    counts = np.bincount(expert, minlength=experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return token[order], offsets


def make_moe_inputs(wl: Workload, seed: int | None = None, with_dy: bool = True):
    """(inputs, offsets) of a grouped workload, drawn in a fixed order from
    ``default_rng(seed)``: the router, x [tokens, H] (gathered into the routed
    rows), the stacked weights W_gate, W_up [E, I, H], W_down [E, H, I] (int4:
    codes then scales per expert), A_gate, B_gate, A_up, B_up, A_down, B_down
    stacked [E, ...], and dY [rows, H]."""
    seed = wl.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    E, H, I, r, dt = wl.experts, wl.hidden, wl.inter, wl.rank, wl.dtype
    if E < 1 or wl.top_k < 1 or wl.top_k > E:
        raise ValueError("a grouped workload needs 1 <= top_k <= experts")
    tok, offsets = route_counts(rng, wl.tokens, E, wl.top_k)
    x = _normal(rng, (wl.tokens, H), wl.x_std)
    out = {"x": _store(np.ascontiguousarray(x[tok]), dt)}
    del x
    for name, (o, i) in (("w_gate", (I, H)), ("w_up", (I, H)), ("w_down", (H, I))):
        if wl.wfmt == "dense":
            out[name] = _store(_normal(rng, (E, o, i), wl.w_std), dt)
        else:
            qs = [_draw_int4(rng, o, i, wl.qscale_std) for _ in range(E)]
            out[name] = np.stack([q for q, _ in qs])
            out[name + "_scales"] = np.stack([s for _, s in qs])
    out["a_gate"] = _store(_normal(rng, (E, r, H), wl.a_std), dt)
    out["b_gate"] = _store(_normal(rng, (E, I, r), wl.b_std), dt)
    out["a_up"] = _store(_normal(rng, (E, r, H), wl.a_std), dt)
    out["b_up"] = _store(_normal(rng, (E, I, r), wl.b_std), dt)
    out["a_down"] = _store(_normal(rng, (E, r, I), wl.a_std), dt)
    out["b_down"] = _store(_normal(rng, (E, H, r), wl.b_std), dt)
    if with_dy:
        out["dy"] = _store(_normal(rng, (int(offsets[-1]), H), wl.dy_std), dt)
    return out, offsets


def draw_int4_codes(seed: int, out: int, inn: int, qscale_std: float = 0.003):
    """Packed codes and fp16 scales for one weight matrix (dequant tests)."""
    rng = np.random.default_rng(seed)
    return _draw_int4(rng, out, inn, qscale_std)
