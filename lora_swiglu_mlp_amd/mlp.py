"""Torch-side plumbing around the C ABI: device buffers and one call per pass.

PyTorch provides device memory and the stream; every step of the forward and
backward runs in the HIP library (:mod:`lora_swiglu_mlp_amd.abi`).
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import abi

WEIGHTS = ("w_gate", "w_up", "w_down")
ADAPTERS = ("a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")
GRADS = ("dx", "da_gate", "db_gate", "da_up", "db_up", "da_down", "db_down")


def tensor_from_storage(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Device tensor from a stored numpy array (bf16 bits, fp32, u8 codes, fp16 scales)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16 and dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device)


class LoraMLP:
    """One LoRA SwiGLU MLP (frozen W, trainable A/B) bound to device tensors.

    With ``norm_eps`` set, an RMSNorm with the frozen weight ``tensors["gamma"]``
    runs in front of the MLP (the library's norm entry points)."""

    def __init__(self, tensors: Dict[str, torch.Tensor], tokens: int, hidden: int, inter: int,
                 rank: int, scale: float, dtype: str = "bf16", wfmt: str = "dense", flags: int = 0,
                 norm_eps: Optional[float] = None):
        self.t = tensors
        self.norm_eps = norm_eps
        if norm_eps is not None:
            flags |= abi.LMLP_RMSNORM
        self.dtype, self.wfmt = dtype, wfmt
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.hidden, self.inter, self.rank, self.scale, self.flags = hidden, inter, rank, scale, flags
        self.set_tokens(tokens)
        self._ws: Optional[torch.Tensor] = None

    def set_tokens(self, tokens: int):
        self.tokens = tokens
        self.dims = abi.make_dims(tokens, self.hidden, self.inter, self.rank, self.scale,
                                  self.dtype, self.wfmt, self.flags)

    def _scale_ptr(self, name):
        return self.t.get(name + "_scales") if self.wfmt == "int4_b64" else None

    def workspace(self, backward: bool) -> torch.Tensor:
        need = max(abi.lora_mlp_workspace_bytes(self.dims, False),
                   abi.lora_mlp_workspace_bytes(self.dims, True))
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.t["a_gate"].device)
        return self._ws

    def new_saved(self) -> torch.Tensor:
        n = abi.lora_mlp_saved_bytes(self.dims)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.t["a_gate"].device)

    def forward(self, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                saved: Optional[torch.Tensor] = None, stream=None):
        t = self.t
        if y is None:
            y = torch.empty((self.tokens, self.hidden), dtype=self.tdtype, device=x.device)
        if saved is None:
            saved = self.new_saved()
        w = (t["w_gate"], self._scale_ptr("w_gate"), t["w_up"], self._scale_ptr("w_up"), t["w_down"],
             self._scale_ptr("w_down"), t["a_gate"], t["b_gate"], t["a_up"], t["b_up"], t["a_down"],
             t["b_down"])
        if self.norm_eps is None:
            abi.lora_mlp_forward(self.dims, x, *w, y, saved, self.workspace(False), stream=stream)
        else:
            abi.lora_mlp_norm_forward(self.dims, self.norm_eps, x, t["gamma"], *w, y, saved,
                                      self.workspace(False), stream=stream)
        return y, saved

    def new_grads(self, device) -> Dict[str, torch.Tensor]:
        T, H, I, r = self.tokens, self.hidden, self.inter, self.rank
        shapes = {"dx": (T, H), "da_gate": (r, H), "db_gate": (I, r), "da_up": (r, H),
                  "db_up": (I, r), "da_down": (r, I), "db_down": (H, r)}
        return {k: torch.empty(s, dtype=self.tdtype, device=device) for k, s in shapes.items()}

    def backward(self, dy: torch.Tensor, x: torch.Tensor, saved: torch.Tensor,
                 grads: Optional[Dict[str, torch.Tensor]] = None, stream=None):
        t = self.t
        if grads is None:
            grads = self.new_grads(dy.device)
        g = grads
        w = (t["w_gate"], self._scale_ptr("w_gate"), t["w_up"], self._scale_ptr("w_up"), t["w_down"],
             self._scale_ptr("w_down"), t["a_gate"], t["b_gate"], t["a_up"], t["b_up"], t["a_down"],
             t["b_down"])
        outs = (g["dx"], g["da_gate"], g["db_gate"], g["da_up"], g["db_up"], g["da_down"], g["db_down"])
        if self.norm_eps is None:
            abi.lora_mlp_backward(self.dims, dy, x, *w, saved, *outs, self.workspace(True), stream=stream)
        else:
            abi.lora_mlp_norm_backward(self.dims, dy, x, t["gamma"], *w, saved, *outs, self.workspace(True),
                                       stream=stream)
        return grads


def from_inputs(inp: Dict[str, np.ndarray], wl, device="cuda", flags: int = 0,
                norm_eps: Optional[float] = None):
    """LoraMLP plus device x, dy from a generated workload (see inputs.make_inputs;
    with ``norm_eps``, ``inp["gamma"]`` from inputs.make_norm_gamma)."""
    tens = {k: tensor_from_storage(v, wl.dtype, device) for k, v in inp.items()}
    m = LoraMLP(tens, wl.tokens, wl.hidden, wl.inter, wl.rank, wl.scale, wl.dtype, wl.wfmt, flags, norm_eps)
    return m, tens["x"], tens.get("dy")


class LoraMoE:
    """E LoRA SwiGLU MLP experts (stacked tensors [E, ...]) over token rows
    grouped by expert: rows offsets[e] .. offsets[e+1]-1 belong to expert e."""

    def __init__(self, tensors: Dict[str, torch.Tensor], offsets, hidden: int, inter: int, rank: int,
                 scale: float, dtype: str = "bf16", wfmt: str = "dense", flags: int = 0):
        self.t = tensors
        self.offsets = [int(v) for v in offsets]
        self.experts = len(self.offsets) - 1
        self.dtype, self.wfmt = dtype, wfmt
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.rows, self.hidden, self.inter, self.rank = self.offsets[-1], hidden, inter, rank
        self.dims = abi.make_dims(self.rows, hidden, inter, rank, scale, dtype, wfmt, flags)
        self._ws: Optional[torch.Tensor] = None

    def _scale_ptr(self, name):
        return self.t.get(name + "_scales") if self.wfmt == "int4_b64" else None

    def _w(self):
        t = self.t
        return (t["w_gate"], self._scale_ptr("w_gate"), t["w_up"], self._scale_ptr("w_up"), t["w_down"],
                self._scale_ptr("w_down"), t["a_gate"], t["b_gate"], t["a_up"], t["b_up"], t["a_down"],
                t["b_down"])

    def workspace(self) -> torch.Tensor:
        need = max(abi.lora_moe_workspace_bytes(self.dims, self.offsets, False),
                   abi.lora_moe_workspace_bytes(self.dims, self.offsets, True))
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.t["a_gate"].device)
        return self._ws

    def new_saved(self) -> torch.Tensor:
        n = abi.lora_moe_saved_bytes(self.dims, self.offsets)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.t["a_gate"].device)

    def forward(self, x, y=None, saved=None, stream=None):
        if y is None:
            y = torch.empty((self.rows, self.hidden), dtype=self.tdtype, device=x.device)
        if saved is None:
            saved = self.new_saved()
        abi.lora_moe_forward(self.dims, self.offsets, x, *self._w(), y, saved, self.workspace(), stream=stream)
        return y, saved

    def new_grads(self, device) -> Dict[str, torch.Tensor]:
        E, T, H, I, r = self.experts, self.rows, self.hidden, self.inter, self.rank
        shapes = {"dx": (T, H), "da_gate": (E, r, H), "db_gate": (E, I, r), "da_up": (E, r, H),
                  "db_up": (E, I, r), "da_down": (E, r, I), "db_down": (E, H, r)}
        return {k: torch.empty(s, dtype=self.tdtype, device=device) for k, s in shapes.items()}

    def backward(self, dy, x, saved, grads=None, stream=None):
        g = self.new_grads(dy.device) if grads is None else grads
        abi.lora_moe_backward(self.dims, self.offsets, dy, x, *self._w(), saved, g["dx"], g["da_gate"],
                              g["db_gate"], g["da_up"], g["db_up"], g["da_down"], g["db_down"], self.workspace(),
                              stream=stream)
        return g


def moe_from_inputs(inp: Dict[str, np.ndarray], offsets, wl, device="cuda", flags: int = 0):
    """LoraMoE plus device x, dy from inputs.make_moe_inputs."""
    tens = {k: tensor_from_storage(v, wl.dtype, device) for k, v in inp.items()}
    m = LoraMoE(tens, offsets, wl.hidden, wl.inter, wl.rank, wl.scale, wl.dtype, wl.wfmt, flags)
    return m, tens["x"], tens.get("dy")


class LoraLinear:
    """One fused LoRA linear y = x W^T + s (x A^T) B^T (frozen W, trainable A/B)
    bound to device tensors ``w`` [out, in] (or 4-bit codes + ``w_scales``),
    ``a`` [r, in], ``b`` [out, r]."""

    def __init__(self, tensors: Dict[str, torch.Tensor], tokens: int, inn: int, out: int, rank: int,
                 scale: float, dtype: str = "bf16", wfmt: str = "dense", flags: int = 0):
        self.t = tensors
        self.dtype, self.wfmt = dtype, wfmt
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.inn, self.out, self.rank, self.scale, self.flags = inn, out, rank, scale, flags
        self.tokens = tokens
        self.dims = abi.make_dims(tokens, inn, out, rank, scale, dtype, wfmt, flags)
        self._ws: Optional[torch.Tensor] = None

    def workspace(self) -> torch.Tensor:
        need = max(abi.lora_linear_workspace_bytes(self.dims, False),
                   abi.lora_linear_workspace_bytes(self.dims, True))
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.t["a"].device)
        return self._ws

    def new_saved(self) -> torch.Tensor:
        n = abi.lora_linear_saved_bytes(self.dims)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.t["a"].device)

    def forward(self, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                saved: Optional[torch.Tensor] = None, stream=None):
        t = self.t
        if y is None:
            y = torch.empty((self.tokens, self.out), dtype=self.tdtype, device=x.device)
        if saved is None:
            saved = self.new_saved()
        abi.lora_linear_forward(self.dims, x, t["w"], t.get("w_scales") if self.wfmt == "int4_b64" else None,
                                t["a"], t["b"], y, saved, self.workspace(), stream=stream)
        return y, saved

    def new_grads(self, device) -> Dict[str, torch.Tensor]:
        T, r = self.tokens, self.rank
        shapes = {"dx": (T, self.inn), "da": (r, self.inn), "db": (self.out, r)}
        return {k: torch.empty(s, dtype=self.tdtype, device=device) for k, s in shapes.items()}

    def backward(self, dy: torch.Tensor, x: torch.Tensor, saved: torch.Tensor,
                 grads: Optional[Dict[str, torch.Tensor]] = None, stream=None):
        t = self.t
        g = grads if grads is not None else self.new_grads(dy.device)
        abi.lora_linear_backward(self.dims, dy, x, t["w"], t.get("w_scales") if self.wfmt == "int4_b64" else None,
                                 t["a"], t["b"], saved, g["dx"], g["da"], g["db"], self.workspace(),
                                 stream=stream)
        return g


def linear_from_inputs(inp: Dict[str, np.ndarray], wl, device="cuda", flags: int = 0):
    """LoraLinear plus device x, dy from a generated linear workload
    (inputs.make_linear_inputs; ``hidden`` = in, ``inter`` = out)."""
    tens = {k: tensor_from_storage(v, wl.dtype, device) for k, v in inp.items()}
    m = LoraLinear(tens, wl.tokens, wl.hidden, wl.inter, wl.rank, wl.scale, wl.dtype, wl.wfmt, flags)
    return m, tens["x"], tens.get("dy")
