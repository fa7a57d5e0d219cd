"""The allocation-free fused LoRA linear forward (lora_linear_forward_noalloc,
workspace in the library's own device array) against lora_linear_forward
with a caller workspace: the same kernels in the same order, so y and every
byte of `saved` must agree bit for bit. Two calls in a row, the second with
fewer tokens and other widths (the array keeps the first call's contents),
then the larger shape again, and a 4-bit case with the in-kernel decode.
y is also checked against the fp64 oracle (max|gpu-ref| / max|ref| <= 2e-2
for bf16)."""
import numpy as np
import pytest

from oracle import lora_linear_oracle as L
from lora_swiglu_mlp_amd import abi, mlp
from lora_swiglu_mlp_amd import inputs as I
from lmlp_testutil import TOL, oracle_inputs, relerr

pytestmark = pytest.mark.gpu


def _case(T, n_in, n_out, r, alpha, wfmt="dense", flags=0):
    import torch
    base = I.LINEAR_WORKLOADS["linear_llama3_qo"]
    wl = base.replace(name="noalloc", tokens=T, hidden=n_in, inter=n_out, rank=r, alpha=alpha, wfmt=wfmt)
    print(f"[case] noalloc T={T} in={n_in} out={n_out} r={r} {wfmt} flags={flags}", flush=True)
    inp = I.make_linear_inputs(wl)
    m, x, _ = mlp.linear_from_inputs(inp, wl, "cuda", flags)
    ws = abi.lora_linear_workspace_bytes(m.dims, False)
    assert 0 < ws <= abi.LMLP_NOALLOC_SCRATCH_BYTES
    y0 = torch.empty((T, n_out), dtype=m.tdtype, device="cuda")
    y1 = torch.full_like(y0, float("nan"))
    s0 = torch.zeros(abi.lora_linear_saved_bytes(m.dims), dtype=torch.uint8, device="cuda")
    s1 = torch.zeros_like(s0)
    m.forward(x, y0, s0)
    t = m.t
    abi.lora_linear_forward_noalloc(m.dims, x, t["w"], t.get("w_scales") if wfmt == "int4_b64" else None,
                                    t["a"], t["b"], y1, s1)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    assert torch.equal(s0, s1)
    ref = L.forward_backward(oracle_inputs(inp, wl), wl.scale, row_chunk=2048)["y"]
    err = relerr(y1.float().cpu().numpy().astype(np.float64), ref)
    print(f"[parity] noalloc y={err:.2e}", flush=True)
    assert err <= TOL["bf16"]


def test_noalloc_linear_forward_matches_the_workspace_entry_point():
    _case(1000, 1024, 1536, 16, 16.0)   # several tiles, ragged T
    _case(77, 320, 264, 8, 16.0)        # smaller: the scratch holds the previous call's bytes
    _case(1000, 1024, 1536, 16, 16.0)   # the first shape again after the small one
    _case(300, 256, 384, 12, 24.0, "int4_b64", abi.LMLP_INT4_INKERNEL)
