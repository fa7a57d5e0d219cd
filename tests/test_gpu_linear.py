"""GPU parity of the fused LoRA linear (through the C ABI) against its fp64
oracle: ragged shapes over several tiles, every rank padding case, the
smallest sizes, an empty batch, both dtypes, both 4-bit modes, the Llama-3-8B
projection sizes in full. Tolerance as for the MLP: max|gpu-ref| / max|ref|
<= 1e-4 (fp32), <= 2e-2 (bf16) per output tensor."""
import numpy as np
import pytest

from oracle import lora_linear_oracle as L
from lora_swiglu_mlp_amd import abi
from lora_swiglu_mlp_amd import inputs as I
from lmlp_testutil import LIN_KEYS, TOL, compare, oracle_inputs, run_hip_linear

pytestmark = pytest.mark.gpu

CASES = {
    # name: (T, in, out, r, alpha, dtype, wfmt)
    "tiny_fp32": (256, 128, 344, 8, 16.0, "f32", "dense"),
    "f32_ragged": (100, 36, 52, 3, 6.0, "f32", "dense"),
    "bf16_ragged": (300, 320, 600, 16, 32.0, "bf16", "dense"),
    "bf16_multi": (520, 512, 1088, 16, 16.0, "bf16", "dense"),
    "bf16_narrow_out": (777, 1024, 136, 8, 16.0, "bf16", "dense"),
    "bf16_rank1": (64, 128, 256, 1, 2.0, "bf16", "dense"),
    "bf16_rank64": (384, 256, 512, 64, 128.0, "bf16", "dense"),
    "bf16_rank256": (128, 256, 256, 256, 256.0, "bf16", "dense"),
    "bf16_one_token": (1, 64, 128, 8, 16.0, "bf16", "dense"),
    "bf16_min_width": (40, 8, 8, 2, 4.0, "bf16", "dense"),
    # few output tiles: the forward product splits K (8 splits with a K tail
    # in the last; 3 even splits)
    "bf16_splitk8": (300, 4136, 264, 16, 32.0, "bf16", "dense"),
    "bf16_splitk3": (2000, 1536, 520, 8, 16.0, "bf16", "dense"),
    "int4_small": (192, 256, 384, 16, 16.0, "bf16", "int4_b64"),
    "int4_ragged": (300, 192, 320, 12, 24.0, "bf16", "int4_b64"),
}


def workload(name):
    T, n_in, n_out, r, alpha, dt, wf = CASES[name]
    base = I.LINEAR_WORKLOADS["linear_tiny_fp32" if dt == "f32" else "linear_llama3_qo"]
    return base.replace(name=name, tokens=T, hidden=n_in, inter=n_out, rank=r, alpha=alpha, dtype=dt, wfmt=wf)


def _oracle(inp, wl):
    return L.forward_backward(oracle_inputs(inp, wl), wl.scale, row_chunk=2048)


@pytest.mark.parametrize("name", list(CASES))
def test_linear_parity(name):
    wl = workload(name)
    print(f"[case] linear {name} {CASES[name]}", flush=True)
    inp = I.make_linear_inputs(wl)
    got, _ = run_hip_linear(inp, wl)
    compare(got, _oracle(inp, wl), TOL[wl.dtype], "linear " + name)
    assert np.linalg.norm(got["da"]) > 0 and np.linalg.norm(got["db"]) > 0
    assert all(np.isfinite(v).all() for v in got.values())


@pytest.mark.parametrize("name", ["bf16_splitk8", "bf16_splitk3", "bf16_narrow_out"])
def test_linear_split_k_forward(name):
    """Products whose output tiles do not fill the GPU split K and sum fp32
    partials in split order: the split path runs (its sum launch is
    recorded), matches the oracle, and repeats bit for bit."""
    wl = workload(name)
    inp = I.make_linear_inputs(wl)
    print(f"[case] linear split-K {name} {CASES[name]}", flush=True)
    abi.lora_mlp_profile_begin()
    a, _ = run_hip_linear(inp, wl)
    names = [n for n, _ in abi.lora_mlp_profile_end()]
    assert "sum(y)" in names, names
    b, _ = run_hip_linear(inp, wl)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    compare(a, _oracle(inp, wl), TOL[wl.dtype], "linear split-K " + name)


@pytest.mark.parametrize("name", ["int4_small", "int4_ragged"])
def test_linear_int4_modes_bitwise_equal(name):
    """Decoding inside the products' staging (the default) gives the same
    weights as the bf16 copy, in the same k order."""
    wl = workload(name)
    inp = I.make_linear_inputs(wl)
    a, _ = run_hip_linear(inp, wl)
    b, _ = run_hip_linear(inp, wl, flags=abi.LMLP_INT4_BF16_COPIES)
    for k in LIN_KEYS:
        assert np.array_equal(a[k], b[k]), k
    compare(b, _oracle(inp, wl), TOL[wl.dtype], "linear " + name + " copies")


def test_linear_empty_batch_gives_zero_adapter_gradients():
    import torch
    from lora_swiglu_mlp_amd import mlp
    wl = workload("bf16_rank1").replace(tokens=0)
    inp = I.make_linear_inputs(wl)
    m, x, dy = mlp.linear_from_inputs(inp, wl)
    y, saved = m.forward(x)
    g = m.new_grads(x.device)
    for v in g.values():
        v.fill_(7.0)
    m.backward(dy, x, saved, g)
    torch.cuda.synchronize()
    assert y.numel() == 0 and torch.all(g["da"] == 0) and torch.all(g["db"] == 0)


def test_linear_deterministic_b_zero_and_dy_linearity():
    wl = workload("bf16_ragged")
    inp = I.make_linear_inputs(wl)
    a, _ = run_hip_linear(inp, wl)
    b, _ = run_hip_linear(inp, wl)
    for k in LIN_KEYS:
        assert np.array_equal(a[k], b[k]), k
    inp2 = dict(inp, dy=I.f32_to_bf16_bits(I.bf16_bits_to_f32(inp["dy"]) * 2.0))
    c, _ = run_hip_linear(inp2, wl)
    assert np.array_equal(c["y"], a["y"])
    for k in ("dx", "da", "db"):
        assert np.array_equal(c[k], 2.0 * a[k]), k
    z = dict(inp, b=np.zeros_like(inp["b"]))
    p, _ = run_hip_linear(z, wl)
    q, _ = run_hip_linear(z, wl.replace(alpha=0.0))
    assert np.array_equal(p["y"], q["y"]) and np.all(p["da"] == 0)


@pytest.mark.parametrize("name", ["linear_llama3_qo", "linear_llama3_kv", "linear_llama3_up_int4"])
def test_linear_fullsize_parity(name):
    """The Llama-3-8B projection sizes, in the bench's launch configuration,
    every element against the chunked oracle."""
    wl = I.LINEAR_WORKLOADS[name]
    print(f"[case] {name} T={wl.tokens} in={wl.hidden} out={wl.inter} r={wl.rank}", flush=True)
    inp = I.make_linear_inputs(wl)
    got, _ = run_hip_linear(inp, wl)
    compare(got, _oracle(inp, wl), TOL[wl.dtype], name)
