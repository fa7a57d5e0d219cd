"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Shapes span several 256x256 tiles with ragged M, N and K tails, every rank
padding case, the smallest legal sizes, an empty token batch, both dtypes and
the 4-bit weight path. Tolerance per output tensor: max|gpu-ref| / max|ref|
<= 1e-4 (fp32) and <= 2e-2 (bf16); the 4-bit decode is compared bit for bit.
"""
import os

import numpy as np
import pytest

import oracle
from lora_swiglu_mlp_amd import abi
from lora_swiglu_mlp_amd import inputs as I
from lmlp_testutil import OUT_KEYS, TOL, compare, oracle_inputs, run_hip

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

CASES = {
    # name: (T, H, I, r, alpha, dtype, wfmt)
    "tiny_fp32": (256, 128, 344, 8, 16.0, "f32", "dense"),        # the tiny fp32 workload itself
    "f32_ragged": (100, 36, 52, 3, 6.0, "f32", "dense"),
    "bf16_ragged": (300, 320, 600, 16, 32.0, "bf16", "dense"),    # ragged M, N and K tails
    "bf16_multi": (520, 512, 1088, 16, 16.0, "bf16", "dense"),    # 3 x 9 gate/up tiles, 17 K tiles
    "bf16_rank1": (64, 128, 256, 1, 2.0, "bf16", "dense"),
    "bf16_rank8": (96, 64, 136, 8, 16.0, "bf16", "dense"),
    "bf16_rank64": (384, 256, 512, 64, 128.0, "bf16", "dense"),
    "bf16_rank256": (128, 256, 256, 256, 256.0, "bf16", "dense"),  # largest supported rank
    "bf16_one_token": (1, 64, 128, 8, 16.0, "bf16", "dense"),
    "bf16_min_width": (40, 8, 8, 2, 4.0, "bf16", "dense"),
    "int4_small": (192, 256, 384, 16, 16.0, "bf16", "int4_b64"),
    "int4_ragged": (300, 192, 320, 12, 24.0, "bf16", "int4_b64"),
    # dZ has 2 x 129 tiles of 256 columns: on 256 CUs the last column goes to
    # the second launch of 128-wide tiles (ragged: 232 columns), rank 16 with
    # the fused rank products and rank 32 without
    "bf16_dz_tail": (512, 64, 33000, 16, 16.0, "bf16", "dense"),
    "bf16_dz_tail_r32": (512, 64, 33000, 32, 32.0, "bf16", "dense"),
}


def workload(name):
    T, H, Iw, r, alpha, dt, wf = CASES[name]
    base = I.WORKLOADS["tiny_fp32"] if dt == "f32" else I.WORKLOADS["llama3_8b"]
    return base.replace(name=name, tokens=T, hidden=H, inter=Iw, rank=r, alpha=alpha, dtype=dt,
                        wfmt=wf)


@pytest.mark.parametrize("name", list(CASES))
def test_parity_against_oracle(name):
    wl = workload(name)
    print(f"[case] {name} {CASES[name]}", flush=True)
    inp = I.make_inputs(wl)
    got, _ = run_hip(inp, wl)
    ref = oracle.forward_backward(oracle_inputs(inp, wl), wl.scale)
    errs = compare(got, ref, TOL[wl.dtype], name)
    for k in ("da_gate", "db_gate", "da_up", "db_up", "da_down", "db_down"):
        assert np.linalg.norm(got[k]) > 0, k  # gradients flow into every adapter factor
    assert all(np.isfinite(v).all() for v in got.values())
    assert errs


def _random_shapes(n, seed=20261203):
    """Seeded random shapes: ragged M, N and K at every tile size the kernels
    use, ranks 1..64, both dtypes (fp32 smaller)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        f32 = i % 4 == 3
        T = int(rng.integers(1, 700 if not f32 else 200))
        H = 8 * int(rng.integers(1, 90 if not f32 else 20))
        Iw = 8 * int(rng.integers(1, 150 if not f32 else 30))
        r = int(rng.choice([1, 3, 8, 13, 16, 16, 24, 32, 48, 64]))
        out.append((f"rand{i}", T, H, Iw, r, float(2 * r), "f32" if f32 else "bf16"))
    return out


@pytest.mark.parametrize("case", _random_shapes(12), ids=lambda c: c[0])
def test_parity_random_shapes(case):
    name, T, H, Iw, r, alpha, dt = case
    base = I.WORKLOADS["tiny_fp32"] if dt == "f32" else I.WORKLOADS["llama3_8b"]
    wl = base.replace(name=name, tokens=T, hidden=H, inter=Iw, rank=r, alpha=alpha, dtype=dt, wfmt="dense")
    print(f"[case] {case}", flush=True)
    inp = I.make_inputs(wl)
    got, _ = run_hip(inp, wl)
    ref = oracle.forward_backward(oracle_inputs(inp, wl), wl.scale)
    compare(got, ref, TOL[dt], name)


def test_dz_tail_launch_taken():
    """On a 256-CU device the bf16_dz_tail shape runs dZ as two launches (256-
    and 128-wide tiles); the parity cases above then cover the second one."""
    import torch
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the split point depends on the CU count")
    wl = workload("bf16_dz_tail")
    inp = I.make_inputs(wl)
    abi.lora_mlp_profile_begin()
    run_hip(inp, wl)
    names = [n for n, _ in abi.lora_mlp_profile_end()]
    assert names.count("gemm(dZ)") == 1 and names.count("gemm(dZ tail)") == 1, names


def test_empty_token_batch():
    import torch
    from lora_swiglu_mlp_amd import mlp
    wl = workload("bf16_rank8").replace(tokens=0)
    inp = I.make_inputs(wl)
    m, x, dy = mlp.from_inputs(inp, wl)
    y, saved = m.forward(x)
    grads = m.new_grads(x.device)
    for g in grads.values():
        g.fill_(7.0)
    m.backward(dy, x, saved, grads)
    torch.cuda.synchronize()
    assert y.numel() == 0
    for k, g in grads.items():
        if k != "dx":
            assert torch.all(g == 0), k


def test_b_zero_equals_scale_zero_and_zero_da():
    import torch
    wl = workload("bf16_ragged")
    inp = I.make_inputs(wl)
    for k in ("b_gate", "b_up", "b_down"):
        inp[k] = np.zeros_like(inp[k])
    a, _ = run_hip(inp, wl)
    b, _ = run_hip(inp, wl.replace(alpha=0.0))
    assert np.array_equal(a["y"], b["y"])  # the adapter K-steps add exact zeros
    for k in ("da_gate", "da_up", "da_down"):
        assert np.all(a[k] == 0), k
    ref = oracle.forward_backward(oracle_inputs(inp, wl), wl.scale)
    compare(a, ref, TOL["bf16"], "B=0")
    torch.cuda.synchronize()


def test_bitwise_deterministic_and_consume_flag():
    from lora_swiglu_mlp_amd import abi
    wl = workload("bf16_multi")
    inp = I.make_inputs(wl)
    a, _ = run_hip(inp, wl)
    b, _ = run_hip(inp, wl)
    c, _ = run_hip(inp, wl, flags=abi.LMLP_CONSUME_SAVED)
    for k in OUT_KEYS:
        assert np.array_equal(a[k], b[k]), k
        assert np.array_equal(a[k], c[k]), k


def test_backward_twice_without_consume():
    import torch
    from lora_swiglu_mlp_amd import mlp
    wl = workload("bf16_ragged")
    inp = I.make_inputs(wl)
    m, x, dy = mlp.from_inputs(inp, wl)
    y, saved = m.forward(x)
    g1 = {k: v.clone() for k, v in m.backward(dy, x, saved).items()}
    g2 = m.backward(dy, x, saved)
    torch.cuda.synchronize()
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_dy_linearity_bitwise():
    wl = workload("bf16_ragged")
    inp = I.make_inputs(wl)
    a, _ = run_hip(inp, wl)
    inp2 = dict(inp)
    inp2["dy"] = I.f32_to_bf16_bits(I.bf16_bits_to_f32(inp["dy"]) * 2.0)
    b, _ = run_hip(inp2, wl)
    assert np.array_equal(a["y"], b["y"])
    for k in OUT_KEYS[1:]:
        assert np.array_equal(b[k], 2.0 * a[k]), k


def _dequant_gpu(packed, scales, out, inn):
    import torch
    from lora_swiglu_mlp_amd import abi
    p = torch.from_numpy(packed).cuda()
    s = torch.from_numpy(scales).cuda()
    w = torch.empty((out, inn), dtype=torch.bfloat16, device="cuda")
    abi.lora_mlp_dequant_int4(p, s, out, inn, w)
    torch.cuda.synchronize()
    return w.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("name", ["int4_small", "int4_ragged"])
def test_int4_bf16_copies_parity(name):
    """4-bit weights decoded once into bf16 copies (LMLP_INT4_BF16_COPIES)
    instead of inside the GEMM staging."""
    wl = workload(name)
    print(f"[case] {name} bf16 copies", flush=True)
    inp = I.make_inputs(wl)
    got, _ = run_hip(inp, wl, flags=abi.LMLP_INT4_BF16_COPIES)
    ref = oracle.forward_backward(oracle_inputs(inp, wl), wl.scale)
    compare(got, ref, TOL["bf16"], name + "_copies")


def test_int4_decode_modes_bitwise_equal():
    """Decoding in the staging (all four products) and decoding to bf16
    copies first give the same weights, fed to the same MFMA sequence in the
    same k order."""
    wl = workload("int4_ragged")
    inp = I.make_inputs(wl)
    a, _ = run_hip(inp, wl)
    b, _ = run_hip(inp, wl, flags=abi.LMLP_INT4_BF16_COPIES)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    compare(b, oracle.forward_backward(oracle_inputs(inp, wl), wl.scale), TOL["bf16"], "int4_ragged_copies")


@pytest.mark.parametrize("name,flags", [
    ("tiny_fp32", 0), ("f32_ragged", 0), ("bf16_ragged", 0), ("bf16_multi", 0), ("bf16_rank64", 0),
    ("bf16_dz_tail", 0), ("bf16_rank8", abi.LMLP_CONSUME_SAVED), ("int4_ragged", 0),
    ("int4_ragged", abi.LMLP_INT4_BF16_COPIES)])
def test_recompute_mode_bitwise_equal(name, flags):
    """LMLP_RECOMPUTE_GU (the gradient-checkpointing variant): the backward
    recomputes G and U with the forward's gate/up product from the same
    operand bits (X, the weights, and s P_gu rounded from the saved fp32
    P_gu), so every output equals the default mode's bit for bit; the default
    mode is checked against the oracle above. CONSUME_SAVED has no effect
    with it."""
    wl = workload(name)
    print(f"[case] {name} recompute flags={flags}", flush=True)
    inp = I.make_inputs(wl)
    a, _ = run_hip(inp, wl)
    b, _ = run_hip(inp, wl, flags=flags | abi.LMLP_RECOMPUTE_GU)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    ref = oracle.forward_backward(oracle_inputs(inp, wl), wl.scale)
    compare(b, ref, TOL[wl.dtype], f"{name}_recompute")


def test_int4_dequant_bit_exact_random():
    packed, scales = I.draw_int4_codes(5, 384, 1024)
    got = _dequant_gpu(packed, scales, 384, 1024)
    want = oracle.dequant_int4_bits(packed, scales, 1024)
    assert np.array_equal(got, want)


def test_int4_dequant_special_scales():
    # every code with zero, subnormal, tie-making and extreme fp16 scales (incl. negative)
    sbits = [0x0000, 0x8000, 0x0001, 0x0155, 0x03FF, 0x0400, 0x3C00, 0x3C04, 0x3C0C, 0x3800,
             0x7BFF, 0xFBFF, 0xBC00, 0x2E66, 0x1A00, 0x5555]
    rows = len(sbits)
    codes = np.tile(np.arange(-8, 8, dtype=np.int16), (rows, 4))       # [rows, 64]
    packed = I.pack_int4(codes)
    scales = np.array(sbits, dtype=np.uint16).reshape(rows, 1).view(np.float16)
    got = _dequant_gpu(packed, scales, rows, 64)
    want = oracle.dequant_int4_bits(packed, scales, 64)
    assert np.array_equal(got, want)


def test_int4_golden_cases_on_gpu():
    rows = []
    with open(os.path.join(GOLDEN, "int4_dequant_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([c.strip() for c in line.split("|")])
    packed = np.array([[int(r[0], 16)] * 32 for r in rows], dtype=np.uint8)
    scales = np.array([[int(r[2], 16)] for r in rows], dtype=np.uint16).view(np.float16)
    got = _dequant_gpu(packed, scales, len(rows), 64)
    for i, (byte, nib, sb, q, bits, note) in enumerate(rows):
        assert got[i, 0 if nib == "lo" else 1] == int(bits, 16), note
