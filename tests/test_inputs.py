"""Seeded input generator: storage conversions and draw order (no GPU)."""
import numpy as np
import torch

from lora_swiglu_mlp_amd import inputs as inp


def test_bf16_bits_match_torch_rne():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(50000) * 10.0 ** rng.integers(-20, 20, 50000)).astype(np.float32)
    want = torch.tensor(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(inp.f32_to_bf16_bits(v), want)
    back = inp.bf16_bits_to_f32(want)
    assert np.array_equal(back, torch.tensor(v).to(torch.bfloat16).float().numpy())


def test_pack_int4_layout():
    q = np.array([[-1, -8, 7, 0, 3, -3]], dtype=np.int16)
    b = inp.pack_int4(q)
    assert b.tolist() == [[0x8F, 0x07, 0xD3]]


def test_draws_are_seeded_and_shaped():
    wl = inp.WORKLOADS["tiny_fp32"]
    a = inp.make_inputs(wl)
    b = inp.make_inputs(wl)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert a["x"].shape == (256, 128) and a["x"].dtype == np.float32
    assert a["w_down"].shape == (128, 344)
    assert a["a_down"].shape == (8, 344) and a["b_down"].shape == (128, 8)
    q = inp.make_inputs(wl.replace(dtype="bf16", wfmt="int4_b64", inter=384))
    assert q["w_gate"].shape == (384, 64) and q["w_gate"].dtype == np.uint8
    assert q["w_gate_scales"].shape == (384, 2) and q["w_gate_scales"].dtype == np.float16
    assert q["w_down"].shape == (128, 192)
    assert wl.scale == 2.0
