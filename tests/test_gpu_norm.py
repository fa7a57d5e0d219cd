"""GPU parity of RMSNorm then the fused LoRA MLP (through the C ABI's norm
entry points) against the fp64 oracle: ragged token counts (not a multiple
of the four rows a workgroup takes), row widths that fill a wave partially,
exactly, and beyond what stays in registers (the second-read path), both
dtypes, 4-bit weights, the full-recompute mode, an empty batch, and the
Llama-3-8B size in full. Tolerance as for the MLP: max|gpu-ref| / max|ref|
<= 1e-4 (fp32), <= 2e-2 (bf16) per output tensor."""
import time

import numpy as np
import pytest

from lora_swiglu_mlp_amd import abi
from lora_swiglu_mlp_amd import inputs as I
from lmlp_testutil import TOL, compare, norm_oracle, run_hip_norm

pytestmark = pytest.mark.gpu

EPS = I.NORM_EPS
CASES = {
    # name: (T, H, I, r, alpha, dtype, wfmt)
    "tiny_fp32": (256, 128, 344, 8, 16.0, "f32", "dense"),
    "f32_ragged": (101, 36, 52, 3, 6.0, "f32", "dense"),
    "f32_wide_rows": (5, 4100, 40, 4, 8.0, "f32", "dense"),      # 17 chunks per lane: re-read path
    "bf16_ragged": (301, 320, 600, 16, 32.0, "bf16", "dense"),
    "bf16_multi": (517, 1024, 1088, 16, 16.0, "bf16", "dense"),
    "bf16_rows_8192": (9, 8192, 128, 16, 16.0, "bf16", "dense"),  # 16 chunks per lane, the register limit
    "bf16_wide_rows": (6, 8264, 64, 4, 8.0, "bf16", "dense"),     # past it
    "bf16_rank64": (130, 256, 512, 64, 128.0, "bf16", "dense"),
    "bf16_one_token": (1, 64, 128, 8, 16.0, "bf16", "dense"),
    "int4_small": (192, 256, 384, 16, 16.0, "bf16", "int4_b64"),
}


def workload(name):
    T, H, Iw, r, alpha, dt, wf = CASES[name]
    base = I.WORKLOADS["tiny_fp32" if dt == "f32" else "llama3_8b"]
    return base.replace(name=name, tokens=T, hidden=H, inter=Iw, rank=r, alpha=alpha, dtype=dt, wfmt=wf)


def _inputs(wl):
    inp = I.make_inputs(wl)
    inp["gamma"] = I.make_norm_gamma(wl)
    return inp


@pytest.mark.parametrize("name", list(CASES))
def test_norm_mlp_parity(name):
    wl = workload(name)
    print(f"[case] norm {name} {CASES[name]}", flush=True)
    inp = _inputs(wl)
    got, _ = run_hip_norm(inp, wl, EPS)
    compare(got, norm_oracle(inp, wl, EPS), TOL[wl.dtype], "norm " + name)
    assert all(np.isfinite(v).all() for v in got.values())


def test_norm_recompute_mode_and_determinism_bitwise():
    """Bitwise: two runs agree, and LMLP_RECOMPUTE_GU gives the default mode's
    outputs (the backward re-applies the norm from the saved statistics, so
    the recomputed G, U see the forward's normalised rows bit for bit)."""
    wl = workload("bf16_ragged")
    inp = _inputs(wl)
    a, _ = run_hip_norm(inp, wl, EPS)
    b, _ = run_hip_norm(inp, wl, EPS)
    c, _ = run_hip_norm(inp, wl, EPS, flags=abi.LMLP_RECOMPUTE_GU)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
        assert np.array_equal(a[k], c[k]), k
    compare(c, norm_oracle(inp, wl, EPS), TOL[wl.dtype], "norm recompute")


def test_norm_eps_matters_and_zero_eps():
    """Rows of tiny magnitude: eps dominates the statistic, so eps = 0 and
    eps = 1 give very different y, each matching the oracle."""
    wl = workload("tiny_fp32").replace(x_std=1e-3)
    inp = _inputs(wl)
    outs = {}
    for eps in (0.0, 1.0):
        got, _ = run_hip_norm(inp, wl, eps)
        compare(got, norm_oracle(inp, wl, eps), TOL[wl.dtype], f"norm eps={eps}")
        outs[eps] = got["y"]
    assert np.max(np.abs(outs[0.0])) > 100 * np.max(np.abs(outs[1.0]))


def test_norm_empty_batch():
    import torch
    from lora_swiglu_mlp_amd import mlp
    wl = workload("bf16_ragged").replace(tokens=0)
    inp = _inputs(wl)
    m, x, dy = mlp.from_inputs(inp, wl, "cuda", norm_eps=EPS)
    y, saved = m.forward(x)
    g = m.new_grads("cuda")
    for v in g.values():
        v.fill_(7.0)
    m.backward(dy, x, saved, g)
    torch.cuda.synchronize()
    assert y.numel() == 0
    for k, v in g.items():
        assert v.numel() == 0 if k == "dx" else bool((v == 0).all()), k


def test_norm_fullsize_parity():
    """The Llama-3-8B MLP size with the norm in front, in the bench's launch
    configuration, against the oracle over the whole batch."""
    wl = I.WORKLOADS["llama3_8b"]
    print(f"[case] norm llama3_8b T={wl.tokens} H={wl.hidden} I={wl.inter}", flush=True)
    t0 = time.time()
    inp = _inputs(wl)
    got, _ = run_hip_norm(inp, wl, EPS)
    t1 = time.time()
    ref = norm_oracle(inp, wl, EPS)
    print(f"[time] inputs+gpu {t1 - t0:.1f}s oracle {time.time() - t1:.1f}s", flush=True)
    compare(got, ref, TOL[wl.dtype], "norm llama3_8b")
