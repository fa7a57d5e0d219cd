"""Host logic of bench.py and of the grouped workloads' router (no GPU)."""
import os
import subprocess
import sys

import numpy as np

import oracle
from oracle import lora_linear_oracle as LO

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from lora_swiglu_mlp_amd import inputs as I  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_gemm_flops_plus_side_work_give_the_oracle_count():
    T, H, Iw, r = 4096, 4096, 14336, 16
    gemms = sum(bench.kernel_flops(n, T, H, Iw, r) for n in ("gemm(gate/up)", "gemm(down)", "gemm(dZ)", "gemm(dX)"))
    # the four products carry the base FLOPs and the adapter K segments
    # (6 T r (H + I)); the rank-r side products carry the rest, 2 T r per
    # element of: X A_g^T, X A_u^T, dY B_d, dB_d, dA_g, dA_u (6 H) and
    # Z A_d^T, Q_g, Q_u, dB_g, dB_u, dA_d (6 I)
    assert gemms + 12 * T * r * (H + Iw) == oracle.flops(T, H, Iw, r)
    lin = sum(bench.kernel_flops(n, T, H, 1024, r, linear=True) for n in ("gemm(y)", "gemm(dX)"))
    assert lin + 4 * T * r * (H + 1024) == LO.flops(T, H, 1024, r)


def test_router_groups_every_token_top_k_times():
    rng = np.random.default_rng(3)
    tok, off = I.route_counts(rng, 500, 16, 4)
    assert off[0] == 0 and off[-1] == 2000 and np.all(np.diff(off) >= 0)
    # each token appears top_k times, in top_k distinct experts
    assert np.array_equal(np.bincount(tok, minlength=500), np.full(500, 4))
    expert_of_row = np.repeat(np.arange(16), np.diff(off))
    pairs = set(zip(tok.tolist(), expert_of_row.tolist()))
    assert len(pairs) == 2000


def test_moe_inputs_gather_the_token_rows():
    wl = I.MOE_WORKLOADS["moe_tiny_fp32"]
    inp, off = I.make_moe_inputs(wl)
    E, H, Iw, r = wl.experts, wl.hidden, wl.inter, wl.rank
    assert inp["x"].shape == (int(off[-1]), H) and inp["dy"].shape == (int(off[-1]), H)
    assert inp["w_gate"].shape == (E, Iw, H) and inp["w_down"].shape == (E, H, Iw)
    assert inp["a_down"].shape == (E, r, Iw) and inp["b_down"].shape == (E, H, r)
    # the rows are copies of token rows: every row equals some other row top_k - 1 more times
    _, counts = np.unique(inp["x"], axis=0, return_counts=True)
    assert np.all(counts == wl.top_k)
    again, off2 = I.make_moe_inputs(wl)
    assert np.array_equal(off, off2) and all(np.array_equal(inp[k], again[k]) for k in inp)


def test_norm_gamma_is_seeded_and_in_range():
    wl = I.WORKLOADS["tiny_fp32"]
    g = I.make_norm_gamma(wl)
    assert g.shape == (wl.hidden,) and g.min() >= 0.5 and g.max() < 1.5
    assert np.array_equal(g, I.make_norm_gamma(wl))
    # its own stream: the MLP's draws do not move
    assert np.array_equal(I.make_inputs(wl)["x"], I.make_inputs(wl)["x"])
