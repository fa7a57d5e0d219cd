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


def test_dz_split_and_per_launch_flops_at_llama3_8b():
    """On 256 compute units the Llama-3-8B dZ product (16 x 56 tiles of 256,
    3.5 waves) runs 12288 columns in 256-wide tiles and the last 2048 in a
    second launch; each launch is credited with its own columns, and the two
    add up to the whole product."""
    T, H, Iw, r = 4096, 4096, 14336, 16
    n1 = bench.dz_split(T, Iw, 256)
    assert n1 == 12288
    main = bench.kernel_flops("gemm(dZ)", T, H, Iw, r, dz_cols=n1)
    tail = bench.kernel_flops("gemm(dZ tail)", T, H, Iw, r, dz_cols=n1)
    assert main == 2 * T * (H + r) * 12288 and tail == 2 * T * (H + r) * 2048
    assert main + tail == bench.kernel_flops("gemm(dZ)", T, H, Iw, r)
    # full waves (or less than one) keep every column in one launch
    assert bench.dz_split(4096, 8192, 256) == 8192
    assert bench.dz_split(256, 14336, 256) == 14336
    kern = {"gemm(dZ)": {"ms": 0.4, "launches_per_step": 1.0}, "gemm(dZ tail)": {"ms": 0.1, "launches_per_step": 1.0}}
    tab = bench.gemm_table(kern, T, H, Iw, r, 2500.0, dz_cols=n1)
    assert abs(tab["dZ"]["tflops"] - (main + tail) / 0.5e-3 / 1e12) < 1e-9


class _OpCount(np.ndarray):
    """An array that counts the element operations done on full [T, H]
    operands (ufunc calls, and reductions counted at their input size)."""
    full = 0
    ops = 0

    def __array_ufunc__(self, ufunc, method, *inputs, **kw):
        args = [np.asarray(i) if isinstance(i, _OpCount) else i for i in inputs]
        if "out" in kw:
            kw["out"] = tuple(np.asarray(o) if isinstance(o, _OpCount) else o for o in kw["out"])
        res = getattr(ufunc, method)(*args, **kw)
        big = max(np.size(a) for a in args if isinstance(a, np.ndarray))
        if big == _OpCount.full:
            _OpCount.ops += big
        return res.view(_OpCount) if isinstance(res, np.ndarray) else res


def test_norm_flops_count_the_oracles_operations():
    """bench's RMSNorm FLOP figure equals the element operations the norm
    oracle actually performs on [T, H] arrays in its forward and backward."""
    from oracle import rmsnorm_oracle as R
    rng = np.random.default_rng(5)
    T, H = 6, 10
    x = rng.standard_normal((T, H)).view(_OpCount)
    gamma = rng.standard_normal(H).view(_OpCount)
    g = rng.standard_normal((T, H)).view(_OpCount)
    _OpCount.full, _OpCount.ops = T * H, 0
    _, rstd = R.forward(x, gamma, 1e-5)
    fwd = _OpCount.ops
    R.backward(x, gamma, np.asarray(rstd).view(_OpCount), g)
    assert fwd == 4 * T * H
    assert _OpCount.ops == bench.norm_flops(T, H)


def test_moe_bytes_and_bound():
    """The grouped products' algorithmic bytes, counted by hand for a small
    case, and the bound they give: the Qwen3-30B-A3B MoE shape (small
    experts) sits below the ridge point of 2500 TFLOP/s over 8 TB/s, the
    Mixtral-8x7B shape above it."""
    rows, E, H, Iw, r = 10, 3, 8, 6, 2
    # gate/up: X 80, W 3*2*6*8 = 288, P 40, B 3*2*6*2 = 72, G U Z 180 -> 660 elements
    assert bench.moe_gemm_bytes("gemm(gate/up)", rows, E, H, Iw, r, 2) == 2 * 660
    # down: Z 60, W_d 144, P_d 20, B_d 48, y 80 -> 352
    assert bench.moe_gemm_bytes("gemm(down)", rows, E, H, Iw, r, 2) == 2 * 352
    # dZ: dY 80, W_d 144, G U dG dU 240 -> 464
    assert bench.moe_gemm_bytes("gemm(dZ)", rows, E, H, Iw, r, 2) == 2 * 464
    # dX: dG dU 120, W_g W_u 288, Q 40, A_g A_u 96, dx 80 -> 624
    assert bench.moe_gemm_bytes("gemm(dX)", rows, E, H, Iw, r, 2) == 2 * 624
    ridge = bench.PEAK_TFLOPS["bf16"] * 1e12 / (bench.HBM_PEAK_GBS * 1e9)
    for wl, below in (("moe_qwen3", True), ("moe_mixtral", False)):
        w = I.MOE_WORKLOADS[wl]
        n = w.tokens * w.top_k
        for k in ("gemm(gate/up)", "gemm(down)", "gemm(dZ)", "gemm(dX)"):
            f = bench.kernel_flops(k, n, w.hidden, w.inter, w.rank)
            b = bench.moe_gemm_bytes(k, n, w.experts, w.hidden, w.inter, w.rank, 2)
            assert (f / b < ridge) == below, (wl, k, f / b)
