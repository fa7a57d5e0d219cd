"""Pins for the fp64 CPU oracle (no GPU).

Each test checks the oracle against something other than itself: finite
differences, an independent merged-weight route, scalar brute-force loops,
torch autograd in fp64, hand-derived closed forms, invariants that hold
exactly, and planted mistakes that the pins must catch.
"""
import inspect
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import lora_mlp_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
WNAMES = orc.WEIGHT_KEYS


def rand_problem(T=3, H=8, I=12, r=2, seed=0, std=0.6):
    rng = np.random.default_rng(seed)
    n = lambda *s: rng.standard_normal(s) * std  # noqa: E731
    return {"x": n(T, H), "w_gate": n(I, H), "w_up": n(I, H), "w_down": n(H, I),
            "a_gate": n(r, H), "b_gate": n(I, r), "a_up": n(r, H), "b_up": n(I, r),
            "a_down": n(r, I), "b_down": n(H, r), "dy": n(T, H)}


def weights(p):
    return [p[k] for k in WNAMES]


def full(p, s):
    return orc.forward_backward(p, s)


def relerr(a, b):
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


GRAD_KEYS = ("dx",) + orc.ADAPTER_KEYS
ALL_KEYS = ("y",) + GRAD_KEYS


# ---------------------------------------------------------------------------
# finite differences pin the whole backward

def _loss(p, s):
    y = orc.forward(p["x"], *weights(p), s)["y"]
    return float(np.sum(p["dy"] * y))


@pytest.mark.parametrize("s", [0.75, 2.0])
def test_finite_differences(s):
    p = rand_problem(T=3, H=8, I=12, r=2, seed=1)
    got = full(p, s)
    grad_of = {"x": "dx", "a_gate": "da_gate", "b_gate": "db_gate", "a_up": "da_up",
               "b_up": "db_up", "a_down": "da_down", "b_down": "db_down"}
    h = 1e-6
    for name, gk in grad_of.items():
        fd = np.zeros_like(p[name])
        for idx in np.ndindex(p[name].shape):
            q = {k: v.copy() for k, v in p.items()}
            q[name][idx] += h
            lp = _loss(q, s)
            q[name][idx] -= 2 * h
            lm = _loss(q, s)
            fd[idx] = (lp - lm) / (2 * h)
        assert relerr(got[gk], fd) < 1e-7, name


# ---------------------------------------------------------------------------
# independent routes

@pytest.mark.parametrize("shape", [(5, 16, 24, 4), (7, 8, 40, 1), (4, 32, 8, 8)])
def test_merged_weight_route(shape):
    T, H, I, r = shape
    p = rand_problem(T, H, I, r, seed=T + H)
    s = 1.5
    a = full(p, s)
    b = orc.merged_reference(p["x"], *weights(p), s, p["dy"])
    for k in ALL_KEYS:
        assert relerr(a[k], b[k]) < 1e-12, k


def test_bruteforce_loops():
    p = rand_problem(T=3, H=4, I=6, r=2, seed=7)
    s = 2.0
    a = full(p, s)
    b = orc.bruteforce(p["x"], *weights(p), s, p["dy"])
    for k in ALL_KEYS:
        assert relerr(a[k], b[k]) < 1e-12, k


def test_torch_autograd_fp64():
    p = rand_problem(T=6, H=16, I=20, r=3, seed=11)
    s = 0.5
    a = full(p, s)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=(k not in
                         ("w_gate", "w_up", "w_down", "dy"))) for k, v in p.items()}

    def lin(v, w, A, B):
        return v @ w.T + s * (v @ A.T) @ B.T

    g = lin(t["x"], t["w_gate"], t["a_gate"], t["b_gate"])
    u = lin(t["x"], t["w_up"], t["a_up"], t["b_up"])
    y = lin(torch.nn.functional.silu(g) * u, t["w_down"], t["a_down"], t["b_down"])
    (y * t["dy"]).sum().backward()
    ref = {"y": y.detach().numpy(), "dx": t["x"].grad.numpy()}
    for k in ("gate", "up", "down"):
        ref["da_" + k] = t["a_" + k].grad.numpy()
        ref["db_" + k] = t["b_" + k].grad.numpy()
    for k in ALL_KEYS:
        assert relerr(a[k], ref[k]) < 1e-12, k


# ---------------------------------------------------------------------------
# invariants

def _base_mlp(p):
    x = torch.tensor(p["x"])
    g = x @ torch.tensor(p["w_gate"]).T
    u = x @ torch.tensor(p["w_up"]).T
    return (torch.nn.functional.silu(g) * u @ torch.tensor(p["w_down"]).T).numpy()


def test_b_zero_gives_base_mlp_and_zero_da():
    p = rand_problem(T=5, H=12, I=10, r=3, seed=3)
    for k in ("b_gate", "b_up", "b_down"):
        p[k] = np.zeros_like(p[k])
    out = full(p, 2.0)
    assert relerr(out["y"], _base_mlp(p)) < 1e-13
    for k in ("da_gate", "da_up", "da_down"):
        assert np.all(out[k] == 0.0), k
    for k in ("db_gate", "db_up", "db_down"):
        assert np.linalg.norm(out[k]) > 0, k


def test_a_zero_gives_zero_db():
    p = rand_problem(T=5, H=12, I=10, r=3, seed=4)
    for k in ("a_gate", "a_up", "a_down"):
        p[k] = np.zeros_like(p[k])
    out = full(p, 2.0)
    assert relerr(out["y"], _base_mlp(p)) < 1e-13
    for k in ("db_gate", "db_up", "db_down"):
        assert np.all(out[k] == 0.0), k
    for k in ("da_gate", "da_up", "da_down"):
        assert np.linalg.norm(out[k]) > 0, k


def test_adapter_rescaling_is_exact():
    p = rand_problem(T=4, H=8, I=12, r=2, seed=5)
    s = 1.0
    a = full(p, s)
    q = dict(p)
    for k in ("gate", "up", "down"):
        q["a_" + k] = p["a_" + k] * 2.0
        q["b_" + k] = p["b_" + k] / 2.0
    b = full(q, s)
    assert np.array_equal(a["y"], b["y"])
    assert np.array_equal(a["dx"], b["dx"])
    for k in ("gate", "up", "down"):
        assert np.array_equal(b["da_" + k], a["da_" + k] / 2.0), k
        assert np.array_equal(b["db_" + k], a["db_" + k] * 2.0), k


def test_linear_in_dy():
    p = rand_problem(T=4, H=8, I=12, r=2, seed=6)
    a = full(p, 1.25)
    q = dict(p)
    q["dy"] = p["dy"] * 2.0
    b = full(q, 1.25)
    for k in GRAD_KEYS:
        assert np.array_equal(b[k], a[k] * 2.0), k


def test_rows_are_independent():
    p = rand_problem(T=9, H=8, I=12, r=2, seed=8)
    perm = np.random.default_rng(0).permutation(9)
    a = full(p, 1.0)
    q = dict(p)
    q["x"], q["dy"] = p["x"][perm], p["dy"][perm]
    b = full(q, 1.0)
    assert np.array_equal(b["y"], a["y"][perm])
    assert np.array_equal(b["dx"], a["dx"][perm])
    for k in orc.ADAPTER_KEYS:
        assert relerr(b[k], a[k]) < 1e-13, k


def test_row_chunks_match_whole_batch():
    p = rand_problem(T=37, H=16, I=24, r=4, seed=9)
    a = orc.forward_backward(p, 2.0)
    b = orc.forward_backward(p, 2.0, row_chunk=8)
    for k in ALL_KEYS:
        assert relerr(b[k], a[k]) < 1e-13, k
    rows = [0, 5, 36]
    c = orc.base_mlp_rows(p["x"][rows], *weights(p), 2.0, dy=p["dy"][rows])
    assert relerr(c["y"], a["y"][rows]) < 1e-14
    assert relerr(c["dx"], a["dx"][rows]) < 1e-14


def test_sigmoid_extremes_and_library():
    from scipy.special import expit
    g = np.array([-800.0, -40.0, -1e-3, 0.0, 1e-3, 40.0, 800.0])
    with np.errstate(over="raise"):
        sg = orc.sigmoid(g)
    assert np.all(np.isfinite(sg))
    assert np.allclose(sg, expit(g), rtol=1e-15, atol=0)
    assert orc.silu(np.array([0.0]))[0] == 0.0


# ---------------------------------------------------------------------------
# hand-derived closed forms

def _read_cases(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([c.strip() for c in line.split("|")])
    return rows


def test_scalar_closed_form_golden():
    L = math.log(3.0)
    env = {"__builtins__": {}, "L": L}
    cases = _read_cases("scalar_closed_form.txt")
    assert len(cases) >= 2
    for name, ins, exp in cases:
        vals = {kv.split("=")[0]: float(eval(kv.split("=", 1)[1], env))
                for kv in ins.split()}
        s = vals.pop("s")
        p = {"x": [[vals["x"]]], "w_gate": [[vals["wg"]]], "a_gate": [[vals["ag"]]],
             "b_gate": [[vals["bg"]]], "w_up": [[vals["wu"]]], "a_up": [[vals["au"]]],
             "b_up": [[vals["bu"]]], "w_down": [[vals["wd"]]], "a_down": [[vals["ad"]]],
             "b_down": [[vals["bd"]]], "dy": [[vals["dy"]]]}
        p = {k: np.array(v, dtype=np.float64) for k, v in p.items()}
        out = full(p, s)
        for kv in exp.split():
            k, e = kv.split("=", 1)
            want = float(eval(e, env))
            assert abs(out[k][0, 0] - want) <= 1e-14 * max(1.0, abs(want)), (name, k)


# ---------------------------------------------------------------------------
# 4-bit weights

def test_int4_golden_cases():
    for byte, nib, sbits, q, bits, note in _read_cases("int4_dequant_cases.txt"):
        b = int(byte, 16)
        packed = np.array([[b] * 32], dtype=np.uint8)       # one 64-element block
        scales = np.array([[int(sbits, 16)]], dtype=np.uint16).view(np.float16)
        codes = orc.unpack_int4(packed, 64)
        k = 0 if nib == "lo" else 1
        assert codes[0, k] == int(q), note
        got = orc.dequant_int4_bits(packed, scales, 64)[0, k]
        assert got == int(bits, 16), (note, hex(got))


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        np.array([0.0, -0.0, 1.0, 3.0e38, 1e-39, -1e-40])]).astype(np.float32)
    want = torch.tensor(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = orc.bf16_round(v.astype(np.float64))
    assert np.array_equal(np.signbit(got), np.signbit(want))
    assert np.array_equal(got, want)


def test_int4_random_blocks_properties():
    from lora_swiglu_mlp_amd.inputs import draw_int4_codes
    packed, scales = draw_int4_codes(3, 48, 256)
    w = orc.dequant_int4(packed, scales, 256)
    q = orc.unpack_int4(packed, 256)
    assert set(np.unique(q)) == set(range(-8, 8))
    exact = q * np.repeat(scales.astype(np.float64), 64, axis=1)
    # rounding error of one bf16 RNE: at most half a unit in the 8th significant bit
    tol = np.abs(exact) * 2.0 ** -8 + 1e-300
    assert np.all(np.abs(w - exact) <= tol)
    # values lie on the bf16 grid
    assert np.array_equal(orc.bf16_round(w), w)


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by a pin above

MUTANTS = [
    ("backward", "(1.0 + g * (1.0 - sg))", "(1.0 + g * sg)"),            # wrong SiLU'
    ("backward", "(1.0 + g * (1.0 - sg))", "1.0"),                       # dropped term
    ("backward", "db_down = s * (dy.T @ fwd[\"p_down\"])", "db_down = (dy.T @ fwd[\"p_down\"])"),
    ("backward", "da_down = s * (q_down.T @ z)", "da_down = -s * (q_down.T @ z)"),
    ("backward", "+ s * (q_down @ a_down)", ""),                          # dropped adapter path
    ("backward", "q_gate = dg @ b_gate", "q_gate = du @ b_gate"),          # wrong operand
    ("backward", "db_up = s * (du.T @ fwd[\"p_up\"])", "db_up = s * (du.T @ fwd[\"p_gate\"])"),
    ("backward", "q_up @ a_up", "q_up @ a_gate"),
    ("forward", "u = x @ w_up.T + s * (p_up @ b_up.T)", "u = x @ w_up.T + s * (p_gate @ b_up.T)"),
    ("forward", "z = g * sg * u", "z = sg * u"),
    ("forward", "p_down = z @ a_down.T", "p_down = (g * u) @ a_down.T"),
]


@pytest.mark.parametrize("fn,old,new", MUTANTS)
def test_planted_mistakes_are_caught(fn, old, new):
    src = inspect.getsource(getattr(orc, fn))
    assert old in src, "mutant no longer applies"
    ns = dict(vars(orc))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    mutated = ns[fn]
    p = rand_problem(T=4, H=6, I=10, r=2, seed=12)
    s = 1.5
    # the mutated oracle, composed the same way forward_backward does
    fwd_fn = mutated if fn == "forward" else orc.forward
    bwd_fn = mutated if fn == "backward" else orc.backward
    f = fwd_fn(p["x"], *weights(p), s)
    b = bwd_fn(p["dy"], p["x"], *weights(p), s, fwd=f)
    got = {"y": f["y"], **b}
    ref = orc.merged_reference(p["x"], *weights(p), s, p["dy"])
    worst = max(relerr(got[k], ref[k]) for k in ALL_KEYS)
    assert worst > 1e-6, "planted mistake went unnoticed"


def test_flop_count():
    # counted by hand from the matmuls in forward() and backward()
    T, H, I, r = 4096, 4096, 14336, 16
    base = 6 * T * H * I + 6 * T * H * I
    fwd_lora = 2 * T * H * r * 2 + 2 * T * I * r * 2 + 2 * T * I * r + 2 * T * H * r
    bwd_lora = (2 * T * H * r * 2 + 2 * T * I * r * 2 + 2 * T * I * r * 4 + 2 * T * H * r * 4)
    assert orc.flops(T, H, I, r) == base + fwd_lora + bwd_lora
    assert abs(orc.flops(T, H, I, r) / 1e12 - 2.9080) < 1e-3
