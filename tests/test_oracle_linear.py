"""Pins of the fused LoRA linear oracle (no GPU).

Each pin is independent of the oracle's own formulas: finite differences of
L = <dY, y>, the merged-weight route, scalar brute force, invariants of the
adapter (B = 0, A = 0, rescaling, linearity in dY), agreement with the
(separately pinned) MLP oracle's down projection, and planted mistakes that
the finite-difference pin must catch.
"""
import numpy as np
import pytest

import oracle
from oracle import lora_linear_oracle as L


def _draw(T=3, n_in=5, n_out=4, r=2, seed=0, std=1.0):
    rng = np.random.default_rng(seed)
    return {"x": rng.normal(0, std, (T, n_in)), "w": rng.normal(0, std, (n_out, n_in)),
            "a": rng.normal(0, std, (r, n_in)), "b": rng.normal(0, std, (n_out, r)),
            "dy": rng.normal(0, std, (T, n_out))}


def _fd_check(fb, inp, s, h=1e-6):
    """Central differences of L = <dY, y> against fb's gradients for every
    scalar of x, A and B; returns the worst relative error."""
    got = fb(inp, s)
    worst = 0.0
    for name, gname in (("x", "dx"), ("a", "da"), ("b", "db")):
        num = np.zeros_like(inp[name])
        for idx in np.ndindex(*inp[name].shape):
            plus, minus = dict(inp), dict(inp)
            plus[name] = inp[name].copy()
            minus[name] = inp[name].copy()
            plus[name][idx] += h
            minus[name][idx] -= h
            lp = np.sum(inp["dy"] * fb(plus, s)["y"])
            lm = np.sum(inp["dy"] * fb(minus, s)["y"])
            num[idx] = (lp - lm) / (2 * h)
        den = max(1.0, float(np.max(np.abs(num))))
        worst = max(worst, float(np.max(np.abs(num - got[gname]))) / den)
    return worst


@pytest.mark.parametrize("s", [1.0, 2.5, -0.75])
def test_finite_differences(s):
    assert _fd_check(L.forward_backward, _draw(seed=int(s * 10) % 7), s) < 1e-7


@pytest.mark.parametrize("shape", [(7, 24, 16, 4), (33, 40, 72, 8), (5, 16, 8, 1)])
def test_merged_weight_route(shape):
    T, n_in, n_out, r = shape
    inp = _draw(T, n_in, n_out, r, seed=3)
    got = L.forward_backward(inp, 1.7)
    ref = L.merged_reference(inp["x"], inp["w"], inp["a"], inp["b"], 1.7, inp["dy"])
    for k in ref:
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-11, atol=1e-11)


def test_bruteforce_loops():
    inp = _draw(4, 6, 5, 3, seed=5)
    got = L.forward_backward(inp, 0.8)
    ref = L.bruteforce(inp["x"], inp["w"], inp["a"], inp["b"], 0.8, inp["dy"])
    for k in ref:
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-12, atol=1e-12)


def test_b_zero_and_a_zero_invariants():
    inp = _draw(6, 8, 7, 3, seed=9)
    b0 = dict(inp, b=np.zeros_like(inp["b"]))
    g = L.forward_backward(b0, 2.0)
    np.testing.assert_array_equal(g["y"], inp["x"] @ inp["w"].T)
    assert np.all(g["da"] == 0) and np.linalg.norm(g["db"]) > 0
    a0 = dict(inp, a=np.zeros_like(inp["a"]))
    g = L.forward_backward(a0, 2.0)
    assert np.all(g["db"] == 0) and np.linalg.norm(g["da"]) > 0


def test_adapter_rescaling_and_dy_linearity():
    inp = _draw(6, 8, 7, 3, seed=11)
    g1 = L.forward_backward(inp, 1.3)
    g2 = L.forward_backward(dict(inp, a=2 * inp["a"], b=inp["b"] / 2), 1.3)
    np.testing.assert_allclose(g2["y"], g1["y"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(g2["da"], g1["da"] / 2, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(g2["db"], 2 * g1["db"], rtol=1e-13, atol=1e-13)
    g3 = L.forward_backward(dict(inp, dy=2 * inp["dy"]), 1.3)
    for k in ("dx", "da", "db"):
        np.testing.assert_array_equal(g3[k], 2 * g1[k])


def test_row_chunks_match_whole_batch():
    inp = _draw(13, 9, 6, 2, seed=2)
    a = L.forward_backward(inp, 0.9)
    b = L.forward_backward(inp, 0.9, row_chunk=4)
    for k in a:
        np.testing.assert_allclose(a[k], b[k], rtol=1e-13, atol=1e-13)


def test_agrees_with_the_mlp_oracle_down_projection():
    """The MLP's down projection is a LoRA linear applied to Z: same y, and
    the same dB_d, dA_d and dZ (the MLP oracle is pinned on its own)."""
    rng = np.random.default_rng(4)
    T, H, I, r = 5, 6, 10, 2
    w = {k: rng.normal(0, 0.5, sh) for k, sh in (
        ("w_gate", (I, H)), ("w_up", (I, H)), ("w_down", (H, I)), ("a_gate", (r, H)), ("b_gate", (I, r)),
        ("a_up", (r, H)), ("b_up", (I, r)), ("a_down", (r, I)), ("b_down", (H, r)))}
    x, dy = rng.normal(0, 1, (T, H)), rng.normal(0, 1, (T, H))
    args = [w[k] for k in oracle.WEIGHT_KEYS]
    f = oracle.forward(x, *args, 1.5)
    b = oracle.backward(dy, x, *args, 1.5, fwd=f)
    lin = L.forward_backward({"x": f["z"], "w": w["w_down"], "a": w["a_down"], "b": w["b_down"], "dy": dy}, 1.5)
    np.testing.assert_allclose(lin["y"], f["y"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lin["da"], b["da_down"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lin["db"], b["db_down"], rtol=1e-12, atol=1e-12)


def _mutant(kind):
    def fb(inp, s):
        x, w, a, b, dy = inp["x"], inp["w"], inp["a"], inp["b"], inp["dy"]
        p = x @ a.T
        q = dy @ b
        out = {"y": x @ w.T + s * (p @ b.T), "dx": dy @ w + s * (q @ a), "da": s * (q.T @ x),
               "db": s * (dy.T @ p)}
        if kind == "dx_no_adapter":
            out["dx"] = dy @ w
        elif kind == "db_no_scale":
            out["db"] = dy.T @ p
        elif kind == "da_wrong_sign":
            out["da"] = -out["da"]
        elif kind == "db_wrong_factor":
            out["db"] = s * (dy.T @ (x @ w.T)[:, :p.shape[1]])
        return out
    return fb


@pytest.mark.parametrize("kind", ["dx_no_adapter", "db_no_scale", "da_wrong_sign", "db_wrong_factor"])
def test_planted_mistakes_are_caught(kind):
    inp = _draw(seed=1)
    assert _fd_check(_mutant("none"), inp, 1.5) < 1e-7  # the unmutated copy passes
    assert _fd_check(_mutant(kind), inp, 1.5) > 1e-3


def test_flop_count():
    assert L.flops(4096, 4096, 4096, 16) == 4 * 4096 ** 3 + 6 * 4096 * 16 * 8192
    # three linears of the MLP's shapes give the MLP's count
    T, H, I, r = 64, 32, 48, 4
    assert 2 * L.flops(T, H, I, r) + L.flops(T, I, H, r) == oracle.flops(T, H, I, r)
