"""Pins of the RMSNorm oracle and of its composition with the MLP (no GPU).

Each pin is independent of the oracle's own formulas: finite differences of
<g, xn> and of <dY, y> through norm and MLP, scalar brute force with the
chain rule written per element, closed forms (constant rows, H = 1, unit
root mean square), the scale invariance of the normalised row at eps = 0
and the orthogonality of its gradient to x that follows, and planted
mistakes that these pins must catch.
"""
import numpy as np
import pytest

from oracle import lora_mlp_oracle as M
from oracle import rmsnorm_oracle as R


def _draw(T=3, H=6, seed=0):
    rng = np.random.default_rng(seed)
    return rng.normal(0, 1, (T, H)), rng.normal(1, 0.3, H), rng.normal(0, 1, (T, H))


def _fd_norm(fwd, bwd, x, gamma, eps, g, h=1e-6):
    """worst relative error of bwd against central differences of <g, xn>"""
    xn, rstd = fwd(x, gamma, eps)
    got = bwd(x, gamma, rstd, g)
    num = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        num[idx] = (np.sum(g * fwd(xp, gamma, eps)[0]) - np.sum(g * fwd(xm, gamma, eps)[0])) / (2 * h)
    return float(np.max(np.abs(num - got))) / max(1.0, float(np.max(np.abs(num))))


@pytest.mark.parametrize("eps", [0.0, 1e-5, 0.5])
def test_finite_differences(eps):
    x, gamma, g = _draw(4, 7, seed=int(eps * 10) + 1)
    assert _fd_norm(R.forward, R.backward, x, gamma, eps, g) < 1e-8


def test_bruteforce_loops():
    x, gamma, g = _draw(3, 5, seed=4)
    xn, rstd, dx = R.bruteforce(x, gamma, 1e-5, g)
    xn2, rstd2 = R.forward(x, gamma, 1e-5)
    np.testing.assert_allclose(xn2, xn, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(rstd2, rstd, rtol=1e-13)
    np.testing.assert_allclose(R.backward(x, gamma, rstd2, g), dx, rtol=1e-12, atol=1e-12)


def test_closed_forms():
    # constant row c: mean square c^2, xn = gamma * c / sqrt(c^2 + eps)
    H, eps = 8, 1e-5
    gamma = np.linspace(0.5, 2.0, H)
    for c in (3.0, -0.25):
        x = np.full((1, H), c)
        xn, rstd = R.forward(x, gamma, eps)
        np.testing.assert_allclose(rstd, [1 / np.sqrt(c * c + eps)], rtol=1e-15)
        np.testing.assert_allclose(xn[0], gamma * c / np.sqrt(c * c + eps), rtol=1e-15)
    # H = 1: xn = gamma x / sqrt(x^2 + eps); d xn / dx = gamma eps / (x^2 + eps)^(3/2)
    x = np.array([[1.5], [-0.2]])
    gm = np.array([0.7])
    xn, rstd = R.forward(x, gm, 0.1)
    np.testing.assert_allclose(xn[:, 0], 0.7 * x[:, 0] / np.sqrt(x[:, 0] ** 2 + 0.1), rtol=1e-15)
    dx = R.backward(x, gm, rstd, np.ones_like(x))
    np.testing.assert_allclose(dx[:, 0], 0.7 * 0.1 / (x[:, 0] ** 2 + 0.1) ** 1.5, rtol=1e-13)
    # gamma = 1, eps = 0: every normalised row has root mean square 1
    x, _, _ = _draw(5, 9, seed=7)
    xn, _ = R.forward(x, np.ones(9), 0.0)
    np.testing.assert_allclose(np.mean(xn * xn, axis=1), 1.0, rtol=1e-14)


def test_scale_invariance_and_orthogonal_gradient():
    x, gamma, g = _draw(4, 10, seed=9)
    xn, rstd = R.forward(x, gamma, 0.0)
    xn3, rstd3 = R.forward(3.0 * x, gamma, 0.0)
    np.testing.assert_allclose(xn3, xn, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(rstd3, rstd / 3.0, rtol=1e-14)
    dx = R.backward(x, gamma, rstd, g)
    # xn(c x) = xn(x) => its gradient has no component along x, and scales as 1/c
    np.testing.assert_allclose(np.sum(dx * x, axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose(R.backward(3.0 * x, gamma, rstd3, g), dx / 3.0, rtol=1e-12, atol=1e-14)


def _mlp_draw(T=3, H=5, I=4, r=2, seed=0):
    rng = np.random.default_rng(seed)
    inp = {"x": rng.normal(0, 1, (T, H)), "dy": rng.normal(0, 1, (T, H)),
           "w_gate": rng.normal(0, 0.5, (I, H)), "w_up": rng.normal(0, 0.5, (I, H)),
           "w_down": rng.normal(0, 0.5, (H, I)),
           "a_gate": rng.normal(0, 0.5, (r, H)), "b_gate": rng.normal(0, 0.5, (I, r)),
           "a_up": rng.normal(0, 0.5, (r, H)), "b_up": rng.normal(0, 0.5, (I, r)),
           "a_down": rng.normal(0, 0.5, (r, I)), "b_down": rng.normal(0, 0.5, (H, r))}
    return inp, rng.normal(1, 0.3, H)


def test_norm_then_mlp_finite_differences():
    inp, gamma = _mlp_draw(seed=2)
    eps, s, h = 1e-5, 1.3, 1e-6
    got = R.norm_mlp_forward_backward(inp, gamma, eps, s)
    worst = 0.0
    for name, gname in (("x", "dx"), ("a_gate", "da_gate"), ("b_up", "db_up"), ("a_down", "da_down")):
        num = np.zeros_like(inp[name])
        for idx in np.ndindex(*inp[name].shape):
            p, m = dict(inp), dict(inp)
            p[name] = inp[name].copy()
            m[name] = inp[name].copy()
            p[name][idx] += h
            m[name][idx] -= h
            lp = np.sum(inp["dy"] * R.norm_mlp_forward_backward(p, gamma, eps, s)["y"])
            lm = np.sum(inp["dy"] * R.norm_mlp_forward_backward(m, gamma, eps, s)["y"])
            num[idx] = (lp - lm) / (2 * h)
        worst = max(worst, float(np.max(np.abs(num - got[gname]))) / max(1.0, float(np.max(np.abs(num)))))
    assert worst < 1e-7


def test_composition_reduces_to_the_mlp_on_normalised_rows():
    inp, gamma = _mlp_draw(T=6, H=8, I=16, r=3, seed=5)
    got = R.norm_mlp_forward_backward(inp, gamma, 1e-5, 0.9, row_chunk=4)
    xn, _ = R.forward(inp["x"], gamma, 1e-5)
    ref = M.forward_backward(dict(inp, x=xn), 0.9)
    for k in ("y",) + M.ADAPTER_KEYS:
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(got["dxn"], ref["dx"], rtol=1e-13, atol=1e-13)


def _mutant(kind):
    def fwd(x, gamma, eps):
        if kind == "centred":        # variance about the mean instead of the mean square
            ms = np.var(x, axis=1)
        elif kind == "sum":          # sum instead of mean
            ms = np.sum(x * x, axis=1)
        else:
            ms = np.mean(x * x, axis=1)
        rstd = 1.0 / (np.sqrt(ms) + eps) if kind == "eps_outside" else 1.0 / np.sqrt(ms + eps)
        return x * rstd[:, None] * gamma[None, :], rstd

    def bwd(x, gamma, rstd, g):
        xhat = x * rstd[:, None]
        gg = g * gamma[None, :]
        if kind == "no_correction":
            return rstd[:, None] * gg
        c = np.mean((g if kind == "gamma_dropped" else gg) * xhat, axis=1)
        return rstd[:, None] * (gg - xhat * c[:, None])

    return fwd, bwd


@pytest.mark.parametrize("kind", ["centred", "sum", "eps_outside", "no_correction", "gamma_dropped"])
def test_planted_mistakes_are_caught(kind):
    fwd, bwd = _mutant(kind)
    x, gamma, g = _draw(3, 6, seed=11)
    caught = not np.allclose(fwd(x, gamma, 0.5)[0], R.bruteforce(x, gamma, 0.5, g)[0], rtol=1e-9)
    # a mutant with the right forward must fail the gradient check
    caught = caught or _fd_norm(fwd, bwd, x, gamma, 0.5, g) > 1e-6
    assert caught, kind
