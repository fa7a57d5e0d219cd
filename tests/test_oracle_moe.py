"""Pins of the grouped (MoE) LoRA MLP oracle (no GPU).

Independent of the oracle's own code path: finite differences of <dY, y>
for x and for one expert's adapters, the scalar brute force of the (pinned)
MLP checker per expert, the partition identity (E copies of one expert give
the dense MLP, and the adapter gradients summed over experts give the
dense ones), consistency under a permutation of the experts, locality (an
expert's weights touch only its rows), empty groups, and planted mistakes
in the grouping that these pins must catch.
"""
import numpy as np
import pytest

from oracle import lora_mlp_oracle as M
from oracle import moe_oracle as MO


def _draw(E=3, counts=(2, 0, 3), H=5, I=4, r=2, seed=0):
    rng = np.random.default_rng(seed)
    T = int(sum(counts))
    inp = {"x": rng.normal(0, 1, (T, H)), "dy": rng.normal(0, 1, (T, H))}
    shapes = {"w_gate": (I, H), "w_up": (I, H), "w_down": (H, I), "a_gate": (r, H), "b_gate": (I, r),
              "a_up": (r, H), "b_up": (I, r), "a_down": (r, I), "b_down": (H, r)}
    for k, sh in shapes.items():
        inp[k] = rng.normal(0, 0.5, (E,) + sh)
    return inp, np.concatenate([[0], np.cumsum(counts)]).astype(int)


def test_finite_differences():
    inp, off = _draw(seed=1)
    s, h = 1.3, 1e-6
    got = MO.forward_backward(inp, off, s)
    worst = 0.0
    for name, idx_set in (("x", None), ("a_gate", 2), ("b_down", 0), ("a_down", 2), ("b_gate", 1)):
        arr = inp[name]
        sub = np.ndindex(*arr.shape) if idx_set is None else ((idx_set,) + t for t in np.ndindex(*arr.shape[1:]))
        for idx in sub:
            p, m = dict(inp), dict(inp)
            p[name] = arr.copy()
            m[name] = arr.copy()
            p[name][idx] += h
            m[name][idx] -= h
            num = (np.sum(inp["dy"] * MO.forward_backward(p, off, s)["y"])
                   - np.sum(inp["dy"] * MO.forward_backward(m, off, s)["y"])) / (2 * h)
            g = got["dx" if name == "x" else "d" + name][idx]
            worst = max(worst, abs(num - g) / max(1.0, abs(num)))
    assert worst < 1e-7


def test_bruteforce_per_expert():
    inp, off = _draw(seed=2)
    got = MO.forward_backward(inp, off, 0.7)
    for e in range(3):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        w = [inp[k][e] for k in M.WEIGHT_KEYS]
        bf = M.bruteforce(inp["x"][lo:hi], *w, 0.7, inp["dy"][lo:hi])
        for k in ("y", "dx"):
            np.testing.assert_allclose(got[k][lo:hi], bf[k], rtol=1e-10, atol=1e-12)
        for k in M.ADAPTER_KEYS:
            np.testing.assert_allclose(got[k][e], bf[k], rtol=1e-10, atol=1e-12)


def test_identical_experts_partition_the_dense_mlp():
    inp, off = _draw(E=4, counts=(3, 1, 0, 4), seed=3)
    for k in M.WEIGHT_KEYS:
        inp[k] = np.repeat(inp[k][:1], 4, axis=0)
    got = MO.forward_backward(inp, off, 2.0)
    dense = M.forward_backward({**{k: inp[k][0] for k in M.WEIGHT_KEYS}, "x": inp["x"], "dy": inp["dy"]}, 2.0)
    for k in ("y", "dx"):
        np.testing.assert_allclose(got[k], dense[k], rtol=1e-12, atol=1e-13)
    for k in M.ADAPTER_KEYS:
        np.testing.assert_allclose(got[k].sum(axis=0), dense[k], rtol=1e-11, atol=1e-13)
        np.testing.assert_array_equal(got[k][2], 0.0)  # the expert with no rows


def test_expert_permutation_and_locality():
    counts = (2, 3, 1)
    inp, off = _draw(E=3, counts=counts, seed=4)
    got = MO.forward_backward(inp, off, 1.1)
    perm = [2, 0, 1]  # new expert j is old expert perm[j]
    rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in perm])
    p = {k: inp[k][perm] for k in M.WEIGHT_KEYS}
    p["x"], p["dy"] = inp["x"][rows], inp["dy"][rows]
    poff = np.concatenate([[0], np.cumsum([counts[e] for e in perm])])
    q = MO.forward_backward(p, poff, 1.1)
    for k in ("y", "dx"):
        np.testing.assert_allclose(q[k], got[k][rows], rtol=1e-13, atol=1e-14)
    for k in M.ADAPTER_KEYS:
        np.testing.assert_allclose(q[k], got[k][perm], rtol=1e-13, atol=1e-14)
    # changing expert 1's weights leaves the rows and gradients of experts 0 and 2 alone
    inp2 = dict(inp)
    inp2["w_up"] = inp["w_up"].copy()
    inp2["w_up"][1] *= 3.0
    r2 = MO.forward_backward(inp2, off, 1.1)
    keep = np.r_[off[0]:off[1], off[2]:off[3]]
    np.testing.assert_array_equal(r2["y"][keep], got["y"][keep])
    assert not np.allclose(r2["y"][off[1]:off[2]], got["y"][off[1]:off[2]])


def test_rejects_bad_offsets():
    inp, _ = _draw(seed=5)
    for bad in ([0, 2, 1, 5], [1, 2, 2, 5], [0, 2, 2, 4]):
        with pytest.raises(ValueError):
            MO.forward_backward(inp, bad, 1.0)


def _mutant(kind):
    def fb(inp, off, s):
        E = len(off) - 1
        T, H = inp["x"].shape
        y = np.zeros((T, H))
        dx = np.zeros((T, H))
        g = {k: np.zeros((E,) + inp[k.replace("d", "", 1)].shape[1:]) for k in M.ADAPTER_KEYS}
        for e in range(E):
            lo, hi = int(off[e]), int(off[e + 1])
            if hi == lo:
                continue
            if kind == "shifted_rows":
                lo, hi = max(0, lo - 1), hi - 1 if hi - 1 > max(0, lo - 1) else hi
            we = (e + 1) % E if kind == "wrong_expert" else e
            d = {k: inp[k][we] for k in M.WEIGHT_KEYS}
            d["x"], d["dy"] = inp["x"][lo:hi], inp["dy"][lo:hi]
            out = M.forward_backward(d, s)
            y[lo:hi], dx[lo:hi] = out["y"], out["dx"]
            for k in M.ADAPTER_KEYS:
                # "accumulated": a running sum carried over from the earlier experts
                g[k][e] = out[k] + (g[k][e - 1] if kind == "accumulated" and e else 0)
        return {"y": y, "dx": dx, **g}
    return fb


@pytest.mark.parametrize("kind", ["shifted_rows", "wrong_expert", "accumulated"])
def test_planted_mistakes_are_caught(kind):
    inp, off = _draw(E=3, counts=(2, 3, 2), seed=6)
    got = _mutant(kind)(inp, off, 1.0)
    ref = MO.forward_backward(inp, off, 1.0)
    # the brute-force pin, per expert
    bad = False
    for e in range(3):
        lo, hi = off[e], off[e + 1]
        bf = M.bruteforce(inp["x"][lo:hi], *[inp[k][e] for k in M.WEIGHT_KEYS], 1.0, inp["dy"][lo:hi])
        bad |= not np.allclose(got["y"][lo:hi], bf["y"], rtol=1e-9)
        bad |= any(not np.allclose(got[k][e], bf[k], rtol=1e-9) for k in M.ADAPTER_KEYS)
    assert bad, kind
    assert not all(np.allclose(got[k], ref[k]) for k in ref)


def test_flop_count():
    assert MO.flops([0, 5, 9], 16, 32, 4) == M.flops(9, 16, 32, 4)
