"""GPU parity of the grouped (MoE) LoRA MLP (through the C ABI) against its
fp64 oracle: routed groups of uneven size, experts with no rows and with
one row, both dtypes, 4-bit weights, rank 64, the recompute mode and
determinism bitwise, the single-expert case against the plain MLP entry
point bit for bit, and the two full MoE workloads. Tolerance as for the
MLP: max|gpu-ref| / max|ref| <= 1e-4 (fp32), <= 2e-2 (bf16) per output."""
import time

import numpy as np
import pytest

from oracle import moe_oracle as MO
from lora_swiglu_mlp_amd import abi
from lora_swiglu_mlp_amd import inputs as I
from lmlp_testutil import TOL, compare, moe_oracle_inputs, run_hip, run_hip_moe

pytestmark = pytest.mark.gpu

CASES = {
    # name: (tokens, E, top_k, H, I, r, alpha, dtype, wfmt)
    "tiny_fp32": (96, 4, 2, 128, 344, 8, 16.0, "f32", "dense"),
    # more than 8 experts: tables and deferred launches, with products that
    # are not grouped (fp32, 4-bit weights) queued among the grouped ones
    "fp32_12experts": (160, 12, 2, 128, 264, 8, 16.0, "f32", "dense"),
    "int4_12experts": (240, 12, 3, 256, 384, 16, 16.0, "bf16", "int4_b64"),
    "bf16_routed": (300, 6, 2, 256, 520, 16, 32.0, "bf16", "dense"),
    "bf16_many_small": (200, 32, 4, 128, 256, 16, 16.0, "bf16", "dense"),
    "bf16_rank64": (160, 3, 2, 256, 384, 64, 128.0, "bf16", "dense"),
    "int4_routed": (128, 4, 2, 256, 384, 16, 16.0, "bf16", "int4_b64"),
}


def workload(name):
    tok, E, k, H, Iw, r, alpha, dt, wf = CASES[name]
    base = I.MOE_WORKLOADS["moe_tiny_fp32" if dt == "f32" else "moe_qwen3"]
    return base.replace(name=name, tokens=tok, experts=E, top_k=k, hidden=H, inter=Iw, rank=r, alpha=alpha,
                        dtype=dt, wfmt=wf)


def _oracle(inp, off, wl):
    return MO.forward_backward(moe_oracle_inputs(inp, wl), off, wl.scale, row_chunk=2048)


@pytest.mark.parametrize("name", list(CASES))
def test_moe_parity(name):
    wl = workload(name)
    inp, off = I.make_moe_inputs(wl)
    print(f"[case] moe {name} {CASES[name]} rows per expert {np.diff(off).tolist()}", flush=True)
    got, _ = run_hip_moe(inp, off, wl)
    compare(got, _oracle(inp, off, wl), TOL[wl.dtype], "moe " + name)
    assert all(np.isfinite(v).all() for v in got.values())


def _regroup(inp, counts):
    """The same tensors with the rows regrouped by the given per-expert counts."""
    return inp, np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def test_moe_empty_and_single_row_experts():
    wl = workload("bf16_routed")
    inp, off = I.make_moe_inputs(wl)
    T = int(off[-1])
    counts = [0, 1, T - 1 - 130, 0, 130, 0]  # experts 0, 3, 5 get no rows; expert 1 one row
    inp, off = _regroup(inp, counts)
    print(f"[case] moe empty/single rows per expert {counts}", flush=True)
    got, _ = run_hip_moe(inp, off, wl)
    ref = _oracle(inp, off, wl)
    compare(got, ref, TOL[wl.dtype], "moe empty/single")
    for e in (0, 3, 5):
        for k in ("da_gate", "db_gate", "da_up", "db_up", "da_down", "db_down"):
            assert not got[k][e].any(), (e, k)


def test_moe_recompute_consume_and_determinism_bitwise():
    wl = workload("bf16_routed")
    inp, off = I.make_moe_inputs(wl)
    a, _ = run_hip_moe(inp, off, wl)
    b, _ = run_hip_moe(inp, off, wl)
    c, _ = run_hip_moe(inp, off, wl, flags=abi.LMLP_RECOMPUTE_GU)
    d, _ = run_hip_moe(inp, off, wl, flags=abi.LMLP_CONSUME_SAVED)  # dG, dU in place of the saved G, U
    for k in a:
        assert np.array_equal(a[k], b[k]), k
        assert np.array_equal(a[k], c[k]), k
        assert np.array_equal(a[k], d[k]), k
    ref = _oracle(inp, off, wl)
    compare(c, ref, TOL[wl.dtype], "moe recompute")
    compare(d, ref, TOL[wl.dtype], "moe consume-saved")


def test_moe_one_expert_with_all_rows_equals_the_mlp_entry_point():
    """All rows routed to expert 1: its outputs are the plain MLP's on expert
    1's tensors bit for bit, and every other expert's gradients are zero."""
    wl = workload("bf16_routed")
    inp, off = I.make_moe_inputs(wl)
    T = int(off[-1])
    counts = [0, T, 0, 0, 0, 0]
    inp, off = _regroup(inp, counts)
    got, _ = run_hip_moe(inp, off, wl)
    single = {k: (v[1] if k not in ("x", "dy") else v) for k, v in inp.items()}
    ref, _ = run_hip(single, wl.replace(tokens=T))
    assert np.array_equal(got["y"], ref["y"]) and np.array_equal(got["dx"], ref["dx"])
    for k in ("da_gate", "db_gate", "da_up", "db_up", "da_down", "db_down"):
        assert np.array_equal(got[k][1], ref[k]), k
        assert not np.delete(got[k], 1, axis=0).any(), k


@pytest.mark.parametrize("name", ["moe_mixtral", "moe_qwen3"])
def test_moe_fullsize_parity(name):
    """The full MoE shapes against the oracle, and a second run bitwise equal
    to the first. At the Mixtral shape (8 experts, 592 tiles of the dX
    product on 256 compute units) the dX product runs as two K splits summed
    in order: the per-launch profile shows its sum."""
    wl = I.MOE_WORKLOADS[name]
    t0 = time.time()
    inp, off = I.make_moe_inputs(wl)
    print(f"[case] {name} tokens={wl.tokens} E={wl.experts} top{wl.top_k} rows={int(off[-1])} "
          f"H={wl.hidden} I={wl.inter} r={wl.rank}", flush=True)
    abi.lora_mlp_profile_begin()
    got, _ = run_hip_moe(inp, off, wl)
    names = {n for n, _ in abi.lora_mlp_profile_end()}
    again, _ = run_hip_moe(inp, off, wl)
    for k in got:
        assert np.array_equal(got[k], again[k]), k
    if name == "moe_mixtral" and torch_cus() == 256:
        assert "sum(dX)" in names, sorted(names)
    t1 = time.time()
    ref = _oracle(inp, off, wl)
    print(f"[time] inputs+gpu {t1 - t0:.1f}s oracle {time.time() - t1:.1f}s", flush=True)
    compare(got, ref, TOL[wl.dtype], name)


def torch_cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("name", ["int4_routed", "int4_12experts"])
def test_moe_int4_decode_modes_bitwise_equal(name):
    """4-bit weights decoded inside the products' staging (the default; those
    products are launched expert by expert, not grouped) give the outputs of
    the decoded-copy mode bit for bit; both are checked against the oracle."""
    wl = workload(name)
    inp, off = I.make_moe_inputs(wl)
    a, _ = run_hip_moe(inp, off, wl)
    b, _ = run_hip_moe(inp, off, wl, flags=abi.LMLP_INT4_BF16_COPIES)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    compare(b, _oracle(inp, off, wl), TOL[wl.dtype], "moe int4 copies")


def test_moe_more_experts_than_one_grouped_launch_holds():
    """600 experts, over 512 of them with rows (and some without): the grouped
    GEMMs take two launches (512 parameter blocks per launch) and the merged
    side kernels many chunks of their job arrays; against the oracle."""
    wl = workload("bf16_routed").replace(tokens=6000, experts=600, top_k=2, hidden=64, inter=128, rank=4,
                                         alpha=8.0)
    inp, off = I.make_moe_inputs(wl)
    counts = np.diff(off)
    assert (counts > 0).sum() > 512 and (counts == 0).any()
    print(f"[case] moe 600 experts rows {int(off[-1])} empty {int((counts == 0).sum())} max {int(counts.max())}",
          flush=True)
    got, _ = run_hip_moe(inp, off, wl)
    compare(got, _oracle(inp, off, wl), TOL[wl.dtype], "moe 600 experts")


def _moe600():
    wl = workload("bf16_routed").replace(tokens=6000, experts=600, top_k=2, hidden=64, inter=128, rank=4,
                                         alpha=8.0)
    inp, off = I.make_moe_inputs(wl)
    return wl, inp, off


def _moe_buffers(inp, off, wl):
    import torch
    from lora_swiglu_mlp_amd import mlp
    m, x, dy = mlp.moe_from_inputs(inp, off, wl, "cuda")
    saved = m.new_saved()
    y = torch.empty((int(off[-1]), wl.hidden), dtype=m.tdtype, device="cuda")
    grads = m.new_grads(x.device)
    m.workspace()
    return m, x, dy, saved, y, grads


def test_moe_parameter_tables_many_calls_in_flight():
    """Twelve forward+backward calls queued without a host wait, the tables
    over 1 MB per call at 600 experts. Every call gives the synchronised
    call's outputs bit for bit."""
    import torch
    wl, inp, off = _moe600()
    m, x, dy, saved, y, grads = _moe_buffers(inp, off, wl)
    m.forward(x, y, saved)
    m.backward(dy, x, saved, grads)
    torch.cuda.synchronize()
    ref = {"y": y.clone(), **{k: v.clone() for k, v in grads.items()}}
    outs = []
    for _ in range(12):
        yy = torch.empty_like(y)
        gg = {k: torch.empty_like(v) for k, v in grads.items()}
        m.forward(x, yy, saved)
        m.backward(dy, x, saved, gg)
        outs.append({"y": yy, **gg})
    torch.cuda.synchronize()
    for o in outs:
        for k in ref:
            assert torch.equal(o[k], ref[k]), k


def test_moe_deep_queue_of_calls():
    """128 forward+backward steps at the Qwen3-30B-A3B MoE shape queued
    without a host wait: the host can run more than one lap of the 16 MB
    pinned table ring ahead of the device, so tables meet regions whose
    earlier copies have not run yet and go through the copy kernels instead.
    Every eighth step's outputs (and the last step's) equal the synchronised
    step's bit for bit."""
    import torch
    wl = I.MOE_WORKLOADS["moe_qwen3"]
    inp, off = I.make_moe_inputs(wl)
    print(f"[case] moe_qwen3 deep queue: 128 steps, rows {int(off[-1])}", flush=True)
    m, x, dy, saved, y, grads = _moe_buffers(inp, off, wl)
    m.forward(x, y, saved)
    m.backward(dy, x, saved, grads)
    torch.cuda.synchronize()
    ref = {"y": y.clone(), **{k: v.clone() for k, v in grads.items()}}
    scratch = {"y": torch.empty_like(y), **{k: torch.empty_like(v) for k, v in grads.items()}}
    kept = []
    for i in range(128):
        o = {k: torch.empty_like(v) for k, v in ref.items()} if (i % 8 == 0 or i == 127) else scratch
        m.forward(x, o["y"], saved)
        m.backward(dy, x, saved, {k: o[k] for k in grads})
        if o is not scratch:
            kept.append((i, o))
    torch.cuda.synchronize()
    for i, o in kept:
        for k in ref:
            assert torch.equal(o[k], ref[k]), (i, k)


def test_moe_graph_capture_writes_the_tables_with_copy_kernels():
    """Captured into a HIP graph, the grouped GEMMs' parameter tables are
    written by copy kernels on the stream (no host ring). Three replays, with
    eager work and a synchronisation between them, each give the eager
    outputs bit for bit; the eager outputs match the oracle."""
    import torch
    wl, inp, off = _moe600()
    m, x, dy, saved, y, grads = _moe_buffers(inp, off, wl)
    m.forward(x, y, saved)
    m.backward(dy, x, saved, grads)
    torch.cuda.synchronize()
    ref = {"y": y.clone(), **{k: v.clone() for k, v in grads.items()}}
    got = {k: v.float().cpu().numpy().astype(np.float64) for k, v in ref.items()}
    compare(got, _oracle(inp, off, wl), TOL[wl.dtype], "moe 600 experts eager")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        m.forward(x, y, saved)
        m.backward(dy, x, saved, grads)
    torch.cuda.synchronize()
    for i in range(3):
        y.zero_()
        for v in grads.values():
            v.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"[graph] replay {i}", flush=True)
        assert torch.equal(y, ref["y"]), i
        for k, v in grads.items():
            assert torch.equal(v, ref[k]), (i, k)
