"""GPU parity at the full workload sizes, in the launch configuration the bench times.

Every output tensor is compared with the fp64 oracle computed in row chunks
over the whole token batch (the adapter gradients are sums over all tokens,
so no subsampling is possible for them). Each case costs tens of seconds of
host fp64 BLAS time.
"""
import time

import numpy as np
import pytest

import oracle
from lora_swiglu_mlp_amd import abi
from lora_swiglu_mlp_amd import inputs as I
from lmlp_testutil import TOL, compare, oracle_inputs, run_hip

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["llama3_8b", "llama3_8b_int4", "llama3_8b_int4_copies", "tinyllama_long",
                                  "qwen2_7b"])
def test_fullsize_parity(name):
    flags = 0
    if name.endswith("_copies"):  # 4-bit weights decoded into bf16 copies first
        name, flags = name[: -len("_copies")], abi.LMLP_INT4_BF16_COPIES
    wl = I.WORKLOADS[name]
    print(f"[case] {name} T={wl.tokens} H={wl.hidden} I={wl.inter} r={wl.rank} s={wl.scale} "
          f"{wl.dtype} {wl.wfmt}", flush=True)
    t0 = time.time()
    inp = I.make_inputs(wl)
    got, _ = run_hip(inp, wl, flags=flags)
    t1 = time.time()
    ref = oracle.forward_backward(oracle_inputs(inp, wl), wl.scale, row_chunk=2048)
    t2 = time.time()
    print(f"[time] inputs+gpu {t1 - t0:.1f}s oracle {t2 - t1:.1f}s", flush=True)
    compare(got, ref, TOL[wl.dtype], name)
    for k in ("da_gate", "db_gate", "da_up", "db_up", "da_down", "db_down"):
        assert np.linalg.norm(got[k]) > 0, k


def test_fullsize_recompute_mode_bitwise_equal():
    """The recompute mode at the Llama-3-8B MLP size, in the bench's launch
    configuration: bitwise equal to the default mode (checked against the
    oracle above)."""
    wl = I.WORKLOADS["llama3_8b"]
    print(f"[case] llama3_8b recompute", flush=True)
    inp = I.make_inputs(wl)
    a, _ = run_hip(inp, wl)
    b, _ = run_hip(inp, wl, flags=abi.LMLP_RECOMPUTE_GU)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    ref = oracle.forward_backward(oracle_inputs(inp, wl), wl.scale, row_chunk=2048)
    compare(b, ref, TOL[wl.dtype], "llama3_8b recompute")
