"""Code generation of the bf16 GEMM kernels (CPU: hipcc cross-compiles gfx950).

The K loops of the 256-wide-tile kernels keep their 256 fp32 accumulators in
place: no AGPR<->VGPR moves and no scratch traffic between the MFMAs. A change
elsewhere in a kernel (an epilogue, a helper in common.h) can shift register
allocation and put such moves into the loop, which has cost 10-20 % of the
GEMM time without changing any result, so no numerics test would notice.
"""
import collections
import os
import re
import subprocess

import pytest

from lora_swiglu_mlp_amd import build as B

MOVES = ("v_accvgpr_read", "v_accvgpr_write", "v_accvgpr_mov", "scratch_")


def _kernels(asm: str):
    """{kernel symbol: [instructions]} of a gfx950 assembly listing."""
    out = {}
    lines = asm.split("\n")
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\S*kernel\S*):", l)
        if not m:
            continue
        body = []
        for t in lines[i + 1:]:
            if t.startswith(".Lfunc_end"):
                break
            t = t.split(";")[0].strip()
            if t:
                body.append(t)
        out[m.group(1)] = body
    return out


def _k_loop(body):
    """Instructions of the loop (backward branch) that holds the most MFMAs."""
    labels = {l[:-1]: k for k, l in enumerate(body) if re.match(r"^\.LBB\w+:$", l)}
    best = None
    for k, l in enumerate(body):
        m = re.match(r"s_(?:cbranch_\w+|branch)\s+(\.LBB\w+)", l)
        if m and m.group(1) in labels and labels[m.group(1)] < k:
            seg = body[labels[m.group(1)]:k]
            n = sum("v_mfma" in x for x in seg)
            if best is None or n > best[0]:
                best = (n, seg)
    return best


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    try:
        cc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "gemm_bf16.s"
    flags = [f for f in B.HIPFLAGS if f != "-fPIC"]
    cmd = [cc] + flags + ["--cuda-device-only", "-S", os.path.join(B.CSRC, "gemm_bf16.hip"), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-3000:]
    return out.read_text()


def test_wide_tile_k_loops_keep_accumulators_in_place(gemm_asm):
    ks = _kernels(gemm_asm)
    checked = 0
    for name, body in ks.items():
        loop = _k_loop(body)
        assert loop is not None, name
        nmfma, seg = loop
        # 256-wide tiles: 8 x 8 MFMAs per wave and k-tile, two k-tiles per
        # iteration
        if nmfma not in (64, 128) or ("gemm_bf16" in name and nmfma != 128):
            continue
        ops = collections.Counter(i.split()[0] for i in seg)
        bad = {o: c for o, c in ops.items() if o.startswith(MOVES)}
        assert not bad, f"{name}: {bad}"
        checked += 1
    # the four-wave kernels: plain NT and NN, their grouped and table-driven
    # forms (gate/up and dZ run on eight waves, checked below)
    assert checked >= 6, checked


def _dma_loops(body):
    """Backward-branch loops that issue LDS DMA (the K loops of the staged kernels)."""
    labels = {l[:-1]: k for k, l in enumerate(body) if re.match(r"^\.LBB\w+:$", l)}
    out = []
    for k, l in enumerate(body):
        m = re.match(r"s_(?:cbranch_\w+|branch)\s+(\.LBB\w+)", l)
        if m and m.group(1) in labels and labels[m.group(1)] < k:
            seg = body[labels[m.group(1)]:k]
            if any(x.startswith("buffer_load_dwordx4") and x.endswith("lds") for x in seg):
                out.append(seg)
    return out


def test_eight_wave_k_loops_keep_accumulators_in_place(gemm_asm):
    """The eight-wave ping-pong kernels (dense, 4-bit, and the grouped forms
    of the MoE path): 128 accumulators per lane, 32 MFMAs per k-tile, no
    accumulator moves or scratch traffic in the K loop, and at most 256
    registers per lane so that two waves fit one SIMD."""
    ks = _kernels(gemm_asm)
    names = [n for n in ks if "gemm8" in n]
    assert len(names) >= 14, names
    for name in names:
        loops = [x for x in _dma_loops(ks[name]) if sum("v_mfma" in i for i in x) == 32]
        assert loops, name
        seg = max(loops, key=len)
        ops = collections.Counter(i.split()[0] for i in seg)
        bad = {o: c for o, c in ops.items() if o.startswith(MOVES)}
        assert not bad, f"{name}: {bad}"
        assert ops["s_barrier"] == 2, (name, ops["s_barrier"])
    for name in names:
        m = re.search(r"\.set " + re.escape(name) + r"\.num_vgpr, (\d+)", gemm_asm)
        a = re.search(r"\.set " + re.escape(name) + r"\.num_agpr, (\d+)", gemm_asm)
        assert m and a, name
        assert int(m.group(1)) + int(a.group(1)) <= 256, (name, m.group(1), a.group(1))
