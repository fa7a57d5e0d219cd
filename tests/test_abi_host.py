"""C ABI checks that need no GPU: symbols, size queries, argument validation.

Validation runs before any HIP call, so every error path below returns
without touching a device. Pointers here are fake aligned addresses; no call
in this file reaches a kernel launch.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from lora_swiglu_mlp_amd import abi

FAKE = 0x10000  # 16-byte aligned, never dereferenced (validation fails first)


def dims(**kw):
    base = dict(tokens=256, hidden=128, inter=344, rank=8, scale=2.0, dtype="bf16", wfmt="dense")
    base.update(kw)
    return abi.make_dims(**base)


def test_library_exports_every_header_symbol():
    names = abi.header_functions()
    assert set(names) == {"lora_mlp_saved_bytes", "lora_mlp_workspace_bytes", "lora_mlp_forward",
                          "lora_mlp_backward", "lora_mlp_dequant_int4", "lora_mlp_status_string",
                          "lora_mlp_last_error", "lora_mlp_profile_begin", "lora_mlp_profile_end",
                          "lora_linear_saved_bytes", "lora_linear_workspace_bytes", "lora_linear_forward",
                          "lora_linear_backward", "lora_linear_forward_noalloc", "lora_mlp_mfma_probe",
                          "lora_mlp_norm_forward", "lora_mlp_norm_backward",
                          "lora_moe_saved_bytes", "lora_moe_workspace_bytes", "lora_moe_forward",
                          "lora_moe_backward"}
    L = abi.lib()
    for n in names:
        assert hasattr(L, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", abi.LIB_PATH], capture_output=True, text=True)
    exported = {l.split()[-1] for l in nm.stdout.splitlines() if " T " in l}
    assert set(names) <= exported


def test_header_compiles_as_c():
    src = '#include "lora_mlp.h"\nint main(void){lmlp_dims d; (void)d; return 0;}\n'
    out = subprocess.run(["gcc", "-x", "c", "-std=c99", "-Wall", "-Werror", "-fsyntax-only",
                          "-I", os.path.dirname(abi.HEADER), "-"], input=src, capture_output=True,
                         text=True)
    assert out.returncode == 0, out.stderr


def align(n):
    return (n + 255) // 256 * 256


@pytest.mark.parametrize("T,H,I,r,dt", [(256, 128, 344, 8, "f32"), (4096, 4096, 14336, 16, "bf16"),
                                        (8192, 3584, 18944, 64, "bf16"), (0, 64, 64, 4, "bf16")])
def test_saved_bytes_formula(T, H, I, r, dt):
    eb = 2 if dt == "bf16" else 4
    r16 = (r + 15) // 16 * 16
    # G, U; P_gu, P_d (fp32); the adapter factors packed for both passes:
    # [A_g; A_u], A_d, B_d^T, B_g^T, B_u^T (rank rows padded to r16)
    # and B_g, B_u as [I, 2 r16], the gate/up product's adapter segment
    packed = (align(2 * r16 * H * eb) + align(r16 * I * eb) + align(r16 * H * eb) + 2 * align(r16 * I * eb)
              + 2 * align(I * 2 * r16 * eb))
    want = 2 * align(T * I * eb) + align(T * 2 * r16 * 4) + align(T * r16 * 4) + packed
    assert abi.lora_mlp_saved_bytes(dims(tokens=T, hidden=H, inter=I, rank=r, dtype=dt)) == want
    # only the gate/up pre-activations are kept at activation size: no SiLU(G), no Z
    assert want <= 2 * T * I * eb + 3 * T * r16 * 4 + 7 * r16 * (H + I) * eb + 11 * 256
    # full recompute: no activation-sized tensor at all
    rc = abi.lora_mlp_saved_bytes(dims(tokens=T, hidden=H, inter=I, rank=r, dtype=dt, flags=abi.LMLP_RECOMPUTE_GU))
    assert rc == want - 2 * align(T * I * eb)


def test_workspace_sizes_positive_and_consume_flag_saves_memory():
    d = dims(tokens=4096, hidden=4096, inter=14336, rank=16)
    fw, bw = abi.lora_mlp_workspace_bytes(d, False), abi.lora_mlp_workspace_bytes(d, True)
    assert fw > 4096 * 14336 * 2 and bw > fw
    dc = dims(tokens=4096, hidden=4096, inter=14336, rank=16, flags=abi.LMLP_CONSUME_SAVED)
    assert abi.lora_mlp_workspace_bytes(dc, True) == bw - 2 * align(4096 * 14336 * 2)
    # full recompute: G, U come back into the backward workspace and dG, dU
    # overwrite them, so it is as large as without the flag; the forward's
    # does not change
    dr = dims(tokens=4096, hidden=4096, inter=14336, rank=16, flags=abi.LMLP_RECOMPUTE_GU)
    assert abi.lora_mlp_workspace_bytes(dr, True) == bw
    assert abi.lora_mlp_workspace_bytes(dr, False) == fw


@pytest.mark.parametrize("kw,code", [
    (dict(rank=0), abi.LMLP_ERR_INVALID_ARG),
    (dict(tokens=-1), abi.LMLP_ERR_INVALID_ARG),
    (dict(hidden=0), abi.LMLP_ERR_INVALID_ARG),
    (dict(scale=float("nan")), abi.LMLP_ERR_INVALID_ARG),
    (dict(scale=float("inf")), abi.LMLP_ERR_INVALID_ARG),
    (dict(dtype=7), abi.LMLP_ERR_INVALID_ARG),
    (dict(wfmt=3), abi.LMLP_ERR_INVALID_ARG),
    (dict(flags=0x20), abi.LMLP_ERR_INVALID_ARG),
    (dict(flags=abi.LMLP_INT4_INKERNEL | abi.LMLP_INT4_BF16_COPIES), abi.LMLP_ERR_INVALID_ARG),
    (dict(flags=0x8), abi.LMLP_ERR_INVALID_ARG),  # the norm flag on the plain entry point
    (dict(rank=257), abi.LMLP_ERR_UNSUPPORTED),
    (dict(hidden=132), abi.LMLP_ERR_UNSUPPORTED),          # not a multiple of 8 for bf16
    (dict(inter=346, dtype="f32"), abi.LMLP_ERR_UNSUPPORTED),  # not a multiple of 4
    (dict(wfmt="int4_b64", dtype="f32"), abi.LMLP_ERR_UNSUPPORTED),
    (dict(wfmt="int4_b64", inter=344), abi.LMLP_ERR_UNSUPPORTED),  # not a multiple of 64
    # 128 token-contiguous bf16 rows of roundup(T, 64) must stay below 2^32 bytes
    (dict(tokens=(1 << 24) - 63), abi.LMLP_ERR_UNSUPPORTED),
    (dict(tokens=1 << 24), abi.LMLP_ERR_UNSUPPORTED),
    (dict(hidden=(1 << 22) + 8), abi.LMLP_ERR_UNSUPPORTED),
])
def test_invalid_dims_rejected(kw, code):
    d = dims(**kw)
    if kw.get("flags") != abi.LMLP_RMSNORM:  # valid dims, wrong entry point
        assert abi.lora_mlp_saved_bytes(d) == 0
        assert abi.lora_mlp_workspace_bytes(d, True) == 0
    rc = _forward_raw(d, saved_bytes=1 << 40, workspace_bytes=1 << 40)
    assert rc == code, abi.lora_mlp_last_error()
    assert abi.lora_mlp_last_error()


def test_largest_token_count_is_accepted():
    d = dims(tokens=(1 << 24) - 64, hidden=64, inter=64, rank=64)
    assert abi.lora_mlp_saved_bytes(d) > 0 and abi.lora_mlp_workspace_bytes(d, True) > 0


def _forward_raw(d, ptrs=None, saved_bytes=0, workspace_bytes=0, scales=(None, None, None)):
    p = dict.fromkeys(["x", "wg", "wu", "wd", "ag", "bg", "au", "bu", "ad", "bd", "y", "saved", "ws"],
                      FAKE)
    p.update(ptrs or {})
    return abi.lib().lora_mlp_forward(
        ctypes.byref(d), p["x"], p["wg"], scales[0], p["wu"], scales[1], p["wd"], scales[2],
        p["ag"], p["bg"], p["au"], p["bu"], p["ad"], p["bd"], p["y"], p["saved"], saved_bytes,
        p["ws"], workspace_bytes, None)


def _backward_raw(d, ptrs=None, saved_bytes=0, workspace_bytes=0):
    names = ["dy", "x", "wg", "wu", "wd", "ag", "bg", "au", "bu", "ad", "bd", "saved", "dx", "dag",
             "dbg", "dau", "dbu", "dad", "dbd", "ws"]
    p = dict.fromkeys(names, FAKE)
    p.update(ptrs or {})
    return abi.lib().lora_mlp_backward(
        ctypes.byref(d), p["dy"], p["x"], p["wg"], None, p["wu"], None, p["wd"], None, p["ag"],
        p["bg"], p["au"], p["bu"], p["ad"], p["bd"], p["saved"], saved_bytes, p["dx"], p["dag"],
        p["dbg"], p["dau"], p["dbu"], p["dad"], p["dbd"], p["ws"], workspace_bytes, None)


@pytest.mark.parametrize("name", ["x", "wg", "ag", "bd", "y", "saved", "ws"])
def test_forward_null_and_misaligned_pointers(name):
    d = dims()
    big = 1 << 40
    assert _forward_raw(d, {name: None}, big, big) == abi.LMLP_ERR_INVALID_ARG
    assert "NULL" in abi.lora_mlp_last_error()
    assert _forward_raw(d, {name: FAKE + 8}, big, big) == abi.LMLP_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ["dy", "dx", "dag", "dbd", "saved", "ws"])
def test_backward_null_pointers(name):
    big = 1 << 40
    assert _backward_raw(dims(), {name: None}, big, big) == abi.LMLP_ERR_INVALID_ARG


def test_scale_pointer_rules():
    big = 1 << 40
    d = dims()
    assert _forward_raw(d, None, big, big, scales=(FAKE, None, None)) == abi.LMLP_ERR_INVALID_ARG
    d4 = dims(wfmt="int4_b64", hidden=128, inter=384)
    assert _forward_raw(d4, None, big, big, scales=(FAKE, None, FAKE)) == abi.LMLP_ERR_INVALID_ARG


def test_small_buffers_rejected():
    d = dims()
    sb = abi.lora_mlp_saved_bytes(d)
    wb = abi.lora_mlp_workspace_bytes(d, False)
    assert _forward_raw(d, None, sb - 1, wb) == abi.LMLP_ERR_WORKSPACE
    assert _forward_raw(d, None, sb, wb - 1) == abi.LMLP_ERR_WORKSPACE
    bb = abi.lora_mlp_workspace_bytes(d, True)
    assert _backward_raw(d, None, sb, bb - 1) == abi.LMLP_ERR_WORKSPACE


def test_dequant_argument_checks():
    L = abi.lib()
    assert L.lora_mlp_dequant_int4(FAKE, FAKE, 4, 96, FAKE, None) == abi.LMLP_ERR_UNSUPPORTED
    assert L.lora_mlp_dequant_int4(FAKE, FAKE, -1, 64, FAKE, None) == abi.LMLP_ERR_INVALID_ARG
    assert L.lora_mlp_dequant_int4(None, FAKE, 4, 64, FAKE, None) == abi.LMLP_ERR_INVALID_ARG
    assert L.lora_mlp_dequant_int4(None, None, 0, 64, None, None) == abi.LMLP_OK  # empty


def test_status_strings():
    assert abi.lora_mlp_status_string(0) == "LMLP_OK"
    assert abi.lora_mlp_status_string(3) == "LMLP_ERR_WORKSPACE"
    assert abi.lora_mlp_status_string(99) == "LMLP_UNKNOWN_STATUS"


def test_python_binding_raises():
    with pytest.raises(abi.LoraMLPError) as e:
        abi.lora_mlp_forward(dims(rank=0), *([FAKE] * 14), saved=FAKE, workspace=FAKE, stream=0,
                             saved_bytes=0, workspace_bytes=0)
    assert e.value.status == abi.LMLP_ERR_INVALID_ARG


def test_profile_session_without_launches():
    abi.lora_mlp_profile_begin()
    assert abi.lora_mlp_profile_end() == []


@pytest.mark.parametrize("T,n_in,n_out,r,dt", [(256, 128, 344, 8, "f32"), (4096, 4096, 1024, 16, "bf16"),
                                               (0, 64, 64, 4, "bf16")])
def test_linear_saved_bytes_formula(T, n_in, n_out, r, dt):
    eb = 2 if dt == "bf16" else 4
    r16 = (r + 15) // 16 * 16
    ldT = (T + 63) // 64 * 64
    want = (align(T * r16 * 4) + (align(r16 * ldT * eb) if dt == "bf16" else 0) + align(r16 * n_in * eb)
            + align(n_out * r16 * eb) + align(r16 * n_out * eb))
    d = dims(tokens=T, hidden=n_in, inter=n_out, rank=r, dtype=dt)
    assert abi.lora_linear_saved_bytes(d) == want
    if T > 0:
        assert abi.lora_linear_workspace_bytes(d, False) > 0 and abi.lora_linear_workspace_bytes(d, True) > 0


def test_linear_rejects_the_mlp_only_flags():
    for f in (abi.LMLP_CONSUME_SAVED, abi.LMLP_RECOMPUTE_GU):
        assert abi.lora_linear_saved_bytes(dims(flags=f)) == 0
    assert abi.lora_linear_saved_bytes(dims(inter=384, wfmt="int4_b64", flags=abi.LMLP_INT4_INKERNEL)) > 0


def _norm_forward_raw(d, eps=1e-5, gamma=FAKE, saved_bytes=1 << 40, workspace_bytes=1 << 40):
    return abi.lib().lora_mlp_norm_forward(
        ctypes.byref(d), eps, FAKE, gamma, FAKE, None, FAKE, None, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
        FAKE, FAKE, saved_bytes, FAKE, workspace_bytes, None)


def _norm_backward_raw(d, gamma=FAKE, saved_bytes=1 << 40, workspace_bytes=1 << 40):
    return abi.lib().lora_mlp_norm_backward(
        ctypes.byref(d), FAKE, FAKE, gamma, FAKE, None, FAKE, None, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
        FAKE, FAKE, saved_bytes, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, workspace_bytes, None)


@pytest.mark.parametrize("T,H,I,r,dt", [(256, 128, 344, 8, "f32"), (4096, 4096, 14336, 16, "bf16"), (0, 64, 64, 4, "bf16")])
def test_norm_sizes(T, H, I, r, dt):
    eb = 2 if dt == "bf16" else 4
    base = dims(tokens=T, hidden=H, inter=I, rank=r, dtype=dt)
    nd = dims(tokens=T, hidden=H, inter=I, rank=r, dtype=dt, flags=abi.LMLP_RMSNORM)
    # saved: one fp32 statistic per token row; each workspace: the normalised rows
    assert abi.lora_mlp_saved_bytes(nd) == abi.lora_mlp_saved_bytes(base) + align(4 * T)
    for bwd in (False, True):
        assert abi.lora_mlp_workspace_bytes(nd, bwd) == abi.lora_mlp_workspace_bytes(base, bwd) + align(T * H * eb)


def test_norm_entry_point_argument_checks():
    nd = dims(flags=abi.LMLP_RMSNORM)
    plain = dims()
    assert _norm_forward_raw(plain) == abi.LMLP_ERR_INVALID_ARG      # flag missing
    assert "LMLP_RMSNORM" in abi.lora_mlp_last_error()
    assert _norm_backward_raw(plain) == abi.LMLP_ERR_INVALID_ARG
    for eps in (float("nan"), float("inf"), -1e-6):
        assert _norm_forward_raw(nd, eps=eps) == abi.LMLP_ERR_INVALID_ARG
    assert _norm_forward_raw(nd, gamma=None) == abi.LMLP_ERR_INVALID_ARG
    assert _norm_forward_raw(nd, gamma=FAKE + 4) == abi.LMLP_ERR_INVALID_ARG
    assert _norm_backward_raw(nd, gamma=None) == abi.LMLP_ERR_INVALID_ARG
    assert _norm_forward_raw(nd, saved_bytes=16) == abi.LMLP_ERR_WORKSPACE
    assert _norm_backward_raw(nd, workspace_bytes=16) == abi.LMLP_ERR_WORKSPACE
    assert _backward_raw(nd, saved_bytes=1 << 40, workspace_bytes=1 << 40) == abi.LMLP_ERR_INVALID_ARG
    assert abi.lora_linear_saved_bytes(dims(flags=abi.LMLP_RMSNORM)) == 0


def _moe_forward_raw(d, offsets, saved_bytes=1 << 40, workspace_bytes=1 << 40):
    off = abi.offsets_array(offsets) if offsets is not None else None
    n = len(offsets) - 1 if offsets is not None else 1
    return abi.lib().lora_moe_forward(
        ctypes.byref(d), n, off, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
        FAKE, FAKE, saved_bytes, FAKE, workspace_bytes, None)


@pytest.mark.parametrize("counts,dt", [((3, 0, 5, 1), "bf16"), ((4096, 2048, 2048, 0), "bf16"), ((7, 9), "f32"),
                                       (tuple(range(10)), "bf16")])
def test_moe_sizes(counts, dt):
    T = sum(counts)
    off = [0] + list(np.cumsum(counts))
    d = dims(tokens=T, hidden=256, inter=512, rank=16, dtype=dt)
    per = [dims(tokens=c, hidden=256, inter=512, rank=16, dtype=dt) for c in counts]
    # one saved and one workspace region per expert (an expert without rows
    # needs no workspace): every expert's intermediates stay resident across
    # the phases of the grouped launches
    assert abi.lora_moe_saved_bytes(d, off) == sum(abi.lora_mlp_saved_bytes(p) for p in per)
    # more experts than one launch's arguments hold (8): the region for one
    # pass's tables follows, room for four GEMM kinds' 416-byte parameter
    # blocks and four side launches of 10 jobs of at most 96 bytes per expert
    table = 4 * (align(len(counts) * 416) + align(len(counts) * 10 * 96)) if len(counts) > 8 else 0
    for bwd in (False, True):
        assert abi.lora_moe_workspace_bytes(d, off, bwd) == table + sum(abi.lora_mlp_workspace_bytes(p, bwd)
                                                                        for c, p in zip(counts, per) if c > 0)


def test_moe_argument_checks():
    d = dims(tokens=10)
    good = [0, 4, 10]
    assert abi.lora_moe_saved_bytes(d, good) > 0
    for bad in ([0, 5, 4, 10], [1, 4, 10], [0, 4, 9], [0, 4, 11]):
        assert abi.lora_moe_saved_bytes(d, bad) == 0
        assert _moe_forward_raw(d, bad) == abi.LMLP_ERR_INVALID_ARG
    assert _moe_forward_raw(d, None) == abi.LMLP_ERR_INVALID_ARG  # offsets NULL
    assert "offsets" in abi.lora_mlp_last_error()
    assert abi.lib().lora_moe_saved_bytes(ctypes.byref(d), 0, abi.offsets_array([0])) == 0  # no experts
    assert abi.lora_moe_saved_bytes(dims(tokens=10, flags=abi.LMLP_RMSNORM), good) == 0
    assert _moe_forward_raw(d, good, saved_bytes=16) == abi.LMLP_ERR_WORKSPACE
    assert _moe_forward_raw(d, good, workspace_bytes=16) == abi.LMLP_ERR_WORKSPACE


def test_binding_argument_counts_match_the_header():
    """Every ctypes signature has as many arguments as the header prototype."""
    import re
    with open(abi.HEADER) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    for name, (_, args) in abi._SIGS.items():
        m = re.search(r"\b" + name + r"\s*\(([^)]*)\)", text)
        assert m, name
        params = [p for p in m.group(1).split(",") if p.strip() and p.strip() != "void"]
        assert len(params) == len(args), (name, len(params), len(args))


def test_noalloc_linear_rejects_workspace_beyond_the_scratch():
    """lora_linear_forward_noalloc refuses, before any device call, dims whose
    forward workspace exceeds the library's scratch array; the header's size
    is the binding's."""
    with open(abi.HEADER) as f:
        m = re.search(r"#define LMLP_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == abi.LMLP_NOALLOC_SCRATCH_BYTES
    big = dims(tokens=1 << 20, hidden=4096, inter=4096, rank=64, scale=2.0)
    assert abi.lora_linear_workspace_bytes(big, False) > abi.LMLP_NOALLOC_SCRATCH_BYTES
    rc = abi.lib().lora_linear_forward_noalloc(ctypes.byref(big), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                                               1 << 40, None)
    assert rc == abi.LMLP_ERR_UNSUPPORTED and "scratch" in abi.lora_mlp_last_error()
    bad = dims(rank=0)
    rc = abi.lib().lora_linear_forward_noalloc(ctypes.byref(bad), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                                               1 << 40, None)
    assert rc == abi.LMLP_ERR_INVALID_ARG


def test_int4_workspaces_hold_no_bf16_weights_by_default():
    """4-bit weights decoded in the GEMM staging (the default): the forward
    and backward workspaces of the Llama-3-8B MLP are within a few MB of the
    dense bf16 ones (fp32 block scales only); the decoded-copy mode adds the
    2 (2 I H + H I) bytes of bf16 weights to each."""
    T, H, I, r = 4096, 4096, 14336, 16
    dense = dims(tokens=T, hidden=H, inter=I, rank=r, scale=1.0)
    q4 = dims(tokens=T, hidden=H, inter=I, rank=r, scale=1.0, wfmt="int4_b64")
    cp = dims(tokens=T, hidden=H, inter=I, rank=r, scale=1.0, wfmt="int4_b64", flags=abi.LMLP_INT4_BF16_COPIES)
    for bwd in (False, True):
        wd = abi.lora_mlp_workspace_bytes(dense, bwd)
        wq = abi.lora_mlp_workspace_bytes(q4, bwd)
        assert wd < wq < wd + 16 * 2**20, (bwd, wd, wq)
        assert abi.lora_mlp_workspace_bytes(cp, bwd) >= wd + 2 * (2 * I * H + H * I), bwd


def test_mfma_probe_validates_before_launching():
    L = abi.lib()
    assert L.lora_mlp_mfma_probe(None, 1 << 20, FAKE, 1, 1, None) == abi.LMLP_ERR_INVALID_ARG
    assert L.lora_mlp_mfma_probe(FAKE, 1 << 20, FAKE, 0, 1, None) == abi.LMLP_ERR_INVALID_ARG
    assert L.lora_mlp_mfma_probe(FAKE, 1 << 20, FAKE, 1, 0, None) == abi.LMLP_ERR_INVALID_ARG
    assert L.lora_mlp_mfma_probe(FAKE, 8 * 768 * 16 - 1, FAKE, 1, 1, None) == abi.LMLP_ERR_INVALID_ARG
