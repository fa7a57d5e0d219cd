#!/usr/bin/env python3
"""Throughput of the fused LoRA SwiGLU MLP forward + backward on one MI355X.

One step = lora_mlp_forward + lora_mlp_backward over one batch of synthetic
tokens (inputs resident in HBM before timing starts). Default workload: the
Llama-3-8B MLP (hidden 4096, intermediate 14336, rank 16, alpha 16) over 4096
tokens (batch 2 x seq 2048) in bf16. Prints one JSON line.

Also reported:
  roofline      the dominant kernel's algorithmic TFLOP/s against the MI355X
                dense MFMA peak of the workload dtype, from HIP events recorded
                around each library launch on the launch stream (a second pass
                of the same steps, so event records do not touch `value`)
  cpu_baseline  the fp64 CPU oracle on a bounded token sample of the same
                workload, on this host's cores
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LoRA-SwiGLU MLP fwd+bwd tokens/sec + TFLOP/s as % of MI355X bf16 peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}    # MI355X published dense MFMA peaks
HBM_PEAK_GBS = 8000.0


def dz_split(T: int, I: int, ncu: int) -> int:
    """Columns of the bf16 dZ product that the library gives 256-wide tiles
    (the rest runs as a second launch of 128-wide tiles): the rule of the
    library's dZ launch, restated for the FLOP accounting of each launch."""
    tm, tn = (T + 255) // 256, (I + 255) // 256
    tiles = tm * tn
    rem = tiles % ncu
    if tiles <= ncu or rem == 0 or 2 * rem > ncu:
        return I
    ntail = (rem + tm - 1) // tm
    if ntail >= tn or tm * ntail * 2 > ncu:
        return I
    return (tn - ntail) * 256


def kernel_flops(name: str, T: int, H: int, I: int, r: int, linear: bool = False, dz_cols=None) -> int:
    """Algorithmic FLOPs of one launch (2mnk per product, real rank, no padding).
    For the fused LoRA linear, H is the input and I the output width. The dZ
    product may run as two launches over the columns [0, dz_cols) and
    [dz_cols, I); each is credited with its own columns."""
    if linear:
        return {"gemm(y)": 2 * T * H * I + 2 * T * r * I, "gemm(dX)": 2 * T * I * H + 2 * T * r * H}.get(name, 0)
    n1 = I if dz_cols is None else dz_cols
    return {
        "gemm(gate/up)": 4 * T * H * I + 4 * T * I * r,
        "gemm(gate/up, recompute)": 4 * T * H * I + 4 * T * I * r,
        "gemm(down)": 2 * T * I * H + 2 * T * H * r,
        "gemm(dZ)": 2 * T * H * n1 + 2 * T * r * n1,
        "gemm(dZ tail)": 2 * T * H * (I - n1) + 2 * T * r * (I - n1),
        "gemm(dX)": 4 * T * I * H + 4 * T * r * H,
    }.get(name, 0)


# the four products of the step, each summed over its launches
GEMM_GROUPS = {"gate/up": ("gemm(gate/up)",), "down": ("gemm(down)",), "dZ": ("gemm(dZ)", "gemm(dZ tail)"),
               "dX": ("gemm(dX)",)}


def gemm_table(kern: dict, T: int, H: int, I: int, r: int, peak: float, dz_cols=None) -> dict:
    """ms per step, TFLOP/s and fraction of peak of each of the four products
    (a product launched twice is one product over both launches' time)."""
    out = {}
    for g, names in GEMM_GROUPS.items():
        ms = sum(kern[n]["ms"] * kern[n]["launches_per_step"] for n in names if n in kern)
        f = sum(kernel_flops(n, T, H, I, r, dz_cols=dz_cols) for n in names if n in kern)
        if ms > 0 and f > 0:
            tf = f / (ms * 1e-3) / 1e12
            out[g] = {"ms": ms, "tflops": tf, "frac": tf / peak}
    return out


def kernel_bytes(name: str, T: int, H: int, I: int, r: int, eb: int) -> int:
    """Algorithmic HBM bytes of one launch of the rank-r side kernels. bf16 at
    rank <= 16 forms the products of dG, dU and Z in the dZ epilogue, and the
    column projection then reads only X and dY."""
    fused = eb == 2 and r <= 16
    return {
        "rowproj(X A^T)": T * H * eb + T * 2 * r * (4 + eb),
        "rowproj(Z A_d^T)": T * I * eb + T * r * (4 + eb),
        "rowproj(dY B_d)": T * H * eb + T * r * (4 + eb),
        "rowproj(dG B_g, dU B_u)": 2 * T * I * eb + 2 * T * r * (4 + eb),
        "colproj": (2 * T * H if fused else 3 * T * I + 2 * T * H) * eb,
        # RMSNorm in front of the MLP: x in, xn out (+ the fp32 row statistic);
        # the backward reads x and g and writes dx
        "rmsnorm(fwd)": 2 * T * H * eb + 4 * T,
        "rmsnorm(apply)": 2 * T * H * eb + 4 * T,
        "rmsnorm(bwd)": 3 * T * H * eb + 4 * T,
    }.get(name, 0)


def moe_gemm_bytes(name: str, rows: int, experts: int, H: int, I: int, r: int, eb: int) -> int:
    """Algorithmic HBM bytes of one grouped (MoE) product over all routed
    rows: every operand read once (the weights of each expert with rows, the
    activations of every routed row, the rank-r adapter segments) and every
    output written once."""
    return {
        # X, W_g and W_u; P_g, P_u [rows, 2r] and the B_g, B_u segments; G, U, Z out
        "gemm(gate/up)": (rows * H + experts * 2 * I * H + rows * 2 * r + experts * 2 * I * r + 3 * rows * I) * eb,
        # Z, W_d, the adapter segments; y out
        "gemm(down)": (rows * I + experts * H * I + rows * r + experts * H * r + rows * H) * eb,
        # dY, W_d, G, U in; dG, dU out
        "gemm(dZ)": (rows * H + experts * H * I + 4 * rows * I) * eb,
        # dG, dU, W_g, W_u, the adapter segments in; dX out
        "gemm(dX)": (2 * rows * I + experts * 2 * I * H + rows * 2 * r + experts * 2 * r * H + rows * H) * eb,
    }.get(name, 0)


# sources of the bf16 GEMM kernels: a measured HBM traffic figure applies only
# while these are unchanged
GEMM_SOURCES = ("lora_swiglu_mlp_amd/csrc/gemm_bf16.hip", "lora_swiglu_mlp_amd/csrc/lds_dma.h",
                "lora_swiglu_mlp_amd/csrc/common.h")


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the counter summary in profiles/
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading), or None when
    there is none for the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    want = gemm_source_hash()
    with open(path) as f:
        for line in f:
            m = re.match(r"^traffic_json: (\{.*\})\s*$", line)
            if m:
                rec = json.loads(m.group(1))
                if rec.get("kernel") == kernel and rec.get("source_sha256_16") == want:
                    return float(rec["bytes_per_launch"])
    return None


def mfma_ceiling(reps: int = 40, iters: int = 4096) -> dict:
    """The bf16 matrix-core ceiling measured on this GPU: the library's probe
    (8 waves per compute unit, 32 independent 16x16x32 MFMAs each on random
    operand bits, no memory traffic) launched `reps` times on the current
    stream; the rate is the median of the last 10 launches, after the clock
    has settled under the load."""
    import torch
    from lora_swiglu_mlp_amd import abi
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    gen = torch.Generator().manual_seed(1)
    ops = torch.randn(ncu * 8 * 768 * 8, generator=gen).to(torch.bfloat16).to("cuda:0")
    sink = torch.empty(ncu * 512, dtype=torch.float32, device="cuda:0")
    flops = ncu * 8 * iters * 32 * 16384
    ms = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        abi.lora_mlp_mfma_probe(ops, sink, ncu, iters)
        e1.record()
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    last = sorted(ms[-10:])
    med = (last[4] + last[5]) / 2
    return {"tflops": flops / (med * 1e-3) / 1e12, "ms_per_launch": med, "launches": reps,
            "first_launch_tflops": flops / (ms[0] * 1e-3) / 1e12,
            "what": f"{ncu} workgroups x 8 waves x {iters} x 32 MFMA 16x16x32 bf16 on random operands, "
                    f"median of the last 10 of {reps} launches"}


def copy_probe(mib: int):
    """A plain elementwise pass over `mib` MiB (reads and writes that many
    bytes): the reference reading for the HBM byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b


def host_cpu() -> dict:
    """What the CPU baseline ran on: logical CPUs of this process and the
    processor model as lscpu names it."""
    import subprocess
    model = ""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except Exception:  # pragma: no cover - lscpu missing
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        nproc = os.cpu_count() or 1
    return {"nproc": nproc, "model": model}


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def median3(run, n):
    ts = sorted(run(n) for _ in range(3))
    return ts[1]


def cpu_baseline(inp, wl, seconds: float, norm_eps=None):
    """The oracle as it stands on the first n tokens: n grows until one
    forward+backward takes about seconds/3, then the median of 3 runs."""
    import oracle
    from lora_swiglu_mlp_amd import inputs as I
    w = {}
    for k in oracle.WEIGHT_KEYS:
        if wl.wfmt == "int4_b64" and k in ("w_gate", "w_up", "w_down"):
            inn = wl.inter if k == "w_down" else wl.hidden
            w[k] = oracle.dequant_int4(inp[k], inp[k + "_scales"], inn)
        else:
            w[k] = I.to_f64(inp[k], wl.dtype)

    def run(n):
        d = dict(w)
        d["x"] = I.to_f64(inp["x"][:n], wl.dtype)
        d["dy"] = I.to_f64(inp["dy"][:n], wl.dtype)
        t0 = time.perf_counter()
        if norm_eps is None:
            oracle.forward_backward(d, wl.scale)
        else:
            oracle.rmsnorm.norm_mlp_forward_backward(d, I.to_f64(inp["gamma"], wl.dtype), norm_eps, wl.scale)
        return time.perf_counter() - t0

    target = seconds / 3
    n, t = 32, run(32)
    while t < target / 4 and n < wl.tokens:
        n = min(wl.tokens, n * 2)
        t = run(n)
    if t < target and n < wl.tokens:
        n = min(wl.tokens, max(n, int(n * target / max(t, 1e-3))))
    t = median3(run, n)
    out = {"value": n / t, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
           "sample": f"first {n} of {wl.tokens} tokens of {wl.name}, "
                     f"{'RMSNorm then ' if norm_eps is not None else ''}forward+backward, "
                     f"fp64 numpy (row-local work per token is the full path), median of 3 runs of {t:.1f} s",
           "gflops": oracle.flops(n, wl.hidden, wl.inter, wl.rank) / t / 1e9,
           "host": host_cpu()}
    return out


def cpu_baseline_tiny_single_thread():
    """The oracle on the whole tiny fp32 workload with one BLAS thread
    (median of 3 runs)."""
    import oracle
    from lora_swiglu_mlp_amd import inputs as I
    from threadpoolctl import threadpool_limits
    wl = I.WORKLOADS["tiny_fp32"]
    inp = I.make_inputs(wl)
    d = {k: I.to_f64(v, wl.dtype) for k, v in inp.items()}
    with threadpool_limits(limits=1):
        def run(_):
            t0 = time.perf_counter()
            oracle.forward_backward(d, wl.scale)
            return time.perf_counter() - t0
        t = median3(run, 0)
    return {"workload": wl.name, "tokens_per_s": wl.tokens / t, "ms": t * 1e3, "cores": 1}


def cpu_baseline_linear(inp, wl, seconds: float):
    from oracle import lora_linear_oracle as L
    from lora_swiglu_mlp_amd import inputs as I
    w = {k: I.to_f64(inp[k], wl.dtype) for k in ("w", "a", "b")}
    if wl.wfmt == "int4_b64":
        import oracle
        w["w"] = oracle.dequant_int4(inp["w"], inp["w_scales"], wl.hidden)

    def run(n):
        d = dict(w, x=I.to_f64(inp["x"][:n], wl.dtype), dy=I.to_f64(inp["dy"][:n], wl.dtype))
        t0 = time.perf_counter()
        L.forward_backward(d, wl.scale)
        return time.perf_counter() - t0

    n, t = 64, run(64)
    while t < seconds / 4 and n < wl.tokens:
        n = min(wl.tokens, n * 2)
        t = run(n)
    return {"value": n / t, "unit": "tokens/s", "cores": os.cpu_count() or 1, "kind": "oracle",
            "sample": f"first {n} of {wl.tokens} tokens of {wl.name}, forward+backward, fp64 numpy, {t:.1f} s"}


def cpu_baseline_moe(inp, offsets, wl, seconds: float):
    """The MoE oracle on the first experts (all their rows) until about
    `seconds` of CPU work; reported per input token (routed rows / top_k)."""
    from oracle import moe_oracle as MO
    from lora_swiglu_mlp_amd import inputs as I
    keys = ("w_gate", "w_up", "w_down", "a_gate", "b_gate", "a_up", "b_up", "a_down", "b_down")
    rows = t = 0.0
    e = 0
    while e < wl.experts and t < seconds:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        d = {k: I.to_f64(inp[k][e:e + 1], wl.dtype) for k in keys}
        d["x"] = I.to_f64(inp["x"][lo:hi], wl.dtype)
        d["dy"] = I.to_f64(inp["dy"][lo:hi], wl.dtype)
        t0 = time.perf_counter()
        MO.forward_backward(d, [0, hi - lo], wl.scale)
        t += time.perf_counter() - t0
        rows += hi - lo
        e += 1
    return {"value": rows / wl.top_k / t, "unit": "tokens/s", "cores": os.cpu_count() or 1, "kind": "oracle",
            "sample": f"experts 0..{e - 1} of {wl.experts} with all their rows ({int(rows)} of "
                      f"{int(offsets[-1])} routed rows) of {wl.name}, forward+backward, fp64 numpy, {t:.1f} s"}


def bench_moe(args, wl):
    """The grouped (MoE) LoRA MLP on a MOE_WORKLOADS shape."""
    import torch
    from lora_swiglu_mlp_amd import abi, mlp
    from lora_swiglu_mlp_amd import inputs as I
    H, Iw, r = wl.hidden, wl.inter, wl.rank
    torch.cuda.set_device(0)
    inp, offsets = I.make_moe_inputs(wl)
    rows = int(offsets[-1])
    m, x, dy = mlp.moe_from_inputs(inp, offsets, wl, "cuda:0")
    saved = m.new_saved()
    y = torch.empty((rows, H), dtype=m.tdtype, device="cuda:0")
    grads = m.new_grads(x.device)
    m.workspace()

    def step():
        m.forward(x, y, saved)
        m.backward(dy, x, saved, grads)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    flops = 12 * rows * H * Iw + 18 * rows * r * (H + Iw)
    peak = PEAK_TFLOPS[wl.dtype]
    tflops = flops / (ms * 1e-3) / 1e12
    counts = [int(c) for c in (offsets[1:] - offsets[:-1])]
    out = {"metric": "grouped (MoE) LoRA-SwiGLU MLP fwd+bwd tokens/sec + TFLOP/s as % of MI355X bf16 peak",
           "value": wl.tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": wl.dtype,
           "data": "synthetic (seeded normal draws; random-init weights; synthetic top-k router)",
           "config": {"workload": wl.name, "tokens": wl.tokens, "experts": wl.experts, "top_k": wl.top_k,
                      "routed_rows": rows, "rows_per_expert_min_max": [min(counts), max(counts)],
                      "hidden": H, "inter": Iw, "rank": r, "alpha": wl.alpha, "weights": wl.wfmt,
                      "parallelism": "single-gpu"},
           "tflops": tflops, "pct_of_peak": 100.0 * tflops / peak}
    if not args.no_profile:
        nprof = max(1, min(args.steps, 5))
        abi.lora_mlp_profile_begin()
        for _ in range(nprof):
            step()
        recs = abi.lora_mlp_profile_end()
        agg = {}
        for name, t in recs:
            a = agg.setdefault(name, [0.0, 0])
            a[0] += t
            a[1] += 1
        # per kernel: time per step summed over the experts' launches; FLOPs over all routed rows
        kern = {name: {"ms_per_step": tot / nprof, "launches_per_step": cnt / nprof}
                for name, (tot, cnt) in agg.items()}
        active = sum(1 for c in counts if c > 0)
        eb = 2 if wl.dtype == "bf16" else 4
        for name, e in kern.items():
            f = kernel_flops(name, rows, H, Iw, r)
            if f:
                e["tflops"] = f / (e["ms_per_step"] * 1e-3) / 1e12
                b = moe_gemm_bytes(name, rows, active, H, Iw, r, eb)
                if b:
                    e["gbps"] = b / (e["ms_per_step"] * 1e-3) / 1e9
                    # below the ridge point (peak FLOP/s over peak bytes/s) HBM bounds the product
                    e["bound"] = "hbm" if f / b < peak * 1e12 / (HBM_PEAK_GBS * 1e9) else "mfma"
        out["kernels"] = kern
        out["kernel_ms_per_step"] = sum(e["ms_per_step"] for e in kern.values())
        dom = max((n for n in kern if "tflops" in kern[n]), key=lambda n: kern[n]["ms_per_step"])
        if kern[dom].get("bound") == "hbm":
            out["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": kern[dom]["gbps"], "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": kern[dom]["gbps"] / HBM_PEAK_GBS, "traffic": None,
                               "tflops": kern[dom]["tflops"]}
        else:
            out["roofline"] = {"kernel": dom, "bound": "mfma", "achieved": kern[dom]["tflops"], "peak": peak,
                               "unit": "TFLOP/s", "frac": kern[dom]["tflops"] / peak, "traffic": None}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_moe(inp, offsets, wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def bench_linear(args, wl):
    """The fused LoRA linear (one projection) on a LINEAR_WORKLOADS shape."""
    import torch
    from lora_swiglu_mlp_amd import abi, mlp
    from lora_swiglu_mlp_amd import inputs as I
    T, n_in, n_out, r = wl.tokens, wl.hidden, wl.inter, wl.rank
    torch.cuda.set_device(0)
    inp = I.make_linear_inputs(wl)
    m, x, dy = mlp.linear_from_inputs(inp, wl, "cuda:0")
    saved = m.new_saved()
    y = torch.empty((T, n_out), dtype=m.tdtype, device="cuda:0")
    grads = m.new_grads(x.device)
    m.workspace()

    def step():
        m.forward(x, y, saved)
        m.backward(dy, x, saved, grads)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    flops = 4 * T * n_in * n_out + 6 * T * r * (n_in + n_out)
    peak = PEAK_TFLOPS[wl.dtype]
    tflops = flops / (ms * 1e-3) / 1e12
    out = {"metric": "fused LoRA linear fwd+bwd tokens/sec + TFLOP/s as % of MI355X bf16 peak",
           "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": wl.dtype, "data": "synthetic (seeded normal draws; random-init weights)",
           "config": {"workload": wl.name, "tokens": T, "in": n_in, "out": n_out, "rank": r, "alpha": wl.alpha,
                      "weights": wl.wfmt, "parallelism": "single-gpu"},
           "tflops": tflops, "pct_of_peak": 100.0 * tflops / peak}
    if not args.no_profile:
        nprof = max(1, min(args.steps, 10))
        abi.lora_mlp_profile_begin()
        for _ in range(nprof):
            step()
        recs = abi.lora_mlp_profile_end()
        agg = {}
        for name, t in recs:
            a = agg.setdefault(name, [0.0, 0])
            a[0] += t
            a[1] += 1
        kern = {}
        for name, (tot, cnt) in agg.items():
            e = {"ms": tot / cnt, "launches_per_step": cnt / nprof}
            f = kernel_flops(name, T, n_in, n_out, r, linear=True)
            if f:
                e["tflops"] = f / (e["ms"] * 1e-3) / 1e12
            kern[name] = e
        out["kernels"] = kern
        dom = max((n for n in kern if "tflops" in kern[n]), key=lambda n: kern[n]["ms"])
        out["roofline"] = {"kernel": dom, "bound": "mfma", "achieved": kern[dom]["tflops"], "peak": peak,
                           "unit": "TFLOP/s", "frac": kern[dom]["tflops"] / peak, "traffic": None}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_linear(inp, wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true")
    ap.add_argument("--recompute", action="store_true",
                    help="full-recompute mode: G, U are not saved, the backward recomputes them "
                         "(its FLOPs are not counted in the metric)")
    ap.add_argument("--norm", action="store_true",
                    help="RMSNorm (eps 1e-5) in front of the MLP: the library's norm entry points")
    ap.add_argument("--no-configs", action="store_true",
                    help="measure only the named workload (no sub-lines for the other workloads)")
    ap.add_argument("--int4-copies", action="store_true",
                    help="4-bit weights decoded once per call into bf16 workspace copies "
                         "(LMLP_INT4_BF16_COPIES) instead of inside the products' operand staging")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run a plain copy of this many MiB first (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from lora_swiglu_mlp_amd import abi, mlp
    from lora_swiglu_mlp_amd import inputs as I

    if args.workload in I.LINEAR_WORKLOADS:
        bench_linear(args, I.LINEAR_WORKLOADS[args.workload])
        return
    if args.workload in I.MOE_WORKLOADS:
        bench_moe(args, I.MOE_WORKLOADS[args.workload])
        return
    wl = I.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)
    norm_eps = I.NORM_EPS if args.norm else None
    flags = abi.LMLP_RECOMPUTE_GU if args.recompute else 0
    if args.int4_copies:
        flags |= abi.LMLP_INT4_BF16_COPIES
    res = measure_mlp(wl, args.steps, args.warmup, flags, norm_eps, profile=not args.no_profile)
    T, H, Iw, r = wl.tokens, wl.hidden, wl.inter, wl.rank
    ms = res["ms"]
    flops = mlp_flops(wl, norm_eps)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[wl.dtype]

    out = {"metric": METRIC, "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": wl.dtype, "data": "synthetic (seeded normal draws; random-init weights)",
           "config": {"workload": wl.name, "tokens": T, "hidden": H, "inter": Iw, "rank": r,
                      "alpha": wl.alpha, "weights": wl.wfmt, "parallelism": "single-gpu",
                      "saved": "recompute G, U" if args.recompute else "G, U",
                      "norm": f"rmsnorm eps={norm_eps}" if args.norm else "none"},
           "tflops": tflops, "pct_of_peak": 100.0 * tflops / peak,
           "workspace_bytes": res["workspace_bytes"], "saved_bytes": res["saved_bytes"]}
    if wl.wfmt != "dense":
        out["config"]["int4_decode"] = "bf16 copies" if args.int4_copies else "in the operand staging"

    if "kern" in res:
        kern = res["kern"]
        out["kernels"] = kern
        out["kernel_ms_per_step"] = sum(v["ms"] * v["launches_per_step"] for v in kern.values())
        dom = max((n for n in kern if kernel_flops(n, T, H, Iw, r, dz_cols=res["dz_cols"])),
                  key=lambda n: kern[n]["ms"] * kern[n]["launches_per_step"])
        achieved = kern[dom]["tflops"]
        out["roofline"] = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": peak,
                           "unit": "TFLOP/s", "frac": achieved / peak,
                           "traffic": measured_traffic(dom, wl.name)}
        out["gemms"] = res["gemms"]
        if wl.dtype == "bf16":
            ceil = mfma_ceiling()
            out["mfma_ceiling"] = ceil
            out["roofline"]["frac_of_mfma_ceiling"] = achieved / ceil["tflops"]
            for g in out["gemms"].values():
                g["frac_of_mfma_ceiling"] = g["tflops"] / ceil["tflops"]
            out["pct_of_mfma_ceiling"] = 100.0 * tflops / ceil["tflops"]
        out["fwd_kernel_ms"] = res["fwd_kernel_ms"]
        out["bwd_kernel_ms"] = out["kernel_ms_per_step"] - out["fwd_kernel_ms"]

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(res["inp"], wl, args.cpu_seconds, norm_eps)
        out["cpu_baseline"]["single_thread"] = cpu_baseline_tiny_single_thread()
    del res

    # the other workloads of the metric, one sub-line each (fewer steps)
    if args.workload == "llama3_8b" and not (args.recompute or args.norm or args.no_configs):
        subs = {}
        for name in ("tiny_fp32", "qwen2_7b", "tinyllama_long", "llama3_8b_int4", "llama3_8b_int4 (bf16 copies)"):
            copies = name.endswith("(bf16 copies)")
            w2 = I.WORKLOADS[name.split()[0]]
            r2 = measure_mlp(w2, min(args.steps, 10), min(args.warmup, 3),
                             abi.LMLP_INT4_BF16_COPIES if copies else 0, None, profile=not args.no_profile)
            f2 = mlp_flops(w2, None)
            tf2 = f2 / (r2["ms"] * 1e-3) / 1e12
            e = {"ms_per_step": r2["ms"], "tokens_per_s": w2.tokens / (r2["ms"] * 1e-3), "tflops": tf2,
                 "pct_of_peak": 100.0 * tf2 / PEAK_TFLOPS[w2.dtype], "dtype": w2.dtype, "weights": w2.wfmt,
                 "tokens": w2.tokens, "hidden": w2.hidden, "inter": w2.inter, "rank": w2.rank,
                 "alpha": w2.alpha, "workspace_bytes": r2["workspace_bytes"], "saved_bytes": r2["saved_bytes"]}
            if w2.wfmt != "dense":
                e["int4_decode"] = "bf16 copies" if copies else "in the operand staging"
            if "gemms" in r2:
                e["gemms"] = {g: round(v["frac"], 4) for g, v in r2["gemms"].items()}
                e["fwd_kernel_ms"] = r2["fwd_kernel_ms"]
                e["kernel_ms_per_step"] = sum(v["ms"] * v["launches_per_step"] for v in r2["kern"].values())
            subs[name] = e
            del r2
            torch.cuda.empty_cache()
        out["configs"] = subs

    print(json.dumps(out), flush=True)


FWD_NAMES = ("rmsnorm(fwd)", "pack(fwd)", "rowproj(X A^T)", "gemm(gate/up)", "rowproj(Z A_d^T)", "gemm(down)",
)


def mlp_flops(wl, norm_eps) -> int:
    T, H, Iw, r = wl.tokens, wl.hidden, wl.inter, wl.rank
    return 12 * T * H * Iw + 18 * T * r * (H + Iw) + (norm_flops(T, H) if norm_eps is not None else 0)


def norm_flops(T: int, H: int) -> int:
    """Useful FLOPs of the RMSNorm forward + backward, one per element
    operation on [T, H] arrays (a sum over H counts H adds): forward x*x, its
    row sum, x*rstd, *gamma (4); backward x*rstd, g*gamma, their product, its
    row sum, xhat*c, the difference, *rstd (7). Per-row scalar work (eps,
    square root, reciprocal, the mean's divide) is not counted."""
    return 11 * T * H


def measure_mlp(wl, steps: int, warmup: int, flags: int, norm_eps, profile: bool = True) -> dict:
    """Time `steps` forward+backward steps of the MLP on workload wl (after
    `warmup` untimed ones); with `profile`, a second pass of the same steps
    records per-launch HIP events for the per-kernel table."""
    import torch
    from lora_swiglu_mlp_amd import abi, mlp
    from lora_swiglu_mlp_amd import inputs as I
    T, H, Iw, r = wl.tokens, wl.hidden, wl.inter, wl.rank
    inp = I.make_inputs(wl)
    if norm_eps is not None:
        inp["gamma"] = I.make_norm_gamma(wl)
    m, x, dy = mlp.from_inputs(inp, wl, "cuda:0", flags, norm_eps=norm_eps)
    saved = m.new_saved()
    y = torch.empty((T, H), dtype=m.tdtype, device="cuda:0")
    grads = m.new_grads(x.device)
    m.workspace(True)

    def step():
        m.forward(x, y, saved)
        m.backward(dy, x, saved, grads)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    res = {"ms": (time.perf_counter() - t0) * 1e3 / steps, "inp": inp}
    res["workspace_bytes"] = max(abi.lora_mlp_workspace_bytes(m.dims, False),
                                 abi.lora_mlp_workspace_bytes(m.dims, True))
    res["saved_bytes"] = abi.lora_mlp_saved_bytes(m.dims)
    if profile:
        ncu = torch.cuda.get_device_properties(0).multi_processor_count
        nprof = max(1, min(steps, 10))
        abi.lora_mlp_profile_begin()
        for _ in range(nprof):
            step()
        recs = abi.lora_mlp_profile_end()
        agg = {}
        for name, t in recs:
            a = agg.setdefault(name, [0.0, 0])
            a[0] += t
            a[1] += 1
        # the library's column split of the dZ product, when it ran as two launches
        dz_cols = dz_split(T, Iw, ncu) if "gemm(dZ tail)" in agg else None
        kern = {}
        for name, (tot, cnt) in agg.items():
            avg = tot / cnt
            e = {"ms": avg, "launches_per_step": cnt / nprof}
            f = kernel_flops(name, T, H, Iw, r, dz_cols=dz_cols)
            if f:
                e["tflops"] = f / (avg * 1e-3) / 1e12
            b = kernel_bytes(name, T, H, Iw, r, 2 if wl.dtype == "bf16" else 4)
            if b:
                e["gbps"] = b / (avg * 1e-3) / 1e9
            kern[name] = e
        res["kern"] = kern
        res["dz_cols"] = dz_cols
        res["gemms"] = gemm_table(kern, T, H, Iw, r, PEAK_TFLOPS[wl.dtype], dz_cols)
        res["fwd_kernel_ms"] = sum(kern[n]["ms"] * kern[n]["launches_per_step"] for n in kern if n in FWD_NAMES)
    del m, x, dy, saved, y, grads
    return res


if __name__ == "__main__":
    main()
