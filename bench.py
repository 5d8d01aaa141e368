#!/usr/bin/env python3
"""Benchmark of the CODA GEMM-epilogue path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--all] [--out FILE]

One step = the whole 8B-like non-attention block (the largest of the five
synthetic workloads: M = 8192 tokens, d = 4096, ffn = 14336), forward and
reverse-fused backward, on seeded synthetic bf16 inputs already resident in
HBM:

  forward   u1 = x W0 + z (+ sum-of-squares partials)      coda_gemm_res_sumsq  8192 x 4096 x 4096
            r1 = 1/sqrt(sum/d + eps)                        coda_row_rms
            a1 = SwiGLU(r1 (h2_1 Wgu1)), pre1 kept          coda_gemm_swiglu     8192 x 28672 x 4096
            u2 = a1 Wd1 + u1 (+ partials), r2               coda_gemm_res_sumsq  8192 x 4096 x 14336
            a2 = SwiGLU(r2 (h2_2 Wgu2)); out = a2 Wd2 + u2  (same calls)
  backward  per layer (2, then 1): dWd = a^T dres; dpre = dSwiGLU(dres Wd^T) with s partials;
            s; du = dres + r(G*gamma) - r^2 s u with n2 and dgamma partials (G = dpre Wgu^T);
            dgamma; dWgu = n2^T dpre; finally dx = du1 W0^T and dW0 = x^T du1.

The metric counts only the GEMMs' algorithmic 2*M*N*K FLOPs (18.14 TFLOP per
step).  The dominant kernel (the call with the largest time per step in the
warmup) is timed with HIP events recorded on its launch stream around every
one of its launches inside the timed region; that gives the roofline entry.
Rank 0 prints ONE JSON line on stdout; tables go to stderr.  The line also
carries the unfused sequence of the same block, the config-2 (1B) block
forward as a secondary workload, the measured matrix-core clock, and the fp64
oracle timed on the host on a bounded sample of the same block.  ``--all``
also measures every fused call of the five synthetic workloads against the
plain GEMM of the same shape and writes them to ``--out``.
"""

from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "fused GEMM+epilogue TFLOP/s and % of bf16 MFMA peak (1 MI355X)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


_CODE_TOKENS = re.compile(r'"(?:\\.|[^"\\\n])*"|//[^\n]*|/\*.*?\*/', re.S)


def code_text(src: str) -> str:
    """C++ source without its comments and with runs of whitespace folded
    (string literals kept), so that edits to comments alone leave it equal."""
    out = _CODE_TOKENS.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", src)
    return " ".join(out.split())


def src_hash(files=None) -> str:
    """Hash of the kernel sources (csrc/, comments and layout ignored): a
    measurement taken at one hash belongs to the kernels of that hash.
    files: optional {name: text} to hash instead of the tree's csrc/."""
    if files is None:
        csrc = os.path.join(ROOT, "gemm_epilogue_transformer_mainloop_amd", "csrc")
        files = {}
        for name in sorted(os.listdir(csrc)):
            with open(os.path.join(csrc, name), encoding="utf-8") as f:
                files[name] = f.read()
    h = hashlib.sha256()
    for name in sorted(files):
        h.update(name.encode())
        h.update(b"\0")
        h.update(code_text(files[name]).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------
# timing helpers
# ----------------------------------------------------------------------------


class OpTimer:
    """Per-op HIP event pairs recorded on the current stream, averaged after sync."""

    def __init__(self, torch, only=None):
        self.torch = torch
        self.ev = {}
        self.only = only  # names to time (None: every op); the others run bare

    def run(self, name, fn):
        t = self.torch
        if self.only is not None and name not in self.only:
            return fn()
        s = t.cuda.Event(enable_timing=True)
        e = t.cuda.Event(enable_timing=True)
        s.record()
        out = fn()
        e.record()
        self.ev.setdefault(name, []).append((s, e))
        return out

    def times_ms(self):
        return {k: [s.elapsed_time(e) for s, e in v] for k, v in self.ev.items()}

    def mean_ms(self):
        return {k: float(np.mean(t)) for k, t in self.times_ms().items()}

    def stats_ms(self):
        """Per op: (mean, median, min, launches) over the recorded launches."""
        return {k: (float(np.mean(t)), float(np.median(t)), float(np.min(t)), len(t))
                for k, t in self.times_ms().items()}


def bare(name, fn):
    return fn()


def time_fn(torch, fn, iters=20, warmup=5):
    """Median and min over `iters` back-to-back calls, each bracketed by HIP
    events on the current stream (one synchronisation at the end, so the
    host never makes the GPU wait between calls)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for s, e in ev:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    times = [s.elapsed_time(e) for s, e in ev]
    return float(np.median(times)), float(np.min(times))


def timed_steps(torch, step, steps, tm=None):
    """`steps` back-to-back steps between two events; returns ms per step."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        step(tm)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


# ----------------------------------------------------------------------------
# the 8B-like block (config 5): forward + reverse-fused backward
# ----------------------------------------------------------------------------

BLOCK_DIMS = (8192, 4096, 14336)  # tokens M, model width d, ffn width F


def block_op_flops(M, d, F):
    """Algorithmic 2*M*N*K FLOPs per launch of each GEMM call of the step."""
    return {
        "res_sumsq W0": 2.0 * M * d * d,
        "swiglu": 2.0 * M * 2 * F * d,
        "down+res_sumsq": 2.0 * M * d * F,
        "down+residual": 2.0 * M * d * F,
        "wgrad dWd": 2.0 * F * d * M,
        "swiglu_bwd+s": 2.0 * M * F * d,
        "rowscale_bwd": 2.0 * M * d * 2 * F,
        "wgrad dWgu": 2.0 * d * 2 * F * M,
        "dgrad+wgrad W0": 2 * 2.0 * M * d * d,
    }


# launches per step of each GEMM call
BLOCK_LAUNCHES = {"res_sumsq W0": 1, "swiglu": 2, "down+res_sumsq": 1, "down+residual": 1, "wgrad dWd": 2,
                  "swiglu_bwd+s": 2, "rowscale_bwd": 2, "wgrad dWgu": 2, "dgrad+wgrad W0": 1}

BLOCK_SHAPES = {  # (M, N, K) of each call's GEMM as the user sees it
    "res_sumsq W0": "8192x4096x4096", "swiglu": "8192x28672x4096", "down+res_sumsq": "8192x4096x14336",
    "down+residual": "8192x4096x14336", "wgrad dWd": "14336x4096x8192 (reduction over tokens)",
    "swiglu_bwd+s": "8192x14336x4096", "rowscale_bwd": "8192x4096x28672",
    "wgrad dWgu": "4096x28672x8192 (reduction over tokens)", "dgrad+wgrad W0": "8192x4096x4096 twice",
}

BLOCK_KERNELS = {  # C entry point of each call
    "res_sumsq W0": "coda_gemm_res_sumsq", "swiglu": "coda_gemm_swiglu", "down+res_sumsq": "coda_gemm_res_sumsq",
    "down+residual": "coda_gemm_res_sumsq", "wgrad dWd": "coda_gemm_wgrad", "swiglu_bwd+s": "coda_gemm_swiglu_bwd",
    "rowscale_bwd": "coda_gemm_rowscale_bwd", "wgrad dWgu": "coda_gemm_wgrad",
    "dgrad+wgrad W0": "coda_gemm_res_sumsq_bwd",
}


def block_inputs_device(torch, synth, M, d, F, config=5):
    """Seeded synthetic inputs of the block (synth.block_inputs), on the GPU."""
    p = synth.block_inputs(config, M, d, F)
    T = {k: v.torch("cuda") for k, v in p.items() if hasattr(v, "bits")}
    return p, T


def make_block(torch, coda, T, M, d, F, eps):
    """The fused step and the unfused step of the block on the tensors T.
    Each step takes an optional OpTimer (None: bare launches)."""
    bf, f32 = torch.bfloat16, torch.float32

    def emp(*shape, dtype=bf):
        return torch.empty(*shape, dtype=dtype, device="cuda")

    A = [dict(u=emp(M, d), h=emp(M, d), part=emp(M, coda.coda_nparts(d), dtype=f32), r=emp(M, dtype=f32),
              pre=emp(M, 2 * F), a=emp(M, F), dpre=emp(M, 2 * F), du=emp(M, d), n2=emp(M, d),
              sp=emp(M, coda.coda_nparts(F), dtype=f32), s=emp(M, dtype=f32),
              gp=emp(coda.coda_mparts(M), d, dtype=f32), gpu=emp(coda.coda_unfused_rmsnorm_bwd_parts(M), d, dtype=f32),
              dg=emp(d, dtype=f32), dWgu=emp(d, 2 * F, dtype=f32), dWd=emp(F, d, dtype=f32), da=emp(M, F),
              G=emp(M, d)) for _ in range(2)]
    out, dx, dW0, Y0, Tm = emp(M, d), emp(M, d), emp(d, d, dtype=f32), emp(M, d), emp(M, d)
    Lw = [dict(g=T["gamma1"], Wgu=T["Wgu1"], Wd=T["Wd1"]), dict(g=T["gamma2"], Wgu=T["Wgu2"], Wd=T["Wd2"])]
    x, z, dOut, W0 = T["x"], T["z"], T["dOut"], T["W0"]

    def fused(tm=None):
        run = tm.run if tm is not None else bare
        a1, a2 = A
        run("res_sumsq W0", lambda: coda.coda_gemm_res_sumsq(x, W0, z, Lw[0]["g"], a1["u"], a1["h"], a1["part"]))
        run("row_rms", lambda: coda.coda_row_rms(a1["part"], d, eps, a1["r"]))
        run("swiglu", lambda: coda.coda_gemm_swiglu(a1["h"], Lw[0]["Wgu"], a1["r"], a1["a"], a1["pre"]))
        run("down+res_sumsq", lambda: coda.coda_gemm_res_sumsq(a1["a"], Lw[0]["Wd"], a1["u"], Lw[1]["g"], a2["u"],
                                                                 a2["h"], a2["part"]))
        run("row_rms", lambda: coda.coda_row_rms(a2["part"], d, eps, a2["r"]))
        run("swiglu", lambda: coda.coda_gemm_swiglu(a2["h"], Lw[1]["Wgu"], a2["r"], a2["a"], a2["pre"]))
        run("down+residual", lambda: coda.coda_gemm_res_sumsq(a2["a"], Lw[1]["Wd"], a2["u"], U=out, want_part=False))
        dres = dOut
        for l in (1, 0):
            c, W = A[l], Lw[l]
            run("wgrad dWd", lambda: coda.coda_gemm_wgrad(c["a"], dres, c["dWd"]))
            run("swiglu_bwd+s", lambda: coda.coda_gemm_swiglu_bwd(dres, W["Wd"], c["pre"], c["dpre"], c["sp"]))
            run("row_rms_bwd", lambda: coda.coda_row_rms_bwd(c["sp"], d, c["s"]))
            run("rowscale_bwd", lambda: coda.coda_gemm_rowscale_bwd(c["dpre"], W["Wgu"], c["u"], W["g"], c["r"],
                                                                    c["s"], dres, c["du"], c["n2"], c["gp"]))
            run("col_reduce", lambda: coda.coda_col_reduce(c["gp"], c["dg"]))
            run("wgrad dWgu", lambda: coda.coda_gemm_wgrad(c["n2"], c["dpre"], c["dWgu"]))
            dres = c["du"]
        run("dgrad+wgrad W0", lambda: coda.coda_gemm_res_sumsq_bwd(A[0]["du"], W0, X=x, dX=dx, dW=dW0))

    def unfused(tm=None):
        run = tm.run if tm is not None else bare
        a1, a2 = A
        run("gemm W0", lambda: coda.coda_gemm(x, W0, Y0))
        run("add_rmsnorm", lambda: coda.coda_unfused_add_rmsnorm(Y0, z, Lw[0]["g"], eps, a1["u"], a1["n2"], a1["r"]))
        run("gemm gate/up", lambda: coda.coda_gemm(a1["n2"], Lw[0]["Wgu"], a1["pre"]))
        run("swiglu", lambda: coda.coda_unfused_swiglu(a1["pre"], a1["a"]))
        run("gemm down", lambda: coda.coda_gemm(a1["a"], Lw[0]["Wd"], Tm))
        run("add_rmsnorm", lambda: coda.coda_unfused_add_rmsnorm(Tm, a1["u"], Lw[1]["g"], eps, a2["u"], a2["n2"],
                                                                 a2["r"]))
        run("gemm gate/up", lambda: coda.coda_gemm(a2["n2"], Lw[1]["Wgu"], a2["pre"]))
        run("swiglu", lambda: coda.coda_unfused_swiglu(a2["pre"], a2["a"]))
        run("gemm down", lambda: coda.coda_gemm(a2["a"], Lw[1]["Wd"], Tm))
        run("add", lambda: coda.coda_unfused_add(Tm, a2["u"], out))
        dres = dOut
        for l in (1, 0):
            c, W = A[l], Lw[l]
            run("wgrad dWd", lambda: coda.coda_gemm_wgrad(c["a"], dres, c["dWd"]))
            run("dgrad down", lambda: coda.coda_gemm_res_sumsq_bwd(dres, W["Wd"], dX=c["da"], want_dw=False))
            run("swiglu_bwd", lambda: coda.coda_unfused_swiglu_bwd(c["da"], c["pre"], c["dpre"]))
            run("dgrad gate/up", lambda: coda.coda_gemm_res_sumsq_bwd(c["dpre"], W["Wgu"], dX=c["G"], want_dw=False))
            run("rmsnorm_bwd", lambda: coda.coda_unfused_rmsnorm_bwd(c["G"], c["u"], W["g"], c["r"], dres, c["du"],
                                                                     c["gpu"]))
            run("col_reduce", lambda: coda.coda_col_reduce(c["gpu"], c["dg"]))
            run("wgrad dWgu", lambda: coda.coda_gemm_wgrad(c["n2"], c["dpre"], c["dWgu"]))
            dres = c["du"]
        run("dgrad+wgrad W0", lambda: coda.coda_gemm_res_sumsq_bwd(A[0]["du"], W0, X=x, dX=dx, dW=dW0))

    tensors = list(T.values()) + [v for a in A for v in a.values()] + [out, dx, dW0]
    ws_bytes = sum(t.numel() * t.element_size() for t in tensors)
    return fused, unfused, ws_bytes


def block_cpu_baseline(p, M, d, F, rows=256, min_seconds=12.0, max_steps=20):
    """The fp64 oracle's block forward + backward timed on the host, on a
    bounded sample of the same workload: the first `rows` tokens of the same
    seeded inputs with the full weights (at least min_seconds, at most
    max_steps steps)."""
    from oracle import coda_oracle as O
    from threadpoolctl import threadpool_info

    q = {k: (v.f64() if hasattr(v, "bits") else v) for k, v in p.items()}
    for k in ("x", "z", "dOut"):
        q[k] = q[k][:rows]
    flops = sum(block_op_flops(rows, d, F)[k] * BLOCK_LAUNCHES[k] for k in BLOCK_LAUNCHES)
    steps = 0
    t0 = time.perf_counter()
    while True:
        f = O.block_fwd(q)
        O.block_bwd(q, f)
        steps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or steps >= max_steps:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(flops * steps / el / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{steps} whole block forward+backward steps (W0 + 2 residual/RMSNorm/SwiGLU layers, d={d}, "
                      f"ffn={F}, full weights) on the first {rows} of the {M} tokens, {flops / 1e12:.3f} TFLOP "
                      f"each, fp64 numpy, {el:.1f} s"}


# ----------------------------------------------------------------------------
# config-2 step (the Llama-3-1B-like block forward): a secondary workload
# ----------------------------------------------------------------------------


def c2_inputs(torch, synth):
    c = synth.CONFIGS[2]
    M, d, K, N, NR = c["M"], c["d"], c["K"], c["N"], c["n_rope_cols"]
    p = synth.norm_block_inputs(2, M, d, K, N, n_rope_cols=NR)
    T = {k: v.torch("cuda") for k, v in p.items() if hasattr(v, "bits")}
    T["pos"] = torch.from_numpy(p["pos"]).cuda()
    return p, T, (M, d, K, N, NR)


def c2_flops(M, d, K, N, NR):
    return {"res_sumsq": 2.0 * M * d * K, "rowscale": 2.0 * M * N * d, "rope": 2.0 * M * NR * d}


def make_c2_step(torch, coda, T, dims, eps):
    M, d, K, N, NR = dims
    n_rope = 2560  # Q (32 heads) and K (8 heads) of the 2048:512:512 QKV split; V passes through
    bf = torch.bfloat16
    buf = {
        "U": torch.empty(M, d, dtype=bf, device="cuda"),
        "H2": torch.empty(M, d, dtype=bf, device="cuda"),
        "part": torch.empty(M, coda.coda_nparts(d), dtype=torch.float32, device="cuda"),
        "r": torch.empty(M, dtype=torch.float32, device="cuda"),
        "Y": torch.empty(M, N, dtype=bf, device="cuda"),
        "Yr": torch.empty(M, NR, dtype=bf, device="cuda"),
    }

    def step(tm=None):
        run = tm.run if tm is not None else bare
        run("res_sumsq", lambda: coda.coda_gemm_res_sumsq(T["x"], T["W0"], T["z"], T["gamma"], U=buf["U"],
                                                           H2=buf["H2"], part=buf["part"]))
        run("row_rms", lambda: coda.coda_row_rms(buf["part"], d, eps, r=buf["r"]))
        run("rowscale", lambda: coda.coda_gemm_rowscale(buf["H2"], T["W1"], buf["r"], Y=buf["Y"]))
        run("rope", lambda: coda.coda_gemm_rope(buf["H2"], T["W1r"], buf["r"], T["pos"], 500000.0, 64, n_rope,
                                                 Y=buf["Yr"]))

    return step, buf, n_rope


def make_c2_unfused_step(torch, coda, T, dims, eps, n_rope):
    """The same block as the conventional sequence: plain GEMM, standalone
    residual-add + RMSNorm, plain GEMMs, standalone RoPE."""
    M, d, K, N, NR = dims
    bf = torch.bfloat16
    buf = {
        "Y0": torch.empty(M, d, dtype=bf, device="cuda"),
        "U": torch.empty(M, d, dtype=bf, device="cuda"),
        "N2": torch.empty(M, d, dtype=bf, device="cuda"),
        "r": torch.empty(M, dtype=torch.float32, device="cuda"),
        "Y": torch.empty(M, N, dtype=bf, device="cuda"),
        "Yr": torch.empty(M, NR, dtype=bf, device="cuda"),
    }

    def step(tm=None):
        run = tm.run if tm is not None else bare
        run("gemm0", lambda: coda.coda_gemm(T["x"], T["W0"], buf["Y0"]))
        run("add_rmsnorm", lambda: coda.coda_unfused_add_rmsnorm(buf["Y0"], T["z"], T["gamma"], eps, U=buf["U"],
                                                                 N2=buf["N2"], r=buf["r"]))
        run("gemm1", lambda: coda.coda_gemm(buf["N2"], T["W1"], buf["Y"]))
        run("gemm_qkv", lambda: coda.coda_gemm(buf["N2"], T["W1r"], buf["Yr"]))
        run("rope", lambda: coda.coda_unfused_rope(buf["Yr"], T["pos"], 500000.0, 64, n_rope))

    return step


def c2_cold_cache(torch, coda, T, dims, eps, total_flops, min_bytes=600 << 20, steps=30):
    """Config-2 step with the inputs rotated over enough copies to exceed the MALL."""
    keys = ("x", "W0", "z", "gamma", "W1", "W1r")
    per_set = sum(T[k].numel() * T[k].element_size() for k in keys)
    nsets = max(2, -(-min_bytes // per_set))
    sets = []
    for i in range(nsets):
        Ti = dict(T)
        for k in keys:
            Ti[k] = T[k].clone()
        sets.append(make_c2_step(torch, coda, Ti, dims, eps)[0])
    for st in sets:
        st()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        sets[i % nsets]()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    del sets
    return {"ms_per_step": round(ms, 5), "value": round(total_flops / (ms * 1e-3) / 1e12, 2), "input_sets": nsets,
            "bytes_rotated": int(nsets * per_set), "steps": steps}


def bench_c2(torch, coda, synth, steps=100, warmup=20):
    """The config-2 block forward: fused step, per-op times, unfused sequence, cold cache."""
    p, T, dims = c2_inputs(torch, synth)
    M, d, K, N, NR = dims
    step, buf, n_rope = make_c2_step(torch, coda, T, dims, p["eps"])
    flops = c2_flops(*dims)
    total = sum(flops.values())
    for _ in range(warmup):
        step()
    ms = timed_steps(torch, step, steps)
    tm = OpTimer(torch)
    for _ in range(steps):
        step(tm)
    torch.cuda.synchronize()
    ops = {}
    for k, (mean, med, mn, n) in tm.stats_ms().items():
        ent = {"us": round(mean * 1e3, 2), "us_median": round(med * 1e3, 2), "us_min": round(mn * 1e3, 2)}
        if k in flops:
            tf = flops[k] / (mean * 1e-3) / 1e12
            ent.update(tflops=round(tf, 1), pct_peak=round(100 * tf / PEAK_BF16_TFLOPS, 2))
        if k == "row_rms":
            nb = M * coda.coda_nparts(d) * 4 + M * 4
            ent.update(bytes=nb, gbs=round(nb / (mean * 1e-3) / 1e9, 1),
                       pct_hbm=round(100 * nb / (mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 2))
        ops[k] = ent
    ustep = make_c2_unfused_step(torch, coda, T, dims, p["eps"], n_rope)
    for _ in range(warmup):
        ustep()
    ums = timed_steps(torch, ustep, steps)
    cold = c2_cold_cache(torch, coda, T, dims, p["eps"], total)
    res = {
        "workload": "GEMM->residual->RMSNorm->GEMM forward, Llama-3-1B-like: M=8192 tokens (4x2048), d=2048, "
                    "W1 2048x2048 (rowscale) and QKV W1 2048x3072 with RoPE (theta=5e5, hd=64)",
        "gflop_per_step": round(total / 1e9, 2), "steps": steps, "ms_per_step": round(ms, 5),
        "value": round(total / (ms * 1e-3) / 1e12, 2), "pct_peak": round(100 * total / (ms * 1e-3) / 1e12 /
                                                                         PEAK_BF16_TFLOPS, 2),
        "ops": ops,
        "unfused": {"ms_per_step": round(ums, 5), "fused_speedup": round(ums / ms, 4)},
        "cold_cache": cold,
    }
    del T, buf
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------
# the matrix-core clock of this device, measured
# ----------------------------------------------------------------------------


def mfma_probe(torch, coda, cus, iters=20000):
    coda.coda_probe_mfma(cus, 100)  # warm
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    out = coda.coda_probe_mfma(cus, iters)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    t = out.double().cpu().numpy()
    mem, real = float(np.mean(t[:, 0])), float(np.mean(t[:, 1]))
    flops = cus * 4 * iters * 8 * 32768.0
    ref_mhz = real / (ms * 1e3)  # reference ticks per microsecond of the event-timed launch
    return {"sclk_mhz": round(mem / real * 100.0, 1), "refclk_mhz_check": round(ref_mhz, 2),
            "mfma_only_tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "note": "s_memtime / s_memrealtime ticks (reference clock 100 MHz) over an MFMA-only loop on every CU "
                    f"({iters} x 8 bf16 32x32x16 MFMAs per wave); refclk_mhz_check = reference ticks per event-timed "
                    "microsecond"}


def device_info(torch):
    pr = torch.cuda.get_device_properties(0)
    rocm = None
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        if os.path.exists(path):
            with open(path) as f:
                rocm = f.read().strip()
            break
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", None), "cus": pr.multi_processor_count,
            "hbm_gib": round(pr.total_memory / 2 ** 30, 1), "rocm": rocm, "hip_runtime": torch.version.hip,
            "torch": torch.__version__}


def load_traffic(kernel_key):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    ent = t.get(kernel_key)
    if not ent or ent.get("src_hash") != src_hash():
        return None
    return ent.get("bytes_per_launch")


# ----------------------------------------------------------------------------
# --all: every fused call of the five workloads vs the plain GEMM of the same shape
# ----------------------------------------------------------------------------


def bench_all(torch, coda, synth, iters=20):
    bf = torch.bfloat16
    rows = []

    def rnd(*shape, std=1.0):
        return (torch.randn(*shape, device="cuda") * std).to(bf)

    def rec(cfg, op, M, N, K, fn, plain=None, aux_bytes=None):
        med, mn = time_fn(torch, fn, iters)
        ent = {"config": cfg, "op": op, "M": M, "N": N, "K": K, "us_median": med * 1e3, "us_min": mn * 1e3}
        if K:
            tf = 2.0 * M * N * K / (med * 1e-3) / 1e12
            ent.update(tflops=tf, pct_peak=100 * tf / PEAK_BF16_TFLOPS)
        if aux_bytes:
            ent.update(gbs=aux_bytes / (med * 1e-3) / 1e9, pct_hbm=100 * aux_bytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS)
        if plain is not None:
            pm, _ = time_fn(torch, plain, iters)
            ent.update(plain_us=pm * 1e3, ratio_to_plain=med / pm)
        rows.append(ent)
        log(json.dumps(ent))

    def plain_nn(M, N, K):
        X, W, Y = rnd(M, K), rnd(K, N), torch.empty(M, N, dtype=bf, device="cuda")
        return lambda: coda.coda_gemm(X, W, Y)

    def plain_nt(M, N, K):  # Y[M,N] = A[M,K] B[N,K]^T
        A, B, Y = rnd(M, K), rnd(N, K), torch.empty(M, N, dtype=bf, device="cuda")
        return lambda: coda.coda_gemm_res_sumsq_bwd(A, B, dX=Y, want_dw=False)

    for cfg, (M, d, K, N) in {1: (256, 512, 512, 1024), 2: (8192, 2048, 2048, 2048)}.items():
        x, W0, z, g = rnd(M, K), rnd(K, d, std=K ** -0.5), rnd(M, d), torch.ones(d, dtype=bf, device="cuda")
        U, H2 = torch.empty(M, d, dtype=bf, device="cuda"), torch.empty(M, d, dtype=bf, device="cuda")
        part = torch.empty(M, coda.coda_nparts(d), device="cuda")
        rec(cfg, "res_sumsq", M, d, K, lambda: coda.coda_gemm_res_sumsq(x, W0, z, g, U, H2, part), plain_nn(M, d, K))
        r = torch.empty(M, device="cuda")
        rec(cfg, "row_rms", M, 0, 0, lambda: coda.coda_row_rms(part, d, 1e-6, r), aux_bytes=M * part.shape[1] * 4 + M * 4)
        W1, Y = rnd(d, N, std=d ** -0.5), torch.empty(M, N, dtype=bf, device="cuda")
        rec(cfg, "rowscale", M, N, d, lambda: coda.coda_gemm_rowscale(H2, W1, r, Y), plain_nn(M, N, d))
        if cfg == 2:
            W1r, Yr = rnd(d, 3072, std=d ** -0.5), torch.empty(M, 3072, dtype=bf, device="cuda")
            pos = torch.arange(M, device="cuda", dtype=torch.int32) % 2048
            rec(cfg, "rope", M, 3072, d, lambda: coda.coda_gemm_rope(H2, W1r, r, pos, 5e5, 64, 2560, Yr),
                plain_nn(M, 3072, d))
    # config 3: SwiGLU MLP fwd + bwd
    M, d, F = 8192, 2048, 8192
    x, Wgu, Wd, dY = rnd(M, d), rnd(d, 2 * F, std=d ** -0.5), rnd(F, d, std=F ** -0.5), rnd(M, d)
    act, pre = torch.empty(M, F, dtype=bf, device="cuda"), torch.empty(M, 2 * F, dtype=bf, device="cuda")
    rec(3, "swiglu", M, 2 * F, d, lambda: coda.coda_gemm_swiglu(x, Wgu, None, act, pre), plain_nn(M, 2 * F, d))
    out = torch.empty(M, d, dtype=bf, device="cuda")
    rec(3, "down+residual", M, d, F, lambda: coda.coda_gemm_res_sumsq(act, Wd, x, U=out, want_part=False),
        plain_nn(M, d, F))
    dpre = torch.empty(M, 2 * F, dtype=bf, device="cuda")
    rec(3, "swiglu_bwd", M, F, d, lambda: coda.coda_gemm_swiglu_bwd(dY, Wd, pre, dpre, want_spart=False),
        plain_nt(M, F, d))
    rec(3, "swiglu_bwd overlap", M, F, d,
        lambda: coda.coda_gemm_swiglu_bwd_overlap(dY, Wd, pre, dpre, want_spart=False), plain_nt(M, F, d))
    dX = torch.empty(M, d, dtype=bf, device="cuda")
    rec(3, "dgrad+residual", M, d, 2 * F, lambda: coda.coda_gemm_res_sumsq_bwd(dpre, Wgu, dRes=dY, dX=dX, want_dw=False),
        plain_nt(M, d, 2 * F))
    dWgu = torch.empty(d, 2 * F, device="cuda")
    rec(3, "wgrad dWgu", d, 2 * F, M, lambda: coda.coda_gemm_wgrad(x, dpre, dWgu))
    dWd = torch.empty(F, d, device="cuda")
    rec(3, "wgrad dWd", F, d, M, lambda: coda.coda_gemm_wgrad(act, dY, dWd))
    del x, Wgu, Wd, dY, act, pre, dpre, dX, dWgu, dWd, out
    # config 4: LM head + CE
    M, d, V = 8192, 2048, 128256
    h, W = rnd(M, d), rnd(d, V, std=d ** -0.5)
    labels = torch.randint(0, V, (M,), device="cuda", dtype=torch.int32)
    ws = torch.empty(coda.coda_lmhead_ce_workspace(M, V), dtype=torch.uint8, device="cuda")
    lse, lr, lm = (torch.empty(M, device="cuda"), torch.empty(M, device="cuda"), torch.empty(1, device="cuda"))
    rec(4, "lmhead_ce", M, V, d, lambda: coda.coda_lmhead_ce(h, W, labels, lse, lr, lm, ws), plain_nn(M, V, d))
    dH, dW = torch.empty(M, d, dtype=bf, device="cuda"), torch.empty(d, V, device="cuda")
    wsb = torch.empty(M * V * 2, dtype=torch.uint8, device="cuda")
    med, mn = time_fn(torch, lambda: coda.coda_lmhead_ce_bwd(h, W, labels, lse, 1.0 / M, dH, dW, wsb), 5, 2)
    ent = {"config": 4, "op": "lmhead_ce_bwd (3 GEMMs)", "M": M, "N": V, "K": d, "us_median": med * 1e3,
           "tflops": 3 * 2.0 * M * V * d / (med * 1e-3) / 1e12}
    ent["pct_peak"] = 100 * ent["tflops"] / PEAK_BF16_TFLOPS
    rows.append(ent)
    log(json.dumps(ent))
    del wsb
    for vc in (4096, 8192, 16384):
        wsv = torch.empty(coda.coda_lmhead_ce_bwd_vchunk_workspace(M, V, d, vc), dtype=torch.uint8, device="cuda")
        med, mn = time_fn(torch, lambda: coda.coda_lmhead_ce_bwd_vchunk(h, W, labels, lse, 1.0 / M, vc, dH, dW, wsv),
                          5, 2)
        ent = {"config": 4, "op": f"lmhead_ce_bwd_vchunk {vc} (3 GEMMs per chunk)", "M": M, "N": V, "K": d,
               "us_median": med * 1e3, "tflops": 3 * 2.0 * M * V * d / (med * 1e-3) / 1e12,
               "workspace_bytes": int(wsv.numel())}
        ent["pct_peak"] = 100 * ent["tflops"] / PEAK_BF16_TFLOPS
        rows.append(ent)
        log(json.dumps(ent))
        del wsv
    L = torch.empty(M, V, dtype=bf, device="cuda")
    rec(4, "lmhead_ce_logits", M, V, d, lambda: coda.coda_lmhead_ce_logits(h, W, labels, lse, lr, lm, L, ws),
        plain_nn(M, V, d))
    # each timed call turns the buffer's dlogits into dlogits again: same work
    med, mn = time_fn(torch, lambda: coda.coda_lmhead_ce_bwd_logits(h, W, labels, lse, 1.0 / M, L, dH, dW), 5, 2)
    ent = {"config": 4, "op": "lmhead_ce_bwd_logits (dlogits + 2 GEMMs)", "M": M, "N": V, "K": d,
           "us_median": med * 1e3, "tflops": 2 * 2.0 * M * V * d / (med * 1e-3) / 1e12}
    ent["pct_peak"] = 100 * ent["tflops"] / PEAK_BF16_TFLOPS
    rows.append(ent)
    log(json.dumps(ent))
    del h, W, ws, L, dH, dW
    # config 5: the block-backward fused calls at 8B-like shape
    M, d, F = 8192, 4096, 14336
    dOut, Wd, Wgu = rnd(M, d), rnd(F, d, std=F ** -0.5), rnd(d, 2 * F, std=d ** -0.5)
    pre, dpre = rnd(M, 2 * F), torch.empty(M, 2 * F, dtype=bf, device="cuda")
    act5, r5 = torch.empty(M, F, dtype=bf, device="cuda"), torch.ones(M, device="cuda")
    rec(5, "swiglu+r", M, 2 * F, d, lambda: coda.coda_gemm_swiglu(dOut, Wgu, r5, act5, dpre), plain_nn(M, 2 * F, d))
    del act5, r5
    spart = torch.empty(M, coda.coda_nparts(F), device="cuda")
    rec(5, "swiglu_bwd+s", M, F, d, lambda: coda.coda_gemm_swiglu_bwd(dOut, Wd, pre, dpre, spart), plain_nt(M, F, d))
    rec(5, "swiglu_bwd+s overlap", M, F, d, lambda: coda.coda_gemm_swiglu_bwd_overlap(dOut, Wd, pre, dpre, spart),
        plain_nt(M, F, d))
    s = torch.empty(M, device="cuda")
    rec(5, "row_rms_bwd", M, 0, 0, lambda: coda.coda_row_rms_bwd(spart, d, s), aux_bytes=spart.numel() * 4 + M * 4)
    u, gam, r = rnd(M, d), torch.ones(d, dtype=bf, device="cuda"), torch.ones(M, device="cuda")
    dU, N2 = torch.empty(M, d, dtype=bf, device="cuda"), torch.empty(M, d, dtype=bf, device="cuda")
    gpart = torch.empty(coda.coda_mparts(M), d, device="cuda")
    rec(5, "rowscale_bwd", M, d, 2 * F, lambda: coda.coda_gemm_rowscale_bwd(dpre, Wgu, u, gam, r, s, dOut, dU, N2, gpart),
        plain_nt(M, d, 2 * F))
    dg = torch.empty(d, device="cuda")
    rec(5, "col_reduce", 0, d, 0, lambda: coda.coda_col_reduce(gpart, dg), aux_bytes=gpart.numel() * 4 + d * 4)
    dW = torch.empty(d, 2 * F, device="cuda")
    rec(5, "wgrad dWgu", d, 2 * F, M, lambda: coda.coda_gemm_wgrad(N2, dpre, dW))
    del dOut, Wd, Wgu, pre, dpre, spart, s, u, gam, r, dU, N2, gpart, dg, dW
    torch.cuda.empty_cache()
    rows += bench_sequences(torch, coda, iters)
    return rows


def bench_sequences(torch, coda, iters=20):
    """Each workload's fused call sequence against its unfused sequence (plain
    GEMMs + standalone kernels) on the same tensors."""
    bf = torch.bfloat16
    rows = []

    def rnd(*shape, std=1.0):
        return (torch.randn(*shape, device="cuda") * std).to(bf)

    def emp(*shape, dtype=bf):
        return torch.empty(*shape, dtype=dtype, device="cuda")

    def seq(cfg, name, flops, fused, unfused, it=iters):
        fm, fmin = time_fn(torch, fused, it, 3)
        um, umin = time_fn(torch, unfused, it, 3)
        ent = {"config": cfg, "sequence": name, "gflop": round(flops / 1e9, 1),
               "fused_us_median": round(fm * 1e3, 1), "fused_us_min": round(fmin * 1e3, 1),
               "unfused_us_median": round(um * 1e3, 1), "unfused_us_min": round(umin * 1e3, 1),
               "fused_tflops": round(flops / (fm * 1e-3) / 1e12, 1),
               "unfused_tflops": round(flops / (um * 1e-3) / 1e12, 1),
               "speedup": round(um / fm, 3)}
        rows.append(ent)
        log(json.dumps(ent))

    # configs 1 and 2: GEMM -> residual -> RMSNorm -> GEMM (+ QKV GEMM with RoPE)
    for cfg, (M, d, K, N, NR) in {1: (256, 512, 512, 1024, 0), 2: (8192, 2048, 2048, 2048, 3072)}.items():
        x, W0, z, g = rnd(M, K), rnd(K, d, std=K ** -0.5), rnd(M, d), torch.ones(d, dtype=bf, device="cuda")
        W1 = rnd(d, N, std=d ** -0.5)
        U, H2, N2, Y0, Y = emp(M, d), emp(M, d), emp(M, d), emp(M, d), emp(M, N)
        part, r = emp(M, coda.coda_nparts(d), dtype=torch.float32), emp(M, dtype=torch.float32)
        if NR:
            W1r, Yr = rnd(d, NR, std=d ** -0.5), emp(M, NR)
            pos = torch.arange(M, device="cuda", dtype=torch.int32) % 2048

        def fused():
            coda.coda_gemm_res_sumsq(x, W0, z, g, U, H2, part)
            coda.coda_row_rms(part, d, 1e-6, r)
            coda.coda_gemm_rowscale(H2, W1, r, Y)
            if NR:
                coda.coda_gemm_rope(H2, W1r, r, pos, 5e5, 64, 2560, Yr)

        def unfused():
            coda.coda_gemm(x, W0, Y0)
            coda.coda_unfused_add_rmsnorm(Y0, z, g, 1e-6, U, N2, r)
            coda.coda_gemm(N2, W1, Y)
            if NR:
                coda.coda_gemm(N2, W1r, Yr)
                coda.coda_unfused_rope(Yr, pos, 5e5, 64, 2560)

        seq(cfg, "norm block forward", 2.0 * M * K * d + 2.0 * M * d * N + 2.0 * M * d * NR, fused, unfused)
    # config 3: SwiGLU MLP forward and backward
    M, d, F = 8192, 2048, 8192
    x, Wgu, Wd, dY = rnd(M, d), rnd(d, 2 * F, std=d ** -0.5), rnd(F, d, std=F ** -0.5), rnd(M, d)
    act, pre, out, o = emp(M, F), emp(M, 2 * F), emp(M, d), emp(M, d)

    def f_fwd():
        coda.coda_gemm_swiglu(x, Wgu, None, act, pre)
        coda.coda_gemm_res_sumsq(act, Wd, x, U=out, want_part=False)

    def u_fwd():
        coda.coda_gemm(x, Wgu, pre)
        coda.coda_unfused_swiglu(pre, act)
        coda.coda_gemm(act, Wd, o)
        coda.coda_unfused_add(o, x, out)

    seq(3, "MLP forward", 2.0 * M * d * 2 * F + 2.0 * M * F * d, f_fwd, u_fwd)
    da, dpre, dX, dX0 = emp(M, F), emp(M, 2 * F), emp(M, d), emp(M, d)
    dWgu, dWd = emp(d, 2 * F, dtype=torch.float32), emp(F, d, dtype=torch.float32)

    def f_bwd():
        coda.coda_gemm_swiglu_bwd(dY, Wd, pre, dpre, want_spart=False)
        coda.coda_gemm_res_sumsq_bwd(dpre, Wgu, X=x, dRes=dY, dX=dX, dW=dWgu)
        coda.coda_gemm_wgrad(act, dY, dWd)

    def u_bwd():
        coda.coda_gemm_res_sumsq_bwd(dY, Wd, dX=da, want_dw=False)
        coda.coda_unfused_swiglu_bwd(da, pre, dpre)
        coda.coda_gemm_res_sumsq_bwd(dpre, Wgu, dX=dX0, want_dw=False)
        coda.coda_unfused_add(dX0, dY, dX)
        coda.coda_gemm_wgrad(x, dpre, dWgu)
        coda.coda_gemm_wgrad(act, dY, dWd)

    seq(3, "MLP backward", 2.0 * M * d * F + 2 * 2.0 * M * d * 2 * F + 2.0 * M * F * d, f_bwd, u_bwd, 10)
    del x, Wgu, Wd, dY, act, pre, out, o, da, dpre, dX, dX0, dWgu, dWd
    torch.cuda.empty_cache()
    # config 4: LM head + cross-entropy, forward and backward
    M, d, V = 8192, 2048, 128256
    h, W = rnd(M, d), rnd(d, V, std=d ** -0.5)
    labels = torch.randint(0, V, (M,), device="cuda", dtype=torch.int32)
    ws = torch.empty(coda.coda_lmhead_ce_workspace(M, V), dtype=torch.uint8, device="cuda")
    lse, lr, lm = emp(M, dtype=torch.float32), emp(M, dtype=torch.float32), emp(1, dtype=torch.float32)
    L = emp(M, V)
    seq(4, "LM head + CE forward", 2.0 * M * d * V, lambda: coda.coda_lmhead_ce(h, W, labels, lse, lr, lm, ws),
        lambda: (coda.coda_gemm(h, W, L), coda.coda_unfused_cross_entropy(L, labels, lse, lr, lm)), 5)
    dH, dW = emp(M, d), emp(d, V, dtype=torch.float32)
    wsb = torch.empty(M * V * 2, dtype=torch.uint8, device="cuda")

    def u_ce_bwd():
        coda.coda_gemm(h, W, L)
        coda.coda_unfused_cross_entropy(L, labels, lse, lr, lm)
        coda.coda_unfused_cross_entropy_bwd(L, labels, lse, 1.0 / M, L)
        coda.coda_gemm_res_sumsq_bwd(L, W, dX=dH, want_dw=False)
        coda.coda_gemm_wgrad(h, L, dW)

    def f_ce_bwd():
        coda.coda_lmhead_ce(h, W, labels, lse, lr, lm, ws)
        coda.coda_lmhead_ce_bwd(h, W, labels, lse, 1.0 / M, dH, dW, wsb)

    # algorithmic work: the forward GEMM and the two gradient GEMMs (the fused
    # backward's logit recomputation is not counted)
    seq(4, "LM head + CE forward+backward", 3 * 2.0 * M * d * V, f_ce_bwd, u_ce_bwd, 3)

    def f_ce_bwd_logits():
        coda.coda_lmhead_ce_logits(h, W, labels, lse, lr, lm, L, ws)
        coda.coda_lmhead_ce_bwd_logits(h, W, labels, lse, 1.0 / M, L, dH, dW)

    del wsb
    seq(4, "LM head + CE forward+backward, stored logits", 3 * 2.0 * M * d * V, f_ce_bwd_logits, u_ce_bwd, 3)
    wsv = torch.empty(coda.coda_lmhead_ce_bwd_vchunk_workspace(M, V, d, 8192), dtype=torch.uint8, device="cuda")

    def f_ce_bwd_vchunk():
        coda.coda_lmhead_ce(h, W, labels, lse, lr, lm, ws)
        coda.coda_lmhead_ce_bwd_vchunk(h, W, labels, lse, 1.0 / M, 8192, dH, dW, wsv)

    seq(4, "LM head + CE forward+backward, dlogits in 8192-column vocabulary chunks", 3 * 2.0 * M * d * V,
        f_ce_bwd_vchunk, u_ce_bwd, 3)
    del wsv
    del h, W, ws, L, dH, dW
    torch.cuda.empty_cache()
    # config 5: one layer of the block backward (SwiGLU MLP + RMSNorm) at 8B-like shape
    M, d, F = 8192, 4096, 14336
    dOut, Wd, Wgu = rnd(M, d), rnd(F, d, std=F ** -0.5), rnd(d, 2 * F, std=d ** -0.5)
    pre, act, u, N2 = rnd(M, 2 * F), rnd(M, F), rnd(M, d), rnd(M, d)
    gam, r = torch.ones(d, dtype=bf, device="cuda"), torch.ones(M, device="cuda")
    dpre, da, G, dU, N2f = emp(M, 2 * F), emp(M, F), emp(M, d), emp(M, d), emp(M, d)
    spart, s_ = emp(M, coda.coda_nparts(F), dtype=torch.float32), emp(M, dtype=torch.float32)
    gpart = emp(coda.coda_mparts(M), d, dtype=torch.float32)
    gpu_ = emp(coda.coda_unfused_rmsnorm_bwd_parts(M), d, dtype=torch.float32)
    dg, dWgu, dWd = emp(d, dtype=torch.float32), emp(d, 2 * F, dtype=torch.float32), emp(F, d, dtype=torch.float32)

    def f_l():
        coda.coda_gemm_swiglu_bwd(dOut, Wd, pre, dpre, spart)
        coda.coda_row_rms_bwd(spart, d, s_)
        coda.coda_gemm_rowscale_bwd(dpre, Wgu, u, gam, r, s_, dOut, dU, N2f, gpart)
        coda.coda_col_reduce(gpart, dg)
        coda.coda_gemm_wgrad(N2f, dpre, dWgu)
        coda.coda_gemm_wgrad(act, dOut, dWd)

    def u_l():
        coda.coda_gemm_res_sumsq_bwd(dOut, Wd, dX=da, want_dw=False)
        coda.coda_unfused_swiglu_bwd(da, pre, dpre)
        coda.coda_gemm_res_sumsq_bwd(dpre, Wgu, dX=G, want_dw=False)
        coda.coda_unfused_rmsnorm_bwd(G, u, gam, r, dOut, dU, gpu_)
        coda.coda_col_reduce(gpu_, dg)
        coda.coda_gemm_wgrad(N2, dpre, dWgu)
        coda.coda_gemm_wgrad(act, dOut, dWd)

    seq(5, "layer backward (SwiGLU MLP + RMSNorm)", 2.0 * M * d * F * 2 + 2 * 2.0 * M * d * 2 * F, f_l, u_l, 5)
    del dOut, Wd, Wgu, pre, act, u, N2, gam, r, dpre, da, G, dU, N2f, spart, s_, gpart, gpu_, dg, dWgu, dWd
    torch.cuda.empty_cache()
    bench_block(torch, coda, seq)
    return rows


def bench_block(torch, coda, seq_fn):
    """The whole config-5 block (W0 projection + two residual/RMSNorm/SwiGLU-MLP
    layers), forward and backward as one stream ("CODA" paper Figure 11):
    the fused calls against the unfused sequence."""
    from gemm_epilogue_transformer_mainloop_amd import synth

    M, d, F = BLOCK_DIMS
    _, T = block_inputs_device(torch, synth, M, d, F)
    fused, unfused, _ = make_block(torch, coda, T, M, d, F, 1e-6)
    total = sum(block_op_flops(M, d, F)[k] * BLOCK_LAUNCHES[k] for k in BLOCK_LAUNCHES)
    seq_fn(5, "block forward+backward (W0 + 2 layers)", total, lambda: fused(), lambda: unfused(), 3)


# ----------------------------------------------------------------------------


class TimelineRunner:
    """Runs each op of a step alone with the tile-timeline buffer installed
    (timeline build of the library) and keeps, per op name, the per-tile
    figures of every GEMM launch (ops without a GEMM leave no records)."""

    def __init__(self, torch, coda, waves=1 << 16):
        self.torch, self.coda = torch, coda
        self.buf = torch.zeros((waves, coda.coda_timeline_words()), dtype=torch.int64, device="cuda")
        self.rows = {}

    def run(self, name, fn):
        t = self.torch
        t.cuda.synchronize()
        self.buf.zero_()
        self.coda.coda_timeline_set(self.buf)
        out = fn()
        t.cuda.synchronize()
        self.coda.coda_timeline_set(None)
        rec = self.buf.cpu().numpy()
        rec = rec[rec[:, 0] != 0]
        if len(rec):
            self.rows.setdefault(name, []).append(timeline_summary(rec))
        return out


def timeline_summary(rec):
    """Per-launch figures from timeline records (one row per wave; words as in
    coda_probe.h).  Times in microseconds of the 100 MHz reference clock."""
    rt, ct = rec[:, 0:4].astype(np.int64), rec[:, 4:8].astype(np.int64)
    bt, nk, hw, xcc = rec[:, 8], rec[:, 9], rec[:, 10], rec[:, 11]
    t0 = rt[:, 0].min()
    us = lambda x: x / 100.0
    kloop_ct = ct[:, 2] - ct[:, 1]
    kloop_rt = np.maximum(rt[:, 2] - rt[:, 1], 1)
    mfma_cyc = 2048.0 * bt / 256.0 * nk  # 4 x 4 (or 4 x 2) MFMA 32x32x16 per k-step, 8 passes of 4 clocks
    # One record per wave; a tile's four waves run on one compute unit.
    cu = (xcc.astype(np.int64) << 16) | (((hw >> 13) & 7) << 8) | (((hw >> 12) & 1) << 4) | ((hw >> 8) & 15)
    wave0 = np.arange(len(rec)) % 4 == 0  # records are dense from block 0: every 4th is a wave 0
    starts, ends, cus = rt[wave0, 0], rt[wave0, 3], cu[wave0]
    gaps = []
    for c in np.unique(cus):
        i = np.argsort(starts[cus == c])
        s_, e_ = starts[cus == c][i], ends[cus == c][i]
        gaps.extend((s_[1:] - e_[:-1]).tolist())
    span = us(rt[:, 3].max() - t0)
    ncu = len(np.unique(cus))
    # the first round of tiles (records of the first ncu tiles) against the rest
    first = np.arange(len(rec)) < 4 * ncu
    kl = us(rt[:, 2] - rt[:, 1])
    rest = float(np.median(kl[~first])) if (~first).any() else None
    return {
        "tiles": int(wave0.sum()), "compute_units": int(ncu), "k_tiles": int(np.median(nk)),
        "span_us": round(float(span), 1),
        "prologue_us": round(float(np.median(us(rt[:, 1] - rt[:, 0]))), 2),
        "kloop_us": round(float(np.median(us(rt[:, 2] - rt[:, 1]))), 2),
        "kloop_us_first_round": round(float(np.median(kl[first])), 2),
        "kloop_us_later_rounds": round(rest, 2) if rest is not None else None,
        "epilogue_us": round(float(np.median(us(rt[:, 3] - rt[:, 2]))), 2),
        "gap_us": round(float(np.median(us(np.array(gaps)))), 2) if gaps else None,
        "cycles_per_ktile": round(float(np.median(kloop_ct / np.maximum(nk, 1))), 0),
        "sclk_ghz": round(float(np.median(kloop_ct / kloop_rt * 0.1)), 3),
        "mfma_issue_in_kloop": round(float(np.median(mfma_cyc / np.maximum(kloop_ct, 1))), 3),
        "cu_busy": round(float(us(ends - starts).sum() / (ncu * span)), 3),
    }


# ----------------------------------------------------------------------------
# board power and clocks under sustained load
# ----------------------------------------------------------------------------


def parse_smi_metric(text):
    """Socket power (W) and the per-XCD graphics clocks (MHz) from the text of
    `amd-smi metric -p -c`; None where absent."""
    m = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", text)
    clocks = [float(c) for c in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*([0-9.]+)\s*MHz", text)]
    return {"socket_w": float(m.group(1)) if m else None, "gfx_mhz": clocks}


def power_cap_w():
    """The board's power cap (W) from `rocm-smi --showmaxpower`, or None."""
    import subprocess
    try:
        out = subprocess.run(["rocm-smi", "--showmaxpower"], capture_output=True, text=True, timeout=30).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    m = re.search(r"Max Graphics Package Power \(W\):\s*([0-9.]+)", out)
    return float(m.group(1)) if m else None


def sustained_load(torch, fn, flops, secs, cap=None, settle=3.0):
    """Run fn back to back for `secs` seconds while a child process samples
    `amd-smi metric -p -c` about once a second (samples from the first
    `settle` seconds dropped).  Returns the call rate, the TFLOP/s of `flops`
    per call, and the median socket power and XCD clock (None where the tool
    gives nothing)."""
    import subprocess
    import threading

    samples, stop = [], threading.Event()
    t_start = [time.time()]

    def sample():
        while not stop.is_set():
            try:
                txt = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True,
                                     timeout=20).stdout
            except (OSError, subprocess.SubprocessError):
                return
            if time.time() - t_start[0] >= settle:
                samples.append(parse_smi_metric(txt))
            stop.wait(1.0)

    fn()
    torch.cuda.synchronize()
    th = threading.Thread(target=sample, daemon=True)
    t_start[0] = time.time()
    th.start()
    n = 0
    while time.time() - t_start[0] < secs:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    el = time.time() - t_start[0]
    stop.set()
    th.join(timeout=30)
    pw = [x["socket_w"] for x in samples if x["socket_w"] is not None]
    ck = [float(np.mean(x["gfx_mhz"])) for x in samples if x["gfx_mhz"]]
    return {"seconds": round(el, 1), "calls": n, "tflops": round(flops * n / el / 1e12, 1), "samples": len(samples),
            "power_cap_w": cap,
            "socket_w_median": round(float(np.median(pw)), 1) if pw else None,
            "socket_w_min": round(float(np.min(pw)), 1) if pw else None,
            "socket_w_max": round(float(np.max(pw)), 1) if pw else None,
            "gfx_mhz_median": round(float(np.median(ck)), 1) if ck else None}


def power_report(torch, coda, synth, secs=12.0, out=None):
    """The headline step, the plain GEMM of the SwiGLU projection's shape
    (8192 x 28672 x 4096) and the MFMA-only clock probe, each under
    sustained_load for `secs` seconds."""
    M, d, F = BLOCK_DIMS
    bf = torch.bfloat16
    p, T = block_inputs_device(torch, synth, M, d, F)
    fused, _, _ = make_block(torch, coda, T, M, d, F, p["eps"])
    g = torch.Generator(device="cuda").manual_seed(7)
    h = torch.randn(M, d, device="cuda", generator=g).to(bf)
    W = (torch.randn(d, 2 * F, device="cuda", generator=g) * d ** -0.5).to(bf)
    Y = torch.empty(M, 2 * F, dtype=bf, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    probe_out = torch.zeros((cus, 2), dtype=torch.int64, device="cuda")
    opf = block_op_flops(M, d, F)
    loads = [
        ("block step", fused, sum(opf[k] * BLOCK_LAUNCHES[k] for k in BLOCK_LAUNCHES)),
        ("plain GEMM 8192x28672x4096", lambda: coda.coda_gemm(h, W, Y), 2.0 * M * 2 * F * d),
        ("MFMA-only probe", lambda: coda.coda_probe_mfma(cus, 20000, probe_out), cus * 4 * 20000 * 8 * 32768.0),
    ]
    cap = power_cap_w()
    lines = []
    for name, fn, flops in loads:
        ln = {"load": name, **sustained_load(torch, fn, flops, secs, cap)}
        print(json.dumps(ln), flush=True)
        lines.append(ln)
    if out:
        with open(out, "w") as f:
            for ln in lines:
                f.write(json.dumps(ln) + "\n")


def timeline_report(torch, coda, synth, out=None):
    """The headline step's GEMMs, one launch each with the tile timeline."""
    M, d, F = BLOCK_DIMS
    p, T = block_inputs_device(torch, synth, M, d, F)
    fused, _, _ = make_block(torch, coda, T, M, d, F, p["eps"])
    for _ in range(3):
        fused()
    tl = TimelineRunner(torch, coda)
    fused(tl)
    # The SwiGLU backward beside its epilogue-overlapped form, at the block's
    # MLP shape and at the 1B-like one (seeded synthetic operands).
    g = torch.Generator(device="cuda").manual_seed(5)
    bf = torch.bfloat16
    for (Mx, dx, Fx) in ((M, d, F), (8192, 2048, 8192)):
        dO = torch.randn(Mx, dx, device="cuda", generator=g).to(bf)
        Wd = (torch.randn(Fx, dx, device="cuda", generator=g) * Fx ** -0.5).to(bf)
        pre = torch.randn(Mx, 2 * Fx, device="cuda", generator=g).to(bf)
        dpre = torch.empty(Mx, 2 * Fx, dtype=bf, device="cuda")
        sp = torch.empty(Mx, coda.coda_nparts(Fx), device="cuda")
        for name, fn in (("swiglu_bwd+s", coda.coda_gemm_swiglu_bwd),
                         ("swiglu_bwd+s overlap", coda.coda_gemm_swiglu_bwd_overlap)):
            for _ in range(2):
                fn(dO, Wd, pre, dpre, sp)
            tl.run(f"{name} {Mx}x{Fx}x{dx}", lambda: fn(dO, Wd, pre, dpre, sp))
        del dO, Wd, pre, dpre, sp
    lines = []
    for name, rows in tl.rows.items():
        for i, r in enumerate(rows):
            lines.append({"op": name, "launch": i, "shape": BLOCK_SHAPES.get(name), **r})
    for ln in lines:
        print(json.dumps(ln), flush=True)
    if out:
        with open(out, "w") as f:
            for ln in lines:
                f.write(json.dumps(ln) + "\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--all", action="store_true", help="also time every fused call of the five workloads")
    ap.add_argument("--out", default=None, help="file for the --all table (JSON lines)")
    ap.add_argument("--iters", type=int, default=20,
                    help="timed calls per --all entry (after 3-5 untimed ones); fewer for counter runs")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="headline step only (no unfused sequence, config-2 block, clock probe)")
    ap.add_argument("--timeline", action="store_true",
                    help="only print per-tile timelines (prologue, k-loop, epilogue, shader clock) of the headline "
                         "step's GEMMs, from the timeline build libcoda_timeline.so")
    ap.add_argument("--no-power", action="store_true",
                    help="no board_power sampling (amd-smi child processes), e.g. under a profiler")
    ap.add_argument("--power", type=float, default=0.0, metavar="SECONDS",
                    help="only run the headline step, the plain GEMM of its largest shape and the MFMA-only probe "
                         "for SECONDS each while sampling board power and clocks (amd-smi)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only; --gpus must be 1 (no multi-GPU path is built).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from gemm_epilogue_transformer_mainloop_amd import coda, synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.timeline:
        coda.use_library(coda.TIMELINE_LIB_PATH)
    coda.lib()  # fails loudly if the HIP library is not built

    if args.timeline:
        timeline_report(torch, coda, synth, args.out)
        return

    if args.power > 0:
        power_report(torch, coda, synth, args.power, args.out)
        return

    if args.copy_calib:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 x {n} bytes read + {n} bytes written")
        return

    dev = device_info(torch)
    log(f"device: {dev}")
    M, d, F = BLOCK_DIMS
    p, T = block_inputs_device(torch, synth, M, d, F)
    eps = p["eps"]
    fused, unfused, ws_bytes = make_block(torch, coda, T, M, d, F, eps)
    opf = block_op_flops(M, d, F)
    total_flops = sum(opf[k] * BLOCK_LAUNCHES[k] for k in BLOCK_LAUNCHES)

    # Warmup.  Its last steps (two, or one extra untimed step when there is
    # no warmup) carry an event pair around every call, to find the call
    # with the largest time per step: the roofline kernel.
    nrank = min(args.warmup, 2)
    for _ in range(args.warmup - nrank):
        fused()
    rank = OpTimer(torch)
    for _ in range(max(nrank, 1)):
        fused(rank)
    torch.cuda.synchronize()
    per_step = {k: sum(t) / max(nrank, 1) for k, t in rank.times_ms().items()}
    dom = max((k for k in per_step if k in opf), key=lambda k: per_step[k])
    log("warmup ranking (ms per step): " + ", ".join(f"{k} {v:.3f}" for k, v in
                                                     sorted(per_step.items(), key=lambda kv: -kv[1])))

    # The timed region: exactly K steps, back to back.  Every launch of the
    # roofline kernel is bracketed by an event pair on its launch stream
    # (its launches per step are a few of about twenty, in a step of ~15 ms).
    dtm = OpTimer(torch, only={dom})
    ms_step = timed_steps(torch, fused, args.steps, dtm)
    d_mean, d_med, d_min, d_n = dtm.stats_ms()[dom]
    value = total_flops / (ms_step * 1e-3) / 1e12
    achieved = opf[dom] / (d_mean * 1e-3) / 1e12
    log(f"block fwd+bwd: {ms_step:.3f} ms/step, {value:.1f} TFLOP/s; {dom}: {d_mean * 1e3:.1f} us/launch "
        f"({achieved:.1f} TFLOP/s)")

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "config": {
            "workload": "8B-like non-attention block forward + reverse-fused backward: M=8192 tokens, d=4096, "
                        "ffn=14336, a d x d projection with residual then two residual+RMSNorm+SwiGLU-MLP layers; "
                        "seeded synthetic bf16 (x, z, dOut ~N(0,1), weights ~N(0,1/fan_in), gamma ~N(1,0.1))",
            "M": M, "d": d, "ffn": F, "layers": 2, "gflop_per_step": round(total_flops / 1e9, 1),
            "calls_per_step": ["coda_gemm_res_sumsq", "coda_row_rms", "coda_gemm_swiglu", "coda_gemm_res_sumsq",
                               "coda_row_rms", "coda_gemm_swiglu", "coda_gemm_res_sumsq",
                               "2 x [coda_gemm_wgrad, coda_gemm_swiglu_bwd, coda_row_rms_bwd, "
                               "coda_gemm_rowscale_bwd, coda_col_reduce, coda_gemm_wgrad]",
                               "coda_gemm_res_sumsq_bwd"],
        },
        "device": dev,
        "roofline": {
            "bound": "mfma",
            "kernel": f"{BLOCK_KERNELS[dom]} ({dom}, {BLOCK_SHAPES[dom]})",
            "flop_per_launch": opf[dom],
            "us_per_launch": round(d_mean * 1e3, 2),
            "us_per_launch_median": round(d_med * 1e3, 2),
            "launches_timed": d_n,
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": load_traffic("c5 " + dom),
        },
    }

    if not args.no_extra:
        # Per-call breakdown: another K steps with an event pair around every
        # call (outside the timed region).
        tm = OpTimer(torch)
        for _ in range(args.steps):
            fused(tm)
        torch.cuda.synchronize()
        ops = {}
        for k, (mean, med, mn, n) in tm.stats_ms().items():
            ent = {"us": round(mean * 1e3, 2), "us_median": round(med * 1e3, 2), "us_min": round(mn * 1e3, 2),
                   "launches_per_step": n // args.steps}
            if k in opf:
                tf = opf[k] / (mean * 1e-3) / 1e12
                ent.update(tflops=round(tf, 1), pct_peak=round(100 * tf / PEAK_BF16_TFLOPS, 2))
            ops[k] = ent
        line["ops"] = ops
        log("per-call (HIP events on the launch stream):")
        for k, v in ops.items():
            log(f"  {k:16s} {v}")
        # The unfused sequence of the same block on the same tensors.
        for _ in range(args.warmup):
            unfused()
        ums = timed_steps(torch, unfused, args.steps)
        utm = OpTimer(torch)
        for _ in range(args.steps):
            unfused(utm)
        torch.cuda.synchronize()
        line["unfused"] = {
            "ms_per_step": round(ums, 5), "value": round(total_flops / (ums * 1e-3) / 1e12, 2),
            "fused_speedup": round(ums / ms_step, 4),
            "ops": {k: {"us_median": round(v[1] * 1e3, 2), "launches_per_step": v[3] // args.steps}
                    for k, v in utm.stats_ms().items()},
        }
        log(f"unfused block: {ums:.3f} ms/step ({ums / ms_step:.3f}x the fused step)")
        # Board power and clocks while the fused step runs for a few seconds
        # (outside the timed region): the rate the step sustains at the cap.
        if not args.no_power:
            line["board_power"] = {"load": "the fused step, back to back",
                                   **sustained_load(torch, fused, total_flops, 6.0, power_cap_w(), settle=2.0)}
            log(f"board power: {line['board_power']}")
        line["cold_cache"] = {
            "working_set_bytes": int(ws_bytes),
            "note": f"the step touches {ws_bytes / 2 ** 30:.1f} GiB of weights, activations and gradients, far "
                    "beyond the 256 MB Infinity Cache: every timed step runs from HBM; the config-2 entry "
                    "carries a rotated-input cold-cache run of its smaller step"}
        del T
        fused = unfused = None
        torch.cuda.empty_cache()
        line["config2_block_forward"] = bench_c2(torch, coda, synth)
        log(f"config-2 block forward: {line['config2_block_forward']['value']} TFLOP/s")
        line["mfma_clock_probe"] = mfma_probe(torch, coda, dev["cus"])
        log(f"clock probe: {line['mfma_clock_probe']}")

    cpu = None
    if not args.no_cpu:
        cpu = block_cpu_baseline(p, M, d, F)
        log(f"cpu oracle: {cpu}")
    line["cpu_baseline"] = cpu

    if args.all:
        torch.cuda.empty_cache()
        rows = bench_all(torch, coda, synth, max(1, args.iters))
        if args.out:
            with open(args.out, "w") as f:
                for r_ in rows:
                    f.write(json.dumps(r_) + "\n")

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
