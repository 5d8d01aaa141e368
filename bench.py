#!/usr/bin/env python3
"""Benchmark of the CODA GEMM-epilogue path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--all] [--out FILE]

One step = one pass of the fused GEMM -> residual -> RMSNorm -> GEMM forward
at the Llama-3-1B-like shape (M = 8192 tokens, d = 2048) on seeded synthetic
bf16 inputs already resident in HBM:

  coda_gemm_res_sumsq  u = x W0 + z, h2 = u*gamma, sum-of-squares partials  (8192 x 2048 x 2048)
  coda_row_rms         r = 1/sqrt(sum/d + eps)                             (aux, 8192 x 16)
  coda_gemm_rowscale   y = r * (h2 W1)                                     (8192 x 2048 x 2048)
  coda_gemm_rope       y_qkv = rope(r * (h2 W1qkv)), Q and K rotated        (8192 x 3072 x 2048)

The metric counts only the GEMMs' algorithmic 2*M*N*K FLOPs.  Each kernel is
timed with HIP events recorded on the stream it is launched on, inside the
timed region.  Rank 0 prints ONE JSON line on stdout; tables go to stderr.
``--all`` also measures every fused call of the five synthetic workloads
against the plain GEMM of the same shape and writes them to ``--out``.
"""

from __future__ import annotations

import argparse
import hashlib
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


def src_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gemm_epilogue_transformer_mainloop_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
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

    def mean_ms(self):
        return {k: float(np.mean([s.elapsed_time(e) for s, e in v])) for k, v in self.ev.items()}

    def stats_ms(self):
        """Per op: (mean, median, min) over the recorded launches."""
        out = {}
        for k, v in self.ev.items():
            t = [s.elapsed_time(e) for s, e in v]
            out[k] = (float(np.mean(t)), float(np.median(t)), float(np.min(t)))
        return out


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


# ----------------------------------------------------------------------------
# config-2 step
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
        run = tm.run if tm is not None else (lambda n, f: f())
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
        run = tm.run if tm is not None else (lambda n, f: f())
        run("gemm0", lambda: coda.coda_gemm(T["x"], T["W0"], buf["Y0"]))
        run("add_rmsnorm", lambda: coda.coda_unfused_add_rmsnorm(buf["Y0"], T["z"], T["gamma"], eps, U=buf["U"],
                                                                 N2=buf["N2"], r=buf["r"]))
        run("gemm1", lambda: coda.coda_gemm(buf["N2"], T["W1"], buf["Y"]))
        run("gemm_qkv", lambda: coda.coda_gemm(buf["N2"], T["W1r"], buf["Yr"]))
        run("rope", lambda: coda.coda_unfused_rope(buf["Yr"], T["pos"], 500000.0, 64, n_rope))

    return step


def cold_cache(torch, coda, synth, p, T, dims, n_rope, total_flops, min_bytes=600 << 20, steps=30):
    """Fused step with the inputs rotated over enough copies to exceed the MALL."""
    M, d, K, N, NR = dims
    keys = ("x", "W0", "z", "gamma", "W1", "W1r")
    per_set = sum(T[k].numel() * T[k].element_size() for k in keys)
    nsets = max(2, -(-min_bytes // per_set))
    sets = []
    for i in range(nsets):
        Ti = dict(T)
        for k in keys:
            Ti[k] = T[k].clone()
        sets.append(make_c2_step(torch, coda, Ti, dims, p["eps"])[0])
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


def cpu_baseline(p, dims, n_rope, min_seconds=12.0, max_steps=60):
    """The fp64 oracle timed on the host on whole config-2 steps (at least
    min_seconds, at most max_steps: about 12-30 s of host work)."""
    from oracle import coda_oracle as O
    from threadpoolctl import threadpool_info

    M, d, K, N, NR = dims
    x, W0, z, g, W1, W1r = (p[k].f64() for k in ("x", "W0", "z", "gamma", "W1", "W1r"))
    pos = p["pos"]
    flops = sum(c2_flops(*dims).values())
    steps = 0
    t0 = time.perf_counter()
    while True:
        u, h2, ss = O.res_sumsq(x, W0, z, g)
        n2, r = O.rmsnorm(u, g, p["eps"])
        y = O.gemm(n2, W1)
        yr = O.rope(O.gemm(n2, W1r), pos, 500000.0, 64, n_rope)
        steps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or steps >= max_steps:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(flops * steps / el / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{steps} whole config-2 steps (M=8192, d=2048; 240.5 GFLOP each) in fp64 numpy, "
                      f"{el:.1f} s"}


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
    spart = torch.empty(M, coda.coda_nparts(F), device="cuda")
    rec(5, "swiglu_bwd+s", M, F, d, lambda: coda.coda_gemm_swiglu_bwd(dOut, Wd, pre, dpre, spart), plain_nt(M, F, d))
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
    rows += bench_block(torch, coda, seq_fn=seq)
    return rows


def bench_block(torch, coda, seq_fn):
    """The whole config-5 block (W0 projection + two residual/RMSNorm/SwiGLU-MLP
    layers), forward and backward as one stream ("CODA" paper Figure 11):
    the fused calls against the unfused sequence."""
    bf, f32 = torch.bfloat16, torch.float32
    M, d, F, eps = 8192, 4096, 14336, 1e-6

    def rnd(*shape, std=1.0):
        return (torch.randn(*shape, device="cuda") * std).to(bf)

    def emp(*shape, dtype=bf):
        return torch.empty(*shape, dtype=dtype, device="cuda")

    x, z, dOut, W0 = rnd(M, d), rnd(M, d), rnd(M, d), rnd(d, d, std=d ** -0.5)
    L = [dict(g=(1.0 + 0.1 * torch.randn(d, device="cuda")).to(bf), Wgu=rnd(d, 2 * F, std=d ** -0.5),
              Wd=rnd(F, d, std=F ** -0.5)) for _ in range(2)]
    # activations (shared shapes by both paths) and gradients
    A = [dict(u=emp(M, d), h=emp(M, d), part=emp(M, coda.coda_nparts(d), dtype=f32), r=emp(M, dtype=f32),
              pre=emp(M, 2 * F), a=emp(M, F), dpre=emp(M, 2 * F), du=emp(M, d), n2=emp(M, d),
              sp=emp(M, coda.coda_nparts(F), dtype=f32), s=emp(M, dtype=f32),
              gp=emp(coda.coda_mparts(M), d, dtype=f32), gpu=emp(coda.coda_unfused_rmsnorm_bwd_parts(M), d, dtype=f32),
              dg=emp(d, dtype=f32), dWgu=emp(d, 2 * F, dtype=f32), dWd=emp(F, d, dtype=f32), da=emp(M, F),
              G=emp(M, d), y=emp(M, d)) for _ in range(2)]
    out, dx, dW0, Y0, T = emp(M, d), emp(M, d), emp(d, d, dtype=f32), emp(M, d), emp(M, d)

    def fused():
        a1, a2 = A
        coda.coda_gemm_res_sumsq(x, W0, z, L[0]["g"], a1["u"], a1["h"], a1["part"])
        coda.coda_row_rms(a1["part"], d, eps, a1["r"])
        coda.coda_gemm_swiglu(a1["h"], L[0]["Wgu"], a1["r"], a1["a"], a1["pre"])
        coda.coda_gemm_res_sumsq(a1["a"], L[0]["Wd"], a1["u"], L[1]["g"], a2["u"], a2["h"], a2["part"])
        coda.coda_row_rms(a2["part"], d, eps, a2["r"])
        coda.coda_gemm_swiglu(a2["h"], L[1]["Wgu"], a2["r"], a2["a"], a2["pre"])
        coda.coda_gemm_res_sumsq(a2["a"], L[1]["Wd"], a2["u"], U=out, want_part=False)
        dres = dOut
        for l in (1, 0):
            c, W = A[l], L[l]
            coda.coda_gemm_wgrad(c["a"], dres, c["dWd"])
            coda.coda_gemm_swiglu_bwd(dres, W["Wd"], c["pre"], c["dpre"], c["sp"])
            coda.coda_row_rms_bwd(c["sp"], d, c["s"])
            coda.coda_gemm_rowscale_bwd(c["dpre"], W["Wgu"], c["u"], W["g"], c["r"], c["s"], dres, c["du"], c["n2"],
                                        c["gp"])
            coda.coda_col_reduce(c["gp"], c["dg"])
            coda.coda_gemm_wgrad(c["n2"], c["dpre"], c["dWgu"])
            dres = c["du"]
        coda.coda_gemm_res_sumsq_bwd(A[0]["du"], W0, X=x, dX=dx, dW=dW0)

    def unfused():
        a1, a2 = A
        coda.coda_gemm(x, W0, Y0)
        coda.coda_unfused_add_rmsnorm(Y0, z, L[0]["g"], eps, a1["u"], a1["n2"], a1["r"])
        coda.coda_gemm(a1["n2"], L[0]["Wgu"], a1["pre"])
        coda.coda_unfused_swiglu(a1["pre"], a1["a"])
        coda.coda_gemm(a1["a"], L[0]["Wd"], T)
        coda.coda_unfused_add_rmsnorm(T, a1["u"], L[1]["g"], eps, a2["u"], a2["n2"], a2["r"])
        coda.coda_gemm(a2["n2"], L[1]["Wgu"], a2["pre"])
        coda.coda_unfused_swiglu(a2["pre"], a2["a"])
        coda.coda_gemm(a2["a"], L[1]["Wd"], T)
        coda.coda_unfused_add(T, a2["u"], out)
        dres = dOut
        for l in (1, 0):
            c, W = A[l], L[l]
            coda.coda_gemm_wgrad(c["a"], dres, c["dWd"])
            coda.coda_gemm_res_sumsq_bwd(dres, W["Wd"], dX=c["da"], want_dw=False)
            coda.coda_unfused_swiglu_bwd(c["da"], c["pre"], c["dpre"])
            coda.coda_gemm_res_sumsq_bwd(c["dpre"], W["Wgu"], dX=c["G"], want_dw=False)
            coda.coda_unfused_rmsnorm_bwd(c["G"], c["u"], W["g"], c["r"], dres, c["du"], c["gpu"])
            coda.coda_col_reduce(c["gpu"], c["dg"])
            coda.coda_gemm_wgrad(c["n2"], c["dpre"], c["dWgu"])
            dres = c["du"]
        coda.coda_gemm_res_sumsq_bwd(A[0]["du"], W0, X=x, dX=dx, dW=dW0)

    fwd = 2.0 * M * d * d + 2 * (2.0 * M * d * 2 * F + 2.0 * M * F * d)
    rows = []
    seq_fn(5, "block forward+backward (W0 + 2 layers)", 3 * fwd, fused, unfused, 3)
    return rows


# ----------------------------------------------------------------------------


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--all", action="store_true", help="also time every fused call of the five workloads")
    ap.add_argument("--out", default=None, help="file for the --all table (JSON lines)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
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
    coda.lib()  # fails loudly if the HIP library is not built

    if args.copy_calib:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 x {n} bytes read + {n} bytes written")
        return

    p, T, dims = c2_inputs(torch, synth)
    M, d, K, N, NR = dims
    step, buf, n_rope = make_c2_step(torch, coda, T, dims, p["eps"])
    flops = c2_flops(*dims)
    total_flops = sum(flops.values())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The timed region holds the K steps.  The roofline kernel (the RoPE
    # call) is timed inside it, back to back with the other kernels: one HIP
    # event pair around it in every tenth step (each pair delays the kernel
    # it brackets by its dispatch after the marker, so fewer pairs disturb
    # the step less).  An event pair around every call would make the host,
    # not the GPU, set the pace.
    dom = "rope"
    dtm = OpTimer(torch, only={dom})
    every = max(1, args.steps // 10)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(dtm if i % every == 0 else None)
    t_end.record()
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    dom_ms = dtm.mean_ms()[dom]

    # Per-op breakdown: another K steps with an event pair around every call,
    # outside the timed region (kernels separated by the event records).
    tm = OpTimer(torch)
    for _ in range(args.steps):
        step(tm)
    torch.cuda.synchronize()
    op_ms = tm.mean_ms()
    op_stats = tm.stats_ms()

    # The unfused sequence of the same block, same inputs, same number of
    # steps, timed the same way.
    ustep = make_c2_unfused_step(torch, coda, T, dims, p["eps"], n_rope)
    for _ in range(args.warmup):
        ustep()
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        ustep()
    t_end.record()
    torch.cuda.synchronize()
    ums_step = t_start.elapsed_time(t_end) / args.steps
    utm = OpTimer(torch)
    for _ in range(args.steps):
        ustep(utm)
    torch.cuda.synchronize()
    uops = {k: {"us_median": round(v[1] * 1e3, 2), "us_min": round(v[2] * 1e3, 2)}
            for k, v in utm.stats_ms().items()}
    log(f"unfused sequence: {ums_step * 1e3:.1f} us/step  {uops}")

    # Cold cache: rotate input sets totalling more than 512 MB, so that no step
    # finds its inputs in the 256 MB Infinity Cache.
    cold = cold_cache(torch, coda, synth, p, T, dims, n_rope, total_flops)
    log(f"cold cache: {cold}")

    value = total_flops / (ms_step * 1e-3) / 1e12
    achieved = flops[dom] / (dom_ms * 1e-3) / 1e12
    ops = {}
    for k, v in op_ms.items():
        ent = {"us": round(v * 1e3, 2), "us_median": round(op_stats[k][1] * 1e3, 2),
               "us_min": round(op_stats[k][2] * 1e3, 2)}
        if k in flops:
            tf = flops[k] / (v * 1e-3) / 1e12
            ent.update(tflops=round(tf, 1), pct_peak=round(100 * tf / PEAK_BF16_TFLOPS, 2))
        if k == "row_rms":  # aux reduction: algorithmic bytes (partials in, r out) per time
            nb = M * coda.coda_nparts(d) * 4 + M * 4
            ent.update(bytes=nb, gbs=round(nb / (v * 1e-3) / 1e9, 1),
                       pct_hbm=round(100 * nb / (v * 1e-3) / 1e9 / PEAK_HBM_GBS, 2))
        ops[k] = ent
    log("per-op (HIP events on the launch stream):")
    for k, v in ops.items():
        log(f"  {k:10s} {v}")

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(p, dims, n_rope)
        log(f"cpu oracle: {cpu}")

    if args.all:
        rows = bench_all(torch, coda, synth)
        if args.out:
            with open(args.out, "w") as f:
                for r_ in rows:
                    f.write(json.dumps(r_) + "\n")

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
            "workload": "GEMM->residual->RMSNorm->GEMM forward, Llama-3-1B-like: M=8192 tokens (4x2048), d=2048, "
                        "W1 2048x2048 (rowscale) and QKV W1 2048x3072 with RoPE (theta=5e5, hd=64)",
            "M": M, "d": d, "K": K, "N": N, "N_qkv": NR, "n_rope": n_rope,
            "calls": ["coda_gemm_res_sumsq", "coda_row_rms", "coda_gemm_rowscale", "coda_gemm_rope"],
        },
        "ops": ops,
        "unfused": {
            "ms_per_step": round(ums_step, 5),
            "value": round(total_flops / (ums_step * 1e-3) / 1e12, 2),
            "fused_speedup": round(ums_step / ms_step, 4),
            "calls": ["coda_gemm", "coda_unfused_add_rmsnorm", "coda_gemm", "coda_gemm", "coda_unfused_rope"],
            "ops": uops,
        },
        "cold_cache": cold,
        "roofline": {
            "bound": "mfma",
            "kernel": "coda_gemm_rope (8192x3072x2048)",
            "us_per_launch": round(dom_ms * 1e3, 2),
            "launches_timed": len(dtm.ev[dom]),
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": load_traffic("rope_c2"),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
