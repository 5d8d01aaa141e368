"""Seeded shape fuzz of every fused call against the fp64 oracle.

Each case draws its sizes from a seeded generator within the documented
limits (M arbitrary, widths and K multiples of 8, often not of the 64-deep k
tile or the 256-wide tile) and passes every bf16 matrix as a strided view
into a larger buffer:
  - input padding (columns past the logical width, rows past the last) holds
    NaN, so any element read past the view poisons the result;
  - output padding holds canaries that must survive the call.
Bound: max|gpu - ref| <= 2e-2 * max|ref| per output, as in the parity tests.
"""

import numpy as np
import pytest
import torch

from gpu_util import assert_close, canary_intact, f64, say
from gemm_epilogue_transformer_mainloop_amd import synth as S
from oracle import coda_oracle as O

pytestmark = pytest.mark.gpu

SEEDS = list(range(6))
BF16_NAN = 0x7FC0


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gemm_epilogue_transformer_mainloop_amd import coda

    coda.lib()
    yield


def C():
    from gemm_epilogue_transformer_mainloop_amd import coda

    return coda


def rng_of(call, seed):
    """One generator per (call, seed); the call name only decorrelates the calls."""
    return np.random.default_rng([sum(map(ord, call)), seed])


def m8(rng, lo, hi):
    """A multiple of 8 in [lo, hi]."""
    return 8 * int(rng.integers(max(lo // 8, 1), hi // 8 + 1))


def dims(rng):
    """Token count (any), plus a K that is often not a multiple of 64."""
    M = int(rng.choice([1, 7, 31, 63, 64, 65, 129, 255, 256, 257, 300, 511, 640]))
    K = m8(rng, 8, 600)
    return M, K


def strided_in(b, rng):
    """bf16 matrix (synth.Bf16) -> cuda view with NaN padding (extra columns
    rounded so ld % 8 == 0, and one extra row)."""
    rows, cols = b.bits.shape
    pad = 8 * int(rng.integers(0, 4))
    full = torch.full((rows + 1, cols + pad), BF16_NAN, dtype=torch.int16, device="cuda")
    full[:rows, :cols] = torch.from_numpy(b.bits.view(np.int16)).to("cuda")
    return full.view(torch.bfloat16)[:rows, :cols]


def strided_out(rows, cols, dtype, rng):
    pad_cols = (8 if dtype == torch.bfloat16 else 4) * int(rng.integers(1, 4))
    fill = -1024.0 if dtype == torch.bfloat16 else 12345.0
    full = torch.full((rows + 2, cols + pad_cols), fill, dtype=dtype, device="cuda")
    return full, full[:rows, :cols]


def intact(full, view):
    return canary_intact(full, view.shape[0], view.shape[1])


def vec(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_gemm(seed):
    rng = rng_of("gemm", seed)
    M, K = dims(rng)
    N = m8(rng, 8, 800)
    say(f"case: fuzz gemm seed={seed} M={M} N={N} K={K}")
    X = S.normal_bf16(rng.integers(1 << 30), (M, K))
    W = S.normal_bf16(rng.integers(1 << 30), (K, N), std=K ** -0.5)
    Yf, Y = strided_out(M, N, torch.bfloat16, rng)
    C().coda_gemm(strided_in(X, rng), strided_in(W, rng), Y=Y)
    torch.cuda.synchronize()
    assert_close(f64(Y), O.gemm(X.f64(), W.f64()), "Y")
    assert intact(Yf, Y)


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_res_sumsq_rowscale(seed):
    rng = rng_of("norm", seed)
    M, K = dims(rng)
    d = m8(rng, 8, 800)
    N = m8(rng, 8, 600)
    eps = 1e-6
    say(f"case: fuzz res_sumsq + row_rms + rowscale seed={seed} M={M} K={K} d={d} N={N}")
    x = S.normal_bf16(rng.integers(1 << 30), (M, K))
    W0 = S.normal_bf16(rng.integers(1 << 30), (K, d), std=K ** -0.5)
    z = S.normal_bf16(rng.integers(1 << 30), (M, d))
    g = S.normal_bf16(rng.integers(1 << 30), (d,), std=0.1, mean=1.0)
    W1 = S.normal_bf16(rng.integers(1 << 30), (d, N), std=d ** -0.5)
    coda = C()
    Uf, U = strided_out(M, d, torch.bfloat16, rng)
    Hf, H2 = strided_out(M, d, torch.bfloat16, rng)
    coda.coda_gemm_res_sumsq(strided_in(x, rng), strided_in(W0, rng), Z=strided_in(z, rng),
                             gamma=g.torch("cuda"), U=U, H2=H2)
    _, _, part = coda.coda_gemm_res_sumsq(strided_in(x, rng), strided_in(W0, rng), Z=strided_in(z, rng),
                                          gamma=g.torch("cuda"), want_h2=False)
    r = coda.coda_row_rms(part, d, eps)
    Yf, Y = strided_out(M, N, torch.bfloat16, rng)
    coda.coda_gemm_rowscale(H2, strided_in(W1, rng), r, Y=Y)
    torch.cuda.synchronize()
    u, h2, ss = O.res_sumsq(x.f64(), W0.f64(), z.f64(), g.f64())
    assert_close(f64(U), u, "u")
    assert_close(f64(H2), h2, "h2")
    assert_close(part.double().sum(1).cpu().numpy(), ss, "sum of partials")
    y, _, r_ref = O.norm_block_fwd(x.f64(), W0.f64(), z.f64(), g.f64(), W1.f64(), eps)
    assert_close(f64(r), r_ref, "r")
    assert_close(f64(Y), y, "y")
    assert intact(Uf, U) and intact(Hf, H2) and intact(Yf, Y)


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_rope(seed):
    rng = rng_of("rope", seed)
    M, K = dims(rng)
    hd = int(rng.choice([2, 8, 24, 64, 128]))
    N = m8(rng, 8, 800)
    unit = int(np.lcm(hd, 8))  # n_rope is a multiple of head_dim and of 8
    n_rope = unit * int(rng.integers(0, N // unit + 1))
    theta = float(rng.choice([10000.0, 500000.0]))
    say(f"case: fuzz rope seed={seed} M={M} K={K} N={N} head_dim={hd} n_rope={n_rope}")
    A = S.normal_bf16(rng.integers(1 << 30), (M, K))
    W = S.normal_bf16(rng.integers(1 << 30), (K, N), std=K ** -0.5)
    r = (0.5 + rng.random(M)).astype(np.float32)
    pos = rng.integers(0, 8192, M).astype(np.int32)
    coda = C()
    Yf, Y = strided_out(M, N, torch.bfloat16, rng)
    Bf, Yb = strided_out(M, N, torch.bfloat16, rng)
    coda.coda_gemm_rope(strided_in(A, rng), strided_in(W, rng), vec(r), vec(pos), theta, hd, n_rope, Y=Y)
    coda.coda_gemm_rope_bwd(strided_in(A, rng), strided_in(W, rng), None, vec(pos), theta, hd, n_rope, Y=Yb)
    torch.cuda.synchronize()
    t = O.gemm(A.f64(), W.f64())
    assert_close(f64(Y), O.rope(O.row_scale(r, t), pos, theta, hd, n_rope), "rope")
    assert_close(f64(Yb), O.rope(t, pos, theta, hd, n_rope, inverse=True), "rope_bwd")
    assert intact(Yf, Y) and intact(Bf, Yb)


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_swiglu_fwd_bwd(seed):
    rng = rng_of("swiglu", seed)
    M, K = dims(rng)
    F = m8(rng, 8, 520)
    N = m8(rng, 8, 520)
    with_r = bool(rng.integers(0, 2))
    say(f"case: fuzz swiglu fwd/bwd seed={seed} M={M} K={K} F={F} N={N} r={with_r}")
    A = S.normal_bf16(rng.integers(1 << 30), (M, K))
    Wgu = S.normal_bf16(rng.integers(1 << 30), (K, 2 * F), std=K ** -0.5)
    dOut = S.normal_bf16(rng.integers(1 << 30), (M, N))
    Wd = S.normal_bf16(rng.integers(1 << 30), (F, N), std=F ** -0.5)
    r = (0.5 + rng.random(M)).astype(np.float32) if with_r else None
    coda = C()
    Af, act = strided_out(M, F, torch.bfloat16, rng)
    Pf, pre = strided_out(M, 2 * F, torch.bfloat16, rng)
    coda.coda_gemm_swiglu(strided_in(A, rng), strided_in(Wgu, rng), None if r is None else vec(r), Act=act, Pre=pre)
    torch.cuda.synchronize()
    t = O.gemm(A.f64(), Wgu.f64())
    if with_r:
        t = O.row_scale(r, t)
    assert_close(f64(pre), t, "pre")
    assert_close(f64(act), O.swiglu(t), "act")
    assert intact(Af, act) and intact(Pf, pre)
    # backward over the (bf16) pre-activations just produced
    Df, dpre = strided_out(M, 2 * F, torch.bfloat16, rng)
    _, spart = coda.coda_gemm_swiglu_bwd(strided_in(dOut, rng), strided_in(Wd, rng), pre, dPre=dpre)
    s = coda.coda_row_rms_bwd(spart, 2 * F)
    torch.cuda.synchronize()
    pre64 = f64(pre)
    ref = O.swiglu_bwd(O.gemm(dOut.f64(), Wd.f64().T), pre64)
    assert_close(f64(dpre), ref, "dpre")
    assert_close(f64(s), np.sum(ref * pre64, axis=1) / (2 * F), "s")
    assert intact(Df, dpre)


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_rowscale_bwd(seed):
    rng = rng_of("rowscale_bwd", seed)
    M, _ = dims(rng)
    d = m8(rng, 8, 600)
    N = m8(rng, 8, 600)
    with_res = bool(rng.integers(0, 2))
    eps = 1e-6
    say(f"case: fuzz rowscale bwd seed={seed} M={M} d={d} N={N} dres={with_res}")
    dY = S.normal_bf16(rng.integers(1 << 30), (M, N))
    W1 = S.normal_bf16(rng.integers(1 << 30), (d, N), std=d ** -0.5)
    u = S.normal_bf16(rng.integers(1 << 30), (M, d))
    gamma = S.normal_bf16(rng.integers(1 << 30), (d,), std=0.1, mean=1.0)
    dres = S.normal_bf16(rng.integers(1 << 30), (M, d)) if with_res else None
    G = O.gemm(dY.f64(), W1.f64().T)
    du_ref, dg_ref, s_ref, r_ref = O.rmsnorm_bwd(G, u.f64(), gamma.f64(), eps,
                                                 dres=None if dres is None else dres.f64())
    n2_ref, _ = O.rmsnorm(u.f64(), gamma.f64(), eps)
    coda = C()
    Uf, dU = strided_out(M, d, torch.bfloat16, rng)
    Nf, N2 = strided_out(M, d, torch.bfloat16, rng)
    _, _, gpart = coda.coda_gemm_rowscale_bwd(
        strided_in(dY, rng), strided_in(W1, rng), strided_in(u, rng), gamma.torch("cuda"),
        vec(r_ref.astype(np.float32)), vec(s_ref.astype(np.float32)),
        dRes=None if dres is None else strided_in(dres, rng), dU=dU, N2=N2)
    dgamma = coda.coda_col_reduce(gpart)
    torch.cuda.synchronize()
    assert_close(f64(dU), du_ref, "du")
    assert_close(f64(N2), n2_ref, "n2")
    assert_close(f64(dgamma), dg_ref, "dgamma")
    assert intact(Uf, dU) and intact(Nf, N2)


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_res_bwd_and_wgrad(seed):
    rng = rng_of("res_bwd", seed)
    M, _ = dims(rng)
    N = m8(rng, 8, 600)
    K = m8(rng, 8, 600)
    with_res = bool(rng.integers(0, 2))
    say(f"case: fuzz res_sumsq_bwd + wgrad seed={seed} M={M} N={N} K={K} dres={with_res}")
    dU = S.normal_bf16(rng.integers(1 << 30), (M, N))
    W = S.normal_bf16(rng.integers(1 << 30), (K, N), std=K ** -0.5)
    X = S.normal_bf16(rng.integers(1 << 30), (M, K))
    dres = S.normal_bf16(rng.integers(1 << 30), (M, K)) if with_res else None
    coda = C()
    Xf, dX = strided_out(M, K, torch.bfloat16, rng)
    Wf, dW = strided_out(K, N, torch.float32, rng)
    coda.coda_gemm_res_sumsq_bwd(strided_in(dU, rng), strided_in(W, rng), X=strided_in(X, rng),
                                 dRes=None if dres is None else strided_in(dres, rng), dX=dX, dW=dW)
    acc = dW.clone()
    coda.coda_gemm_wgrad(strided_in(X, rng), strided_in(dU, rng), dW=acc, accumulate=True)
    torch.cuda.synchronize()
    dx_ref = O.gemm(dU.f64(), W.f64().T) + (0.0 if dres is None else dres.f64())
    assert_close(f64(dX), dx_ref, "dX")
    ref = O.gemm(X.f64().T, dU.f64())
    assert_close(dW.cpu().numpy(), ref, "dW")
    assert_close(acc.cpu().numpy(), 2 * ref, "dW accumulate")
    assert intact(Xf, dX) and intact(Wf, dW)


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_lmhead_ce(seed):
    rng = rng_of("lmhead", seed)
    M, _ = dims(rng)
    d = m8(rng, 8, 520)
    V = m8(rng, 8, 1600)
    say(f"case: fuzz lmhead ce seed={seed} M={M} d={d} V={V}")
    h = S.normal_bf16(rng.integers(1 << 30), (M, d))
    W = S.normal_bf16(rng.integers(1 << 30), (d, V), std=d ** -0.5)
    labels = rng.integers(0, V, M).astype(np.int32)
    labels[: min(M, 2)] = [0, V - 1][: min(M, 2)]
    coda = C()
    H, Wt, lab = strided_in(h, rng), strided_in(W, rng), vec(labels)
    lse, loss_row, loss_mean = coda.coda_lmhead_ce(H, Wt, lab)
    Hf, dH = strided_out(M, d, torch.bfloat16, rng)
    Wf, dW = strided_out(d, V, torch.float32, rng)
    rows = int(rng.choice([M, 256, 512]))  # 256-row chunks are the minimum
    coda.coda_lmhead_ce_bwd(H, Wt, lab, lse, 1.0 / M, dH=dH, dW=dW, ws_rows=rows)
    torch.cuda.synchronize()
    lse_r, loss_r, mean_r = O.lmhead_ce(h.f64(), W.f64(), labels)
    assert_close(f64(lse), lse_r, "lse")
    assert_close(f64(loss_row), loss_r, "loss_row")
    assert abs(float(loss_mean.item()) - mean_r) <= 1e-3 * abs(mean_r)
    dh_r, dW_r, _ = O.lmhead_ce_bwd(h.f64(), W.f64(), labels, 1.0 / M)
    assert_close(f64(dH), dh_r, "dh")
    assert_close(dW.cpu().numpy(), dW_r, "dW")
    assert intact(Hf, dH) and intact(Wf, dW)


@pytest.mark.parametrize("seed", SEEDS)
def test_fuzz_lmhead_ce_logits(seed):
    """The stored-logits forward and its backward (dlogits in place)."""
    rng = rng_of("lmhead_logits", seed)
    M, _ = dims(rng)
    d = m8(rng, 8, 520)
    V = m8(rng, 8, 1600)
    say(f"case: fuzz lmhead ce (stored logits) seed={seed} M={M} d={d} V={V}")
    h = S.normal_bf16(rng.integers(1 << 30), (M, d))
    W = S.normal_bf16(rng.integers(1 << 30), (d, V), std=d ** -0.5)
    labels = rng.integers(0, V, M).astype(np.int32)
    labels[: min(M, 2)] = [0, V - 1][: min(M, 2)]
    coda = C()
    H, Wt, lab = strided_in(h, rng), strided_in(W, rng), vec(labels)
    Lf, logits = strided_out(M, V, torch.bfloat16, rng)
    lse, loss_row, loss_mean, _ = coda.coda_lmhead_ce_logits(H, Wt, lab, logits=logits)
    torch.cuda.synchronize()
    l_gpu = f64(logits)
    Hf, dH = strided_out(M, d, torch.bfloat16, rng)
    Wf, dW = strided_out(d, V, torch.float32, rng)
    coda.coda_lmhead_ce_bwd_logits(H, Wt, lab, lse, 1.0 / M, logits, dH=dH, dW=dW)
    torch.cuda.synchronize()
    assert_close(l_gpu, O.gemm(h.f64(), W.f64()), "logits")
    lse_r, loss_r, mean_r = O.lmhead_ce(h.f64(), W.f64(), labels)
    assert_close(f64(lse), lse_r, "lse")
    assert_close(f64(loss_row), loss_r, "loss_row")
    assert abs(float(loss_mean.item()) - mean_r) <= 1e-3 * abs(mean_r)
    dh_r, dW_r, D_r = O.lmhead_ce_bwd(h.f64(), W.f64(), labels, 1.0 / M)
    assert_close(f64(logits), D_r, "dlogits (in place of the logits)")
    assert_close(f64(dH), dh_r, "dh")
    assert_close(dW.cpu().numpy(), dW_r, "dW")
    assert intact(Lf, logits) and intact(Hf, dH) and intact(Wf, dW)
