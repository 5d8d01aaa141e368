"""The LayerNorm variant of the GEMM -> residual -> norm -> GEMM composition
(the paper's review page: LayerNorm gradients as an epilogue composition)
against the fp64 oracle, through the C ABI.

Forward: GEMM1 emits per-tile (mean, M2) partials, an auxiliary kernel merges
them into mu and r, and GEMM2's epilogue applies r (h3 - mu c) + b with
c = gamma^T W, b = beta^T W.  Backward: the next layer's SwiGLU-backward
epilogue accumulates the two row statistics, and the data-gradient epilogue
forms the delayed LayerNorm backward with the dgamma / dbeta column partials.
Sizes span several tiles with ragged tails; the residual z has mean 0.5, so
the mean term matters.  Bound: max|gpu - ref| <= 2e-2 max|ref| per output.
"""

import numpy as np
import pytest
import torch

from gpu_util import assert_close, dev, f64, say
from gemm_epilogue_transformer_mainloop_amd import synth as S
from oracle import coda_oracle as O

pytestmark = pytest.mark.gpu


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


def f32np(t):
    return t.detach().double().cpu().numpy()


def test_ln_colvec():
    K, N = 520, 264
    say(f"case: ln_colvec K={K} N={N}")
    W = S.normal_bf16(71, (K, N), std=K ** -0.5)
    g = S.normal_bf16(72, (K,), std=0.1, mean=1.0)
    b = S.normal_bf16(73, (K,), std=0.1)
    c, bv = C().coda_ln_colvec(dev(W), dev(g), dev(b))
    c0, bv0 = C().coda_ln_colvec(dev(W), dev(g))
    torch.cuda.synchronize()
    assert bv0 is None
    assert_close(f32np(c), O.gemm(g.f64()[None, :], W.f64())[0], "c = gamma^T W")
    assert_close(f32np(bv), O.gemm(b.f64()[None, :], W.f64())[0], "b = beta^T W")
    assert torch.equal(c, c0)


def ln_forward(p, with_beta=True):
    coda = C()
    T = {k: dev(v) for k, v in p.items() if k != "eps"}
    d = T["W0"].shape[1]
    beta = T["beta"] if with_beta else None
    U, H2, pm, pq = coda.coda_gemm_res_lnstats(T["x"], T["W0"], T["z"], T["gamma"])
    mu, r = coda.coda_row_ln(pm, pq, d, p["eps"])
    c, b = coda.coda_ln_colvec(T["W1"], T["gamma"], beta)
    Y = coda.coda_gemm_ln_rowscale(H2, T["W1"], r, mu, c, b)
    torch.cuda.synchronize()
    return U, H2, mu, r, Y


@pytest.mark.parametrize("with_beta", [True, False])
def test_ln_norm_block_forward(with_beta):
    M, K, d, N = 700, 256, 520, 264
    say(f"case: LayerNorm block forward M={M} K={K} d={d} N={N} beta={with_beta}")
    p = S.ln_norm_block_inputs(61, M, d, K, N)
    U, H2, mu, r, Y = ln_forward(p, with_beta)
    q = {k: (v.f64() if hasattr(v, "bits") else v) for k, v in p.items()}
    beta = q["beta"] if with_beta else np.zeros(d)
    y, u, mu_r, r_r = O.ln_norm_block_fwd(q["x"], q["W0"], q["z"], q["gamma"], beta, q["W1"], q["eps"])
    assert_close(f64(U), u, "u")
    assert_close(f64(H2), u * q["gamma"][None, :], "h2")
    assert_close(f32np(mu), mu_r, "mu")
    assert_close(f32np(r), r_r, "r")
    assert_close(f64(Y), y, "y")


@pytest.mark.slow
def test_ln_norm_block_forward_1b_shape():
    """The LayerNorm block forward at the 1B shape (M = 8192, d = 2048), sampled rows."""
    M, K, d, N = 8192, 2048, 2048, 2048
    say(f"case: LayerNorm block forward M={M} K={K} d={d} N={N}")
    p = S.ln_norm_block_inputs(62, M, d, K, N)
    U, H2, mu, r, Y = ln_forward(p)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, M - 1], np.random.default_rng(62).choice(M, 12, replace=False)]))
    q = {k: (v.f64() if hasattr(v, "bits") else v) for k, v in p.items()}
    y, u, mu_r, r_r = O.ln_norm_block_fwd(q["x"][rows], q["W0"], q["z"][rows], q["gamma"], q["beta"], q["W1"],
                                          q["eps"])
    idx = torch.as_tensor(rows, device="cuda")
    assert_close(f64(U[idx]), u, "u")
    assert_close(f32np(mu[idx]), mu_r, "mu")
    assert_close(f32np(r[idx]), r_r, "r")
    assert_close(f64(Y[idx]), y, "y")


def run_ln_block_gpu(p, M, d, F, with_beta=True):
    """Forward + reverse-fused backward of the two-layer LayerNorm block through the C ABI."""
    coda = C()
    T = {k: dev(v) for k, v in p.items() if k != "eps"}
    eps = p["eps"]
    be = {l: (T[f"beta{l}"] if with_beta else None) for l in (1, 2)}
    cv, bv = {}, {}
    for l in (1, 2):
        cv[l], bv[l] = coda.coda_ln_colvec(T[f"Wgu{l}"], T[f"gamma{l}"], be[l])
    f = {}
    f["u1"], h2_1, pm1, pq1 = coda.coda_gemm_res_lnstats(T["x"], T["W0"], T["z"], T["gamma1"])
    f["mu1"], f["r1"] = coda.coda_row_ln(pm1, pq1, d, eps)
    f["a1"], f["pre1"] = coda.coda_gemm_ln_swiglu(h2_1, T["Wgu1"], f["r1"], f["mu1"], cv[1], bv[1])
    f["u2"], h2_2, pm2, pq2 = coda.coda_gemm_res_lnstats(f["a1"], T["Wd1"], f["u1"], T["gamma2"])
    f["mu2"], f["r2"] = coda.coda_row_ln(pm2, pq2, d, eps)
    f["a2"], f["pre2"] = coda.coda_gemm_ln_swiglu(h2_2, T["Wgu2"], f["r2"], f["mu2"], cv[2], bv[2])
    f["out"], _, _ = coda.coda_gemm_res_sumsq(f["a2"], T["Wd2"], f["u2"], want_part=False)
    g = {}
    dres = T["dOut"]
    for l in (2, 1):
        g[f"dWd{l}"] = coda.coda_gemm_wgrad(f[f"a{l}"], dres)
        g[f"dpre{l}"], sp, ap = coda.coda_gemm_swiglu_bwd_ln(dres, T[f"Wd{l}"], f[f"pre{l}"], cv[l], bv[l])
        g[f"s{l}"], g[f"a{l}"] = coda.coda_row_ln_bwd(sp, ap, d)
        g[f"du{l}"], n2, gp, bp = coda.coda_gemm_ln_bwd(g[f"dpre{l}"], T[f"Wgu{l}"], f[f"u{l}"], T[f"gamma{l}"],
                                                        be[l], f[f"r{l}"], f[f"mu{l}"], g[f"s{l}"], g[f"a{l}"],
                                                        dRes=dres)
        g[f"dgamma{l}"] = coda.coda_col_reduce(gp)
        g[f"dbeta{l}"] = coda.coda_col_reduce(bp)
        g[f"dWgu{l}"] = coda.coda_gemm_wgrad(n2, g[f"dpre{l}"])
        dres = g[f"du{l}"]
    g["dx"], g["dW0"] = coda.coda_gemm_res_sumsq_bwd(g["du1"], T["W0"], X=T["x"])
    torch.cuda.synchronize()
    return f, g


@pytest.mark.parametrize("M,d,F,with_beta", [(520, 264, 392, True), (300, 384, 136, False)])
def test_ln_block_chain(M, d, F, with_beta):
    say(f"case: LayerNorm block fwd+bwd M={M} d={d} F={F} beta={with_beta}")
    p = S.ln_block_inputs(63, M, d, F)
    f, g = run_ln_block_gpu(p, M, d, F, with_beta)
    q = {k: (v.f64() if hasattr(v, "bits") else v) for k, v in p.items()}
    if not with_beta:
        q["beta1"] = np.zeros(d)
        q["beta2"] = np.zeros(d)
    fr = O.ln_block_fwd(q)
    gr = O.ln_block_bwd(q, fr)
    for k in ("u1", "mu1", "r1", "pre1", "a1", "u2", "mu2", "r2", "pre2", "a2", "out"):
        got = f32np(f[k]) if f[k].dtype == torch.float32 else f64(f[k])
        assert_close(got, fr[k], k)
    for k in ("dWd2", "dpre2", "s2", "a2", "du2", "dgamma2", "dbeta2", "dWgu2", "dWd1", "dpre1", "s1", "a1", "du1",
              "dgamma1", "dbeta1", "dWgu1", "dx", "dW0"):
        got = f32np(g[k]) if g[k].dtype == torch.float32 else f64(g[k])
        assert_close(got, gr[k], k)
