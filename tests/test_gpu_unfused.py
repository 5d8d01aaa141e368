"""GPU parity of the unfused baseline (include/coda_unfused.h) against the fp64
oracle: every standalone kernel on ragged sizes, and the unfused sequences of
the norm block, the SwiGLU MLP and the LM head (plain GEMMs + standalone
kernels) against the same oracle chains the fused calls are tested on.

Bound (per output): max|gpu - ref| <= 2e-2 * max|ref|; scalar loss relative
error <= 1e-3.
"""

import numpy as np
import pytest
import torch

from gpu_util import LOSS_RTOL, assert_close, dev, f64, say
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


@pytest.mark.parametrize("M,d,with_z", [(300, 520, True), (33, 4104, True), (9, 8192, False)])
def test_unfused_add_rmsnorm(M, d, with_z):
    say(f"case: unfused add+rmsnorm M={M} d={d} z={with_z}")
    y = S.normal_bf16(301, (M, d))
    z = S.normal_bf16(302, (M, d)) if with_z else None
    gamma = S.normal_bf16(303, (d,), std=0.1, mean=1.0)
    U, N2, r = C().coda_unfused_add_rmsnorm(dev(y), None if z is None else dev(z), dev(gamma), 1e-6)
    torch.cuda.synchronize()
    u = y.f64() + (z.f64() if z is not None else 0.0)
    n2, r_ref = O.rmsnorm(u, gamma.f64(), 1e-6)
    assert_close(f64(U), u, "U")
    assert_close(r.cpu().numpy(), r_ref, "r")
    assert_close(f64(N2), n2, "N2")


@pytest.mark.parametrize("inverse,hd,n_rope", [(False, 64, 256), (True, 64, 256), (False, 2, 6), (True, 6, 18),
                                                (False, 128, 384)])
def test_unfused_rope(inverse, hd, n_rope):
    """n_rope need not be a multiple of 8 here: the last chunk rotates only its leading pairs."""
    M, N = 130, 384
    say(f"case: unfused rope M={M} N={N} head_dim={hd} n_rope={n_rope} inverse={inverse}")
    t = S.normal_bf16(311, (M, N))
    pos = S.positions_int32(M, 2048)
    Y = dev(t)
    C().coda_unfused_rope(Y, dev(pos), S.ROPE_THETA, hd, n_rope, inverse)
    torch.cuda.synchronize()
    assert_close(f64(Y), O.rope(t.f64(), pos, S.ROPE_THETA, hd, n_rope, inverse), "Y")


def test_unfused_swiglu_fwd_bwd():
    M, F = 70, 264
    say(f"case: unfused swiglu fwd/bwd M={M} F={F}")
    pre = S.normal_bf16(321, (M, 2 * F), std=2.0)
    da = S.normal_bf16(322, (M, F))
    coda = C()
    act = coda.coda_unfused_swiglu(dev(pre))
    dpre = coda.coda_unfused_swiglu_bwd(dev(da), dev(pre))
    torch.cuda.synchronize()
    assert_close(f64(act), O.swiglu(pre.f64()), "act")
    assert_close(f64(dpre), O.swiglu_bwd(da.f64(), pre.f64()), "dpre")


@pytest.mark.parametrize("M,d,with_res", [(70, 520, True), (33, 4096, False)])
def test_unfused_rmsnorm_bwd(M, d, with_res):
    say(f"case: unfused rmsnorm bwd M={M} d={d} dres={with_res}")
    G = S.normal_bf16(331, (M, d))
    u = S.normal_bf16(332, (M, d))
    gamma = S.normal_bf16(333, (d,), std=0.1, mean=1.0)
    dres = S.normal_bf16(334, (M, d)) if with_res else None
    eps = 1e-6
    du_ref, dg_ref, _, r_ref = O.rmsnorm_bwd(G.f64(), u.f64(), gamma.f64(), eps,
                                             dres=None if dres is None else dres.f64())
    coda = C()
    r = torch.tensor(r_ref, dtype=torch.float32, device="cuda")
    dU, gpart = coda.coda_unfused_rmsnorm_bwd(dev(G), dev(u), dev(gamma), r, None if dres is None else dev(dres))
    assert gpart.shape[0] == coda.coda_unfused_rmsnorm_bwd_parts(M)
    dgamma = coda.coda_col_reduce(gpart)
    torch.cuda.synchronize()
    assert_close(f64(dU), du_ref, "dU")
    assert_close(dgamma.cpu().numpy(), dg_ref, "dgamma")


def test_unfused_cross_entropy_and_bwd():
    M, d, V = 37, 64, 1000
    say(f"case: unfused CE fwd/bwd over materialised logits M={M} V={V}")
    h = S.normal_bf16(341, (M, d))
    W = S.normal_bf16(342, (d, V), std=d ** -0.5)
    labels = S.labels_int32(343, M, V)
    coda = C()
    L = coda.coda_gemm(dev(h), dev(W))
    lse, loss_row, loss_mean = coda.coda_unfused_cross_entropy(L, dev(labels))
    D = coda.coda_unfused_cross_entropy_bwd(L, dev(labels), lse, 1.0 / M)
    torch.cuda.synchronize()
    lse_ref, loss_ref, mean_ref = O.lmhead_ce(h.f64(), W.f64(), labels)
    assert_close(lse.cpu().numpy(), lse_ref, "lse")
    assert_close(loss_row.cpu().numpy(), loss_ref, "loss_row")
    assert abs(float(loss_mean.item()) - mean_ref) <= LOSS_RTOL * abs(mean_ref)
    _, _, D_ref = O.lmhead_ce_bwd(h.f64(), W.f64(), labels, 1.0 / M)
    assert_close(f64(D), D_ref, "dlogits")
    # a label outside [0, V) gives a NaN row loss
    bad = labels.copy()
    bad[4] = V
    _, lr, _ = coda.coda_unfused_cross_entropy(L, dev(bad))
    torch.cuda.synchronize()
    lr = lr.cpu().numpy()
    assert np.isnan(lr[4]) and np.all(np.isfinite(np.delete(lr, 4)))


def test_unfused_norm_block_sequence():
    """Plain GEMM -> add+RMSNorm -> plain GEMM (+ plain GEMM -> RoPE): the unfused
    form of the norm block, against the canonical oracle chain."""
    M, d, K, N, NR = 264, 256, 256, 520, 384
    say(f"case: unfused norm-block sequence M={M} d={d} N={N} N_rope={NR}")
    p = S.norm_block_inputs(1, M, d, K, N)
    coda = C()
    x, W0, z, gamma, W1 = (dev(p[k]) for k in ("x", "W0", "z", "gamma", "W1"))
    W1r = dev(S.normal_bf16(351, (d, NR), std=d ** -0.5))
    pos = S.positions_int32(M, 2048)
    Y0 = coda.coda_gemm(x, W0)
    U, N2, r = coda.coda_unfused_add_rmsnorm(Y0, z, gamma, p["eps"])
    y = coda.coda_gemm(N2, W1)
    q = coda.coda_gemm(N2, W1r)
    coda.coda_unfused_rope(q, dev(pos), S.ROPE_THETA, 64, 256)
    torch.cuda.synchronize()
    y_ref, u_ref, r_ref = O.norm_block_fwd(p["x"].f64(), p["W0"].f64(), p["z"].f64(), p["gamma"].f64(),
                                           p["W1"].f64(), p["eps"])
    n2_ref, _ = O.rmsnorm(u_ref, p["gamma"].f64(), p["eps"])
    assert_close(f64(U), u_ref, "u")
    assert_close(r.cpu().numpy(), r_ref, "r")
    assert_close(f64(y), y_ref, "y")
    q_ref = O.rope(O.gemm(n2_ref, f64(W1r)), pos, S.ROPE_THETA, 64, 256)
    assert_close(f64(q), q_ref, "q")


def test_unfused_mlp_sequence():
    """Plain GEMMs + standalone SwiGLU / add kernels, forward and backward."""
    M, d, F = 264, 256, 264
    say(f"case: unfused MLP sequence M={M} d={d} F={F}")
    p = S.mlp_inputs(3, M, d, F)
    coda = C()
    x, Wgu, Wd, dY = (dev(p[k]) for k in ("x", "Wgu", "Wd", "dY"))
    pre = coda.coda_gemm(x, Wgu)
    a = coda.coda_unfused_swiglu(pre)
    out = coda.coda_unfused_add(coda.coda_gemm(a, Wd), x)
    da, _ = coda.coda_gemm_res_sumsq_bwd(dY, Wd, want_dw=False)
    dpre = coda.coda_unfused_swiglu_bwd(da, pre)
    dX0, _ = coda.coda_gemm_res_sumsq_bwd(dpre, Wgu, want_dw=False)
    dX = coda.coda_unfused_add(dX0, dY)
    dWgu = coda.coda_gemm_wgrad(x, dpre)
    dWd = coda.coda_gemm_wgrad(a, dY)
    torch.cuda.synchronize()
    o_ref, _, _ = O.mlp_fwd(p["x"].f64(), p["Wgu"].f64(), p["Wd"].f64())
    g = O.mlp_bwd(p["x"].f64(), p["Wgu"].f64(), p["Wd"].f64(), p["dY"].f64())
    assert_close(f64(out), o_ref, "out")
    assert_close(f64(dpre), g["dpre"], "dpre")
    assert_close(f64(dX), g["dX"], "dX")
    assert_close(dWgu.cpu().numpy(), g["dWgu"], "dWgu")
    assert_close(dWd.cpu().numpy(), g["dWd"], "dWd")
