"""Parity at the full sizes of the five synthetic workloads, with the same
kernels and tile configuration the benchmark times.

The GPU computes every output in full; the fp64 oracle recomputes a seeded
sample of rows (row-independent outputs) and of columns (weight gradients and
dgamma, whose columns only need column slices of the inputs).  The LM head's
statistics (lse, row loss, mean loss) are recomputed by the oracle for all
8192 rows, row chunk by row chunk, and the RMSNorm backward of the 8B-like
block for all rows.  Every expected value comes from an oracle function.
Bounds: max|gpu - ref| <= 2e-2 * max|ref| per output; scalar loss relative
error <= 1e-3.
"""

import numpy as np
import pytest
import torch

from gpu_util import LOSS_RTOL, assert_close, dev, f64, say
from gemm_epilogue_transformer_mainloop_amd import synth as S
from oracle import coda_oracle as O

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


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


def sample(n, k=12, seed=7):
    """Edge rows/columns plus seeded random ones."""
    edge = [0, 1, 31, 32, 127, 128, 255, 256, n // 2, n - 2, n - 1]
    rng = np.random.default_rng(seed)
    rnd = rng.choice(n, size=k, replace=False).tolist()
    return np.array(sorted(set(i for i in edge + rnd if 0 <= i < n)))


def rows_of(t, rows):
    return f64(t[torch.as_tensor(rows, device=t.device)])


# ---------------------------------------------------------------------------
# config 2: GEMM -> residual -> RMSNorm -> GEMM (+ RoPE on the QKV projection)
# ---------------------------------------------------------------------------


def test_config2_fullsize():
    c = S.CONFIGS[2]
    M, d, K, N, NR = c["M"], c["d"], c["K"], c["N"], c["n_rope_cols"]
    say(f"case: config 2 full size M={M} d={d} K={K} N={N} N_qkv={NR}")
    p = S.norm_block_inputs(2, M, d, K, N, n_rope_cols=NR)
    coda = C()
    x, W0, z, g, W1, W1r = (dev(p[k]) for k in ("x", "W0", "z", "gamma", "W1", "W1r"))
    pos = dev(p["pos"])
    U, H2, part = coda.coda_gemm_res_sumsq(x, W0, z, g)
    r = coda.coda_row_rms(part, d, p["eps"])
    Y = coda.coda_gemm_rowscale(H2, W1, r)
    Yr = coda.coda_gemm_rope(H2, W1r, r, pos, S.ROPE_THETA, S.HEAD_DIM, 2560)
    torch.cuda.synchronize()
    rows = sample(M)
    xs, zs = p["x"].f64()[rows], p["z"].f64()[rows]
    u, h2, ss = O.res_sumsq(xs, p["W0"].f64(), zs, p["gamma"].f64())
    n2, rr = O.rmsnorm(u, p["gamma"].f64(), p["eps"])
    assert_close(rows_of(U, rows), u, "u")
    assert_close(rows_of(H2, rows), h2, "h2")
    assert_close(part[torch.as_tensor(rows, device="cuda")].double().sum(1).cpu().numpy(), ss, "sum of partials")
    assert_close(rows_of(r, rows), rr, "r")
    assert_close(rows_of(Y, rows), O.gemm(n2, p["W1"].f64()), "y")
    yr = O.rope(O.gemm(n2, p["W1r"].f64()), p["pos"][rows], S.ROPE_THETA, S.HEAD_DIM, 2560)
    assert_close(rows_of(Yr, rows), yr, "y (QKV + RoPE)")


# ---------------------------------------------------------------------------
# config 3: SwiGLU MLP forward + backward
# ---------------------------------------------------------------------------


def test_config3_fullsize():
    c = S.CONFIGS[3]
    M, d, F = c["M"], c["d"], c["F"]
    say(f"case: config 3 full size M={M} d={d} F={F}")
    p = S.mlp_inputs(3, M, d, F)
    coda = C()
    x, Wgu, Wd, dY = (dev(p[k]) for k in ("x", "Wgu", "Wd", "dY"))
    act, pre = coda.coda_gemm_swiglu(x, Wgu)
    out, _, _ = coda.coda_gemm_res_sumsq(act, Wd, Z=x, want_part=False)
    dpre, _ = coda.coda_gemm_swiglu_bwd(dY, Wd, pre, want_spart=False)
    dX, dWgu = coda.coda_gemm_res_sumsq_bwd(dpre, Wgu, X=x, dRes=dY)
    dWd = coda.coda_gemm_wgrad(act, dY)
    torch.cuda.synchronize()
    X64, Wgu64, Wd64, dY64 = (p[k].f64() for k in ("x", "Wgu", "Wd", "dY"))
    rows = sample(M)
    pre_r = O.gemm(X64[rows], Wgu64)
    a_r = O.swiglu(pre_r)
    assert_close(rows_of(pre, rows), pre_r, "pre")
    assert_close(rows_of(act, rows), a_r, "act")
    assert_close(rows_of(out, rows), O.gemm(a_r, Wd64) + X64[rows], "out")
    dpre_r = O.swiglu_bwd(O.gemm(dY64[rows], Wd64.T), pre_r)
    assert_close(rows_of(dpre, rows), dpre_r, "dpre")
    assert_close(rows_of(dX, rows), O.gemm(dpre_r, Wgu64.T) + dY64[rows], "dX")
    # weight gradients on sampled columns: every row of the column is needed
    js = sample(F, k=6, seed=8)
    cols = np.stack([2 * js, 2 * js + 1], axis=1).reshape(-1)
    pre_c = O.gemm(X64, Wgu64[:, cols])
    dpre_c = O.swiglu_bwd(O.gemm(dY64, Wd64[js].T), pre_c)
    assert_close(dWgu[:, torch.as_tensor(cols, device="cuda")].cpu().numpy(), O.gemm(X64.T, dpre_c), "dWgu columns")
    a_c = O.swiglu(pre_c)
    ns = sample(d, k=6, seed=9)
    assert_close(dWd[torch.as_tensor(js, device="cuda")][:, torch.as_tensor(ns, device="cuda")].cpu().numpy(),
                 O.gemm(a_c.T, dY64[:, ns]), "dWd entries")


# ---------------------------------------------------------------------------
# config 4: LM head + cross-entropy
# ---------------------------------------------------------------------------


@pytest.fixture(scope="module")
def c4_ref():
    """The oracle's cross-entropy over all 8192 rows of the LM-head workload
    (row chunks, fp64), and what the sampled dW columns need: for every row,
    the log-sum-exp of the logits outside the sampled columns."""
    c = S.CONFIGS[4]
    M, d, V = c["M"], c["d"], c["V"]
    p = S.lmhead_inputs(4, M, d, V)
    h64, W64 = p["h"].f64(), p["W"].f64()
    js = sample(V, k=10, seed=12)
    rest = np.setdiff1d(np.arange(V), js)
    lse = np.empty(M)
    loss = np.empty(M)
    lrest = np.empty(M)
    for m0 in range(0, M, 512):
        lg = O.gemm(h64[m0:m0 + 512], W64)
        lse[m0:m0 + 512], loss[m0:m0 + 512], _ = O.cross_entropy(lg, p["labels"][m0:m0 + 512])
        lrest[m0:m0 + 512] = O.logsumexp_rows(lg[:, rest])
        del lg
    say(f"  oracle: lse/loss over all {M} rows, mean loss {loss.mean():.6f}")
    return dict(p=p, h64=h64, W64=W64, lse=lse, loss=loss, mean=float(loss.mean()), js=js, lrest=lrest)


def dw_columns_ref(ref, M):
    """dW[:, js] of the mean loss from the oracle's lmhead_ce_bwd on a reduced
    head: the sampled columns plus one extra logit that carries, per row, the
    log-sum-exp of every other column (an extra input feature equal to it and
    a weight column selecting that feature).  The softmax of the sampled
    columns is then exactly the full softmax's, so the reduced head's dW
    columns are the full head's."""
    h64, W64, js, lrest, labels = ref["h64"], ref["W64"], ref["js"], ref["lrest"], ref["p"]["labels"]
    d = h64.shape[1]
    k = len(js)
    h_aug = np.concatenate([h64, lrest[:, None]], axis=1)
    W_aug = np.zeros((d + 1, k + 1))
    W_aug[:d, :k] = W64[:, js]
    W_aug[d, k] = 1.0
    pos = {int(j): q for q, j in enumerate(js)}
    lab_aug = np.array([pos.get(int(y), k) for y in labels], dtype=np.int64)
    _, dW_aug, _ = O.lmhead_ce_bwd(h_aug, W_aug, lab_aug, 1.0 / M)
    return dW_aug[:d, :k]


def check_c4(ref, lse, loss_row, loss_mean, dH, dW, tag=""):
    M = lse.shape[0]
    p, h64, W64 = ref["p"], ref["h64"], ref["W64"]
    assert_close(f64(lse), ref["lse"], "lse (all rows)" + tag)
    assert_close(f64(loss_row), ref["loss"], "loss_row (all rows)" + tag)
    got = float(loss_mean.item())
    rel = abs(got - ref["mean"]) / abs(ref["mean"])
    say(f"  mean loss{tag}: gpu {got:.6f} oracle {ref['mean']:.6f} rel err {rel:.3e}")
    assert rel <= LOSS_RTOL
    rows = sample(M)
    dh_r, _, _ = O.lmhead_ce_bwd(h64[rows], W64, p["labels"][rows], 1.0 / M)
    assert_close(rows_of(dH, rows), dh_r, "dh" + tag)
    js = ref["js"]
    assert_close(dW[:, torch.as_tensor(js, device="cuda")].double().cpu().numpy(), dw_columns_ref(ref, M),
                 "dW sampled columns (all rows)" + tag)


def test_config4_fullsize(c4_ref):
    c = S.CONFIGS[4]
    M, d, V = c["M"], c["d"], c["V"]
    say(f"case: config 4 full size M={M} d={d} V={V}")
    p = c4_ref["p"]
    coda = C()
    H, W, lab = dev(p["h"]), dev(p["W"]), dev(p["labels"])
    lse, loss_row, loss_mean = coda.coda_lmhead_ce(H, W, lab)
    dH, dW = coda.coda_lmhead_ce_bwd(H, W, lab, lse, 1.0 / M)
    torch.cuda.synchronize()
    check_c4(c4_ref, lse, loss_row, loss_mean, dH, dW)


def test_config4_fullsize_stored_logits(c4_ref):
    """The stored-logits forward and backward at the full LM-head shape."""
    c = S.CONFIGS[4]
    M, d, V = c["M"], c["d"], c["V"]
    say(f"case: config 4 full size, stored logits, M={M} d={d} V={V}")
    p = c4_ref["p"]
    coda = C()
    H, W, lab = dev(p["h"]), dev(p["W"]), dev(p["labels"])
    lse, loss_row, loss_mean, logits = coda.coda_lmhead_ce_logits(H, W, lab)
    rows = sample(M, seed=8)
    h64, W64 = c4_ref["h64"], c4_ref["W64"]
    l_rows = rows_of(logits, rows)
    dH, dW = coda.coda_lmhead_ce_bwd_logits(H, W, lab, lse, 1.0 / M, logits)
    torch.cuda.synchronize()
    assert_close(l_rows, O.gemm(h64[rows], W64), "logits")
    _, _, D_r = O.lmhead_ce_bwd(h64[rows], W64, p["labels"][rows], 1.0 / M)
    assert_close(rows_of(logits, rows), D_r, "dlogits")
    check_c4(c4_ref, lse, loss_row, loss_mean, dH, dW, " [stored logits]")


def test_config4_fullsize_vchunk(c4_ref):
    """The vocabulary-chunked backward (8192-column chunks of dlogits, which
    stay in the Infinity Cache) at the full LM-head shape."""
    c = S.CONFIGS[4]
    M, d, V = c["M"], c["d"], c["V"]
    say(f"case: config 4 full size, vocabulary-chunked backward, M={M} d={d} V={V}")
    p = c4_ref["p"]
    coda = C()
    H, W, lab = dev(p["h"]), dev(p["W"]), dev(p["labels"])
    lse, loss_row, loss_mean = coda.coda_lmhead_ce(H, W, lab)
    dH, dW = coda.coda_lmhead_ce_bwd_vchunk(H, W, lab, lse, 1.0 / M, vchunk=8192)
    torch.cuda.synchronize()
    check_c4(c4_ref, lse, loss_row, loss_mean, dH, dW, " [vocabulary chunks]")


def test_config4_full_vocab_wgrad_small_m():
    """The full 2048 x 128256 weight gradient, exactly, at M = 64 rows."""
    M, d, V = 64, 2048, 128256
    say(f"case: LM-head backward full vocabulary M={M}")
    p = S.lmhead_inputs(4, 8192, d, V)
    coda = C()
    h = S.Bf16(p["h"].bits[:M])
    labels = p["labels"][:M]
    H, W, lab = dev(h), dev(p["W"]), dev(labels)
    lse, _, _ = coda.coda_lmhead_ce(H, W, lab)
    dH, dW = coda.coda_lmhead_ce_bwd(H, W, lab, lse, 1.0 / M)
    torch.cuda.synchronize()
    dh_r, dW_r, _ = O.lmhead_ce_bwd(h.f64(), p["W"].f64(), labels, 1.0 / M)
    assert_close(f64(dH), dh_r, "dh")
    assert_close(dW.cpu().numpy(), dW_r, "dW")


# ---------------------------------------------------------------------------
# config 5: the fused backward calls at the 8B-like block shape
# ---------------------------------------------------------------------------


def test_config5_fullsize_backward_calls():
    c = S.CONFIGS[5]
    M, d, F = c["M"], c["d"], c["F"]
    say(f"case: config 5 full size fused backward calls M={M} d={d} F={F}")
    b = S.block_inputs(5, M, d, F)
    u = S.normal_bf16(5050, (M, d))
    pre = S.normal_bf16(5051, (M, 2 * F))
    coda = C()
    dOut, Wd2, Wgu2, g2 = dev(b["dOut"]), dev(b["Wd2"]), dev(b["Wgu2"]), dev(b["gamma2"])
    dpre, spart = coda.coda_gemm_swiglu_bwd(dOut, Wd2, dev(pre))
    s = coda.coda_row_rms_bwd(spart, d)
    torch.cuda.synchronize()
    # swiglu_bwd + s on sampled rows
    rows = sample(M)
    dOut64, Wd64, Wgu64, g64, u64 = b["dOut"].f64(), b["Wd2"].f64(), b["Wgu2"].f64(), b["gamma2"].f64(), u.f64()
    eps = b["eps"]
    pre64 = pre.f64()
    dpre_r = O.swiglu_bwd(O.gemm(dOut64[rows], Wd64.T), pre64[rows])
    assert_close(rows_of(dpre, rows), dpre_r, "dpre")
    # s is the RMSNorm statistic of the layer whose output pre is (y = pre)
    assert_close(rows_of(s, rows), np.sum(dpre_r * pre64[rows], axis=1) / d, "s")
    del spart, s
    # RMSNorm backward of n2 = rmsnorm(u) at K = 28672, against the oracle's
    # canonical backward on every row.  Its own upstream gradient is a seeded
    # dpre-shaped dY: dn2 = dY W_gu^T; r and s are the oracle's for this u and dn2.
    dY = S.normal_bf16(5053, (M, 2 * F))
    dY64 = dY.f64()
    n2_r, r64 = O.rmsnorm(u64, g64, eps)
    dn2 = O.gemm(dY64, Wgu64.T)
    du_r, dg_r, s64, _ = O.rmsnorm_bwd(dn2, u64, g64, eps, dres=dOut64)
    say("  oracle: canonical RMSNorm backward over all rows")
    r32 = dev(r64.astype(np.float32))
    s32 = dev(s64.astype(np.float32))
    dU, N2, gpart = coda.coda_gemm_rowscale_bwd(dev(dY), Wgu2, dev(u), g2, r32, s32, dRes=dOut)
    dgamma = coda.coda_col_reduce(gpart)
    torch.cuda.synchronize()
    assert_close(f64(dU), du_r, "du (all rows)")
    assert_close(f64(N2), n2_r, "n2 (all rows)")
    assert_close(dgamma.double().cpu().numpy(), dg_r, "dgamma")
    del dn2, du_r
    # wgrad dWgu = n2^T dY on sampled entries (the oracle's n2)
    dWgu = coda.coda_gemm_wgrad(N2, dev(dY))
    torch.cuda.synchronize()
    js = sample(d, k=6, seed=10)
    ns = sample(2 * F, k=6, seed=11)
    ref = O.gemm(n2_r[:, js].T, dY64[:, ns])
    got = dWgu[torch.as_tensor(js, device="cuda")][:, torch.as_tensor(ns, device="cuda")].cpu().numpy()
    assert_close(got, ref, "dWgu entries")
