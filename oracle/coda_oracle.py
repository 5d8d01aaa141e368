"""Plain fp64 CPU oracle for the CODA GEMM-epilogue path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call
this module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark do.  It shares no code with the HIP kernels and imports nothing
from the package that holds them.

Every function computes the *canonical*, unfused form of an operation in
float64 numpy, with no blocking, fusion or reordering beyond what its
definition states.  Inputs are plain float64 arrays (the exact widening of
the bfloat16 inputs the GPU also consumes).  Sources:

* [N2]  "CODA GEMM-Epilogue Programming" (reading notes), section 2
        "Forward-Pass Reparameterizations": GEMM -> Residual -> RMSNorm -> GEMM,
        pairwise activations (SwiGLU, RoPE), cross-entropy loss.
* [N3]  same page, section 3 "The Backward Pass: Reverse Fusion" and
        "Eliminating the RMSNorm backward kernel".
* [F4]  "CODA: Rewriting Transformer Blocks as GEMM-Epilogue Programs",
        Figure 4 (two-level RMSNorm reduction) and Figure 5's caption
        (r = 1/sqrt(reduce(partials) + eps)).
* [F7]  same paper, Figure 7 (pairwise maps: RoPE 2->2, SwiGLU 2->1,
        SwiGLU backward 1->2).
* [L2]  same paper, Listing 2 (residual D = acc + C, partial statistic on the
        unscaled D, per-column RMSNorm weight applied to a side output).
* [RoF] RoFormer (Su et al.), cited by the paper for rotary embeddings:
        rotate each adjacent feature pair by pos * theta^(-2k/head_dim).
* [LN]  the paper's review page: the referee report (major comment 1) asks
        for LayerNorm gradients as an epilogue composition and the simulated
        rebuttal (point 1) promises the LayerNorm backward pass with its
        residual-gradient path.  LayerNorm itself is the textbook one (Ba et
        al.): n = ((u - mean) / sqrt(var + eps)) * gamma + beta with the
        biased row variance.

Readings where the pages leave a step open (each also listed in the design
notes): RMSNorm is r = (mean_j u_ij^2 + eps)^(-1/2) with gamma applied after
normalisation; SwiGLU pairs are adjacent columns (gate even, up odd) with
a = silu(gate) * up; RoPE rotates adjacent pairs inside each head of the
first ``n_rope`` columns; the LM-head loss is the mean over all rows with no
ignore index; a label outside [0, V) gives a NaN row loss.  LayerNorm uses
the biased variance with eps inside the root, like the RMSNorm reading.

Parity pins: every public function here is pinned by tests/test_oracle_pins.py
against closed forms, brute force, library special cases, algebraic identities
or finite differences.
"""

from __future__ import annotations

import numpy as np

F64 = np.float64


def _f(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


# --------------------------------------------------------------------------
# GEMM
# --------------------------------------------------------------------------


def gemm(a, b) -> np.ndarray:
    """C = A @ B in float64 (the GEMM mainloop's result before any epilogue)."""
    return _f(a) @ _f(b)


# --------------------------------------------------------------------------
# Forward: GEMM -> residual -> RMSNorm -> GEMM   [N2], [F4], [L2]
# --------------------------------------------------------------------------


def residual(x, w0, z) -> np.ndarray:
    """u = x W0 + z (the residual stream entering RMSNorm)."""
    return gemm(x, w0) + _f(z)


def row_sumsq(u) -> np.ndarray:
    """Per-row sum of squares sum_j u_ij^2 of the unscaled residual stream [L2]."""
    u = _f(u)
    return np.sum(u * u, axis=1)


def row_rms(sumsq, d: int, eps: float) -> np.ndarray:
    """r_i = 1 / sqrt(sumsq_i / d + eps)  [F4 / Figure 5 caption]."""
    return 1.0 / np.sqrt(_f(sumsq) / d + eps)


def res_sumsq(x, w0, z, gamma):
    """GEMM1 quantities: u = xW0 + z, h2 = u * gamma, and sum_j u_ij^2  [N2], [L2]."""
    u = residual(x, w0, z)
    return u, u * _f(gamma)[None, :], row_sumsq(u)


def rmsnorm(u, gamma, eps: float):
    """Canonical RMSNorm: n2 = (r * u) * gamma with r = (mean_j u^2 + eps)^(-1/2).

    Returns (n2, r)."""
    u = _f(u)
    r = 1.0 / np.sqrt(np.mean(u * u, axis=1) + eps)
    return (r[:, None] * u) * _f(gamma)[None, :], r


def norm_block_fwd(x, w0, z, gamma, w1, eps: float):
    """Canonical y = (r (xW0 + z) * gamma) W1  [N2].  Returns (y, u, r)."""
    u = residual(x, w0, z)
    n2, r = rmsnorm(u, gamma, eps)
    return gemm(n2, w1), u, r


def row_scale(r, t) -> np.ndarray:
    """y_ij = r_i t_ij (the delayed row scale of GEMM2's epilogue) [N2]."""
    return _f(r)[:, None] * _f(t)


# --------------------------------------------------------------------------
# Pairwise maps  [F7], [N2 "Pairwise activations"], [RoF]
# --------------------------------------------------------------------------


def rope_angles(pos, theta: float, head_dim: int, n_cols: int) -> np.ndarray:
    """ang[i, c//2] for each even column c < n_cols: pos_i * theta^(-2k/head_dim), k = (c mod head_dim)/2."""
    c = np.arange(0, n_cols, 2)
    k = (c % head_dim) // 2
    inv_freq = np.power(F64(theta), -2.0 * k / head_dim)
    return _f(pos)[:, None] * inv_freq[None, :]


def rope(t, pos, theta: float, head_dim: int, n_rope: int, inverse: bool = False) -> np.ndarray:
    """Rotate adjacent pairs (2k', 2k'+1) of the first n_rope columns; pass the rest through.

    (y_c, y_c+1) = (t_c cos - t_c+1 sin, t_c sin + t_c+1 cos); ``inverse`` uses -ang.
    """
    t = _f(t)
    y = t.copy()
    ang = rope_angles(pos, theta, head_dim, n_rope)
    if inverse:
        ang = -ang
    cs, sn = np.cos(ang), np.sin(ang)
    a = t[:, 0:n_rope:2]
    b = t[:, 1:n_rope:2]
    y[:, 0:n_rope:2] = a * cs - b * sn
    y[:, 1:n_rope:2] = a * sn + b * cs
    return y


def sigmoid(g) -> np.ndarray:
    g = _f(g)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-g))


def swiglu(pre) -> np.ndarray:
    """a_j = silu(g_j) * v_j with g = pre[:, 0::2] (gate), v = pre[:, 1::2] (up)  [F7]."""
    pre = _f(pre)
    g = pre[:, 0::2]
    v = pre[:, 1::2]
    return g * sigmoid(g) * v


# --------------------------------------------------------------------------
# LM head + cross-entropy  [N2 "Cross-entropy loss"]
# --------------------------------------------------------------------------


def logsumexp_rows(logits) -> np.ndarray:
    """lse_i = m_i + log sum_k exp(l_ik - m_i), m_i = max_k l_ik."""
    l = _f(logits)
    m = np.max(l, axis=1)
    return m + np.log(np.sum(np.exp(l - m[:, None]), axis=1))


def cross_entropy(logits, labels):
    """loss_i = -l_{i,y_i} + log sum_k exp(l_ik); returns (lse, loss_rows, mean)."""
    l = _f(logits)
    labels = np.asarray(labels)
    V = l.shape[1]
    lse = logsumexp_rows(l)
    ok = (labels >= 0) & (labels < V)
    tgt = np.full(l.shape[0], np.nan)
    rows = np.nonzero(ok)[0]
    tgt[rows] = l[rows, labels[rows]]
    loss = lse - tgt
    return lse, loss, float(np.mean(loss))


def lmhead_ce(h, w, labels):
    """Logits h W (fp64, never rounded) followed by cross_entropy."""
    return cross_entropy(gemm(h, w), labels)


# --------------------------------------------------------------------------
# Backward  [N3], [F7]
# --------------------------------------------------------------------------


def swiglu_bwd(da, pre) -> np.ndarray:
    """d(pre) from d(a): dg = da v s (1 + g (1 - s)), dv = da g s, s = sigmoid(g); interleaved like pre."""
    da = _f(da)
    pre = _f(pre)
    g = pre[:, 0::2]
    v = pre[:, 1::2]
    s = sigmoid(g)
    out = np.empty_like(pre)
    out[:, 0::2] = da * v * s * (1.0 + g * (1.0 - s))
    out[:, 1::2] = da * g * s
    return out


def rmsnorm_bwd(dn2, u, gamma, eps: float, dres=None):
    """Canonical RMSNorm backward of n2 = (r u) * gamma, given dn2 = dL/dn2.

    du = dres + r (dn2 * gamma) - r^3 u mean_j((dn2 * gamma) u)
    dgamma_j = sum_i dn2_ij (r_i u_ij)
    Also returns the row statistic s_i = (1/d) sum_j dn2_ij n2_ij  [N3].
    Returns (du, dgamma, s, r).
    """
    dn2 = _f(dn2)
    u = _f(u)
    gamma = _f(gamma)
    d = u.shape[1]
    r = 1.0 / np.sqrt(np.mean(u * u, axis=1) + eps)
    gn = dn2 * gamma[None, :]
    du = r[:, None] * gn - (r ** 3)[:, None] * u * np.mean(gn * u, axis=1)[:, None]
    if dres is not None:
        du = du + _f(dres)
    dgamma = np.sum(dn2 * (r[:, None] * u), axis=0)
    n2 = (r[:, None] * u) * gamma[None, :]
    s = np.sum(dn2 * n2, axis=1) / d
    return du, dgamma, s, r


def lmhead_ce_bwd(h, w, labels, scale: float):
    """Gradients of scale * sum_i loss_i w.r.t. h and W.

    D = (softmax(hW) - onehot(labels)) * scale; dh = D W^T; dW = h^T D.
    Returns (dh, dW, D)."""
    h = _f(h)
    w = _f(w)
    l = gemm(h, w)
    lse = logsumexp_rows(l)
    p = np.exp(l - lse[:, None])
    labels = np.asarray(labels)
    p[np.arange(l.shape[0]), labels] -= 1.0
    D = p * scale
    return gemm(D, w.T), gemm(h.T, D), D


# --------------------------------------------------------------------------
# Chains of the synthetic workloads (compositions of the above)
# --------------------------------------------------------------------------


def mlp_fwd(x, wgu, wd):
    """out = x + swiglu(x Wgu) Wd (SwiGLU MLP with its residual).  Returns (out, pre, a)."""
    pre = gemm(x, wgu)
    a = swiglu(pre)
    return gemm(a, wd) + _f(x), pre, a


def mlp_bwd(x, wgu, wd, dY):
    """Backward of mlp_fwd: returns dict(dpre, dX, dWgu, dWd)."""
    _, pre, a = mlp_fwd(x, wgu, wd)
    dY = _f(dY)
    da = gemm(dY, _f(wd).T)
    dpre = swiglu_bwd(da, pre)
    dX = gemm(dpre, _f(wgu).T) + dY
    return {"dpre": dpre, "dX": dX, "dWgu": gemm(_f(x).T, dpre), "dWd": gemm(a.T, dY), "pre": pre, "a": a}


def block_fwd(p):
    """Two stacked (residual, RMSNorm, SwiGLU MLP) layers behind a d x d projection.

    u1 = x W0 + z; pre_l = rmsnorm(u_l; gamma_l) Wgu_l; a_l = swiglu(pre_l);
    u2 = a1 Wd1 + u1; out = a2 Wd2 + u2.  Returns a dict of every intermediate.
    """
    eps = p["eps"]
    u1 = residual(p["x"], p["W0"], p["z"])
    n2_1, r1 = rmsnorm(u1, p["gamma1"], eps)
    pre1 = gemm(n2_1, p["Wgu1"])
    a1 = swiglu(pre1)
    u2 = gemm(a1, p["Wd1"]) + u1
    n2_2, r2 = rmsnorm(u2, p["gamma2"], eps)
    pre2 = gemm(n2_2, p["Wgu2"])
    a2 = swiglu(pre2)
    out = gemm(a2, p["Wd2"]) + u2
    return dict(u1=u1, r1=r1, n2_1=n2_1, pre1=pre1, a1=a1, u2=u2, r2=r2, n2_2=n2_2, pre2=pre2, a2=a2, out=out)


def block_bwd(p, f=None):
    """Canonical chain-rule backward of block_fwd from dOut; returns every gradient and the s statistics."""
    if f is None:
        f = block_fwd(p)
    eps = p["eps"]
    dOut = _f(p["dOut"])
    g = {}
    g["dWd2"] = gemm(f["a2"].T, dOut)
    da2 = gemm(dOut, _f(p["Wd2"]).T)
    g["dpre2"] = swiglu_bwd(da2, f["pre2"])
    g["dWgu2"] = gemm(f["n2_2"].T, g["dpre2"])
    dn2_2 = gemm(g["dpre2"], _f(p["Wgu2"]).T)
    g["du2"], g["dgamma2"], g["s2"], _ = rmsnorm_bwd(dn2_2, f["u2"], p["gamma2"], eps, dres=dOut)
    g["dWd1"] = gemm(f["a1"].T, g["du2"])
    da1 = gemm(g["du2"], _f(p["Wd1"]).T)
    g["dpre1"] = swiglu_bwd(da1, f["pre1"])
    g["dWgu1"] = gemm(f["n2_1"].T, g["dpre1"])
    dn2_1 = gemm(g["dpre1"], _f(p["Wgu1"]).T)
    g["du1"], g["dgamma1"], g["s1"], _ = rmsnorm_bwd(dn2_1, f["u1"], p["gamma1"], eps, dres=g["du2"])
    g["dx"] = gemm(g["du1"], _f(p["W0"]).T)
    g["dW0"] = gemm(_f(p["x"]).T, g["du1"])
    g["dz"] = g["du1"]
    return g


# --------------------------------------------------------------------------
# LayerNorm variant  [LN]
# --------------------------------------------------------------------------


def layernorm(u, gamma, beta, eps: float):
    """Canonical LayerNorm over each row: n = (r (u - mu)) * gamma + beta with
    mu = mean_j u, r = (mean_j (u - mu)^2 + eps)^(-1/2).  Returns (n, mu, r)."""
    u = _f(u)
    mu = np.mean(u, axis=1)
    cu = u - mu[:, None]
    r = 1.0 / np.sqrt(np.mean(cu * cu, axis=1) + eps)
    return (r[:, None] * cu) * _f(gamma)[None, :] + _f(beta)[None, :], mu, r


def ln_norm_block_fwd(x, w0, z, gamma, beta, w1, eps: float):
    """Canonical y = layernorm(x W0 + z) W1.  Returns (y, u, mu, r)."""
    u = residual(x, w0, z)
    n, mu, r = layernorm(u, gamma, beta, eps)
    return gemm(n, w1), u, mu, r


def layernorm_bwd(dn, u, gamma, eps: float, dres=None):
    """Canonical LayerNorm backward of n = xhat * gamma + beta, xhat = r (u - mu),
    given dn = dL/dn:

    gn = dn * gamma;  du = dres + r (gn - mean_j gn - xhat mean_j(gn xhat))
    dgamma_j = sum_i dn_ij xhat_ij;  dbeta_j = sum_i dn_ij
    Also returns the two row statistics a_i = mean_j gn_ij and
    s_i = mean_j gn_ij xhat_ij.  Returns (du, dgamma, dbeta, a, s).
    """
    dn = _f(dn)
    u = _f(u)
    gamma = _f(gamma)
    mu = np.mean(u, axis=1)
    centered = u - mu[:, None]
    r = 1.0 / np.sqrt(np.mean(centered * centered, axis=1) + eps)
    xhat = r[:, None] * centered
    gn = dn * gamma[None, :]
    a = np.mean(gn, axis=1)
    s = np.mean(gn * xhat, axis=1)
    du = r[:, None] * (gn - a[:, None] - xhat * s[:, None])
    if dres is not None:
        du = du + _f(dres)
    dgamma = np.sum(dn * xhat, axis=0)
    dbeta = np.sum(dn, axis=0)
    return du, dgamma, dbeta, a, s


def ln_block_fwd(p):
    """block_fwd with LayerNorm (gamma_l, beta_l) in place of RMSNorm:
    u1 = x W0 + z; pre_l = layernorm(u_l) Wgu_l; a_l = swiglu(pre_l);
    u2 = a1 Wd1 + u1; out = a2 Wd2 + u2.  Returns a dict of every intermediate."""
    eps = p["eps"]
    u1 = residual(p["x"], p["W0"], p["z"])
    n_1, mu1, r1 = layernorm(u1, p["gamma1"], p["beta1"], eps)
    pre1 = gemm(n_1, p["Wgu1"])
    a1 = swiglu(pre1)
    u2 = u1 + gemm(a1, p["Wd1"])
    n_2, mu2, r2 = layernorm(u2, p["gamma2"], p["beta2"], eps)
    pre2 = gemm(n_2, p["Wgu2"])
    a2 = swiglu(pre2)
    out = u2 + gemm(a2, p["Wd2"])
    return dict(u1=u1, mu1=mu1, r1=r1, n_1=n_1, pre1=pre1, a1=a1, u2=u2, mu2=mu2, r2=r2, n_2=n_2, pre2=pre2,
                a2=a2, out=out)


def ln_block_bwd(p, f=None):
    """Canonical chain-rule backward of ln_block_fwd from dOut; returns every
    gradient and each layer's row statistics a_l, s_l."""
    if f is None:
        f = ln_block_fwd(p)
    eps = p["eps"]
    dOut = _f(p["dOut"])
    g = {}
    g["dWd2"] = gemm(f["a2"].T, dOut)
    da2 = gemm(dOut, _f(p["Wd2"]).T)
    g["dpre2"] = swiglu_bwd(da2, f["pre2"])
    g["dWgu2"] = gemm(f["n_2"].T, g["dpre2"])
    dn_2 = gemm(g["dpre2"], _f(p["Wgu2"]).T)
    g["du2"], g["dgamma2"], g["dbeta2"], g["a2"], g["s2"] = layernorm_bwd(dn_2, f["u2"], p["gamma2"], eps,
                                                                          dres=dOut)
    g["dWd1"] = gemm(f["a1"].T, g["du2"])
    da1 = gemm(g["du2"], _f(p["Wd1"]).T)
    g["dpre1"] = swiglu_bwd(da1, f["pre1"])
    g["dWgu1"] = gemm(f["n_1"].T, g["dpre1"])
    dn_1 = gemm(g["dpre1"], _f(p["Wgu1"]).T)
    g["du1"], g["dgamma1"], g["dbeta1"], g["a1"], g["s1"] = layernorm_bwd(dn_1, f["u1"], p["gamma1"], eps,
                                                                          dres=g["du2"])
    g["dx"] = gemm(g["du1"], _f(p["W0"]).T)
    g["dW0"] = gemm(_f(p["x"]).T, g["du1"])
    g["dz"] = g["du1"]
    return g
