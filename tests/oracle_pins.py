"""Pins of the fp64 oracle against facts fixed outside it.

Each ``check_*`` takes the oracle module ``O`` and raises AssertionError when
``O`` disagrees with a closed form, a brute-force evaluation, a library
special case, an algebraic identity stated on the pages, or a central finite
difference.  ``test_oracle_pins`` runs them on the real oracle and
``test_oracle_mutants`` runs them on copies with planted mistakes, to show
that each plausible slip (dropped term, wrong sign or index, transposed
operand) is caught by at least one pin.

Sources: "CODA GEMM-Epilogue Programming" (reading notes) sections 2 and 3;
"CODA: Rewriting Transformer Blocks as GEMM-Epilogue Programs", Figures 4,
5 and 7, and its review page (referee report, major comment 1; simulated
rebuttal, point 1: the LayerNorm backward as an epilogue composition);
RoFormer for the rotary map; Ba et al. for LayerNorm.
"""

from __future__ import annotations

import math

import numpy as np

RNG = np.random.default_rng(12345)


def _rand(*shape, scale=1.0, seed=None):
    rng = np.random.default_rng(seed) if seed is not None else RNG
    return rng.standard_normal(shape) * scale


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    ref = max(np.max(np.abs(b)) if b.size else 0.0, 1e-300)
    assert err <= tol * max(ref, 1.0), f"{what}: max err {err:.3e} (ref {ref:.3e}, tol {tol})"


# ----------------------------------------------------------------------------
# GEMM
# ----------------------------------------------------------------------------


def check_gemm_bruteforce(O):
    """A triple loop with exactly rounded sums (math.fsum) on a small shape."""
    a = _rand(5, 7, seed=1)
    b = _rand(7, 3, seed=2)
    c = O.gemm(a, b)
    for i in range(5):
        for j in range(3):
            ref = math.fsum(a[i, k] * b[k, j] for k in range(7))
            assert abs(c[i, j] - ref) <= 1e-13, ("gemm", i, j)


def check_gemm_integer_exact(O):
    rng = np.random.default_rng(3)
    a = rng.integers(-4, 5, size=(6, 9))
    b = rng.integers(-4, 5, size=(9, 4))
    c = O.gemm(a, b)
    for i in range(6):
        for j in range(4):
            assert c[i, j] == sum(int(a[i, k]) * int(b[k, j]) for k in range(9))


# ----------------------------------------------------------------------------
# residual + sum of squares + rms
# ----------------------------------------------------------------------------


def check_res_sumsq_integer(O):
    """Integer operands: u, h2 and sum u^2 are exact; compare with Python ints."""
    rng = np.random.default_rng(4)
    x = rng.integers(-3, 4, size=(4, 6))
    w0 = rng.integers(-3, 4, size=(6, 5))
    z = rng.integers(-3, 4, size=(4, 5))
    g = rng.integers(-2, 3, size=(5,))
    u, h2, ss = O.res_sumsq(x, w0, z, g)
    for i in range(4):
        row = [sum(int(x[i, k]) * int(w0[k, j]) for k in range(6)) + int(z[i, j]) for j in range(5)]
        assert list(u[i]) == row
        assert list(h2[i]) == [row[j] * int(g[j]) for j in range(5)]
        assert ss[i] == sum(v * v for v in row)


def check_res_identity_weight(O):
    """W0 = I and z = 0 give u = x."""
    x = _rand(3, 8, seed=5)
    u, h2, ss = O.res_sumsq(x, np.eye(8), np.zeros((3, 8)), np.ones(8))
    _close(u, x, 0, "u=x")
    _close(h2, x, 0, "h2=x")


def check_row_rms_closed_form(O):
    """Constant rows u_ij = c give r = 1/sqrt(c^2 + eps)."""
    d, eps = 16, 1e-6
    cs = np.array([0.5, 1.0, 3.0, 0.0])
    u = np.repeat(cs[:, None], d, axis=1)
    r = O.row_rms(O.row_sumsq(u), d, eps)
    for i, c in enumerate(cs):
        assert abs(r[i] - 1.0 / math.sqrt(c * c + eps)) <= 1e-12 * (1.0 / math.sqrt(c * c + eps))
    # gamma = 1: the normalised rows have mean square sumsq/d / (sumsq/d + eps)
    u = _rand(5, 32, seed=6)
    n2, r2 = O.rmsnorm(u, np.ones(32), eps)
    ms = np.mean(u * u, axis=1)
    _close(np.mean(n2 * n2, axis=1), ms / (ms + eps), 1e-13, "rms of normalised rows")


def check_rmsnorm_bruteforce(O):
    """RMSNorm with Python loops: n2_ij = gamma_j u_ij / sqrt(fsum(u^2)/d + eps)."""
    u = _rand(3, 10, seed=7)
    g = 1.0 + 0.1 * _rand(10, seed=8)
    eps = 1e-6
    n2, r = O.rmsnorm(u, g, eps)
    for i in range(3):
        ri = 1.0 / math.sqrt(math.fsum(v * v for v in u[i]) / 10 + eps)
        assert abs(r[i] - ri) <= 1e-14 * ri
        for j in range(10):
            assert abs(n2[i, j] - g[j] * u[i, j] * ri) <= 1e-13


def check_commutation_identity(O):
    """r((xW0+z)*gamma)W1 == (r(xW0+z)*gamma)W1, the delayed row scale (reading notes sec. 2)."""
    M, K, d, N, eps = 7, 12, 16, 9, 1e-6
    x, w0, z = _rand(M, K, seed=9), _rand(K, d, seed=10) / 4, _rand(M, d, seed=11)
    g, w1 = 1 + 0.1 * _rand(d, seed=12), _rand(d, N, seed=13) / 4
    y, u, r = O.norm_block_fwd(x, w0, z, g, w1, eps)
    u2, h2, ss = O.res_sumsq(x, w0, z, g)
    r2 = O.row_rms(ss, d, eps)
    delayed = O.row_scale(r2, O.gemm(h2, w1))
    _close(delayed, y, 1e-12, "commutation identity")
    _close(r2, r, 1e-13, "r two ways")
    _close(u2, u, 0, "u two ways")


def check_unit_scale_is_plain_gemm(O):
    """Rows with mean(u^2) + eps = 1 have r = 1, so y is the plain GEMM (u*gamma)W1."""
    d, N, eps = 8, 5, 1e-6
    z = _rand(4, d, seed=14)
    z = z / np.sqrt(np.mean(z * z, axis=1, keepdims=True)) * math.sqrt(1 - eps)
    g, w1 = 1 + 0.1 * _rand(d, seed=15), _rand(d, N, seed=16)
    y, u, r = O.norm_block_fwd(np.zeros((4, 3)), np.zeros((3, d)), z, g, w1, eps)
    _close(r, np.ones(4), 1e-14, "r=1")
    ref = np.array([[math.fsum(z[i, j] * g[j] * w1[j, n] for j in range(d)) for n in range(N)] for i in range(4)])
    _close(y, ref, 1e-13, "plain gemm")


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------


def _rope_complex(t, pos, theta, hd, n_rope):
    """Independent formulation: pairs as complex numbers times exp(i * pos * theta^(-2k/hd))."""
    y = np.array(t, dtype=np.float64, copy=True)
    for i in range(t.shape[0]):
        for c in range(0, n_rope, 2):
            k = (c % hd) // 2
            ang = float(pos[i]) * math.pow(theta, -2.0 * k / hd)
            w = complex(t[i, c], t[i, c + 1]) * complex(math.cos(ang), math.sin(ang))
            y[i, c], y[i, c + 1] = w.real, w.imag
    return y


def check_rope_complex(O):
    t = _rand(5, 24, seed=17)
    pos = np.array([0, 1, 7, 100, 2047])
    y = O.rope(t, pos, 500000.0, 8, 16)
    _close(y, _rope_complex(t, pos, 500000.0, 8, 16), 1e-12, "rope vs complex rotation")
    _close(y[:, 16:], t[:, 16:], 0, "pass-through columns")


def check_rope_special_cases(O):
    t = _rand(3, 16, seed=18)
    _close(O.rope(t, np.zeros(3), 10000.0, 16, 16), t, 0, "pos=0 is identity")
    # (1, 0) -> (cos a, sin a) for the first pair of a head, a = pos * theta^0
    e = np.zeros((1, 16))
    e[0, 0] = 1.0
    y = O.rope(e, np.array([3]), 10000.0, 16, 16)
    assert abs(y[0, 0] - math.cos(3.0)) < 1e-15 and abs(y[0, 1] - math.sin(3.0)) < 1e-15
    # second pair of a head rotates by pos * theta^(-2/hd)
    e = np.zeros((1, 16))
    e[0, 2] = 1.0
    a = 3.0 * 10000.0 ** (-2.0 / 16)
    y = O.rope(e, np.array([3]), 10000.0, 16, 16)
    assert abs(y[0, 2] - math.cos(a)) < 1e-15 and abs(y[0, 3] - math.sin(a)) < 1e-15
    # pair norms are preserved
    y = O.rope(t, np.array([5, 9, 1000]), 500000.0, 8, 16)
    _close(y[:, 0:16:2] ** 2 + y[:, 1:16:2] ** 2, t[:, 0:16:2] ** 2 + t[:, 1:16:2] ** 2, 1e-13, "pair norm")
    # the inverse rotation undoes the rotation
    back = O.rope(y, np.array([5, 9, 1000]), 500000.0, 8, 16, inverse=True)
    _close(back, t, 1e-13, "inverse o rope")


def check_rope_relative_position(O):
    """<rope(q, p1), rope(k, p2)> depends only on p1 - p2 (RoFormer)."""
    q = _rand(1, 16, seed=19)
    k = _rand(1, 16, seed=20)
    th, hd = 10000.0, 16
    d1 = np.sum(O.rope(q, [10], th, hd, 16) * O.rope(k, [3], th, hd, 16))
    d2 = np.sum(O.rope(q, [110], th, hd, 16) * O.rope(k, [103], th, hd, 16))
    assert abs(d1 - d2) < 1e-12


# ----------------------------------------------------------------------------
# SwiGLU
# ----------------------------------------------------------------------------


def check_swiglu_closed_forms(O):
    from scipy.special import expit

    pre = np.array([[0.0, 3.0, 1.0, 2.0, -1.0, 5.0, 40.0, 0.5]])
    a = O.swiglu(pre)
    s1 = 1.0 / (1.0 + math.exp(-1.0))
    assert a[0, 0] == 0.0
    assert abs(a[0, 1] - 1.0 * s1 * 2.0) < 1e-15
    assert abs(a[0, 2] - (-1.0) * (1.0 - s1) * 5.0) < 1e-15
    assert abs(a[0, 3] - 40.0 * 0.5) < 1e-12  # silu(g) ~ g for large g
    p = _rand(4, 12, seed=21)
    g, v = p[:, 0::2], p[:, 1::2]
    _close(a=O.swiglu(p), b=g * expit(g) * v, tol=1e-15, what="swiglu vs scipy expit")
    # silu via tanh: g * (1 + tanh(g/2)) / 2
    _close(O.swiglu(p), g * (1.0 + np.tanh(g / 2.0)) / 2.0 * v, 1e-14, "swiglu vs tanh form")


def _fd_grad(f, x, h=1e-6):
    """Central finite differences of scalar f at every entry of x."""
    x = np.array(x, dtype=np.float64, copy=True)
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        x[idx] = old + h
        fp = f(x)
        x[idx] = old - h
        fm = f(x)
        x[idx] = old
        g[idx] = (fp - fm) / (2 * h)
    return g


def check_swiglu_bwd_fd(O):
    pre = _rand(3, 10, seed=22)
    da = _rand(3, 5, seed=23)
    ana = O.swiglu_bwd(da, pre)
    num = _fd_grad(lambda p: float(np.sum(da * O.swiglu(p))), pre)
    _close(ana, num, 1e-7, "swiglu_bwd vs finite differences")


# ----------------------------------------------------------------------------
# Cross-entropy
# ----------------------------------------------------------------------------


def check_ce_bruteforce(O):
    from scipy.special import logsumexp

    l = _rand(4, 13, seed=24) * 3
    labels = np.array([0, 12, 5, 7])
    lse, loss, mean = O.cross_entropy(l, labels)
    for i in range(4):
        ref = math.log(math.fsum(math.exp(v) for v in l[i]))
        assert abs(lse[i] - ref) < 1e-13
        assert abs(loss[i] - (ref - l[i, labels[i]])) < 1e-13
    assert abs(mean - math.fsum(loss) / 4) < 1e-14
    _close(lse, logsumexp(l, axis=1), 1e-14, "lse vs scipy")


def check_ce_tile_merge(O):
    """Two-level (per-tile max / sum-exp, then merge) equals the direct lse for any split."""
    l = _rand(3, 50, seed=25) * 10
    lse, _, _ = O.cross_entropy(l, np.zeros(3, dtype=int))
    for split in ([0, 50], [0, 7, 20, 50], [0, 1, 2, 49, 50]):
        ms, ss = [], []
        for a, b in zip(split[:-1], split[1:]):
            m = l[:, a:b].max(axis=1)
            ms.append(m)
            ss.append(np.sum(np.exp(l[:, a:b] - m[:, None]), axis=1))
        ms, ss = np.array(ms), np.array(ss)
        L = ms.max(axis=0)
        merged = L + np.log(np.sum(ss * np.exp(ms - L[None, :]), axis=0))
        _close(merged, lse, 1e-14, f"tile merge {split}")


def check_ce_zero_hidden(O):
    """h = 0: every logit is 0, loss = ln V; label outside [0, V) gives NaN."""
    V = 37
    lse, loss, mean = O.lmhead_ce(np.zeros((3, 4)), _rand(4, V, seed=26), np.array([0, 36, 5]))
    _close(loss, np.full(3, math.log(V)), 1e-15, "loss = ln V")
    _, loss, _ = O.lmhead_ce(np.zeros((2, 4)), _rand(4, V, seed=27), np.array([V, -1]))
    assert np.all(np.isnan(loss))


def check_ce_bwd_fd(O):
    h = _rand(3, 4, seed=28)
    w = _rand(4, 6, seed=29)
    y = np.array([1, 5, 0])
    c = 1.0 / 3
    dh, dW, D = O.lmhead_ce_bwd(h, w, y, c)
    fh = lambda hh: c * float(np.sum(O.lmhead_ce(hh, w, y)[1]))
    fw = lambda ww: c * float(np.sum(O.lmhead_ce(h, ww, y)[1]))
    _close(dh, _fd_grad(fh, h), 1e-7, "dh vs fd")
    _close(dW, _fd_grad(fw, w), 1e-7, "dW vs fd")


def check_ce_bwd_zero_hidden(O):
    """h = 0: dW = h^T D = 0 and dh_i = c (mean_k W[:, k] - W[:, y_i])."""
    V = 9
    w = _rand(4, V, seed=30)
    y = np.array([2, 8])
    c = 0.5
    dh, dW, D = O.lmhead_ce_bwd(np.zeros((2, 4)), w, y, c)
    _close(dW, np.zeros_like(dW), 0, "dW = 0")
    ref = np.stack([c * (w.mean(axis=1) - w[:, y[i]]) for i in range(2)])
    _close(dh, ref, 1e-14, "dh closed form")
    _close(D.sum(axis=1), np.zeros(2), 1e-15, "dlogits rows sum to 0")


# ----------------------------------------------------------------------------
# RMSNorm backward and the s statistic
# ----------------------------------------------------------------------------


def check_rmsnorm_bwd_fd(O):
    M, d, eps = 3, 6, 1e-3
    u = _rand(M, d, seed=31)
    g = 1 + 0.1 * _rand(d, seed=32)
    dn2 = _rand(M, d, seed=33)
    dres = _rand(M, d, seed=34)
    du, dg, s, r = O.rmsnorm_bwd(dn2, u, g, eps, dres=dres)
    fu = lambda uu: float(np.sum(dn2 * O.rmsnorm(uu, g, eps)[0]) + np.sum(dres * uu))
    fg = lambda gg: float(np.sum(dn2 * O.rmsnorm(u, gg, eps)[0]))
    _close(du, _fd_grad(fu, u), 1e-7, "du vs fd")
    _close(dg, _fd_grad(fg, g), 1e-7, "dgamma vs fd")


def check_s_identity_and_delayed_form(O):
    """s = (1/d) sumcols(dn2 * n2) = (1/d) sumcols(dY * y) with dn2 = dY W1^T, y = n2 W1 (notes sec. 3);
    the delayed du = dres + r (G * gamma) - r^2 s u equals the canonical backward."""
    M, d, N, eps = 4, 8, 5, 1e-6
    u = _rand(M, d, seed=35)
    g = 1 + 0.1 * _rand(d, seed=36)
    w1 = _rand(d, N, seed=37)
    dY = _rand(M, N, seed=38)
    dres = _rand(M, d, seed=39)
    n2, r = O.rmsnorm(u, g, eps)
    y = O.gemm(n2, w1)
    G = O.gemm(dY, w1.T)
    du, dg, s, r2 = O.rmsnorm_bwd(G, u, g, eps, dres=dres)
    _close(s, np.sum(dY * y, axis=1) / d, 1e-12, "s identity")
    delayed = dres + r[:, None] * (G * g[None, :]) - (r ** 2 * s)[:, None] * u
    _close(delayed, du, 1e-12, "delayed RMSNorm backward")
    gp = np.sum(r[:, None] * G * u, axis=0)
    _close(gp, dg, 1e-12, "dgamma from r G u")


# ----------------------------------------------------------------------------
# Chains
# ----------------------------------------------------------------------------


def check_mlp_bwd_fd(O):
    M, d, F = 3, 4, 3
    x = _rand(M, d, seed=40)
    wgu = _rand(d, 2 * F, seed=41) / 2
    wd = _rand(F, d, seed=42) / 2
    dY = _rand(M, d, seed=43)
    g = O.mlp_bwd(x, wgu, wd, dY)
    L = lambda xx, a, b: float(np.sum(dY * O.mlp_fwd(xx, a, b)[0]))
    _close(g["dX"], _fd_grad(lambda v: L(v, wgu, wd), x), 1e-7, "mlp dX")
    _close(g["dWgu"], _fd_grad(lambda v: L(x, v, wd), wgu), 1e-7, "mlp dWgu")
    _close(g["dWd"], _fd_grad(lambda v: L(x, wgu, v), wd), 1e-7, "mlp dWd")


def tiny_block(seed=44, M=3, d=4, F=3):
    rng = np.random.default_rng(seed)
    n = lambda *s: rng.standard_normal(s)
    return dict(x=n(M, d), z=n(M, d), W0=n(d, d) / 2, gamma1=1 + 0.1 * n(d), Wgu1=n(d, 2 * F) / 2,
                Wd1=n(F, d) / 2, gamma2=1 + 0.1 * n(d), Wgu2=n(d, 2 * F) / 2, Wd2=n(F, d) / 2,
                dOut=n(M, d), eps=1e-3)


def check_block_bwd_fd(O):
    p = tiny_block()
    g = O.block_bwd(p)

    def L(name):
        def f(v):
            q = dict(p)
            q[name] = v
            return float(np.sum(p["dOut"] * O.block_fwd(q)["out"]))
        return f

    for name, gname in [("x", "dx"), ("z", "dz"), ("W0", "dW0"), ("gamma1", "dgamma1"), ("Wgu1", "dWgu1"),
                        ("Wd1", "dWd1"), ("gamma2", "dgamma2"), ("Wgu2", "dWgu2"), ("Wd2", "dWd2")]:
        _close(g[gname], _fd_grad(L(name), p[name]), 2e-7, f"block {gname}")


def check_block_s_statistics(O):
    """s_l = (1/d) sumcols(dpre_l * pre_l) for each layer (notes sec. 3)."""
    p = tiny_block(seed=45)
    f = O.block_fwd(p)
    g = O.block_bwd(p, f)
    d = p["x"].shape[1]
    _close(g["s2"], np.sum(g["dpre2"] * f["pre2"], axis=1) / d, 1e-12, "s2")
    _close(g["s1"], np.sum(g["dpre1"] * f["pre1"], axis=1) / d, 1e-12, "s1")


# ----------------------------------------------------------------------------
# LayerNorm variant (the paper's review page: LayerNorm gradients as an
# epilogue composition)
# ----------------------------------------------------------------------------


def check_layernorm_torch(O):
    """Forward against torch's float64 layer_norm, backward against its autograd."""
    import torch

    M, d, eps = 4, 7, 1e-3
    u = _rand(M, d, seed=50) * 2 + 0.7
    g = 1 + 0.1 * _rand(d, seed=51)
    b = 0.2 * _rand(d, seed=52)
    dn = _rand(M, d, seed=53)
    dres = _rand(M, d, seed=54)
    ut = torch.tensor(u, requires_grad=True)
    gt = torch.tensor(g, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True)
    nt = torch.nn.functional.layer_norm(ut, (d,), gt, bt, eps)
    n, mu, r = O.layernorm(u, g, b, eps)
    _close(n, nt.detach().numpy(), 1e-13, "layernorm vs torch")
    (nt * torch.tensor(dn)).sum().backward()
    du, dg, db, a, s = O.layernorm_bwd(dn, u, g, eps, dres=dres)
    _close(du, ut.grad.numpy() + dres, 1e-12, "layernorm du vs torch autograd")
    _close(dg, gt.grad.numpy(), 1e-12, "layernorm dgamma vs torch autograd")
    _close(db, bt.grad.numpy(), 1e-12, "layernorm dbeta vs torch autograd")


def check_layernorm_bruteforce(O):
    """mean, variance, r and n of each row with exactly rounded sums."""
    M, d, eps = 3, 6, 1e-2
    u = _rand(M, d, seed=55) + 1.5
    g = 1 + 0.1 * _rand(d, seed=56)
    b = 0.3 * _rand(d, seed=57)
    n, mu, r = O.layernorm(u, g, b, eps)
    for i in range(M):
        m = math.fsum(u[i]) / d
        v = math.fsum((x - m) ** 2 for x in u[i]) / d
        ri = 1.0 / math.sqrt(v + eps)
        assert abs(mu[i] - m) < 1e-14 and abs(r[i] - ri) < 1e-13, ("layernorm stats", i)
        for j in range(d):
            assert abs(n[i, j] - ((u[i, j] - m) * ri * g[j] + b[j])) < 1e-13, ("layernorm", i, j)


def check_layernorm_special_cases(O):
    """Zero-mean rows with beta = 0 give RMSNorm; constant rows give beta;
    a per-row shift changes nothing; the input gradient sums to 0 over a row
    (apart from the residual path)."""
    M, d, eps = 4, 8, 1e-6
    u = _rand(M, d, seed=58)
    u0 = u - u.mean(axis=1, keepdims=True)
    g = 1 + 0.1 * _rand(d, seed=59)
    b = 0.5 * _rand(d, seed=60)
    _close(O.layernorm(u0, g, np.zeros(d), eps)[0], O.rmsnorm(u0, g, eps)[0], 1e-13, "zero-mean rows = RMSNorm")
    const = np.repeat(np.array([[3.0], [-2.0], [0.0], [7.5]]), d, axis=1)
    _close(O.layernorm(const, g, b, eps)[0], np.broadcast_to(b, (M, d)), 1e-15, "constant rows -> beta")
    shift = _rand(M, 1, seed=61) * 5
    _close(O.layernorm(u + shift, g, b, eps)[0], O.layernorm(u, g, b, eps)[0], 1e-12, "row shift invariance")
    du, _, _, _, _ = O.layernorm_bwd(_rand(M, d, seed=62), u, g, eps)
    _close(du.sum(axis=1), np.zeros(M), 1e-12, "du rows sum to 0")


def check_ln_mean_corrected_commutation(O):
    """layernorm(u) W1 = r (h3 - mu (gamma^T W1)) + beta^T W1 with h3 = (u * gamma) W1:
    the row scale and the mean correction both move past the projection."""
    M, K, d, N, eps = 5, 6, 8, 7, 1e-6
    x = _rand(M, K, seed=63)
    w0 = _rand(K, d, seed=64)
    z = _rand(M, d, seed=65) + 0.8
    g = 1 + 0.1 * _rand(d, seed=66)
    b = 0.3 * _rand(d, seed=67)
    w1 = _rand(d, N, seed=68)
    y, u, mu, r = O.ln_norm_block_fwd(x, w0, z, g, b, w1, eps)
    h3 = O.gemm(u * g[None, :], w1)
    cvec = O.gemm(g[None, :], w1)[0]
    bvec = O.gemm(b[None, :], w1)[0]
    _close(r[:, None] * (h3 - mu[:, None] * cvec[None, :]) + bvec[None, :], y, 1e-12, "mean-corrected commutation")


def check_layernorm_bwd_fd(O):
    M, d, eps = 3, 6, 1e-3
    u = _rand(M, d, seed=69) + 0.4
    g = 1 + 0.1 * _rand(d, seed=70)
    b = 0.2 * _rand(d, seed=71)
    dn = _rand(M, d, seed=72)
    dres = _rand(M, d, seed=73)
    du, dg, db, _, _ = O.layernorm_bwd(dn, u, g, eps, dres=dres)
    fu = lambda uu: float(np.sum(dn * O.layernorm(uu, g, b, eps)[0]) + np.sum(dres * uu))
    fg = lambda gg: float(np.sum(dn * O.layernorm(u, gg, b, eps)[0]))
    fb = lambda bb: float(np.sum(dn * O.layernorm(u, g, bb, eps)[0]))
    _close(du, _fd_grad(fu, u), 1e-7, "layernorm du vs fd")
    _close(dg, _fd_grad(fg, g), 1e-7, "layernorm dgamma vs fd")
    _close(db, _fd_grad(fb, b), 1e-7, "layernorm dbeta vs fd")


def check_ln_delayed_statistics(O):
    """With y = n W1 and G = dY W1^T, the two row statistics come from the
    next GEMM's output side: a = (1/d) dY (gamma^T W1)^T and
    s = (1/d) (sumcols(dY * y) - dY (beta^T W1)^T); the delayed
    du = dres + r (G * gamma) - r a - r^2 s (u - mu) is the canonical one;
    dgamma = sum_i r G (u - mu), dbeta = sum_i G."""
    M, d, N, eps = 4, 8, 5, 1e-6
    u = _rand(M, d, seed=74) + 0.6
    g = 1 + 0.1 * _rand(d, seed=75)
    b = 0.3 * _rand(d, seed=76)
    w1 = _rand(d, N, seed=77)
    dY = _rand(M, N, seed=78)
    dres = _rand(M, d, seed=79)
    n, mu, r = O.layernorm(u, g, b, eps)
    y = O.gemm(n, w1)
    G = O.gemm(dY, w1.T)
    du, dg, db, a, s = O.layernorm_bwd(G, u, g, eps, dres=dres)
    cvec = O.gemm(g[None, :], w1)[0]
    bvec = O.gemm(b[None, :], w1)[0]
    _close(a, O.gemm(dY, cvec[:, None])[:, 0] / d, 1e-12, "a from dY and gamma^T W1")
    _close(s, (np.sum(dY * y, axis=1) - O.gemm(dY, bvec[:, None])[:, 0]) / d, 1e-12, "s from dY, y and beta^T W1")
    c = u - mu[:, None]
    delayed = dres + r[:, None] * (G * g[None, :]) - (r * a)[:, None] - (r ** 2 * s)[:, None] * c
    _close(delayed, du, 1e-12, "delayed LayerNorm backward")
    _close(np.sum(r[:, None] * G * c, axis=0), dg, 1e-12, "dgamma from r G (u - mu)")
    _close(np.sum(G, axis=0), db, 1e-12, "dbeta from G")


def tiny_ln_block(seed=46, M=3, d=4, F=3):
    p = tiny_block(seed=seed, M=M, d=d, F=F)
    rng = np.random.default_rng(seed + 1000)
    p["beta1"] = 0.3 * rng.standard_normal(d)
    p["beta2"] = 0.3 * rng.standard_normal(d)
    p["z"] = p["z"] + 0.5
    return p


def check_ln_block_bwd_fd(O):
    p = tiny_ln_block()
    g = O.ln_block_bwd(p)

    def L(name):
        def f(v):
            q = dict(p)
            q[name] = v
            return float(np.sum(p["dOut"] * O.ln_block_fwd(q)["out"]))
        return f

    for name, gname in [("x", "dx"), ("z", "dz"), ("W0", "dW0"), ("gamma1", "dgamma1"), ("beta1", "dbeta1"),
                        ("Wgu1", "dWgu1"), ("Wd1", "dWd1"), ("gamma2", "dgamma2"), ("beta2", "dbeta2"),
                        ("Wgu2", "dWgu2"), ("Wd2", "dWd2")]:
        _close(g[gname], _fd_grad(L(name), p[name]), 2e-7, f"LayerNorm block {gname}")


def check_ln_block_statistics(O):
    """Each layer's a_l and s_l from its SwiGLU backward's dpre_l and pre_l."""
    p = tiny_ln_block(seed=47)
    f = O.ln_block_fwd(p)
    g = O.ln_block_bwd(p, f)
    d = p["x"].shape[1]
    for l in (1, 2):
        cvec = O.gemm(p[f"gamma{l}"][None, :], p[f"Wgu{l}"])[0]
        bvec = O.gemm(p[f"beta{l}"][None, :], p[f"Wgu{l}"])[0]
        dpre, pre = g[f"dpre{l}"], f[f"pre{l}"]
        _close(g[f"a{l}"], O.gemm(dpre, cvec[:, None])[:, 0] / d, 1e-12, f"a{l}")
        _close(g[f"s{l}"], (np.sum(dpre * pre, axis=1) - O.gemm(dpre, bvec[:, None])[:, 0]) / d, 1e-12, f"s{l}")


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
