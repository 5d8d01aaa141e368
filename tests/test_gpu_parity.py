"""GPU parity of every CODA call against the fp64 oracle, at sizes the oracle
finishes in seconds that still span several 256x256 tiles and ragged tails.

Inputs are seeded (gemm_epilogue_transformer_mainloop_amd.synth); the HIP path
and the oracle consume the same bfloat16 bits.  Bound (per output):
max|gpu - ref| <= 2e-2 * max|ref|; scalar loss relative error <= 1e-3;
integer-exact cases are bit-exact.
"""

import math

import numpy as np
import pytest
import torch

from gpu_util import LOSS_RTOL, assert_close, canary_intact, dev, f64, padded, rel_err, say
from gemm_epilogue_transformer_mainloop_amd import synth as S
from oracle import coda_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gemm_epilogue_transformer_mainloop_amd import coda

    coda.lib()
    name = torch.cuda.get_device_properties(0).gcnArchName
    say(f"device: {name}")
    yield


def C():
    from gemm_epilogue_transformer_mainloop_amd import coda

    return coda


# ---------------------------------------------------------------------------
# mainloop: accumulator layout probe and exact-integer GEMMs
# ---------------------------------------------------------------------------


def test_layout_probe_identity():
    """X = I: Y = X W must reproduce W bit-for-bit (every feature/token lands in its place)."""
    say("case: layout probe identity 256x520x256")
    K = 256
    W = S.normal_bf16(11, (K, 520))
    X = S.Bf16(S.f32_to_bf16_bits(np.eye(K, dtype=np.float32)))
    Y = C().coda_gemm(dev(X), dev(W))
    torch.cuda.synchronize()
    assert np.array_equal(Y.cpu().view(torch.int16).numpy().view(np.uint16), W.bits)


@pytest.mark.parametrize("M,N,K", [(300, 264, 32), (17, 8, 8), (513, 776, 48)])
def test_gemm_integer_exact(M, N, K):
    say(f"case: integer gemm M={M} N={N} K={K}")
    X = S.int_bf16(21, (M, K), -2, 2)
    W = S.int_bf16(22, (K, N), -2, 2)
    Y = C().coda_gemm(dev(X), dev(W))
    torch.cuda.synchronize()
    ref = O.gemm(X.f64(), W.f64())
    assert np.max(np.abs(ref)) <= 256
    assert np.array_equal(f64(Y), ref)


@pytest.mark.parametrize("M,K,N", [(300, 264, 520), (1000, 8, 16), (77, 512, 256)])
def test_wgrad_integer_exact(M, K, N):
    """fp32 output: dW = X^T dY is exact for small integers at any reduction length."""
    say(f"case: integer wgrad M={M} K={K} N={N}")
    X = S.int_bf16(23, (M, K), -3, 3)
    dY = S.int_bf16(24, (M, N), -3, 3)
    dW = C().coda_gemm_wgrad(dev(X), dev(dY))
    torch.cuda.synchronize()
    assert np.array_equal(dW.cpu().numpy().astype(np.float64), O.gemm(X.f64().T, dY.f64()))


def test_dgrad_integer_exact():
    say("case: integer dgrad")
    M, N, K = 260, 136, 520
    dU = S.int_bf16(25, (M, N), -1, 1)
    W = S.int_bf16(26, (K, N), -1, 1)
    dX, _ = C().coda_gemm_res_sumsq_bwd(dev(dU), dev(W), want_dw=False)
    torch.cuda.synchronize()
    assert np.array_equal(f64(dX), O.gemm(dU.f64(), W.f64().T))


def test_gemm_random_ragged():
    say("case: random gemm 1000x776x384")
    M, N, K = 1000, 776, 384
    X = S.normal_bf16(31, (M, K))
    W = S.normal_bf16(32, (K, N), std=K ** -0.5)
    Y = C().coda_gemm(dev(X), dev(W))
    torch.cuda.synchronize()
    assert_close(f64(Y), O.gemm(X.f64(), W.f64()), "Y")


# ---------------------------------------------------------------------------
# GEMM -> residual -> RMSNorm -> GEMM (config 1 at full size, config 2 reduced)
# ---------------------------------------------------------------------------


def _norm_block(p, M, d, K, N, rope=None):
    coda = C()
    x, W0, z, g, W1 = (dev(p[k]) for k in ("x", "W0", "z", "gamma", "W1"))
    U, H2, part = coda.coda_gemm_res_sumsq(x, W0, z, g)
    r = coda.coda_row_rms(part, d, p["eps"])
    Y = coda.coda_gemm_rowscale(H2, W1, r)
    out = {"U": U, "H2": H2, "part": part, "r": r, "Y": Y}
    if rope is not None:
        out["Yr"] = coda.coda_gemm_rope(H2, dev(p["W1r"]), r, dev(rope["pos"]), S.ROPE_THETA, S.HEAD_DIM,
                                        rope["n_rope"])
    torch.cuda.synchronize()
    return out


def _check_norm_block(p, out, d, rope=None):
    u, h2, ss = O.res_sumsq(p["x"].f64(), p["W0"].f64(), p["z"].f64(), p["gamma"].f64())
    assert_close(f64(out["U"]), u, "u")
    assert_close(f64(out["H2"]), h2, "h2")
    assert_close(out["part"].double().sum(1).cpu().numpy(), ss, "sum of partials")
    y, u2, r = O.norm_block_fwd(p["x"].f64(), p["W0"].f64(), p["z"].f64(), p["gamma"].f64(), p["W1"].f64(), p["eps"])
    assert_close(f64(out["r"]), r, "r")
    assert_close(f64(out["Y"]), y, "y")
    if rope is not None:
        n2, _ = O.rmsnorm(u, p["gamma"].f64(), p["eps"])
        t = O.gemm(n2, p["W1r"].f64())
        yr = O.rope(t, rope["pos"], S.ROPE_THETA, S.HEAD_DIM, rope["n_rope"])
        assert_close(f64(out["Yr"]), yr, "y rope")


def test_norm_block_config1():
    say("case: config 1 (M=256, d=512, out=1024)")
    c = S.CONFIGS[1]
    p = S.norm_block_inputs(1, c["M"], c["d"], c["K"], c["N"])
    out = _norm_block(p, c["M"], c["d"], c["K"], c["N"])
    _check_norm_block(p, out, c["d"])


def test_norm_block_reduced_config2_rope():
    """Config 2's structure (QKV-shaped W1 with RoPE on Q and K) at a ragged reduced size."""
    M, d, K, N = 1000, 520, 384, 776
    say(f"case: reduced config 2 M={M} d={d} K={K} N={N} + rope")
    p = S.norm_block_inputs(2, M, d, K, N, n_rope_cols=776)
    rope = {"pos": ((np.arange(M) * 7) % 2048).astype(np.int32), "n_rope": 640}
    out = _norm_block(p, M, d, K, N, rope=rope)
    _check_norm_block(p, out, d, rope=rope)


def test_rope_without_rowscale_and_inverse():
    M, K, N = 300, 256, 520
    say("case: rope without r, rope_bwd")
    A = S.normal_bf16(41, (M, K))
    W = S.normal_bf16(42, (K, N), std=K ** -0.5)
    r = (1.0 + 0.5 * np.random.default_rng(43).random(M)).astype(np.float32)
    pos = np.random.default_rng(44).integers(0, 2048, M).astype(np.int32)
    coda = C()
    Y = coda.coda_gemm_rope(dev(A), dev(W), None, dev(pos), 10000.0, 64, 512)
    Yb = coda.coda_gemm_rope_bwd(dev(A), dev(W), dev(r), dev(pos), 10000.0, 64, 512)
    torch.cuda.synchronize()
    t = O.gemm(A.f64(), W.f64())
    assert_close(f64(Y), O.rope(t, pos, 10000.0, 64, 512), "rope")
    assert_close(f64(Yb), O.rope(O.row_scale(r, t), pos, 10000.0, 64, 512, inverse=True), "rope_bwd")


# ---------------------------------------------------------------------------
# SwiGLU forward / backward, RMSNorm backward
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("with_r", [False, True])
def test_swiglu_fwd(with_r):
    M, K, F = 700, 256, 520
    say(f"case: swiglu fwd M={M} K={K} F={F} r={with_r}")
    A = S.normal_bf16(51, (M, K))
    Wgu = S.normal_bf16(52, (K, 2 * F), std=K ** -0.5)
    r = (0.5 + np.random.default_rng(53).random(M)).astype(np.float32) if with_r else None
    act, pre = C().coda_gemm_swiglu(dev(A), dev(Wgu), None if r is None else dev(r))
    torch.cuda.synchronize()
    t = O.gemm(A.f64(), Wgu.f64())
    if with_r:
        t = O.row_scale(r, t)
    assert_close(f64(pre), t, "pre")
    assert_close(f64(act), O.swiglu(t), "act")


@pytest.mark.parametrize("with_pre", [True, False])
def test_swiglu_fwd_half_chunk_width(with_pre):
    """Activation width F % 8 == 4 with ldact % 8 == 4 (rows end on half a
    16-byte chunk); act and pre in canary-padded strided buffers."""
    M, K, F = 300, 192, 260
    say(f"case: swiglu fwd half-chunk act width M={M} K={K} F={F} ldact={F + 4} pre={with_pre}")
    A = S.normal_bf16(54, (M, K))
    Wgu = S.normal_bf16(55, (K, 2 * F), std=K ** -0.5)
    r = (0.5 + np.random.default_rng(56).random(M)).astype(np.float32)
    act_full, act = padded(M, F, torch.bfloat16, pad_cols=8)
    assert act.stride(0) % 8 == 4
    pre_full, pre = padded(M, 2 * F, torch.bfloat16) if with_pre else (None, None)
    C().coda_gemm_swiglu(dev(A), dev(Wgu), dev(r), Act=act, Pre=pre, want_pre=with_pre)
    torch.cuda.synchronize()
    t = O.row_scale(r, O.gemm(A.f64(), Wgu.f64()))
    assert_close(f64(act), O.swiglu(t), "act")
    assert canary_intact(act_full, M, F)
    if with_pre:
        assert_close(f64(pre), t, "pre")
        assert canary_intact(pre_full, M, 2 * F)


def test_swiglu_bwd_and_s():
    M, N, F, d = 600, 264, 520, 264
    say(f"case: swiglu bwd M={M} N={N} F={F}")
    dOut = S.normal_bf16(61, (M, N))
    Wd = S.normal_bf16(62, (F, N), std=F ** -0.5)
    pre = S.normal_bf16(63, (M, 2 * F), std=2.0)
    coda = C()
    dpre, spart = coda.coda_gemm_swiglu_bwd(dev(dOut), dev(Wd), dev(pre))
    s = coda.coda_row_rms_bwd(spart, d)
    torch.cuda.synchronize()
    da = O.gemm(dOut.f64(), Wd.f64().T)
    ref = O.swiglu_bwd(da, pre.f64())
    assert_close(f64(dpre), ref, "dpre")
    assert_close(f64(s), np.sum(ref * pre.f64(), axis=1) / d, "s")


def test_rowscale_bwd_and_dgamma():
    M, d, N = 700, 520, 776
    say(f"case: rowscale bwd M={M} d={d} N={N}")
    dY = S.normal_bf16(71, (M, N))
    W1 = S.normal_bf16(72, (d, N), std=d ** -0.5)
    u = S.normal_bf16(73, (M, d))
    gamma = S.normal_bf16(74, (d,), std=0.1, mean=1.0)
    dres = S.normal_bf16(75, (M, d))
    eps = 1e-6
    G = O.gemm(dY.f64(), W1.f64().T)
    du_ref, dg_ref, s_ref, r_ref = O.rmsnorm_bwd(G, u.f64(), gamma.f64(), eps, dres=dres.f64())
    n2_ref, _ = O.rmsnorm(u.f64(), gamma.f64(), eps)
    coda = C()
    r_t = torch.tensor(r_ref, dtype=torch.float32, device="cuda")
    s_t = torch.tensor(s_ref, dtype=torch.float32, device="cuda")
    dU, N2, gpart = coda.coda_gemm_rowscale_bwd(dev(dY), dev(W1), dev(u), dev(gamma), r_t, s_t, dRes=dev(dres))
    dgamma = coda.coda_col_reduce(gpart)
    torch.cuda.synchronize()
    assert_close(f64(dU), du_ref, "du")
    assert_close(f64(N2), n2_ref, "n2")
    assert_close(f64(dgamma), dg_ref, "dgamma")


def test_wgrad_and_res_bwd():
    M, N, K = 1000, 264, 520
    say(f"case: res_sumsq_bwd M={M} N={N} K={K}")
    dU = S.normal_bf16(81, (M, N))
    W = S.normal_bf16(82, (K, N), std=K ** -0.5)
    X = S.normal_bf16(83, (M, K))
    dres = S.normal_bf16(84, (M, K))
    dX, dW = C().coda_gemm_res_sumsq_bwd(dev(dU), dev(W), X=dev(X), dRes=dev(dres))
    dW2 = C().coda_gemm_wgrad(dev(X), dev(dU), dW=dW.clone(), accumulate=True)
    torch.cuda.synchronize()
    assert_close(f64(dX), O.gemm(dU.f64(), W.f64().T) + dres.f64(), "dX")
    ref = O.gemm(X.f64().T, dU.f64())
    assert_close(dW.cpu().numpy(), ref, "dW")
    assert_close(dW2.cpu().numpy(), 2 * ref, "dW accumulate")


# ---------------------------------------------------------------------------
# LM head + cross-entropy
# ---------------------------------------------------------------------------


def test_lmhead_ce_fwd_bwd():
    M, d, V = 300, 256, 1000
    say(f"case: lmhead ce M={M} d={d} V={V}")
    p = S.lmhead_inputs(4, M, d, V)
    labels = p["labels"].copy()
    labels[:4] = [0, V - 1, 255, 256]
    coda = C()
    H, W, lab = dev(p["h"]), dev(p["W"]), dev(labels)
    lse, loss_row, loss_mean = coda.coda_lmhead_ce(H, W, lab)
    dH, dW = coda.coda_lmhead_ce_bwd(H, W, lab, lse, 1.0 / M, ws_rows=256)  # two row chunks
    dH1, dW1 = coda.coda_lmhead_ce_bwd(H, W, lab, lse, 1.0 / M)               # one chunk
    torch.cuda.synchronize()
    lse_r, loss_r, mean_r = O.lmhead_ce(p["h"].f64(), p["W"].f64(), labels)
    assert_close(f64(lse), lse_r, "lse")
    assert_close(f64(loss_row), loss_r, "loss_row")
    e = abs(float(loss_mean.item()) - mean_r) / abs(mean_r)
    say(f"  loss mean rel err {e:.3e}")
    assert e <= LOSS_RTOL
    dh_r, dW_r, _ = O.lmhead_ce_bwd(p["h"].f64(), p["W"].f64(), labels, 1.0 / M)
    assert_close(f64(dH), dh_r, "dh")
    assert_close(dW.cpu().numpy(), dW_r, "dW")
    assert_close(f64(dH1), dh_r, "dh (1 chunk)")
    assert_close(dW1.cpu().numpy(), dW_r, "dW (1 chunk)")


@pytest.mark.parametrize("vchunk", [256, 1000, 4096])
def test_lmhead_ce_bwd_vchunk(vchunk):
    """The vocabulary-chunked backward: 5 chunks with a ragged last one (24
    columns), 2 chunks (the second 48 columns wide), and a single chunk."""
    M, d, V = 520, 256, 1048
    say(f"case: lmhead ce bwd, vocabulary chunks of {vchunk}, M={M} d={d} V={V}")
    p = S.lmhead_inputs(44, M, d, V)
    labels = p["labels"].copy()
    labels[:6] = [0, V - 1, 255, 256, 1023, 1024]
    coda = C()
    H, W, lab = dev(p["h"]), dev(p["W"]), dev(labels)
    lse, _, _ = coda.coda_lmhead_ce(H, W, lab)
    dH, dW = coda.coda_lmhead_ce_bwd_vchunk(H, W, lab, lse, 1.0 / M, vchunk=vchunk)
    torch.cuda.synchronize()
    dh_r, dW_r, _ = O.lmhead_ce_bwd(p["h"].f64(), p["W"].f64(), labels, 1.0 / M)
    assert_close(f64(dH), dh_r, "dh")
    assert_close(dW.cpu().numpy(), dW_r, "dW")


def test_lmhead_bad_label_is_nan():
    M, d, V = 40, 64, 264
    say("case: lmhead out-of-range label")
    p = S.lmhead_inputs(4, M, d, V)
    labels = p["labels"].copy()
    labels[3] = V
    labels[5] = -1
    lse, loss_row, _ = C().coda_lmhead_ce(dev(p["h"]), dev(p["W"]), dev(labels))
    _, loss_row2, _, _ = C().coda_lmhead_ce_logits(dev(p["h"]), dev(p["W"]), dev(labels))
    torch.cuda.synchronize()
    for lr in (loss_row.cpu().numpy(), loss_row2.cpu().numpy()):
        assert np.isnan(lr[3]) and np.isnan(lr[5])
        assert np.all(np.isfinite(np.delete(lr, [3, 5])))


# ---------------------------------------------------------------------------
# Chains: SwiGLU MLP (config 3 structure) and the two-layer block (config 5)
# ---------------------------------------------------------------------------


def test_mlp_chain_reduced_config3():
    M, d, F = 520, 256, 392
    say(f"case: reduced config 3 chain M={M} d={d} F={F}")
    p = S.mlp_inputs(3, M, d, F)
    coda = C()
    x, Wgu, Wd, dY = (dev(p[k]) for k in ("x", "Wgu", "Wd", "dY"))
    act, pre = coda.coda_gemm_swiglu(x, Wgu)
    out, _, _ = coda.coda_gemm_res_sumsq(act, Wd, Z=x, want_part=False)
    dpre, _ = coda.coda_gemm_swiglu_bwd(dY, Wd, pre, want_spart=False)
    dX, dWgu = coda.coda_gemm_res_sumsq_bwd(dpre, Wgu, X=x, dRes=dY)
    dWd = coda.coda_gemm_wgrad(act, dY)
    torch.cuda.synchronize()
    o_r, pre_r, a_r = O.mlp_fwd(p["x"].f64(), p["Wgu"].f64(), p["Wd"].f64())
    g = O.mlp_bwd(p["x"].f64(), p["Wgu"].f64(), p["Wd"].f64(), p["dY"].f64())
    assert_close(f64(out), o_r, "out")
    assert_close(f64(dpre), g["dpre"], "dpre")
    assert_close(f64(dX), g["dX"], "dX")
    assert_close(dWgu.cpu().numpy(), g["dWgu"], "dWgu")
    assert_close(dWd.cpu().numpy(), g["dWd"], "dWd")


def run_block_gpu(p, M, d, F):
    """Forward + reverse-fused backward of the two-layer block through the C ABI."""
    coda = C()
    T = {k: dev(v) for k, v in p.items() if k != "eps"}
    eps = p["eps"]
    f = {}
    f["u1"], f["h2_1"], part1 = coda.coda_gemm_res_sumsq(T["x"], T["W0"], T["z"], T["gamma1"])
    f["r1"] = coda.coda_row_rms(part1, d, eps)
    f["a1"], f["pre1"] = coda.coda_gemm_swiglu(f["h2_1"], T["Wgu1"], f["r1"])
    f["u2"], f["h2_2"], part2 = coda.coda_gemm_res_sumsq(f["a1"], T["Wd1"], f["u1"], T["gamma2"])
    f["r2"] = coda.coda_row_rms(part2, d, eps)
    f["a2"], f["pre2"] = coda.coda_gemm_swiglu(f["h2_2"], T["Wgu2"], f["r2"])
    f["out"], _, _ = coda.coda_gemm_res_sumsq(f["a2"], T["Wd2"], f["u2"], want_part=False)
    g = {}
    dOut = T["dOut"]
    g["dWd2"] = coda.coda_gemm_wgrad(f["a2"], dOut)
    g["dpre2"], sp2 = coda.coda_gemm_swiglu_bwd(dOut, T["Wd2"], f["pre2"])
    g["s2"] = coda.coda_row_rms_bwd(sp2, d)
    g["du2"], n2_2, gp2 = coda.coda_gemm_rowscale_bwd(g["dpre2"], T["Wgu2"], f["u2"], T["gamma2"], f["r2"], g["s2"],
                                                      dRes=dOut)
    g["dgamma2"] = coda.coda_col_reduce(gp2)
    g["dWgu2"] = coda.coda_gemm_wgrad(n2_2, g["dpre2"])
    g["dWd1"] = coda.coda_gemm_wgrad(f["a1"], g["du2"])
    g["dpre1"], sp1 = coda.coda_gemm_swiglu_bwd(g["du2"], T["Wd1"], f["pre1"])
    g["s1"] = coda.coda_row_rms_bwd(sp1, d)
    g["du1"], n2_1, gp1 = coda.coda_gemm_rowscale_bwd(g["dpre1"], T["Wgu1"], f["u1"], T["gamma1"], f["r1"], g["s1"],
                                                      dRes=g["du2"])
    g["dgamma1"] = coda.coda_col_reduce(gp1)
    g["dWgu1"] = coda.coda_gemm_wgrad(n2_1, g["dpre1"])
    g["dx"], g["dW0"] = coda.coda_gemm_res_sumsq_bwd(g["du1"], T["W0"], X=T["x"])
    torch.cuda.synchronize()
    return f, g


def test_block_chain_reduced_config5():
    M, d, F = 520, 264, 392
    say(f"case: reduced config 5 block fwd+bwd M={M} d={d} F={F}")
    p = S.block_inputs(5, M, d, F)
    f, g = run_block_gpu(p, M, d, F)
    q = {k: (v.f64() if hasattr(v, "bits") else v) for k, v in p.items()}
    fr = O.block_fwd(q)
    gr = O.block_bwd(q, fr)
    for k in ("u1", "r1", "pre1", "a1", "u2", "r2", "pre2", "a2", "out"):
        assert_close(f64(f[k]), fr[k], k)
    for k in ("dWd2", "dpre2", "s2", "du2", "dgamma2", "dWgu2", "dWd1", "dpre1", "s1", "du1", "dgamma1", "dWgu1",
              "dx", "dW0"):
        got = g[k].cpu().numpy().astype(np.float64) if g[k].dtype == torch.float32 else f64(g[k])
        assert_close(got, gr[k], k)


# ---------------------------------------------------------------------------
# Robustness: canaries around masked edge tiles, determinism, empty inputs
# ---------------------------------------------------------------------------


def test_canary_padding_untouched():
    M, N, K = 300, 264, 256
    say("case: canary padding")
    X = S.normal_bf16(91, (M, K))
    W = S.normal_bf16(92, (K, N), std=K ** -0.5)
    z = S.normal_bf16(93, (M, N))
    g = S.normal_bf16(94, (N,), std=0.1, mean=1.0)
    coda = C()
    Uf, U = padded(M, N, torch.bfloat16)
    Hf, H = padded(M, N, torch.bfloat16)
    npart = coda.coda_nparts(N)
    Pf = torch.full((M * npart + 64,), 12345.0, device="cuda")
    P = Pf[: M * npart].view(M, npart)
    coda.coda_gemm_res_sumsq(dev(X), dev(W), dev(z), dev(g), U=U, H2=H, part=P)
    Af, Act = padded(M, N // 2, torch.bfloat16)
    Prf, Pre = padded(M, N, torch.bfloat16)
    coda.coda_gemm_swiglu(dev(X), dev(W), Act=Act, Pre=Pre)
    torch.cuda.synchronize()
    assert canary_intact(Uf, M, N) and canary_intact(Hf, M, N)
    assert bool(torch.all(Pf[M * npart:] == 12345.0))
    assert canary_intact(Af, M, N // 2) and canary_intact(Prf, M, N)
    u, h2, ss = O.res_sumsq(X.f64(), W.f64(), z.f64(), g.f64())
    assert_close(f64(U), u, "u (padded ld)")


def test_deterministic():
    say("case: determinism")
    M, d, V = 300, 256, 1000
    p = S.lmhead_inputs(4, M, d, V)
    coda = C()
    H, W, lab = dev(p["h"]), dev(p["W"]), dev(p["labels"])
    a = coda.coda_lmhead_ce(H, W, lab)
    b = coda.coda_lmhead_ce(H, W, lab)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    q = S.block_inputs(5, 264, 264, 136)
    f1, g1 = run_block_gpu(q, 264, 264, 136)
    f2, g2 = run_block_gpu(q, 264, 264, 136)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_empty_inputs():
    say("case: empty inputs")
    coda = C()
    X = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((64, 128), dtype=torch.bfloat16, device="cuda")
    Y = coda.coda_gemm(X, W)
    assert Y.shape == (0, 128)
    # zero-length reduction of a weight gradient writes zeros
    dW = coda.coda_gemm_wgrad(X, torch.empty((0, 128), dtype=torch.bfloat16, device="cuda"),
                              dW=torch.full((64, 128), 5.0, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(dW == 0)
    # LM head with no rows: the stored-logits pair; the backward writes dW = 0
    H0 = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    W0 = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    lab0 = torch.empty((0,), dtype=torch.int32, device="cuda")
    lse0, _, _, L0 = coda.coda_lmhead_ce_logits(H0, W0, lab0)
    dH0, dW0 = coda.coda_lmhead_ce_bwd_logits(H0, W0, lab0, lse0, 1.0, L0,
                                              dW=torch.full((64, 256), 5.0, device="cuda"))
    torch.cuda.synchronize()
    assert L0.shape == (0, 256) and dH0.shape == (0, 64) and torch.all(dW0 == 0)
