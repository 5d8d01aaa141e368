"""GPU parity of the tile plans: when 256x256 tiles leave the last round
mostly empty, the trailing features (coda_tile_split) or the trailing tokens
(coda_tile_split_tokens) run as 256x128 tiles in the same dispatch, and a
problem of under half a round runs in 256x128 tiles only.  Every call that can
split is run at a shape that splits on the device (asserted), with ragged
tokens (M = 24500: the last 128-token tile holds 52 rows), ragged features
(712 = 2 x 256 + 200, so the half tiles start at feature 512 and end mid-tile)
and a K that is not a multiple of 64; the weight gradient runs under each plan,
plain and accumulating.  Against the fp64 oracle; bound: max|gpu - ref| <=
2e-2 * max|ref|.
"""

import numpy as np
import pytest
import torch

from gpu_util import LOSS_RTOL, assert_close, dev, f64, say
from gemm_epilogue_transformer_mainloop_amd import synth as S
from oracle import coda_oracle as O

pytestmark = pytest.mark.gpu

M, K, N = 24500, 136, 712


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


def splits(F, T):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    s = C().coda_tile_split(F, T, cus)
    say(f"  tile split F={F} T={T} on {cus} CUs: {s} big feature tiles")
    assert s > 0, "shape chosen to split on a 256-CU device"
    return s


@pytest.mark.parametrize("K", [8, 72, 136, 520])
def test_split_gemm_and_rope(K):
    """K = 8, 72, 136, 520: 1, 2, 3 and 9 k-tiles of 64 (the prologue and
    tail cases of the half-tile k-loop, and its steady state)."""
    say(f"case: split gemm + rope M={M} N={N} K={K}")
    splits(N, M)
    A = S.normal_bf16(701, (M, K))
    W = S.normal_bf16(702, (K, N), std=K ** -0.5)
    r = (0.5 + np.random.default_rng(703).random(M)).astype(np.float32)
    pos = (np.arange(M) % 2048).astype(np.int32)
    coda = C()
    Y = coda.coda_gemm(dev(A), dev(W))
    Yr = coda.coda_gemm_rope(dev(A), dev(W), dev(r), dev(pos), S.ROPE_THETA, 64, 640)
    torch.cuda.synchronize()
    t = O.gemm(A.f64(), W.f64())
    assert_close(f64(Y), t, "Y")
    assert_close(f64(Yr), O.rope(O.row_scale(r, t), pos, S.ROPE_THETA, 64, 640), "rope")


def test_split_res_sumsq():
    say(f"case: split res_sumsq M={M} N={N} K={K}")
    splits(N, M)
    x = S.normal_bf16(711, (M, K))
    W0 = S.normal_bf16(712, (K, N), std=K ** -0.5)
    z = S.normal_bf16(713, (M, N))
    g = S.normal_bf16(714, (N,), std=0.1, mean=1.0)
    coda = C()
    U, H2, part = coda.coda_gemm_res_sumsq(dev(x), dev(W0), dev(z), dev(g))
    r = coda.coda_row_rms(part, N, 1e-6)
    torch.cuda.synchronize()
    u, h2, ss = O.res_sumsq(x.f64(), W0.f64(), z.f64(), g.f64())
    assert_close(f64(U), u, "u")
    assert_close(f64(H2), h2, "h2")
    assert_close(part.double().sum(1).cpu().numpy(), ss, "sum of partials")
    assert_close(f64(r), O.row_rms(ss, N, 1e-6), "r")


def test_split_swiglu_fwd_bwd():
    F = 360  # 2F = 720 interleaved gate/up features
    say(f"case: split swiglu fwd/bwd M={M} F={F} K={K}")
    splits(2 * F, M)
    A = S.normal_bf16(721, (M, K))
    Wgu = S.normal_bf16(722, (K, 2 * F), std=K ** -0.5)
    coda = C()
    act, pre = coda.coda_gemm_swiglu(dev(A), dev(Wgu))
    torch.cuda.synchronize()
    t = O.gemm(A.f64(), Wgu.f64())
    assert_close(f64(pre), t, "pre")
    assert_close(f64(act), O.swiglu(t), "act")
    # backward in the F = 712 feature space (dgrad operand order)
    Fb = N
    splits(Fb, M)
    dOut = S.normal_bf16(723, (M, K))
    Wd = S.normal_bf16(724, (Fb, K), std=Fb ** -0.5)
    preb = S.normal_bf16(725, (M, 2 * Fb), std=2.0)
    dpre, spart = coda.coda_gemm_swiglu_bwd(dev(dOut), dev(Wd), dev(preb))
    s = coda.coda_row_rms_bwd(spart, Fb)
    torch.cuda.synchronize()
    ref = O.swiglu_bwd(O.gemm(dOut.f64(), Wd.f64().T), preb.f64())
    assert_close(f64(dpre), ref, "dpre")
    assert_close(f64(s), np.sum(ref * preb.f64(), axis=1) / Fb, "s")


def test_split_res_bwd_dx():
    say(f"case: split res_sumsq_bwd dX M={M} K(out)={N} N(red)={K}")
    splits(N, M)
    dU = S.normal_bf16(731, (M, K))
    W = S.normal_bf16(732, (N, K), std=N ** -0.5)
    dres = S.normal_bf16(733, (M, N))
    dX, _ = C().coda_gemm_res_sumsq_bwd(dev(dU), dev(W), dRes=dev(dres), want_dw=False)
    torch.cuda.synchronize()
    assert_close(f64(dX), O.gemm(dU.f64(), W.f64().T) + dres.f64(), "dX")


def test_split_lmhead_ce():
    V = N
    say(f"case: split lmhead ce M={M} V={V} d={K}")
    splits(V, M)
    h = S.normal_bf16(741, (M, K))
    W = S.normal_bf16(742, (K, V), std=K ** -0.5)
    labels = S.labels_int32(743, M, V)
    coda = C()
    lse, loss_row, loss_mean = coda.coda_lmhead_ce(dev(h), dev(W), dev(labels))
    dH, dW = coda.coda_lmhead_ce_bwd(dev(h), dev(W), dev(labels), lse, 1.0 / M)
    torch.cuda.synchronize()
    lse_r, loss_r, mean_r = O.lmhead_ce(h.f64(), W.f64(), labels)
    assert_close(f64(lse), lse_r, "lse")
    assert_close(f64(loss_row), loss_r, "loss_row")
    assert abs(float(loss_mean.item()) - mean_r) <= LOSS_RTOL * abs(mean_r)
    dh_r, dW_r, _ = O.lmhead_ce_bwd(h.f64(), W.f64(), labels, 1.0 / M)
    assert_close(f64(dH), dh_r, "dh")
    assert_close(dW.cpu().numpy(), dW_r, "dW")


def plan(F, T):
    """The tile plan on this device: ("feature", split), ("small", 0), ("token", split) or ("none", 0)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    s = C().coda_tile_split(F, T, cus)
    if s > 0:
        return "feature", s
    nTF, nTT = -(-F // 256), -(-T // 256)
    if 2 * nTF * nTT <= cus and -(-T // 128) > nTT:
        return "small", 0
    t = C().coda_tile_split_tokens(F, T, cus)
    return ("token", t) if t > 0 else ("none", 0)


# (tokens M, K, features N, big token tiles): 14000 tokens = 55 tiles, 3.4 rounds of
# 16 feature tiles: tokens 0..12287 in 256 x 256 tiles, the rest (1712, the last
# half tile ragged) in 256 x 128 tiles; the others split 20000 (79 token tiles),
# 6000 (24, a 1.5-round problem) and 20000 again at 24 feature tiles; K from 1 to
# 9 k-tiles of 64, never a multiple of 64 but at 8.
TOKEN_SPLITS = [(14000, 136, 4096, 48), (20000, 72, 2048, 64), (6000, 520, 4096, 16), (20000, 8, 6144, 74)]


@pytest.mark.parametrize("Mt,Kt,Nt,tb", TOKEN_SPLITS)
def test_token_split_gemm(Mt, Kt, Nt, tb):
    """Forward GEMM whose plan is the token split."""
    kind, s = plan(Nt, Mt)
    say(f"case: token split gemm M={Mt} N={Nt} K={Kt}: plan {kind} {s}")
    assert kind == "token" and s == tb
    A = S.normal_bf16(731, (Mt, Kt))
    W = S.normal_bf16(732, (Kt, Nt), std=Kt ** -0.5)
    Y = C().coda_gemm(dev(A), dev(W))
    torch.cuda.synchronize()
    assert_close(f64(Y), O.gemm(A.f64(), W.f64()), "Y")


# (N output columns = features, K_in rows of dW = tokens of the launch, plan)
WGRAD_PLANS = [(712, 24504, "feature"), (4096, 14000, "token"), (4096, 6000, "token"), (512, 1000, "small")]


@pytest.mark.parametrize("N,Kin,kind", WGRAD_PLANS)
@pytest.mark.parametrize("accumulate", [False, True])
def test_split_wgrad(N, Kin, kind, accumulate):
    """The weight gradient dW = X^T dY (both operands contiguous along the
    output dims) under each tile plan, now that its token operand also has a
    128-row tile: the 256 x 128 tiles read it through 256-byte k-rows.  The
    reduction (200 tokens) is not a multiple of 64."""
    Mr = 200
    got, s = plan(N, Kin)
    say(f"case: wgrad N={N} Kin={Kin} M={Mr} accumulate={accumulate}: plan {got} {s}")
    assert got == kind
    X = S.normal_bf16(741, (Mr, Kin))
    dY = S.normal_bf16(742, (Mr, N))
    ref = O.gemm(X.f64().T, dY.f64())
    coda = C()
    if accumulate:
        base = np.random.default_rng(743).standard_normal((Kin, N)).astype(np.float32)
        dW = torch.from_numpy(base).cuda()
        coda.coda_gemm_wgrad(dev(X), dev(dY), dW, accumulate=True)
        ref = ref + base.astype(np.float64)
    else:
        dW = coda.coda_gemm_wgrad(dev(X), dev(dY))
    torch.cuda.synchronize()
    assert_close(dW.double().cpu().numpy(), ref, "dW")


def test_token_split_fused():
    """Fused epilogues under the token split (the half tiles start at token
    12288): SwiGLU forward (act and pre, 4096 interleaved gate/up features)
    and res_sumsq (u, h2 and the per-128-feature row partials), at 14000
    ragged tokens and K = 136."""
    Mt, Kt = 14000, 136
    coda = C()
    kind, s = plan(4096, Mt)
    say(f"case: token split swiglu + res_sumsq M={Mt} N=4096 K={Kt}: plan {kind} {s}")
    assert kind == "token"
    A = S.normal_bf16(751, (Mt, Kt))
    Wgu = S.normal_bf16(752, (Kt, 4096), std=Kt ** -0.5)
    act, pre = coda.coda_gemm_swiglu(dev(A), dev(Wgu))
    torch.cuda.synchronize()
    t = O.gemm(A.f64(), Wgu.f64())
    assert_close(f64(pre), t, "pre")
    assert_close(f64(act), O.swiglu(t), "act")
    del act, pre, t
    W0 = S.normal_bf16(753, (Kt, 4096), std=Kt ** -0.5)
    z = S.normal_bf16(754, (Mt, 4096))
    g = S.normal_bf16(755, (4096,), std=0.1, mean=1.0)
    U, H2, part = coda.coda_gemm_res_sumsq(dev(A), dev(W0), dev(z), dev(g))
    torch.cuda.synchronize()
    u, h2, ss = O.res_sumsq(A.f64(), W0.f64(), z.f64(), g.f64())
    assert_close(f64(U), u, "u")
    assert_close(f64(H2), h2, "h2")
    assert_close(part.double().sum(1).cpu().numpy(), ss, "sum of partials")
