"""Numerics of the fused path against the unfused one, on 8B-shaped layers
(paper "CODA: Rewriting Transformer Blocks as GEMM-Epilogue Programs",
Figure 6: relative error against a high-precision reference, normalised by
the error of the conventional path).

Both GPU paths run on the same seeded bf16 inputs at full size (M = 8192
tokens); the fp64 oracle computes the reference on 256 sampled rows (every
output here is row-independent).  For each output the test prints
  rel_l2 = ||gpu - ref||_2 / ||ref||_2  and  max|gpu - ref| / max|ref|
for the fused and the unfused path and their ratio, checks both against the
parity bound and checks that fusing does not lose accuracy (fused rel_l2 at
most 1.25x the unfused one).
"""

import numpy as np
import pytest
import torch

from gpu_util import TOL, f64, say
from gemm_epilogue_transformer_mainloop_amd import synth as S
from oracle import coda_oracle as O

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

M, D, FF, V = 8192, 4096, 14336, 128256
ROWS = np.arange(0, M, M // 256)
RESULTS = []


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gemm_epilogue_transformer_mainloop_amd import coda

    coda.lib()
    yield
    say("numerics summary (fused / unfused relative L2 error vs the fp64 oracle, 256 sampled rows):")
    for r in RESULTS:
        say("  " + r)


def C():
    from gemm_epilogue_transformer_mainloop_amd import coda

    return coda


def compare(name, fused, unfused, ref, ratio_bound=1.25):
    ref = np.asarray(ref, np.float64)
    out = {}
    for tag, g in (("fused", fused), ("unfused", unfused)):
        g = np.asarray(g, np.float64)
        assert np.all(np.isfinite(g)), f"{name} {tag}: non-finite"
        out[tag] = (float(np.linalg.norm(g - ref) / np.linalg.norm(ref)),
                    float(np.max(np.abs(g - ref)) / np.max(np.abs(ref))))
    line = (f"{name:28s} fused rel_l2 {out['fused'][0]:.3e} max {out['fused'][1]:.3e} | unfused rel_l2 "
            f"{out['unfused'][0]:.3e} max {out['unfused'][1]:.3e} | ratio {out['fused'][0] / out['unfused'][0]:.3f}")
    say(line)
    RESULTS.append(line)
    assert out["fused"][1] <= TOL and out["unfused"][1] <= TOL
    assert out["fused"][0] <= ratio_bound * out["unfused"][0] + 1e-12


def rows(t):
    return f64(t)[ROWS]


def test_numerics_norm_block_forward():
    """y = RMSNorm(x W0 + z) W1, d = 4096: delayed r (fused) vs materialised n2."""
    say(f"case: numerics norm block M={M} d={D}")
    p = S.norm_block_inputs(5, M, D, D, D)
    coda = C()
    x, W0, z, g, W1 = (p[k].torch("cuda") for k in ("x", "W0", "z", "gamma", "W1"))
    U, H2, part = coda.coda_gemm_res_sumsq(x, W0, z, g)
    r = coda.coda_row_rms(part, D, p["eps"])
    y_f = coda.coda_gemm_rowscale(H2, W1, r)
    Y0 = coda.coda_gemm(x, W0)
    Uu, N2u, ru = coda.coda_unfused_add_rmsnorm(Y0, z, g, p["eps"])
    y_u = coda.coda_gemm(N2u, W1)
    torch.cuda.synchronize()
    xs = p["x"].f64()[ROWS]
    y_ref, u_ref, r_ref = O.norm_block_fwd(xs, p["W0"].f64(), p["z"].f64()[ROWS], p["gamma"].f64(),
                                           p["W1"].f64(), p["eps"])
    compare("norm block: u", rows(U), rows(Uu), u_ref)
    compare("norm block: r", r.cpu().numpy()[ROWS], ru.cpu().numpy()[ROWS], r_ref)
    compare("norm block: y", rows(y_f), rows(y_u), y_ref)


def test_numerics_mlp_forward_and_dx():
    """SwiGLU MLP out = x + swiglu(x Wgu) Wd and its data gradient dX (d = 4096, F = 14336)."""
    say(f"case: numerics MLP M={M} d={D} F={FF}")
    p = S.mlp_inputs(5, M, D, FF)
    coda = C()
    x, Wgu, Wd, dY = (p[k].torch("cuda") for k in ("x", "Wgu", "Wd", "dY"))
    # fused
    act, pre = coda.coda_gemm_swiglu(x, Wgu)
    out_f, _, _ = coda.coda_gemm_res_sumsq(act, Wd, Z=x, want_part=False)
    dpre_f, _ = coda.coda_gemm_swiglu_bwd(dY, Wd, pre, want_spart=False)
    dX_f, _ = coda.coda_gemm_res_sumsq_bwd(dpre_f, Wgu, dRes=dY, want_dw=False)
    # unfused
    pre_u = coda.coda_gemm(x, Wgu)
    a_u = coda.coda_unfused_swiglu(pre_u)
    out_u = coda.coda_unfused_add(coda.coda_gemm(a_u, Wd), x)
    da_u, _ = coda.coda_gemm_res_sumsq_bwd(dY, Wd, want_dw=False)
    dpre_u = coda.coda_unfused_swiglu_bwd(da_u, pre_u)
    dX0, _ = coda.coda_gemm_res_sumsq_bwd(dpre_u, Wgu, want_dw=False)
    dX_u = coda.coda_unfused_add(dX0, dY)
    torch.cuda.synchronize()
    xs, dYs = p["x"].f64()[ROWS], p["dY"].f64()[ROWS]
    o_ref, _, _ = O.mlp_fwd(xs, p["Wgu"].f64(), p["Wd"].f64())
    g = O.mlp_bwd(xs, p["Wgu"].f64(), p["Wd"].f64(), dYs)
    compare("MLP: out", rows(out_f), rows(out_u), o_ref)
    compare("MLP: dpre", rows(dpre_f), rows(dpre_u), g["dpre"])
    compare("MLP: dX", rows(dX_f), rows(dX_u), g["dX"])


def test_numerics_lmhead_ce():
    """LM head + CE at d = 4096, V = 128256: fp32 logits in the epilogue (fused) vs bf16
    materialised logits (unfused)."""
    say(f"case: numerics LM head M={M} d={D} V={V}")
    h = S.normal_bf16(S.seed_of(5, 20), (M, D))
    W = S.normal_bf16(S.seed_of(5, 21), (D, V), std=D ** -0.5)
    labels = S.labels_int32(S.seed_of(5, 22), M, V)
    coda = C()
    H, Wt, lab = h.torch("cuda"), W.torch("cuda"), torch.from_numpy(labels).cuda()
    lse_f, loss_f, _ = coda.coda_lmhead_ce(H, Wt, lab)
    L = coda.coda_gemm(H, Wt)
    lse_u, loss_u, _ = coda.coda_unfused_cross_entropy(L, lab)
    torch.cuda.synchronize()
    lse_ref, loss_ref, _ = O.lmhead_ce(h.f64()[ROWS], W.f64(), labels[ROWS])
    compare("LM head: lse", lse_f.cpu().numpy()[ROWS], lse_u.cpu().numpy()[ROWS], lse_ref)
    compare("LM head: loss", loss_f.cpu().numpy()[ROWS], loss_u.cpu().numpy()[ROWS], loss_ref)
