"""coda_gemm_swiglu_bwd_overlap, the SwiGLU backward with each tile's
epilogue overlapped with the next tile's MFMA work: a persistent kernel whose
tile epilogue parks da in fp32 in the dPre bytes of its own tile, and whose
next k-loop applies the pair map between MFMA pairs (coda_swiglu_bwd_units
plans it).

Parity against the fp64 oracle on every output element, at shapes the plan
routes to the deferred kernel (asserted; and one it does not, which runs the
plain kernel): ragged tokens and features (partial
wave tiles, and waves with no token or no feature inside the matrix), a
ragged reduction (masked last k-tile), one and two pair-map
units per k-tile, 1.6 rounds of tiles (workgroups with one tile and with two)
and 4 rounds, with and without the s partials.  dPre starts as NaN inside and
a canary outside: every element must come out finite and the canary intact.
Two calls in a row give the same bits.  Bound: max|gpu - ref| <= 2e-2 *
max|ref| per output.
"""

import numpy as np
import pytest
import torch

from gpu_util import assert_close, canary_intact, dev, f64, padded, say
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


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def spart_ref(dpre_ref, pre, nparts):
    """s partials from the oracle's dpre: per token and 128-feature part p,
    the sum over its features j of dpre_2j pre_2j + dpre_2j+1 pre_2j+1."""
    M, two_f = dpre_ref.shape
    prod = (dpre_ref * pre).reshape(M, two_f // 2, 2).sum(axis=2)
    F = two_f // 2
    out = np.zeros((M, nparts))
    for p in range(nparts):
        out[:, p] = prod[:, 128 * p:min(F, 128 * (p + 1))].sum(axis=1)
    return out


CASES = [
    # M, F, N, units, with spart
    (600, 520, 264, 0, True),        # plan 0: the plain kernel
    (5000, 5000, 2048, 2, True),
    (5000, 5000, 4104, 1, True),
    (5000, 5000, 2056, 2, False),
    (4200, 6208, 2048, 2, True),      # last tiles: a wave with no tokens, a wave with no features
    (8192, 8192, 2048, 2, True),
]


@pytest.mark.parametrize("M,F,N,units,with_s", CASES)
def test_swiglu_bwd_deferred(M, F, N, units, with_s):
    coda = C()
    assert coda.coda_swiglu_bwd_units(M, F, N, cus()) == units
    say(f"case: deferred swiglu bwd M={M} F={F} N={N} units={units} spart={with_s}")
    seed = 7000 + M + F + N
    dOut = S.normal_bf16(seed, (M, N))
    Wd = S.normal_bf16(seed + 1, (F, N), std=F ** -0.5)
    pre = S.normal_bf16(seed + 2, (M, 2 * F), std=2.0)
    full, dpre = padded(M, 2 * F, torch.bfloat16, pad_rows=2, pad_cols=16)
    dpre.fill_(float("nan"))
    np_ = coda.coda_nparts(F)
    spart = torch.full((M, np_), float("nan"), device="cuda") if with_s else None
    coda.coda_gemm_swiglu_bwd_overlap(dev(dOut), dev(Wd), dev(pre), dPre=dpre, spart=spart, want_spart=with_s)
    torch.cuda.synchronize()
    assert canary_intact(full, M, 2 * F), "dPre canary overwritten"
    first = dpre.clone()
    s_first = spart.clone() if with_s else None
    # second call into the same buffers: the same bits
    coda.coda_gemm_swiglu_bwd_overlap(dev(dOut), dev(Wd), dev(pre), dPre=dpre, spart=spart, want_spart=with_s)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), dpre.view(torch.int16)), "second call differs"
    if with_s:
        assert torch.equal(s_first, spart), "second call's spart differs"
    da = O.gemm(dOut.f64(), Wd.f64().T)
    ref = O.swiglu_bwd(da, pre.f64())
    assert_close(f64(dpre), ref, "dpre")
    if with_s:
        assert_close(spart.double().cpu().numpy(), spart_ref(ref, pre.f64(), np_), "spart")


def test_swiglu_bwd_deferred_8b_rows():
    """The 8B-like MLP shape with ragged tokens and features (8152 x 14328,
    K = 4096, one unit per k-tile, 7 rounds): every column of a seeded sample
    of rows against the oracle, spart included."""
    M, F, N = 8152, 14328, 4096
    coda = C()
    assert coda.coda_swiglu_bwd_units(M, F, N, cus()) == 1
    say(f"case: deferred swiglu bwd M={M} F={F} N={N} sampled rows")
    dOut = S.normal_bf16(7101, (M, N))
    Wd = S.normal_bf16(7102, (F, N), std=F ** -0.5)
    pre = S.normal_bf16(7103, (M, 2 * F), std=2.0)
    dpre = torch.full((M, 2 * F), float("nan"), dtype=torch.bfloat16, device="cuda")
    dpre, spart = coda.coda_gemm_swiglu_bwd_overlap(dev(dOut), dev(Wd), dev(pre), dPre=dpre)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(dpre.float()).all()), "dPre has elements left unwritten"
    rng = np.random.default_rng(11)
    rows = np.array(sorted(set([0, 1, 31, 32, 255, 256, 4095, M - 40, M - 1] + rng.choice(M, 16, replace=False).tolist())))
    idx = torch.as_tensor(rows, device="cuda")
    pre_r = pre.f64()[rows]
    ref = O.swiglu_bwd(O.gemm(dOut.f64()[rows], Wd.f64().T), pre_r)
    assert_close(f64(dpre[idx]), ref, "dpre rows")
    assert_close(spart[idx].double().cpu().numpy(), spart_ref(ref, pre_r, coda.coda_nparts(F)), "spart rows")


def _random_shapes(n=4, seed=2024):
    """Seeded shapes (M in [3000, 9000), F and N multiples of 8) that the plan
    routes to the overlapped kernel on this device: tile counts that leave
    some workgroups one tile more than others."""
    coda = C()
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.integers(3000, 9000))
        F = int(rng.integers(300, 1400)) * 8
        N = int(rng.integers(256, 700)) * 8
        if coda.coda_swiglu_bwd_units(M, F, N, cus()) > 0:
            out.append((M, F, N))
    return out


def test_swiglu_bwd_overlap_random_shapes():
    """Every column of a seeded sample of rows against the oracle, and the s
    partials, at four random shapes the plan accepts."""
    coda = C()
    for k, (M, F, N) in enumerate(_random_shapes()):
        say(f"case: overlap random shape {k}: M={M} F={F} N={N} units={coda.coda_swiglu_bwd_units(M, F, N, cus())}")
        seed = 7200 + 10 * k
        dOut = S.normal_bf16(seed, (M, N))
        Wd = S.normal_bf16(seed + 1, (F, N), std=F ** -0.5)
        pre = S.normal_bf16(seed + 2, (M, 2 * F), std=2.0)
        dpre = torch.full((M, 2 * F), float("nan"), dtype=torch.bfloat16, device="cuda")
        dpre, spart = coda.coda_gemm_swiglu_bwd_overlap(dev(dOut), dev(Wd), dev(pre), dPre=dpre)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(dpre.float()).all()), "dPre has elements left unwritten"
        rng = np.random.default_rng(seed)
        rows = np.array(sorted(set([0, 255, 256, M - 1] + rng.choice(M, 12, replace=False).tolist())))
        idx = torch.as_tensor(rows, device="cuda")
        pre_r = pre.f64()[rows]
        ref = O.swiglu_bwd(O.gemm(dOut.f64()[rows], Wd.f64().T), pre_r)
        assert_close(f64(dpre[idx]), ref, "dpre rows")
        assert_close(spart[idx].double().cpu().numpy(), spart_ref(ref, pre_r, coda.coda_nparts(F)), "spart rows")
        del dOut, Wd, pre, dpre, spart
