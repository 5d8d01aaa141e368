"""coda_lmhead_ce_noalloc, the LM-head statistics call for callers that
cannot allocate, against coda_lmhead_ce (the same computation with a
caller-provided workspace), called through the C ABI.

Two calls in a row on one GPU share the library's device array: the first at
the full LM-head shape (M = 8192, V = 128256, d = 2048: its 65.8 MB of
partials fill most of the 64 MiB array), the second smaller, so that a stale
entry of the first call would show.  Each result must equal the workspace
form's bit for bit, and meet the oracle on sampled rows.
"""

import ctypes

import numpy as np
import pytest
import torch

from gpu_util import LOSS_RTOL, assert_close, dev, f64, say
from gemm_epilogue_transformer_mainloop_amd import synth as S
from oracle import coda_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def coda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gemm_epilogue_transformer_mainloop_amd import coda as c

    c.lib()
    return c


def run_case(coda, seed, M, V, d, oracle_rows):
    say(f"case: lmhead_ce_noalloc vs lmhead_ce M={M} V={V} d={d} seed={seed}")
    p = S.lmhead_inputs(seed, M, d, V)
    H, W, lab = dev(p["h"]), dev(p["W"]), dev(p["labels"])
    lse0, lr0, lm0 = coda.coda_lmhead_ce(H, W, lab)
    lse1 = torch.full((M,), float("nan"), device="cuda")
    lr1 = torch.full((M,), float("nan"), device="cuda")
    lm1 = torch.full((1,), float("nan"), device="cuda")
    L = coda.lib()
    st = L.coda_lmhead_ce_noalloc(ctypes.c_void_p(H.data_ptr()), H.stride(0), ctypes.c_void_p(W.data_ptr()),
                                  W.stride(0), ctypes.c_void_p(lab.data_ptr()), ctypes.c_void_p(lse1.data_ptr()),
                                  ctypes.c_void_p(lr1.data_ptr()), ctypes.c_void_p(lm1.data_ptr()), M, V, d,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, coda.status_str(st)
    torch.cuda.synchronize()
    assert torch.equal(lse1, lse0) and torch.equal(lr1, lr0) and torch.equal(lm1, lm0)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(seed).choice(M, oracle_rows, replace=False)]))
    lse_r, loss_r, _ = O.lmhead_ce(p["h"].f64()[rows], p["W"].f64(), p["labels"][rows])
    assert_close(f64(lse1)[rows], lse_r, "lse (noalloc)")
    assert_close(f64(lr1)[rows], loss_r, "loss_row (noalloc)")
    if oracle_rows >= M - 2:  # every row: the mean against the oracle's
        _, _, mean_r = O.lmhead_ce(p["h"].f64(), p["W"].f64(), p["labels"])
        assert abs(float(lm1.item()) - mean_r) <= LOSS_RTOL * abs(mean_r)
    return lse1


def test_noalloc_two_calls_second_smaller(coda):
    assert coda.lib().coda_lmhead_ce_noalloc_max_bytes() == 64 << 20
    run_case(coda, 4, 8192, 128256, 2048, oracle_rows=10)
    run_case(coda, 41, 700, 5000, 256, oracle_rows=698)

