"""The tile-timeline build (libcoda_timeline.so): the same GEMM results as
libcoda.so, bit for bit, and well-formed per-wave records; for the persistent
(epilogue-overlapped) SwiGLU backward, one record per wave and tile."""

import ctypes
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gemm_epilogue_transformer_mainloop_amd import coda  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def TL():
    assert torch.cuda.is_available()
    assert os.path.exists(coda.TIMELINE_LIB_PATH), "libcoda_timeline.so is not built (build.py --timeline)"
    lib = ctypes.CDLL(coda.TIMELINE_LIB_PATH)
    for name in ("coda_gemm", "coda_timeline_set", "coda_timeline_words", "coda_gemm_swiglu_bwd_overlap"):
        res, args = coda._SIGS[name]
        getattr(lib, name).restype = res
        getattr(lib, name).argtypes = args
    return lib


def _gemm(lib, X, W, Y):
    M, K = X.shape
    N = W.shape[1]
    st = lib.coda_gemm(ctypes.c_void_p(X.data_ptr()), X.stride(0), ctypes.c_void_p(W.data_ptr()), W.stride(0),
                       ctypes.c_void_p(Y.data_ptr()), Y.stride(0), M, N, K,
                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, coda.status_str(st)


# (M, N, K): a small problem run in 256 x 128 tiles, a ragged multi-round one in 256 x 256 tiles
@pytest.mark.parametrize("M,N,K", [(512, 512, 1024), (2000, 1288, 520)])
def test_timeline_records_and_results(TL, M, N, K):
    g = torch.Generator().manual_seed(7)
    X = torch.randn(M, K, generator=g).to(torch.bfloat16).cuda()
    W = (torch.randn(K, N, generator=g) * K ** -0.5).to(torch.bfloat16).cuda()
    ref = coda.coda_gemm(X, W)
    words = TL.coda_timeline_words()
    assert words == 12
    cap = 4096
    buf = torch.zeros((cap, words), dtype=torch.int64, device="cuda")
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    assert TL.coda_timeline_set(ctypes.c_void_p(buf.data_ptr()), cap) == 0
    _gemm(TL, X, W, Y)
    torch.cuda.synchronize()
    assert TL.coda_timeline_set(None, 0) == 0
    assert torch.equal(Y.view(torch.int16), ref.view(torch.int16))

    rec = buf.cpu().numpy()
    n = int((rec[:, 0] != 0).sum())
    assert n > 0 and n % 4 == 0
    assert (rec[:n, 0] != 0).all() and (rec[n:] == 0).all()   # dense from record 0, nothing past the grid
    r = rec[:n]
    nk = (K + 63) // 64
    assert (r[:, 9] == nk).all()
    assert set(np.unique(r[:, 8])) <= {128, 256}
    # the tiles (one record per wave, four waves each) cover the output: 256 features x their token width
    tiles = r[::4]
    assert (tiles[:, 8] * 256).sum() >= M * N
    assert ((r[:, 8].reshape(-1, 4) == tiles[:, 8:9]).all())
    for c in (0, 4):  # reference clock, shader clock: tile start <= k-loop start <= k-loop end <= epilogue end
        assert (np.diff(r[:, c:c + 4], axis=1) >= 0).all()
    # the shader clock runs between 0.5 and 3 GHz over the k-loop
    kl = (r[:, 6] - r[:, 5]) / np.maximum(r[:, 2] - r[:, 1], 1) * 0.1
    assert ((kl > 0.5) & (kl < 3.0)).mean() > 0.9, np.median(kl)

    # uninstalled: a further launch writes nothing
    buf.zero_()
    _gemm(TL, X, W, Y)
    torch.cuda.synchronize()
    assert int(buf.count_nonzero()) == 0
    assert torch.equal(Y.view(torch.int16), ref.view(torch.int16))


def test_timeline_persistent_overlap(TL):
    """coda_gemm_swiglu_bwd_overlap (a persistent kernel: 256 workgroups run
    400 tiles) in the timeline build: libcoda.so's bits, and records kept per
    tile (record 4 t + w for wave w of tile t), all 400 x 4 of them."""
    M, F, N = 5000, 5000, 2048
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert coda.coda_swiglu_bwd_units(M, F, N, cus) == 2
    g = torch.Generator().manual_seed(9)
    dOut = torch.randn(M, N, generator=g).to(torch.bfloat16).cuda()
    Wd = (torch.randn(F, N, generator=g) * F ** -0.5).to(torch.bfloat16).cuda()
    pre = torch.randn(M, 2 * F, generator=g).to(torch.bfloat16).cuda()
    ref, sref = coda.coda_gemm_swiglu_bwd_overlap(dOut, Wd, pre)
    words = TL.coda_timeline_words()
    cap = 4096
    buf = torch.zeros((cap, words), dtype=torch.int64, device="cuda")
    dpre = torch.empty(M, 2 * F, dtype=torch.bfloat16, device="cuda")
    sp = torch.empty_like(sref)
    assert TL.coda_timeline_set(ctypes.c_void_p(buf.data_ptr()), cap) == 0
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    st = TL.coda_gemm_swiglu_bwd_overlap(ptr(dOut), N, ptr(Wd), N, ptr(pre), 2 * F, ptr(dpre), 2 * F, ptr(sp),
                                         M, F, N, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, coda.status_str(st)
    torch.cuda.synchronize()
    assert TL.coda_timeline_set(None, 0) == 0
    assert torch.equal(dpre.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(sp, sref)
    tiles = -(-F // 256) * -(-M // 256)
    rec = buf.cpu().numpy()
    assert (rec[:4 * tiles, 0] != 0).all() and (rec[4 * tiles:] == 0).all()
    r = rec[:4 * tiles]
    assert (r[:, 8] == 256).all() and (r[:, 9] == N // 64).all()
    for c in (0, 4):
        assert (np.diff(r[:, c:c + 4], axis=1) >= 0).all()
    # a workgroup's next tile (t + grid) starts after its tile t ended, on the same compute unit
    grid = (cus // 8) * 8
    t = np.arange(tiles - grid)
    assert (r[4 * (t + grid), 0] >= r[4 * t, 3]).all()
    assert (r[4 * (t + grid), 10] == r[4 * t, 10]).all() and (r[4 * (t + grid), 11] == r[4 * t, 11]).all()
