"""C-ABI checks that need no GPU: the library loads, exports every function
the public headers (include/coda.h, coda_unfused.h, coda_probe.h) declare,
and rejects bad arguments before any device call."""

import ctypes
import os

import pytest

from gemm_epilogue_transformer_mainloop_amd import coda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(coda.LIB_PATH):
        from gemm_epilogue_transformer_mainloop_amd import build

        build.build()
    return coda.lib()


def test_exports_every_header_function(L):
    names = coda.header_functions()
    assert len(names) >= 20
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    # the binding covers the whole header
    assert set(names) == set(coda._SIGS), set(names) ^ set(coda._SIGS)


def test_status_strings(L):
    for s in range(8):
        assert coda.status_str(s) and coda.status_str(s) != "unknown status"
    assert coda.status_str(8) == "unknown status"
    assert coda.status_str(0) == "ok"
    assert L.coda_version().decode().startswith("coda-gfx950")


def test_queries(L):
    assert coda.coda_nparts(2048) == 16
    assert coda.coda_nparts(1) == 1
    assert coda.coda_nparts(128256) == 1002
    assert coda.coda_nparts(0) == 0
    assert coda.coda_mparts(8192) == 64
    assert coda.coda_mparts(129) == 2
    M, V = 8192, 128256
    assert coda.coda_lmhead_ce_workspace(M, V) == (2 * M * 1002 + 2 * M) * 4
    assert coda.coda_lmhead_ce_bwd_workspace(M, V, 2048) == 256 * V * 2
    assert coda.coda_lmhead_ce_bwd_workspace(100, V, 2048) == 100 * V * 2


def test_tile_split(L):
    """Tile-count quantization plan (host logic; 256 compute units)."""
    cus = 256
    # QKV 8192 x 3072: 384 big tiles = 1.5 rounds -> 8 feature tiles big, 4 in half tiles
    assert coda.coda_tile_split(3072, 8192, cus) == 8
    # whole rounds stay big: 2048, 16384, 8192 and 14336 features at 8192 tokens
    for F in (2048, 4096, 8192, 14336, 16384, 28672):
        assert coda.coda_tile_split(F, 8192, cus) == 0, F
    # LM head: 16032 tiles, the partial last round costs < 1%, no split
    assert coda.coda_tile_split(128256, 8192, cus) == 0
    # one tile, or a single feature tile: nothing to split
    assert coda.coda_tile_split(256, 256, cus) == 0
    assert coda.coda_tile_split(200, 1 << 20, cus) == 0
    # 3 x 96 = 288 tiles (2 rounds) -> 2 big feature tiles (1 round) + 192 half tiles
    assert coda.coda_tile_split(712, 24500, cus) == 2
    # 4 x 96 = 384 tiles: the half tiles would need 2 rounds, no gain worth it
    assert coda.coda_tile_split(776, 24500, cus) == 0
    # unknown CU count or empty problems
    assert coda.coda_tile_split(3072, 8192, 0) == 0
    assert coda.coda_tile_split(0, 8192, cus) == 0
    assert coda.coda_tile_split(3072, 0, cus) == 0
    # other CU counts: the plan always lowers the modelled round count
    for cus2 in (32, 80, 304):
        for F in (768, 3072, 5120):
            s = coda.coda_tile_split(F, 8192, cus2)
            nF, nT = -(-F // 256), 32
            base = -(-nF * nT // cus2)
            if s:
                assert 0 < s < nF
                cost = -(-s * nT // cus2) + 0.6 * -(-(nF - s) * 64 // cus2)
                assert cost <= base - 0.2


# Fake, 256-byte aligned, never dereferenced: every call below fails validation first.
A16 = ctypes.c_void_p(0x100000)
A16b = ctypes.c_void_p(0x200000)
A16c = ctypes.c_void_p(0x300000)
MIS = ctypes.c_void_p(0x100002)


def test_gemm_validation(L):
    f = L.coda_gemm
    assert f(None, 64, A16, 64, A16b, 64, 16, 64, 64, None) == 1               # NULL X
    assert f(A16, 64, A16b, 64, A16c, 64, -1, 64, 64, None) == 2               # M < 0
    assert f(A16, 32, A16b, 64, A16c, 64, 16, 64, 64, None) == 2               # ldx < K
    assert f(A16, 64, A16b, 64, A16c, 64, 16, 60, 64, None) == 2               # N % 8
    assert f(MIS, 64, A16b, 64, A16c, 64, 16, 64, 64, None) == 3               # misaligned
    assert f(A16, 68, A16b, 64, A16c, 64, 16, 64, 64, None) == 3               # ld % 8
    assert f(A16, 64, A16b, 64, A16c, 64, 0, 64, 64, None) == 0                # empty M: no-op


def test_fused_validation(L):
    # res_sumsq: H2 without gamma
    assert L.coda_gemm_res_sumsq(A16, 64, A16b, 64, None, 0, None, A16c, 64, A16, 64, None,
                                 16, 64, 64, None) == 1
    # row_rms: nparts < 1
    assert L.coda_row_rms(A16, 0, 16, 64, ctypes.c_float(1e-6), A16b, None) == 2
    # rope: n_rope not a multiple of head_dim
    assert L.coda_gemm_rope(A16, 64, A16b, 128, None, A16c, ctypes.c_float(1e4), 64, 96, A16, 128,
                            16, 128, 64, None) == 4
    # rope: odd head_dim
    assert L.coda_gemm_rope(A16, 64, A16b, 128, None, A16c, ctypes.c_float(1e4), 63, 0, A16, 128,
                            16, 128, 64, None) == 4
    # swiglu: NULL act
    assert L.coda_gemm_swiglu(A16, 64, A16b, 64, None, None, 64, None, 0, 16, 32, 64, None) == 1
    # lmhead: workspace too small
    assert L.coda_lmhead_ce(A16, 64, A16b, 128, A16c, A16, None, None, A16b, 16, 16, 128, 64,
                            None) == 6
    # swiglu_bwd: ldp < 2F
    assert L.coda_gemm_swiglu_bwd(A16, 64, A16b, 64, A16c, 64, A16, 128, None, 16, 64, 64,
                                  None) == 2
    # rowscale_bwd: NULL s
    assert L.coda_gemm_rowscale_bwd(A16, 64, A16b, 64, A16c, 64, A16, A16b, None, None, 0, A16c,
                                    64, None, 0, None, 16, 64, 64, None) == 1
    # wgrad: misaligned fp32 ld
    assert L.coda_gemm_wgrad(A16, 64, A16b, 64, A16c, 66, 16, 64, 64, 0, None) == 3
    # lmhead bwd: no workspace
    assert L.coda_lmhead_ce_bwd(A16, 64, A16b, 128, A16c, A16, ctypes.c_float(1.0), A16b, 64, A16c,
                                128, None, 0, 16, 128, 64, None) == 6
    # col_reduce: mparts < 1
    assert L.coda_col_reduce(A16, 0, 64, A16b, None) == 2
    # lmhead with stored logits: NULL logits, then ldl < V
    assert L.coda_lmhead_ce_logits(A16, 64, A16b, 128, A16c, A16, None, None, None, 128, A16b,
                                   1 << 20, 16, 128, 64, None) == 1
    assert L.coda_lmhead_ce_logits(A16, 64, A16b, 128, A16c, A16, None, None, A16c, 64, A16b,
                                   1 << 20, 16, 128, 64, None) == 2
    # lmhead bwd from stored logits: NULL logits
    assert L.coda_lmhead_ce_bwd_logits(A16, 64, A16b, 128, A16c, A16, ctypes.c_float(1.0), None,
                                       128, A16b, 64, A16c, 128, 16, 128, 64, None) == 1


def test_unfused_validation(L):
    F = ctypes.c_float
    assert coda.coda_unfused_rmsnorm_bwd_parts(8192) == 512
    assert coda.coda_unfused_rmsnorm_bwd_parts(17) == 2
    assert coda.coda_unfused_rmsnorm_bwd_parts(0) == 0
    # add: N % 8
    assert L.coda_unfused_add(A16, 64, A16b, 64, A16c, 64, 16, 60, None) == 2
    # add_rmsnorm: d too wide for one workgroup per row
    assert L.coda_unfused_add_rmsnorm(A16, 16384, None, 0, A16b, F(1e-6), A16c, 16384, A16, 16384, A16b,
                                      4, 16384, None) == 4
    # add_rmsnorm: NULL r
    assert L.coda_unfused_add_rmsnorm(A16, 64, None, 0, A16b, F(1e-6), A16c, 64, A16, 64, None, 4, 64,
                                      None) == 1
    # rope: n_rope beyond N, odd head_dim
    assert L.coda_unfused_rope(A16, 64, A16b, F(1e4), 64, 128, 0, 4, 64, None) == 4
    assert L.coda_unfused_rope(A16, 64, A16b, F(1e4), 7, 0, 0, 4, 64, None) == 4
    # swiglu: ldp < 2F; misaligned act
    assert L.coda_unfused_swiglu(A16, 64, A16b, 64, 4, 64, None) == 2
    assert L.coda_unfused_swiglu(A16, 128, MIS, 64, 4, 64, None) == 3
    # swiglu_bwd: NULL pre
    assert L.coda_unfused_swiglu_bwd(A16, 64, None, 128, A16b, 128, 4, 64, None) == 1
    # rmsnorm_bwd: misaligned gpart
    assert L.coda_unfused_rmsnorm_bwd(A16, 64, A16b, 64, A16c, A16, None, 0, A16b, 64, MIS, 4, 64,
                                      None) == 3
    # cross entropy: V % 8, ld < V
    assert L.coda_unfused_cross_entropy(A16, 64, A16b, A16c, A16, None, 4, 60, None) == 2
    assert L.coda_unfused_cross_entropy_bwd(A16, 32, A16b, A16c, F(1.0), A16, 64, 4, 64, None) == 2
    # empty M: no-op
    assert L.coda_unfused_cross_entropy(A16, 64, A16b, A16c, A16, None, 0, 64, None) == 0


def test_no_kernel_spills():
    """Every kernel of the built library runs without scratch memory (the build
    records the compiler's resource report next to the library)."""
    import json
    import os
    from gemm_epilogue_transformer_mainloop_amd import build as B
    if not os.path.exists(B.RESOURCES):
        pytest.skip("library not built with the resource report")
    res = json.load(open(B.RESOURCES))
    gemm = {k: v for k, v in res.items() if "gemm_epi_kernel" in k}
    assert len(gemm) >= 20
    for name, v in res.items():
        assert v["scratch"] == 0 and v["vgpr_spill"] == 0, name
    # the main loop holds the 128x128 wave tile in the 256 accumulation
    # registers (also in the tile-count split kernels, whose second tile
    # shape, 256x128, holds 128x64)
    split = [k for k in gemm if "gemm_epi_kernel_split" in k]
    assert split, "no tile-count split kernels"
    assert all(v["agprs"] == 256 for v in gemm.values())
    assert all(v["lds"] <= 160 * 1024 for v in res.values())


def test_probe_validation(L):
    out = A16
    assert L.coda_probe_mfma(0, 10, out, None) == 2          # no workgroups
    assert L.coda_probe_mfma(4, 0, out, None) == 2           # no iterations
    assert L.coda_probe_mfma(4, 10, None, None) == 1         # NULL output


def test_debug_extent_null_or_empty(L):
    # a NULL pointer or an empty extent passes without a device query
    assert L.coda_debug_extent(None, 1 << 20) == 0
    assert L.coda_debug_extent(A16, 0) == 0


def test_noalloc_limits(L):
    """coda_lmhead_ce_noalloc: the array covers the full LM-head workload;
    a larger need or a bad argument is refused before any device call."""
    assert L.coda_lmhead_ce_noalloc_max_bytes() == 64 << 20
    assert coda.coda_lmhead_ce_workspace(8192, 128256) <= L.coda_lmhead_ce_noalloc_max_bytes()
    # V = 200000 at M = 8192 needs (2 * 8192 * 1563 + 2 * 8192) * 4 bytes = 102 MB
    assert L.coda_lmhead_ce_noalloc(A16, 64, A16b, 200000, A16c, A16, None, None, 8192, 200000, 64, None) == 6
    assert L.coda_lmhead_ce_noalloc(None, 64, A16b, 128, A16c, A16, None, None, 16, 128, 64, None) == 1
    assert L.coda_lmhead_ce_noalloc(A16, 64, A16b, 128, A16c, A16, None, None, 16, 124, 64, None) == 2
    # no rows: nothing to do
    assert L.coda_lmhead_ce_noalloc(A16, 64, A16b, 128, A16c, A16, None, None, 0, 128, 64, None) == 0


def test_vchunk_workspace(L):
    M, V, d = 8192, 128256, 2048
    # one chunk of 8192 columns (134 MB) + the fp32 dH accumulator (64 MB)
    assert coda.coda_lmhead_ce_bwd_vchunk_workspace(M, V, d, 8192) == M * 8192 * 2 + M * d * 4
    # a chunk as wide as the vocabulary needs no accumulator
    assert coda.coda_lmhead_ce_bwd_vchunk_workspace(M, V, d, 131072) == M * V * 2
    assert coda.coda_lmhead_ce_bwd_vchunk_workspace(M, V, d, 100) == 0   # vchunk % 8
    assert coda.coda_lmhead_ce_bwd_vchunk_workspace(0, V, d, 8192) == 0
    # workspace too small, then a misaligned one: refused before any device call
    f = L.coda_lmhead_ce_bwd_vchunk
    assert f(A16, 64, A16b, 128, A16c, A16, ctypes.c_float(1.0), A16b, 64, A16c, 128, A16, 16, 16, 128, 64, 64,
             None) == 6
    assert f(A16, 64, A16b, 128, A16c, A16, ctypes.c_float(1.0), A16b, 64, A16c, 128, ctypes.c_void_p(0x100010),
             1 << 20, 16, 128, 64, 64, None) == 6
    assert f(A16, 64, A16b, 128, A16c, A16, ctypes.c_float(1.0), A16b, 64, A16c, 128, A16, 1 << 20, 16, 128, 64, 60,
             None) == 2


def test_timeline_default_build(L):
    """The default library compiles no timeline: installing one is refused."""
    assert L.coda_timeline_words() == 12
    assert L.coda_timeline_set(None, 0) == 4
    assert L.coda_timeline_set(A16, 1024) == 4


def test_timeline_build_validation():
    """libcoda_timeline.so: same exports; the buffer is checked before it is installed."""
    from gemm_epilogue_transformer_mainloop_amd import build

    path = coda.TIMELINE_LIB_PATH
    if not os.path.exists(path):
        build.build(timeline=True)
    T = ctypes.CDLL(path)
    for name in coda.header_functions():
        assert hasattr(T, name), name
    T.coda_timeline_set.argtypes = [ctypes.c_void_p, ctypes.c_int]
    assert T.coda_timeline_words() == 12
    assert T.coda_timeline_set(None, 5) == 2                       # NULL with records
    assert T.coda_timeline_set(A16, -1) == 2
    assert T.coda_timeline_set(ctypes.c_void_p(0x100004), 8) == 3  # not 8-byte aligned
    assert T.coda_timeline_set(A16, 8) == 0
    assert T.coda_timeline_set(None, 0) == 0                       # uninstall


def test_swiglu_bwd_overlap_rejects_aliasing(L):
    """The epilogue-overlapped SwiGLU backward parks da in dPre before its
    inputs are all read: a dPre sharing bytes with Pre, dOut or Wd is refused
    before any device call; disjoint buffers pass this check (and fail later
    only on the missing device or the fake pointers' other checks)."""
    f = L.coda_gemm_swiglu_bwd_overlap
    M, F, N = 16, 64, 64
    big = ctypes.c_void_p(0x10000000)
    # dPre == Pre (in place), dPre inside dOut, dPre overlapping Wd's last row
    assert f(A16, N, A16b, N, big, 2 * F, big, 2 * F, None, M, F, N, None) == 2
    assert f(big, 4096, A16b, N, A16c, 2 * F, ctypes.c_void_p(0x10000000 + 2 * 4096), 2 * F, None,
             M, F, N, None) == 2
    wd_end = 0x20000000 + 2 * ((F - 1) * N + N)
    assert f(A16, N, ctypes.c_void_p(0x20000000), N, A16c, 2 * F, ctypes.c_void_p(wd_end - 16), 2 * F, None,
             M, F, N, None) == 2
    # adjacent but disjoint: not refused for aliasing
    assert f(A16, N, ctypes.c_void_p(0x20000000), N, A16c, 2 * F, ctypes.c_void_p(wd_end), 2 * F, None,
             M, F, N, None) != 2


def test_swiglu_bwd_units(L):
    """The deferred SwiGLU-backward plan: 1 unit per k-tile from 64 k-tiles,
    2 from 32, only for more than one round of 256 x 256 tiles that no tile
    split touches."""
    f = coda.coda_swiglu_bwd_units
    assert f(8192, 14336, 4096, 256) == 1     # the 8B-like MLP: 1792 tiles, 64 k-tiles
    assert f(8192, 8192, 2048, 256) == 2      # the 1B-like MLP: 1024 tiles, 32 k-tiles
    assert f(5000, 5000, 4104, 256) == 1      # ragged: 400 tiles, 65 k-tiles
    assert f(5000, 5000, 2056, 256) == 2
    assert f(8192, 8192, 1024, 256) == 0      # 16 k-tiles cannot carry 64 units
    assert f(512, 1024, 4096, 256) == 0       # a single round (all 256 x 128 tiles)
    assert f(4096, 4096, 4096, 256) == 0      # exactly one round: nothing to overlap
    assert f(8192, 3072, 2048, 256) == 0 and coda.coda_tile_split(3072, 8192, 256) > 0   # feature split
    assert f(9000, 8192, 2056, 256) == 0 and coda.coda_tile_split_tokens(8192, 9000, 256) > 0  # token split
    assert f(8192, 14336, 4096, 4) == 0 and f(0, 14336, 4096, 256) == 0 and f(8192, 14336, 0, 256) == 0


def test_tile_split_tokens(L):
    """The token split: only when neither the feature split nor the all-half-
    tile plan applies, the largest token-tile count that saves 0.2 rounds."""
    f = coda.coda_tile_split_tokens
    assert f(4096, 14336, 256) == 48      # weight gradient dWd: 3.5 rounds -> 3 + 0.6
    assert f(4096, 14000, 256) == 48      # ragged: 47 and 48 cost the same; the larger
    assert f(28672, 8192, 256) == 0       # 14 whole rounds
    assert f(3072, 8192, 256) == 0 and coda.coda_tile_split(3072, 8192, 256) == 8   # the feature split
    assert f(512, 1000, 256) == 0         # 8 tiles: all 256 x 128
    assert f(4096, 14336, 0) == 0 and f(0, 14336, 256) == 0 and f(4096, 0, 256) == 0
    # the cost model, restated: big rounds + 0.6 x half-tile rounds, 0.2 rounds saved
    cdiv = lambda a, b: -(-a // b)
    for F, T in [(4096, 14336), (4096, 14000), (1000, 9000), (2304, 30000)]:
        t = f(F, T, 256)
        if t:
            nTF, nTT = cdiv(F, 256), cdiv(T, 256)
            cost = cdiv(nTF * t, 256) + 0.6 * cdiv(nTF * cdiv(T - 256 * t, 128), 256)
            assert cost <= cdiv(nTF * nTT, 256) - 0.2
