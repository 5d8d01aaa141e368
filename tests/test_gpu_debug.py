"""The host-side switches of the C ABI on a GPU: CODA_DEBUG's extent check
rejects an argument that leaves its device allocation before anything is
launched, and CODA_LOG prints each call.  Both switches are read once per
process, so the checks run in a child process with the variables set."""

import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys, torch
sys.path.insert(0, sys.argv[1])
from gemm_epilogue_transformer_mainloop_amd import coda
L = coda.lib()
# a valid call: the extents of real tensors pass, and the result is the GEMM
X = torch.randint(-2, 3, (96, 64), device="cuda").to(torch.bfloat16)
W = torch.randint(-2, 3, (64, 128), device="cuda").to(torch.bfloat16)
Y = coda.coda_gemm(X, W)
torch.cuda.synchronize()
assert torch.equal(Y.float(), X.float() @ W.float()), "gemm result"
# an output view whose extent leaves its allocation: the first large
# allocation of this process (a fresh 16 MiB block) holding a 1 x 128 view,
# presented as 200000 rows (51 MB).  The extent query must flag it on its
# own before the entry point is called with it.
big = torch.empty(8 << 20, dtype=torch.bfloat16, device="cuda")
small = big[:128]
MB = 200000
bad_bytes = (MB - 1) * 128 * 2 + 128 * 2
assert coda.coda_debug_extent(small.data_ptr(), bad_bytes) == 7, "extent query"
assert coda.coda_debug_extent(small.data_ptr(), 128 * 2) == 0, "extent query (valid)"
Xb = torch.zeros(MB, 64, dtype=torch.bfloat16, device="cuda")
st = L.coda_gemm(coda._ptr(Xb), 64, coda._ptr(W), 128, coda._ptr(small), 128, MB, 128, 64, None)
torch.cuda.synchronize()
print("STATUS", st, flush=True)
'''


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_debug_and_log_switches():
    print("case: CODA_DEBUG=1 CODA_LOG=1 child process", flush=True)
    env = dict(os.environ, CODA_DEBUG="1", CODA_LOG="1")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], capture_output=True, text=True, env=env,
                       timeout=240)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0
    assert "STATUS 7" in r.stdout
    assert "[coda] coda_gemm(M=96 N=128 K=64)" in r.stderr
    assert "[coda] coda_gemm(M=200000 N=128 K=64)" in r.stderr


def test_debug_extent_query():
    from gemm_epilogue_transformer_mainloop_amd import coda

    t = torch.empty(4096, dtype=torch.float32, device="cuda")
    assert coda.coda_debug_extent(t.data_ptr(), 4096 * 4) == 0
    assert coda.coda_debug_extent(t.data_ptr() + 64, 4000 * 4) == 0
    assert coda.coda_debug_extent(t.data_ptr(), 1 << 40) == 7
