"""The GEMM writes its M x N outputs and nothing else.

Y is a view of the first M rows and N columns of a larger buffer whose other
bytes (256 rows below it, and the columns between N and the row stride) hold a
sentinel pattern; after the call the sentinel must be intact and the view must
equal the output of the same call into a plain contiguous tensor. The extra
rows cover a whole tile of every kernel, so a kernel that wrote rows of its
last, ragged tile past M would write into the sentinel (inside the buffer)
and fail here. Covered: the wide 256 x 256 kernel with ragged last m- and
n-tiles, the 128 x 256 kernel, and split-K decode, in bf16 and fp32, with the
row stride equal to N and larger.
"""
import numpy as np
import pytest
import torch

from mxfp4_w4a4_post_amd import binding
from parity_util import log, row_major_to_gemm_layout

pytestmark = pytest.mark.gpu

GUARD_ROWS = 256
# fp32 and bf16 NaN patterns that no GEMM output equals bit for bit
SENTINEL = {torch.float32: (torch.int32, 0x7FC0ABCD), torch.bfloat16: (torch.int16, 0x7FAB)}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    binding.load_library()
    return torch.device("cuda:0")


def _packed(rng, rows, K, dev):
    c = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    s = rng.integers(118, 136, size=(rows, K // 32), dtype=np.uint8)
    tc, ts = row_major_to_gemm_layout(c, s)
    return binding.Packed(torch.from_numpy(tc).to(dev), torch.from_numpy(ts).to(dev), rows, K)


@pytest.mark.parametrize("M,N,K,extra,what", [
    (4100, 4104, 1024, 0, "wide, ragged m- and n-tiles"),
    (3000, 6152, 1024, 8, "wide, ragged, row stride N + 8"),
    (1000, 3000, 1024, 8, "128 x 256 tiles, ragged, row stride N + 8"),
    (40, 4096, 8192, 0, "decode, split-K"),
])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_gemm_writes_only_its_output(dev, M, N, K, extra, what, out_dtype):
    log("output bounds %s M=%d N=%d K=%d ldy=%d %s" % (what, M, N, K, N + extra, out_dtype))
    rng = np.random.default_rng(M + N + K + extra)
    pa, pw = _packed(rng, M, K, dev), _packed(rng, N, K, dev)
    ref = binding.linear_plain_gemm(pa, pw, out_dtype=out_dtype)
    itype, pattern = SENTINEL[out_dtype]
    buf = torch.full((M + GUARD_ROWS, N + extra), pattern, dtype=itype, device=dev)
    y = buf.view(out_dtype)[:M, :N]
    binding.linear_plain_gemm(pa, pw, out=y)
    torch.cuda.synchronize()
    assert torch.equal(y, ref), "%s: output differs from the contiguous call" % what
    below = buf[M:]
    assert bool((below == pattern).all()), "%s: %d values written below row M" % (what, int((below != pattern).sum()))
    if extra:
        right = buf[:M, N:]
        assert bool((right == pattern).all()), "%s: %d values written past column N" % (
            what, int((right != pattern).sum()))
