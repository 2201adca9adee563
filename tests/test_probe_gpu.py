"""The measurement probes compute what they claim, so the rates that bench.py
derives from them count the work they say.

MFMA probe: with every operand byte 0x22 (E2M1 1.0 in each nibble) and every
scale 2^0, each 32x32x64 MFMA adds 64 to every accumulator element, so after
`iters` rounds a thread's sum over its 8 accumulators of 16 elements is
8 * 16 * 64 * iters exactly (fp32 holds these integers exactly). Random
operand bytes must give a finite result.

Read probe: every 16-byte element of the buffer is read by exactly one
thread, which folds it into its word by XOR, so the XOR of all the words
written equals the XOR of every 32-bit word of the buffer, whatever the grid.
"""
import numpy as np
import pytest
import torch

from mxfp4_w4a4_post_amd import binding
from parity_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    binding.load_library()
    return torch.device("cuda:0")


@pytest.mark.parametrize("workgroups,iters", [(1, 1), (3, 10), (256, 37)])
def test_mfma_probe_counts_its_work(dev, workgroups, iters):
    log("mfma probe workgroups=%d iters=%d" % (workgroups, iters))
    ops = torch.full((binding.MFMA_PROBE_OPERAND_BYTES,), 0x22, dtype=torch.uint8, device=dev)
    out = torch.empty(workgroups * 256, dtype=torch.float32, device=dev)
    binding.mfma_probe(ops, workgroups, iters, out)
    torch.cuda.synchronize()
    assert torch.all(out == float(8 * 16 * 64 * iters)), out.unique()
    rnd = torch.randint(0, 256, (binding.MFMA_PROBE_OPERAND_BYTES,), dtype=torch.uint8, device=dev,
                        generator=torch.Generator(device=dev).manual_seed(1))
    binding.mfma_probe(rnd, workgroups, iters, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("words,workgroups", [(4, 1), (4 * 1000 + 4, 3), (1 << 20, 256), ((1 << 22) + 36, 4096)])
def test_read_probe_reads_every_element_once(dev, words, workgroups):
    log("read probe words=%d workgroups=%d" % (words, workgroups))
    rng = np.random.default_rng(words + workgroups)
    host = rng.integers(0, 1 << 31, size=words, dtype=np.int64).astype(np.int32)
    src = torch.from_numpy(host).to(dev)
    out = torch.zeros(workgroups * 256, dtype=torch.int32, device=dev)
    binding.read_probe(src, workgroups, out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host.view(np.uint32))
