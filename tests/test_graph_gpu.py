"""The layer captured in a HIP graph gives, on every replay, exactly what the
eager call gives (the kernels are deterministic and enqueue no memset)."""
import numpy as np
import pytest
import torch

from mxfp4_w4a4_post_amd import binding, inputs
from parity_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    binding.load_library()
    return torch.device("cuda:0")


@pytest.mark.parametrize("cfg,shape,M", [(1, 0, None), (3, 1, 8), (2, 0, 256)])
def test_graph_replays_match_eager(dev, cfg, shape, M):
    case = inputs.linear_case(cfg, shape, M=M)
    log("graph replay %s" % case.name)
    layer = binding.prepare_layer(case.w.to(dev), case.xcal.to(dev), case.b)
    x = case.x.to(dev)
    y_eager = layer(x, out_dtype=torch.float32)
    y = torch.empty_like(y_eager)
    ws = torch.empty(binding.linear_workspace_size(case.M, case.K, case.N), dtype=torch.uint8, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer(x, out=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        layer(x, out=y, workspace=ws)
    for i in range(4):
        y.fill_(float("nan"))
        ws.fill_(0xAB)                      # eager work on the same buffers between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), "replay %d differs from the eager call" % i
        y_again = layer(x, out_dtype=torch.float32)  # eager call between replays
        torch.cuda.synchronize()
        assert torch.equal(y_again, y_eager)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_graph_moe_block_replays_match_eager(dev, out_dtype):
    """The whole MoE block (routing over several chunks with its tile maps, the
    gathered gate/up with the SwiGLU epilogue, the down projection writing each
    tile during the next one, the combine) captured in a graph: every replay
    equals the eager call, with the workspace overwritten between replays (no
    call may rely on what an earlier one left there)."""
    c = inputs.moe_block_case(tokens=1500, experts=16, top_k=4, hidden=2048, ffn=256, b=32)
    log("graph replay moe block T=%d E=%d k=%d H=%d F=%d %s" % (c.T, c.E, c.k, c.H, c.F, out_dtype))
    lay = binding.prepare_moe(c.w_gate.to(dev), c.w_up.to(dev), c.w_dn.to(dev), c.xcal_gu.to(dev),
                              c.xcal_dn.to(dev), c.b)
    x, ids, w = c.x.to(dev), torch.from_numpy(c.ids).to(dev), torch.from_numpy(c.w).to(dev)
    y_eager = lay(x, ids, w, out_dtype=out_dtype)
    y = torch.empty_like(y_eager)
    ws = torch.empty(binding.moe_workspace_size(c.T, c.k, c.E, c.H, c.F), dtype=torch.uint8, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lay(x, ids, w, out=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        lay(x, ids, w, out=y, workspace=ws)
    for i in range(4):
        y.fill_(float("nan"))
        ws.fill_(0xAB)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), "replay %d differs from the eager call" % i
        y_again = lay(x, ids, w, out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(y_again, y_eager)
