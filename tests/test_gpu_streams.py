"""Stream use of the forward pass through the C ABI: the allocation-free entry
point captured into a HIP graph and replayed, and concurrent calls on two
streams with their own workspaces (include/trimul.h: the handle is read-only
after create)."""
import numpy as np
import pytest
import torch

from triangle_multiplication_amd import inputs

from _helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from triangle_multiplication_amd import binding
    return binding


def _tail_mask(N, B=1):
    tm = np.ones(N, np.float32)
    tm[N - N // 10:] = 0
    tm[5] = 0
    return inputs.pair_mask(tm, B, "bf16").cuda()


def test_noalloc_graph_replays(tb):
    """A captured trimul_fwd_noalloc (masked: the mask scan and tile-pair
    kernels are in the graph too) replays to the eager result every time, with
    other eager calls that reuse the same scratch array between the replays."""
    D, N = 128, 256
    w = inputs.make_weights(D, D, "bf16", random_ln=True)
    layer = tb.TriMul(w, "bf16")
    z = inputs.make_z(1, N, D, "bf16", seed=31).cuda()
    z_other = inputs.make_z(1, 200, D, "bf16", seed=32).cuda()
    mask = _tail_mask(N)
    eager = torch.empty_like(z)
    tb.trimul_fwd_noalloc(layer.h, z, mask, "incoming", eager)
    torch.cuda.synchronize()
    out = torch.empty_like(z)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                  # warm-up off the default stream before capture
        tb.trimul_fwd_noalloc(layer.h, z, mask, "incoming", out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):                  # the binding enqueues on the capturing stream
        tb.trimul_fwd_noalloc(layer.h, z, mask, "incoming", out)
    torch.cuda.synchronize()
    for r in range(3):
        say("graph replay", r)
        out.fill_(float("nan"))
        other = torch.empty_like(z_other)
        tb.trimul_fwd_noalloc(layer.h, z_other, None, "outgoing", other)   # leaves other scratch contents
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), r
    del graph


def test_two_streams_concurrently(tb):
    """Two forward calls in flight at once on two streams (one handle, separate
    workspaces and outputs) give the sequential results, three times over."""
    D, N = 128, 512
    w = inputs.make_weights(D, D, "bf16", random_ln=True)
    layer = tb.TriMul(w, "bf16")
    z1 = inputs.make_z(1, N, D, "bf16", seed=33).cuda()
    z2 = inputs.make_z(1, N, D, "bf16", seed=34).cuda()
    mask = _tail_mask(N)
    ref1 = layer.forward(z1, None, "outgoing").clone()
    ref2 = layer.forward(z2, mask, "incoming").clone()
    ws1 = torch.empty(tb.trimul_workspace_size(layer.h, 1, N), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(tb.trimul_workspace_size_lean(layer.h, 1, N), dtype=torch.uint8, device="cuda")
    o1, o2 = torch.empty_like(z1), torch.empty_like(z2)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for r in range(3):
        say("two streams", r)
        o1.fill_(float("nan"))
        o2.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            tb.trimul_fwd(layer.h, z1, None, "outgoing", o1, ws1)
        with torch.cuda.stream(s2):
            tb.trimul_fwd(layer.h, z2, mask, "incoming", o2, ws2)
        torch.cuda.synchronize()
        assert torch.equal(o1, ref1), r
        assert torch.equal(o2, ref2), r
