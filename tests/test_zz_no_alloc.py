"""trimul_fwd_noalloc (include/trimul.h) through the C ABI: the allocation-free
entry point must give the same output as trimul_fwd with a workspace, on two
calls in a row (the second smaller, so it runs over the first call's leftover
scratch contents), and refuse shapes beyond its static scratch array before
enqueueing anything."""
import ctypes

import numpy as np
import pytest
import torch

from triangle_multiplication_amd import inputs

from _helpers import oracle_check, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from triangle_multiplication_amd import binding
    return binding


def _case(N, D, masked, seed):
    z = inputs.make_z(1, N, D, "bf16", seed=seed).cuda()
    mask = None
    if masked:
        tm = np.ones(N, np.float32)
        tm[N - N // 10:] = 0
        tm[3] = 0
        mask = inputs.pair_mask(tm, 1, "bf16").cuda()
    return z, mask


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_noalloc_matches_fwd_on_two_calls(tb, direction):
    D = 128
    w = inputs.make_weights(D, D, "bf16", random_ln=True)
    layer = tb.TriMul(w, "bf16")
    for N, masked, seed in [(384, True, 21), (136, False, 22)]:   # second call smaller
        say("noalloc", direction, N, masked)
        z, mask = _case(N, D, masked, seed)
        ref = layer.forward(z, mask, direction)
        out = torch.full_like(z, float("nan"))
        tb.trimul_fwd_noalloc(layer.h, z, mask, direction, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (N, masked)
        assert oracle_check(z, mask, w, direction, out, full=True) <= 2e-2


def test_noalloc_refuses_shapes_beyond_its_scratch(tb):
    D = 128
    w = inputs.make_weights(D, D, "bf16")
    layer = tb.TriMul(w, "bf16")
    N = 1024
    z = torch.zeros((1, N, N, D), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros_like(z)
    assert tb.trimul_workspace_size_lean(layer.h, 1, N) > tb.NOALLOC_MAX_BYTES
    with pytest.raises(tb.TriMulError) as e:
        tb.trimul_fwd_noalloc(layer.h, z, None, "outgoing", out)
    assert e.value.status == tb.TRIMUL_ERR_UNSUPPORTED and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert (out == 0).all()          # nothing was enqueued


def test_noalloc_largest_shape_fits(tb):
    """The documented limit: at D = C = 128, B = 1, N = 416 fits and N = 424 does
    not; the largest shape runs and matches trimul_fwd bit for bit."""
    w = inputs.make_weights(128, 128, "bf16", random_ln=True)
    layer = tb.TriMul(w, "bf16")
    assert tb.trimul_workspace_size(layer.h, 1, 416) <= tb.NOALLOC_MAX_BYTES
    assert tb.trimul_workspace_size_lean(layer.h, 1, 424) > tb.NOALLOC_MAX_BYTES
    for direction in ("outgoing", "incoming"):
        say("noalloc largest", direction)
        z, mask = _case(416, 128, True, 23)
        ref = layer.forward(z, mask, direction)
        out = torch.full_like(z, float("nan"))
        tb.trimul_fwd_noalloc(layer.h, z, mask, direction, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
