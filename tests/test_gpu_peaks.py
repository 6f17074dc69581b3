"""The measured-ceiling kernels the benchmark reports against
(trimul_internal_peak_stream / _mfma): the streams move exactly the bytes
their mode defines, over sizes that end inside a workgroup (one 16-byte chunk
per thread, 256 threads) and at its edge, and the MFMA-only loop accumulates
linearly in its iteration count."""
import pytest
import torch

from _helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from triangle_multiplication_amd import binding
    return binding


def _bytes(n16, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    return torch.randint(0, 256, (n16 * 16,), generator=g, dtype=torch.uint8).cuda()


@pytest.mark.parametrize("nt", [False, True])
@pytest.mark.parametrize("n16", [1, 3, 255, 256, 1025, 65536 * 4 + 7])
def test_streams_move_the_defined_bytes(tb, n16, nt):
    say("peak streams", n16, nt)
    s0, s1 = _bytes(n16, 1), _bytes(n16, 2)
    d0 = torch.zeros_like(s0)
    d1 = torch.zeros_like(s0)
    tb.trimul_internal_peak_stream(s0, d0, nontemporal=nt)
    torch.cuda.synchronize()
    assert torch.equal(d0, s0)
    d0.zero_()
    tb.trimul_internal_peak_stream(s0, d0, src1=s1, nontemporal=nt)
    torch.cuda.synchronize()
    assert torch.equal(d0, s0 ^ s1)
    d0.zero_()
    tb.trimul_internal_peak_stream(s0, d0, dst1=d1, nontemporal=nt)
    torch.cuda.synchronize()
    assert torch.equal(d0, s0) and torch.equal(d1, s0)


@pytest.mark.parametrize("shape", [0, 1])
def test_mfma_loop_accumulates_linearly(tb, shape):
    g = torch.Generator(device="cpu").manual_seed(5)
    seed = torch.randn(2048, generator=g).to(torch.bfloat16).cuda()
    blocks = 64
    one = torch.full((blocks * 256,), float("nan"), device="cuda")
    two = torch.full((blocks * 256,), float("nan"), device="cuda")
    tb.trimul_internal_peak_mfma(seed, blocks, 1, one, shape=shape)
    tb.trimul_internal_peak_mfma(seed, blocks, 2, two, shape=shape)
    torch.cuda.synchronize()
    assert torch.isfinite(one).all() and torch.isfinite(two).all()
    assert one.abs().max() > 0
    torch.testing.assert_close(two, 2 * one, rtol=1e-5, atol=1e-3)
