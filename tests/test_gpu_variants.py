"""GPU checks of what changes the order of the work but must not change the
result: the mask scan and the masked key skip of the contraction, every
candidate plan, the workspace-lean layout, and trimul_tune with its plan
cache.  All comparisons are bitwise against the plain path (the same per-tile
arithmetic in the same order), and the plain path is held to the oracle by
test_gpu_parity.py; one end-to-end oracle check per feature is repeated here.
"""
import os

import numpy as np
import pytest
import torch

from triangle_multiplication_amd import inputs

from _helpers import _exact_contract_reference, _to_ab_storage, oracle_check, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tb():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from triangle_multiplication_amd import binding
    return binding


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    if torch.cuda.is_available():
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def _ref_ranges(mask, direction):
    """Per 256-row tile, (first live key // 32, last live key // 32 + 1) of
    M = mask (outgoing) or mask^T (incoming), (0, 0) if none (numpy)."""
    m = mask.float().cpu().numpy()
    B, N, _ = m.shape
    tiles = (N + 255) // 256
    out = np.zeros((B, tiles, 2), np.int32)
    for b in range(B):
        M = m[b] if direction == "outgoing" else m[b].T
        for t in range(tiles):
            live = np.nonzero((M[256 * t:min(N, 256 * t + 256)] != 0).any(axis=0))[0]
            if len(live):
                out[b, t] = (live[0] // 32, live[-1] // 32 + 1)
    return out


def _masks(N, dtype):
    """Masks of several structures, each [1, N, N] on the device."""
    tdt = inputs.TORCH_DTYPES[dtype]
    g = torch.Generator("cpu").manual_seed(31)
    res = {}
    res["tail10"] = inputs.pair_mask(inputs.token_mask_tail(N), 1, dtype)
    chains = np.zeros(N, np.float32)
    chains[: N - N // 7] = 1
    res["chains"] = inputs.pair_mask(chains, 1, dtype)
    # Not an outer product: random sparse live pairs, one row block and one
    # column block entirely dead, and -0.0 in dead places (counts as zero).
    r = (torch.rand((1, N, N), generator=g) < 0.002).float()
    r[:, : min(N, 300)] = 0
    r[:, :, N // 2: N // 2 + 40] = 0
    r[0, 5, N - 9] = 1
    r = torch.where(r == 0, torch.tensor(-0.0), r)
    res["sparse"] = r.to(tdt)
    res["empty"] = torch.zeros((1, N, N), dtype=tdt)
    return res


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("N", [384, 600, 1288])
def test_mask_ranges_match_numpy(tb, direction, N):
    say("mask ranges", direction, N)
    w = inputs.make_weights(32, 32, "bf16")
    layer = tb.TriMul(w, "bf16")
    for name, m in _masks(N, "bf16").items():
        table = layer.mask_ranges(m.cuda(), direction)
        got = tb.table_parts(table, 1, N)[0].cpu().numpy()
        ref = _ref_ranges(m, direction)
        assert (got == ref).all(), (name, got.tolist(), ref.tolist())


@pytest.mark.parametrize("gm", [4, 8, 16])
def test_tile_pair_lists(tb, gm):
    """Each batch's list holds every tile pair once, those with a live key step
    first, each part in the walk order of groups of gm row tiles; the header is
    the largest live count."""
    B, N = 3, 1288
    T = (N + 255) // 256
    say("tile pair lists", gm)
    w = inputs.make_weights(32, 32, "bf16")
    layer = tb.TriMul(w, "bf16")
    ms = _masks(N, "bf16")
    mask = torch.cat([ms["tail10"], ms["sparse"], ms["empty"]]).cuda()
    table = layer.mask_ranges(mask, "incoming")
    tb.trimul_internal_set_plan(layer.h, B, N, "incoming", True, (0, 0, gm, 256))
    C = 32
    a = torch.zeros(tb.ab_storage_shape("bf16", B, C, N), dtype=torch.bfloat16, device="cuda")
    layer.contract(a, a, table, "incoming")   # builds the lists with the plan's gm
    torch.cuda.synchronize()
    rng, hdr, pairs = [t.cpu().numpy() for t in tb.table_parts(table, B, N)]
    walk = []
    for first in range(0, T, gm):
        g = min(gm, T - first)
        for tj in range(T):
            for ti in range(first, first + g):
                walk.append((ti, tj))
    counts = []
    for b in range(B):
        def live(p):
            ti, tj = p
            return max(rng[b, ti, 0], rng[b, tj, 0]) < min(rng[b, ti, 1], rng[b, tj, 1])
        want = [p for p in walk if live(p)] + [p for p in walk if not live(p)]
        got = [(int(e) & 0xFFFF, int(e) >> 16) for e in pairs[b].astype(np.uint32)]
        assert got == want, b
        counts.append(sum(live(p) for p in walk))
    assert hdr[0] == max(counts) and counts[2] == 0


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("N", [600, 1288])
def test_masked_contraction_bitwise_equals_dense(tb, direction, N):
    """Integer operands that are zero wherever the mask is: the contraction
    with the skip equals the dense one (and the exact sums) bit for bit."""
    say("masked contraction", direction, N)
    C = 32
    w = inputs.make_weights(C, C, "bf16")
    layer = tb.TriMul(w, "bf16")
    g = torch.Generator(device="cuda").manual_seed(17)
    for name, m in _masks(N, "bf16").items():
        M = m[0].float().cuda()
        M = M if direction == "outgoing" else M.t()
        live = (M != 0).to(torch.bfloat16)
        a = torch.randint(-3, 4, (1, C, N, N), generator=g, device="cuda").to(torch.bfloat16) * live
        b = torch.randint(-3, 4, (1, C, N, N), generator=g, device="cuda").to(torch.bfloat16) * live
        A, Bs = _to_ab_storage(a, "bf16"), _to_ab_storage(b, "bf16")
        table = layer.mask_ranges(m.cuda(), direction)
        o_skip = layer.contract(A, Bs, table, direction)
        o_dense = layer.contract(A, Bs)
        ref = _exact_contract_reference(a, b).to(torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(o_skip, o_dense), name
        assert torch.equal(o_skip, ref), name


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("N,D", [(384, 128), (600, 256)])
def test_masked_forward_bitwise_equals_stages(tb, direction, N, D):
    """trimul_fwd with a mask (scan + skip) equals projection -> dense
    contraction -> output run stage by stage, bit for bit."""
    say("masked forward vs stages", direction, N, D)
    w = inputs.make_weights(D, D, "bf16", random_ln=True)
    layer = tb.TriMul(w, "bf16")
    z = inputs.make_z(1, N, D, "bf16").cuda()
    for name, m in _masks(N, "bf16").items():
        m = m.cuda()
        out = layer.forward(z, m, direction)
        a, b = layer.project(z, m, direction)
        ref = layer.output(z, layer.contract(a, b))
        torch.cuda.synchronize()
        assert torch.equal(out, ref), name


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("masked", [False, True])
def test_every_plan_gives_the_same_bits(tb, direction, masked):
    B, N, D = 1, 1288, 128
    say("every plan", direction, masked)
    w = inputs.make_weights(D, D, "bf16", random_ln=True)
    layer = tb.TriMul(w, "bf16")
    z = inputs.make_z(B, N, D, "bf16").cuda()
    mask = inputs.pair_mask(inputs.token_mask_tail(N), B, "bf16").cuda() if masked else None
    plans = tb.plan_candidates()
    default = (0, 1, 8, 256)
    assert tb.trimul_internal_get_plan(layer.h, B, N, direction, masked) == default
    assert default in plans
    ref = layer.forward(z, mask, direction)
    for plan in [p for p in plans if p != default]:
        tb.trimul_internal_set_plan(layer.h, B, N, direction, masked, plan)
        assert tb.trimul_internal_get_plan(layer.h, B, N, direction, masked) == plan
        out = layer.forward(z, mask, direction)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), plan
    assert oracle_check(z, mask, w, direction, ref, full=False, extra=(N - 1 - N // 10,)) <= 2e-2


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("masked", [False, True])
def test_lean_workspace_gives_the_same_bits(tb, direction, masked):
    """N = 1288, C = 128: the lean layout runs the contraction in two chunks
    (the second stores its o over the first chunk's a slabs)."""
    B, N, D = 1, 1288, 128
    say("lean workspace", direction, masked)
    w = inputs.make_weights(D, D, "bf16", random_ln=True)
    layer = tb.TriMul(w, "bf16")
    z = inputs.make_z(B, N, D, "bf16").cuda()
    mask = inputs.pair_mask(inputs.token_mask_tail(N), B, "bf16").cuda() if masked else None
    full_b = tb.trimul_workspace_size(layer.h, B, N)
    lean_b = tb.trimul_workspace_size_lean(layer.h, B, N)
    o_slab = N * N * 2
    assert lean_b < full_b - 30 * o_slab     # o keeps at most one chunk of slabs of its own
    ref = layer.forward(z, mask, direction)
    ws = torch.empty(lean_b, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(z)
    tb.trimul_fwd(layer.h, z, mask, direction, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    with pytest.raises(tb.TriMulError) as e:
        tb.trimul_fwd(layer.h, z, mask, direction, out, ws[: lean_b - 256])
    assert e.value.status == tb.TRIMUL_ERR_WORKSPACE


def test_lean_workspace_full_size_bitwise(tb):
    """The lean layout at N = 8192, D = C = 128 with the chains mask (incoming):
    16 contraction launches of 8 slabs, each later one storing its o over the
    previous chunk's a slabs, bitwise equal to the full layout."""
    wl = inputs.WORKLOADS["in_bf16_b1_n8192_d128_chains"]
    direction = "incoming"
    say("lean full size")
    z = inputs.make_z(wl.B, wl.N, wl.D, wl.dtype, var=wl.z_var, device="cuda")
    mask = inputs.pair_mask(wl.token_mask(), wl.B, wl.dtype, device="cuda")
    layer = tb.TriMul(inputs.make_weights(wl.D, wl.C, wl.dtype), wl.dtype)
    ref = layer.forward(z, mask, direction)
    torch.cuda.synchronize()
    layer._ws = None
    torch.cuda.empty_cache()
    lean_b = tb.trimul_workspace_size_lean(layer.h, wl.B, wl.N)
    # o keeps a region of 8 slabs (one chunk) of its own instead of C = 128
    assert tb.trimul_workspace_size(layer.h, wl.B, wl.N) - lean_b == (wl.C - 8) * wl.N * wl.N * 2
    ws = torch.empty(lean_b, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(z)
    tb.trimul_fwd(layer.h, z, mask, direction, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("N,tile", [(384, 128), (200, 128), (512, 256), (640, 256), (1288, 256)])
@pytest.mark.parametrize("masked", [False, True])
def test_default_plan_by_shape(tb, N, tile, masked, monkeypatch):
    """Shapes nothing was recorded for: 128-row tiles in XCD bands where
    256-row tiles would be mostly padding (N <= 512, not a multiple of 256);
    else 256-row tiles in per-round XCD blocks, masked or not."""
    monkeypatch.setenv("TRIMUL_PLAN_CACHE", "0")
    layer = tb.TriMul(inputs.make_weights(128, 128, "bf16"), "bf16")
    order = 1 if tile == 256 else 0
    assert tb.trimul_internal_get_plan(layer.h, 1, N, "outgoing", masked) == (0, order, 8, tile)
    layer.close()


def test_tune_records_a_plan_and_the_cache_reloads_it(tb, tmp_path):
    B, N, D = 1, 1288, 128
    direction = "incoming"
    say("tune")
    path = str(tmp_path / "plans.txt")
    old = os.environ.get("TRIMUL_PLAN_CACHE")
    os.environ["TRIMUL_PLAN_CACHE"] = path
    try:
        w = inputs.make_weights(D, D, "bf16", random_ln=True)
        layer = tb.TriMul(w, "bf16")
        z = inputs.make_z(B, N, D, "bf16").cuda()
        mask = inputs.pair_mask(inputs.token_mask_tail(N), B, "bf16").cuda()
        ref = layer.forward(z, mask, direction)
        out = layer.tune(z, mask, direction)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)               # every plan computes the same bits
        plan = tb.trimul_internal_get_plan(layer.h, B, N, direction, True)
        assert plan in tb.plan_candidates()
        dev = torch.cuda.get_device_properties(0)
        key = "%s-%dcu" % (dev.gcnArchName.split(":")[0], dev.multi_processor_count)
        assert tb.cache_lookup(path, key, D, D, "bf16", B, N, direction, True) == plan
        # A new handle (as in a later process) starts from the cached plan.
        layer2 = tb.TriMul(w, "bf16")
        assert tb.trimul_internal_get_plan(layer2.h, B, N, direction, True) == plan
        assert tb.trimul_internal_get_plan(layer2.h, B, N, "outgoing", True) == (0, 1, 8, 256)   # masked default
        assert torch.equal(layer2.forward(z, mask, direction), ref)
    finally:
        if old is None:
            os.environ.pop("TRIMUL_PLAN_CACHE", None)
        else:
            os.environ["TRIMUL_PLAN_CACHE"] = old

