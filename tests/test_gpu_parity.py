"""GPU parity of libtrimul against the fp64 oracle, through the C ABI.

Tolerances (normalised max error, max|got - ref| / max|ref|): 1e-4 for the
fp32 path, 2e-2 for bf16 storage with fp32 statistics and accumulation.
Every output is compared element by element for N <= 1024 (the oracle's full
mode); for N >= 2048 on a seeded 64 x 64 grid of (i, j) outputs per batch
element (4096 output rows), which the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
from triangle_multiplication_amd import inputs

from _helpers import (_exact_contract_reference, _from_ab_storage, _to_ab_storage, oracle_check,
                      rel_err, say, workload_inputs)

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp32": 1e-4}


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


def _layer(tb, w, dtype):
    return tb.TriMul(w, dtype)


# ----------------------------------------------------------------------------
# Contraction kernel alone: exact on small integers (bitwise)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("B,C,N", [(1, 32, 8), (2, 32, 200), (1, 64, 136), (1, 32, 384),
                                   (1, 32, 2056)])
def test_contract_exact_integers(tb, dtype, B, C, N):
    say("contract exact", dtype, B, C, N)
    w = inputs.make_weights(C, C, dtype)
    layer = _layer(tb, w, dtype)
    g = torch.Generator(device="cuda").manual_seed(7)
    tdt = inputs.TORCH_DTYPES[dtype]
    a = torch.randint(-3, 4, (B, C, N, N), generator=g, device="cuda").to(tdt)
    b = torch.randint(-3, 4, (B, C, N, N), generator=g, device="cuda").to(tdt)
    o = layer.contract(_to_ab_storage(a, dtype), _to_ab_storage(b, dtype))
    ref = _exact_contract_reference(a, b).to(tdt)
    torch.cuda.synchronize()
    assert torch.equal(o, ref)


@pytest.mark.parametrize("C,N", [(256, 4096), (128, 8192)])
def test_contract_exact_integers_full_size(tb, C, N):
    """Full workload shapes (every tile and the whole K loop), checked on sampled rows."""
    say("contract exact full size", C, N)
    w = inputs.make_weights(C, C, "bf16")
    layer = _layer(tb, w, "bf16")
    g = torch.Generator(device="cuda").manual_seed(8)
    a = torch.randint(-3, 4, (1, C, N, N), generator=g, device="cuda", dtype=torch.int8).to(torch.bfloat16)
    b = torch.randint(-3, 4, (1, C, N, N), generator=g, device="cuda", dtype=torch.int8).to(torch.bfloat16)
    o = layer.contract(_to_ab_storage(a, "bf16"), _to_ab_storage(b, "bf16"))
    I, _ = inputs.sample_grid(N, 64)
    rows = torch.as_tensor(I, device="cuda")
    chans = torch.as_tensor([0, 1, C // 2 + 3, C - 1], device="cuda")
    ref = _exact_contract_reference(a, b, rows=rows, chans=chans).to(torch.bfloat16)
    got = o[:, chans][:, :, rows]
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


# ----------------------------------------------------------------------------
# Projection kernel alone against the oracle's a and b
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
# The bf16 kernel for D in {128, 256} runs C / 8 weight stages through a
# three-slot ring in a loop unrolled by three: C = 32, 96, 224 give stage
# counts of every residue mod 3; N = 40, 72 leave a ragged k block.
@pytest.mark.parametrize("B,N,D,C", [(2, 40, 64, 64), (1, 72, 128, 32), (1, 16, 96, 160),
                                     (1, 40, 128, 96), (2, 24, 256, 224)])
def test_project_stage(tb, dtype, direction, B, N, D, C):
    say("project stage", dtype, direction, B, N, D, C)
    w = inputs.make_weights(D, C, dtype, random_ln=True)
    z = inputs.make_z(B, N, D, dtype)
    tm = np.ones(N, np.float32)
    tm[N - 5:] = 0
    tm[1] = 0
    mask = inputs.pair_mask(tm, B, dtype)
    ref = oracle.trimul_full(z.float().numpy(), mask.float().numpy(), w, direction, dumps=True)
    layer = _layer(tb, w, dtype)
    a, b = layer.project(z.cuda(), mask.cuda(), direction)
    a, b = _from_ab_storage(a, dtype), _from_ab_storage(b, dtype)
    a, b = a.float().cpu().numpy(), b.float().cpu().numpy()
    ra, rb = ref["a"], ref["b"]  # [B, N, N, C] pair layout
    if direction == "outgoing":
        ea, eb = ra.transpose(0, 3, 1, 2), rb.transpose(0, 3, 1, 2)
    else:
        ea, eb = ra.transpose(0, 3, 2, 1), rb.transpose(0, 3, 2, 1)
    assert rel_err(a, ea) <= TOL[dtype]
    assert rel_err(b, eb) <= TOL[dtype]
    # masked pairs give exact zeros
    dead = np.nonzero(tm == 0)[0]
    if direction == "outgoing":
        assert (a[:, :, dead, :] == 0).all() and (a[:, :, :, dead] == 0).all()
    else:
        assert (a[:, :, :, dead] == 0).all() and (a[:, :, dead, :] == 0).all()


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("B,N,D,C", [(1, 40, 128, 32), (2, 72, 128, 96), (1, 40, 256, 224), (1, 64, 256, 256),
                                     (1, 24, 256, 128), (1, 40, 128, 256)])
def test_project_stage_unmasked(tb, direction, B, N, D, C):
    """The bf16 projection without a mask runs its own instantiation (no mask
    loads or multiply; lanes of pairs past N store to the sink): a and b against
    the oracle, ragged k blocks included."""
    say("project stage unmasked", direction, B, N, D, C)
    w = inputs.make_weights(D, C, "bf16", random_ln=True)
    z = inputs.make_z(B, N, D, "bf16")
    ref = oracle.trimul_full(z.float().numpy(), None, w, direction, dumps=True)
    layer = _layer(tb, w, "bf16")
    a, b = layer.project(z.cuda(), None, direction)
    a, b = _from_ab_storage(a, "bf16"), _from_ab_storage(b, "bf16")
    a, b = a.float().cpu().numpy(), b.float().cpu().numpy()
    ra, rb = ref["a"], ref["b"]
    perm = (0, 3, 1, 2) if direction == "outgoing" else (0, 3, 2, 1)
    assert rel_err(a, ra.transpose(perm)) <= TOL["bf16"]
    assert rel_err(b, rb.transpose(perm)) <= TOL["bf16"]


# ----------------------------------------------------------------------------
# Output kernel alone against the oracle's output stage
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("B,N,D,C", [(1, 24, 64, 64), (2, 40, 32, 96), (1, 16, 256, 256), (1, 8, 160, 224),
                                     (1, 72, 128, 128), (2, 16, 128, 128), (2, 24, 256, 256),
                                     (1, 24, 256, 128), (1, 40, 128, 256), (2, 24, 128, 64), (1, 16, 128, 192)])
def test_output_stage(tb, dtype, B, N, D, C):
    say("output stage", dtype, B, N, D, C)
    w = inputs.make_weights(D, C, dtype, random_ln=True)
    z = inputs.make_z(B, N, D, dtype)
    g = torch.Generator("cpu").manual_seed(9)
    o = (torch.randn((B, C, N, N), generator=g) * 3.0 + 0.5).to(inputs.TORCH_DTYPES[dtype])
    ref = oracle.output_stage(z.float().numpy(), o.float().permute(0, 2, 3, 1).numpy(), w)
    layer = _layer(tb, w, dtype)
    out = layer.output(z.cuda(), o.cuda())
    assert rel_err(out.float().cpu().numpy(), ref) <= TOL[dtype]


@pytest.mark.parametrize("N,D,C", [(200, 256, 128), (328, 256, 256), (456, 128, 128), (264, 128, 256)])
def test_output_stage_multi_run(tb, N, D, C):
    """Sizes at which every workgroup of the folded output kernel walks several
    64-pair runs and the run count does not divide by the workgroup count:
    the strided walk over one moving window (D = 256) and the rotated walk of
    contiguous ranges (D = 128) must each cover every pair exactly once."""
    B = 1
    say("output stage multi-run", N, D, C)
    w = inputs.make_weights(D, C, "bf16", random_ln=True)
    z = inputs.make_z(B, N, D, "bf16")
    g = torch.Generator("cpu").manual_seed(11)
    o = (torch.randn((B, C, N, N), generator=g) * 2.0 - 0.3).to(torch.bfloat16)
    ref = oracle.output_stage(z.float().numpy(), o.float().permute(0, 2, 3, 1).numpy(), w)
    layer = _layer(tb, w, "bf16")
    out = layer.output(z.cuda(), o.cuda())
    err = rel_err(out.float().cpu().numpy(), ref)
    say("  err", err)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("D,C", [(128, 128), (256, 256), (256, 128), (128, 256), (128, 64), (128, 192)])
@pytest.mark.parametrize("mean", [20.0, -40.0])
def test_output_stage_shifted_o_mean(tb, D, C, mean):
    """o channels far from zero mean (sigma 1): the folded output kernel (every
    width it serves) takes LayerNorm_out's statistics in one pass and applies
    -mu * S algebraically on bf16-stored o, so the cancellation must stay
    within tolerance."""
    B, N = 1, 40
    say("output stage shifted o mean", D, C, mean)
    w = inputs.make_weights(D, C, "bf16", random_ln=True)
    z = inputs.make_z(B, N, D, "bf16")
    g = torch.Generator("cpu").manual_seed(10)
    o = (torch.randn((B, C, N, N), generator=g) + mean).to(torch.bfloat16)
    ref = oracle.output_stage(z.float().numpy(), o.float().permute(0, 2, 3, 1).numpy(), w)
    layer = _layer(tb, w, "bf16")
    out = layer.output(z.cuda(), o.cuda())
    err = rel_err(out.float().cpu().numpy(), ref)
    say("  err", err)
    assert err <= TOL["bf16"]


# ----------------------------------------------------------------------------
# End to end
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("B,N,D,C,masked", [(1, 8, 32, 32, False), (3, 24, 64, 96, True),
                                            (1, 72, 128, 128, True), (2, 136, 32, 64, False),
                                            (1, 40, 256, 256, True), (1, 48, 160, 32, True),
                                            (1, 24, 256, 192, True), (1, 40, 128, 256, True),
                                            (2, 24, 256, 128, False), (1, 32, 128, 64, True),
                                            (1, 136, 128, 192, False)])
def test_fwd_small_shapes(tb, dtype, direction, B, N, D, C, masked):
    say("fwd small", dtype, direction, B, N, D, C, masked)
    w = inputs.make_weights(D, C, dtype, random_ln=True)
    z = inputs.make_z(B, N, D, dtype)
    mask = None
    if masked:
        tm = np.ones(N, np.float32)
        tm[N - max(1, N // 10):] = 0
        tm[N // 3] = 0
        mask = inputs.pair_mask(tm, B, dtype)
    layer = _layer(tb, w, dtype)
    out = layer.forward(z.cuda(), None if mask is None else mask.cuda(), direction)
    err = oracle_check(z, mask, w, direction, out, full=True)
    say("  err", err)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("mean", [3.0, -8.0, 64.0, -64.0, 128.0])
def test_fwd_shifted_mean(tb, direction, D, mean):
    """z rows whose mean is up to 128 standard deviations from zero: the bf16
    kernels apply LayerNorm algebraically with one-pass statistics
    (var = E[v^2] - mean^2 in fp32), which must stay within tolerance over the
    range the library documents (|mean| / std <= 128)."""
    B, N, C = 1, 40, D
    say("fwd shifted mean", direction, D, mean)
    w = inputs.make_weights(D, C, "bf16", random_ln=True)
    z = (inputs.make_z(B, N, D, "fp32") + mean).to(torch.bfloat16)
    layer = _layer(tb, w, "bf16")
    out = layer.forward(z.cuda(), None, direction)
    err = oracle_check(z, None, w, direction, out, full=True)
    say("  err", err)
    assert err <= TOL["bf16"]


WL = inputs.WORKLOADS


def _run_workload(tb, name, direction):
    wl = WL[name]
    say("workload", name, direction)
    z, mask, w = workload_inputs(wl)
    layer = _layer(tb, w, wl.dtype)
    out = layer.forward(z, mask, direction)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    err = oracle_check(z, mask, w, direction, out, full=(wl.check == "full"),
                       extra=wl.sample_extra())
    say("  err", err)
    assert err <= wl.tol
    return z, mask, w, layer, out


def test_workload_out_fp32_b1_n64_d32(tb):
    _run_workload(tb, "out_fp32_b1_n64_d32", "outgoing")


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_workload_outin_bf16_b1_n384_d128_tailmask(tb, direction):
    z, mask, w, layer, out = _run_workload(tb, "outin_bf16_b1_n384_d128_tailmask", direction)
    # every pair touching a padded token: o = 0, so out = p_out(beta_out) * gate = 0 with beta = 0
    n_pad = 38
    assert (out[0, -n_pad:, :] == 0).all() and (out[0, :, -n_pad:] == 0).all()


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_workload_outin_bf16_b2_n1024_d128(tb, direction):
    _run_workload(tb, "outin_bf16_b2_n1024_d128", direction)


# ----------------------------------------------------------------------------
# Invariants on the GPU
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_mask_garbage_invariance_bitwise(tb, direction):
    wl = WL["outin_bf16_b1_n384_d128_tailmask"]
    say("mask garbage", direction)
    z, mask, w = workload_inputs(wl)
    layer = _layer(tb, w, "bf16")
    out1 = layer.forward(z, mask, direction)
    g = torch.Generator(device="cuda").manual_seed(11)
    junk = (torch.randn(z.shape, generator=g, device="cuda") * 40.0).to(z.dtype)
    z2 = torch.where((mask == 0)[..., None], junk, z)
    out2 = layer.forward(z2, mask, direction)
    keep = mask[0] != 0
    assert torch.equal(out1[0][keep], out2[0][keep])


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
@pytest.mark.parametrize("D", [128, 256])
def test_permutation_equivariance(tb, direction, D):
    """Permuting the tokens permutes the output: out(pi z pi, pi m pi)[i, j] =
    out(z, m)[pi(i), pi(j)].  The kernels sum over k in a different order on
    the permuted input, so the two agree to the bf16 tolerance, and each agrees
    with the oracle."""
    B, N, C = 1, 136, D
    say("permutation equivariance", direction, D)
    w = inputs.make_weights(D, C, "bf16", random_ln=True)
    z = inputs.make_z(B, N, D, "bf16")
    tm = np.ones(N, np.float32)
    tm[[5, 77, 130]] = 0
    mask = inputs.pair_mask(tm, B, "bf16")
    pi = torch.as_tensor(np.random.default_rng(12).permutation(N))
    zp = z[:, pi][:, :, pi].contiguous()
    mp = mask[:, pi][:, :, pi].contiguous()
    layer = _layer(tb, w, "bf16")
    out = layer.forward(z.cuda(), mask.cuda(), direction)
    outp = layer.forward(zp.cuda(), mp.cuda(), direction)
    torch.cuda.synchronize()
    perm = out.cpu()[:, pi][:, :, pi]
    err = rel_err(outp.float().cpu().numpy(), perm.float().numpy())
    say("  err", err)
    assert err <= TOL["bf16"]
    assert oracle_check(zp, mp, w, direction, outp, full=True) <= TOL["bf16"]


def test_determinism_bitwise(tb):
    wl = WL["outin_bf16_b1_n384_d128_tailmask"]
    z, mask, w = workload_inputs(wl)
    layer = _layer(tb, w, "bf16")
    o1 = layer.forward(z, mask, "incoming")
    o2 = layer.forward(z, mask, "incoming")
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_transpose_identity_bitwise(tb, dtype):
    """With g_out = 0 (gate 1/2 everywhere), incoming on (z, m) equals outgoing on the transposes."""
    B, N, D, C = 2, 72, 64, 64
    w = inputs.make_weights(D, C, dtype, random_ln=True)
    w = w.replace(g_out=np.zeros_like(w.g_out))
    z = inputs.make_z(B, N, D, dtype).cuda()
    tm = np.ones(N, np.float32)
    tm[5] = 0
    mask = inputs.pair_mask(tm, B, dtype).cuda()
    mask[:, 3, :] = 0  # non-symmetric
    layer = _layer(tb, w, dtype)
    o_in = layer.forward(z, mask, "incoming")
    o_out = layer.forward(z.transpose(1, 2).contiguous(), mask.transpose(1, 2).contiguous(), "outgoing")
    assert torch.equal(o_in, o_out)


def test_guard_bands_untouched(tb):
    B, N, D, C = 1, 72, 64, 64
    w = inputs.make_weights(D, C, "bf16")
    layer = _layer(tb, w, "bf16")
    z = inputs.make_z(B, N, D, "bf16").cuda()
    n_out = B * N * N * D
    pad = 4096
    big = torch.full((n_out + 2 * pad,), 1234.0, dtype=torch.bfloat16, device="cuda")
    out = big[pad:pad + n_out].view(B, N, N, D)
    ws_need = tb.trimul_workspace_size(layer.h, B, N)
    wbig = torch.full((ws_need + 2 * pad,), 0x5A, dtype=torch.uint8, device="cuda")
    ws = wbig[pad:pad + ws_need]
    tb.trimul_fwd(layer.h, z, None, "outgoing", out, ws)
    torch.cuda.synchronize()
    assert (big[:pad] == 1234.0).all() and (big[pad + n_out:] == 1234.0).all()
    assert (wbig[:pad] == 0x5A).all() and (wbig[pad + ws_need:] == 0x5A).all()


def test_error_paths_on_device(tb):
    B, N, D, C = 1, 16, 32, 32
    w = inputs.make_weights(D, C, "bf16")
    layer = _layer(tb, w, "bf16")
    z = inputs.make_z(B, N, D, "bf16").cuda()
    out = torch.empty_like(z)
    need = tb.trimul_workspace_size(layer.h, B, N)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    with pytest.raises(tb.TriMulError) as e:
        tb.trimul_fwd(layer.h, z, None, "outgoing", out, ws[: need - 256])
    assert e.value.status == tb.TRIMUL_ERR_WORKSPACE
    with pytest.raises(tb.TriMulError) as e:
        tb.trimul_fwd(layer.h, z, None, "outgoing", z, ws)
    assert e.value.status == tb.TRIMUL_ERR_INVALID_ARG and "overlaps" in str(e.value)
    zbig = torch.empty(z.numel() + 8, dtype=z.dtype, device="cuda")
    zmis = zbig[1:1 + z.numel()].view(z.shape)
    with pytest.raises(tb.TriMulError) as e:
        tb.trimul_fwd(layer.h, zmis, None, "outgoing", out, ws)
    assert e.value.status == tb.TRIMUL_ERR_INVALID_ARG and "aligned" in str(e.value)
    z12 = torch.zeros((1, 12, 12, D), dtype=z.dtype, device="cuda")
    with pytest.raises(tb.TriMulError) as e:
        tb.trimul_fwd(layer.h, z12, None, "outgoing", torch.empty_like(z12), ws)
    assert e.value.status == tb.TRIMUL_ERR_INVALID_ARG and "multiple of 8" in str(e.value)
    with pytest.raises(tb.TriMulError) as e:
        tb.trimul_fwd(layer.h, z, None, 5, out, ws)
    assert e.value.status == tb.TRIMUL_ERR_INVALID_ARG


def test_arch_gate_accepts_this_device(tb):
    name = torch.cuda.get_device_properties(0).gcnArchName
    tb.trimul_check_arch(name)


# ----------------------------------------------------------------------------
# Full-size workloads (last: they hold tens of GB)
# ----------------------------------------------------------------------------
def test_constant_z_full_size(tb):
    """z equal at every pair: every output row is the same vector, equal to the oracle's."""
    B, N, D, C = 1, 4096, 256, 256
    say("constant z full size")
    w = inputs.make_weights(D, C, "bf16", random_ln=True)
    v = inputs.make_z(1, 1, D, "bf16", seed=5)[0, 0, 0]
    z = v.cuda().expand(B, N, N, D).contiguous()
    layer = _layer(tb, w, "bf16")
    out = layer.forward(z, None, "outgoing")
    torch.cuda.synchronize()
    assert (out == out[0, 0, 0]).all()
    vz = v.float().numpy()[None, None]
    zA = np.broadcast_to(vz, (1, N, D))
    ref = oracle.trimul_grid(N, w, zA, None, zA, None, vz)
    assert rel_err(out[0, 0, 0].float().cpu().numpy(), ref[0, 0]) <= 2e-2
    del out, z


def test_workload_out_bf16_b1_n4096_d256(tb):
    _run_workload(tb, "out_bf16_b1_n4096_d256", "outgoing")


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_fwd_ragged_large_tailmask(tb, direction):
    # The large-N kernels on a ragged size: N = 2056 leaves an 8-token k block
    # in the projection and contraction and an 8-row tile edge in the
    # contraction; the last floor(N/10) = 205 tokens are masked, so the mask
    # boundary (token 1851) falls inside a k block.  D = C = 256 selects the
    # folded projection and output kernels.
    wl = inputs.Workload("ragged_bf16_b1_n2056_d256_tailmask", "bf16", (direction,), 1, 2056, 256, 256,
                         mask="tail10", check="grid")
    say("ragged large", direction)
    z, mask, w = workload_inputs(wl)
    layer = _layer(tb, w, "bf16")
    out = layer.forward(z, mask, direction)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    err = oracle_check(z, mask, w, direction, out, full=False, extra=wl.sample_extra())
    say("  err", err)
    assert err <= wl.tol
    n_valid = 2056 - 205
    assert (out[0, n_valid:, ::89] == 0).all() and (out[0, ::89, n_valid:] == 0).all()


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_fwd_largest_n_tailmask(tb, direction):
    # The largest N run here: N = 16384 at D = C = 32 (about 87 GB of device
    # memory with the full workspace).  2.7e8 pairs per batch element and 8.6e9
    # z elements (64-bit pair offsets in every kernel), 64 x 64 contraction
    # tiles with 4096 tile pairs in the mask table's lists, operand slabs of
    # 512 MiB; the last floor(N/10) tokens are masked.  D = 32 selects the
    # generic projection and output kernels.
    wl = inputs.Workload("big_bf16_b1_n16384_d32_tailmask", "bf16", (direction,), 1, 16384, 32, 32,
                         mask="tail10", check="grid")
    say("largest N", direction)
    z, mask, w = workload_inputs(wl)
    layer = _layer(tb, w, "bf16")
    out = layer.forward(z, mask, direction)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    err = oracle_check(z, mask, w, direction, out, full=False, extra=wl.sample_extra())
    say("  err", err)
    assert err <= wl.tol
    n_valid = 16384 - 1638
    assert (out[0, n_valid:, ::997] == 0).all() and (out[0, ::997, n_valid:] == 0).all()


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_fwd_many_batches_full(tb, direction):
    # Many operand slabs: B = 128 at D = C = 128 is B*C = 16384 slabs of one
    # 64 x 64 tile each (the folded kernels), every batch element with its own
    # tail mask row of the mask table; checked in full.
    B, N, D = 128, 64, 128
    say("many batches", direction)
    w = inputs.make_weights(D, D, "bf16", random_ln=True)
    z = inputs.make_z(B, N, D, "bf16")
    tm = np.ones((B, N), np.float32)
    for b in range(B):
        tm[b, N - 1 - (b % 17):] = 0        # 1 .. 17 masked tokens, varying per batch element
    mask = torch.from_numpy(tm[:, :, None] * tm[:, None, :]).to(torch.bfloat16)
    layer = _layer(tb, w, "bf16")
    out = layer.forward(z.cuda(), mask.cuda(), direction)
    torch.cuda.synchronize()
    err = oracle_check(z, mask, w, direction, out, full=True)
    say("  err", err)
    assert err <= TOL["bf16"]


def test_workload_in_bf16_b1_n8192_d128_chains(tb):
    z, mask, w, layer, out = _run_workload(tb, "in_bf16_b1_n8192_d128_chains", "incoming")
    # padded tail rows and columns are exactly zero (beta_out = 0)
    assert (out[0, 7800:, :: 97] == 0).all() and (out[0, ::97, 7800:] == 0).all()
