"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test fixes the oracle to a closed form, an invariant, a hand-worked
example or an independent library routine (torch's layer_norm, numpy matmul,
scipy's expit), so that a dropped term, a wrong sign or index, a transposed
operand or a swapped half of p_in/g_in fails at least one of them.
The layer follows the fold-cp-ops README, section Use (the six submodules and
the direction argument).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
from triangle_multiplication_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_z(B, N, D, seed=0, scale=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    return (torch.randn((B, N, N, D), generator=g) * scale).numpy()


def _weights(D, C, random_ln=True, seed=1):
    return inputs.make_weights(D, C, dtype="fp32", seed=seed, random_ln=random_ln)


def _ln_lib(v, gamma, beta, eps):
    t = torch.as_tensor(np.asarray(v, np.float64))
    return torch.nn.functional.layer_norm(
        t, (t.shape[-1],), torch.as_tensor(gamma, dtype=torch.float64),
        torch.as_tensor(beta, dtype=torch.float64), eps).numpy()


# ----------------------------------------------------------------------------
# P8: LayerNorm invariants and the library routine
# ----------------------------------------------------------------------------
def test_layernorm_invariants_unit_affine():
    z = _rand_z(1, 6, 16, seed=11, scale=3.0) + 0.7
    w = _weights(16, 8, random_ln=False)
    r = oracle.trimul_full(z, None, w, "outgoing", dumps=True)
    x = r["x"]
    zd = z.astype(np.float64)
    v = zd.var(axis=-1)  # biased (population) variance
    np.testing.assert_allclose(x.mean(axis=-1), 0.0, atol=1e-12)
    np.testing.assert_allclose(x.var(axis=-1), v / (v + w.eps), rtol=1e-12)


def test_layernorm_affine_matches_torch():
    z = _rand_z(2, 5, 24, seed=12)
    w = _weights(24, 16, random_ln=True)
    r = oracle.trimul_full(z, None, w, "incoming", dumps=True)
    ref = _ln_lib(z, w.ln_in_w, w.ln_in_b, w.eps)
    np.testing.assert_allclose(r["x"], ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# Gated projection and output stage against numpy matmul / scipy expit
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_projection_and_output_match_library(direction):
    B, N, D, C = 2, 7, 32, 24
    z = _rand_z(B, N, D, seed=13)
    tm = np.ones(N, np.float32)
    tm[[2, 5]] = 0.0
    mask = np.broadcast_to(np.outer(tm, tm), (B, N, N)).copy()
    w = _weights(D, C, random_ln=True)
    r = oracle.trimul_full(z, mask, w, direction, dumps=True)
    x = r["x"]
    p = x @ w.p_in.astype(np.float64).T
    g = x @ w.g_in.astype(np.float64).T
    m = mask[..., None].astype(np.float64)
    np.testing.assert_allclose(r["a"], m * p[..., :C] * expit(g[..., :C]), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["b"], m * p[..., C:] * expit(g[..., C:]), rtol=1e-12, atol=1e-13)
    y = _ln_lib(r["o"], w.ln_out_w, w.ln_out_b, w.eps)
    out = (y @ w.p_out.astype(np.float64).T) * expit(x @ w.g_out.astype(np.float64).T)
    np.testing.assert_allclose(r["out"], out, rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------------------
# P6: each channel's contraction is a plain matrix product
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_contraction_is_matmul(direction):
    B, N, D, C = 2, 9, 16, 8
    z = _rand_z(B, N, D, seed=14)
    w = _weights(D, C, random_ln=False)
    w = w.replace(g_in=np.zeros_like(w.g_in))  # every gate = 1/2
    r = oracle.trimul_full(z, None, w, direction, dumps=True)
    for b in range(B):
        for c in range(C):
            A = r["a"][b, :, :, c]
            Bm = r["b"][b, :, :, c]
            ref = A @ Bm.T if direction == "outgoing" else A.T @ Bm
            np.testing.assert_allclose(r["o"][b, :, :, c], ref, rtol=1e-12, atol=1e-13)
    # g_in = 0 makes a = p_a / 2 exactly
    np.testing.assert_allclose(r["a"], 0.5 * (r["x"] @ w.p_in[:C].astype(np.float64).T),
                               rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------
# P1b: N = 1 closed form, and the hand-worked N = 2 example
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_single_token_closed_form(direction):
    z = _rand_z(3, 1, 32, seed=15)
    w = _weights(32, 32, random_ln=True)
    r = oracle.trimul_full(z, None, w, direction, dumps=True)
    np.testing.assert_array_equal(r["o"], r["a"] * r["b"])


def _golden():
    with open(os.path.join(GOLDEN, "hand_n2_d2_c2.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_hand_worked_example(direction):
    g = _golden()
    f32 = lambda k: np.asarray(g[k], np.float32)
    w = inputs.TriMulWeights(f32("ln_in_w"), f32("ln_in_b"), f32("p_in"), f32("g_in"),
                             f32("ln_out_w"), f32("ln_out_b"), f32("p_out"), f32("g_out"),
                             g["eps"])
    r = oracle.trimul_full(f32("z"), None, w, direction, dumps=True)
    eps = g["eps"]
    sg = lambda t: 1.0 / (1.0 + math.exp(-t))
    rho = (1.0 + eps) ** -0.5
    sp, sm = sg(2 * rho), sg(-2 * rho)
    S = np.asarray(g["S"])
    if direction == "outgoing":
        o = rho ** 2 * np.array([[[sp, -sm], [-sp, sm]], [[-sm, sp], [sm, -sp]]])
        t = np.asarray(g["t_outgoing"])
    else:
        o = np.broadcast_to(rho ** 2 / 2 * np.array([1.0, -1.0]), (2, 2, 2))
        t = np.asarray(g["t_incoming"])
    np.testing.assert_allclose(r["o"][0], o, rtol=1e-14, atol=1e-15)
    kappa = (rho ** 2 / 2) / math.sqrt(rho ** 4 / 4 + eps)
    out = np.empty((2, 2, 2))
    for i in range(2):
        for j in range(2):
            y = t[i, j] * kappa * np.array([1.0, -1.0])
            out[i, j] = y * np.array([sg(S[i, j] * rho), 0.5])
    np.testing.assert_allclose(r["out"][0], out, rtol=1e-14, atol=1e-15)


def _golden_affine_out():
    with open(os.path.join(GOLDEN, "hand_n2_d2_c2_affine_out.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_hand_worked_example_affine_output(direction):
    """Values derived by hand (derivation in the fixture) with gamma_out != gamma_in,
    beta_out != 0 and non-symmetric p_out and g_out: pins the output LayerNorm's own
    parameters and the [out][in] orientation of both output matrices."""
    g = _golden_affine_out()
    f32 = lambda k: np.asarray(g[k], np.float32)
    w = inputs.TriMulWeights(f32("ln_in_w"), f32("ln_in_b"), f32("p_in"), f32("g_in"),
                             f32("ln_out_w"), f32("ln_out_b"), f32("p_out"), f32("g_out"),
                             g["eps"])
    out = oracle.trimul_full(f32("z"), None, w, direction)
    eps = g["eps"]
    sg = lambda t: 1.0 / (1.0 + math.exp(-t))
    rho = (1.0 + eps) ** -0.5
    kappa = (rho ** 2 / 2) / math.sqrt(rho ** 4 / 4 + eps)
    S = np.asarray(g["S"])
    t = np.asarray(g["t_outgoing"] if direction == "outgoing" else g["t_incoming"])
    ref = np.empty((2, 2, 2))
    for i in range(2):
        for j in range(2):
            s, tk = S[i, j], t[i, j] * kappa
            ref[i, j] = (tk / 2 * sg(s * rho), (-8 * tk - 2.5) * sg(0.75 * s * rho))
    np.testing.assert_allclose(out[0], ref, rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------------------
# P2: constant z
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_constant_z_closed_form(direction):
    N, D, C = 6, 16, 8
    v = np.random.default_rng(5).standard_normal(D).astype(np.float32)
    z = np.broadcast_to(v, (1, N, N, D)).copy()
    w = _weights(D, C, random_ln=True)
    r = oracle.trimul_full(z, None, w, direction, dumps=True)
    alpha, beta = r["a"][0, 0, 0], r["b"][0, 0, 0]
    np.testing.assert_allclose(r["o"][0], np.broadcast_to(N * alpha * beta, (N, N, C)),
                               rtol=1e-13)
    # every pair computes the same arithmetic: every output row is bitwise the same
    assert (r["out"][0] == r["out"][0, 0, 0]).all()


# ----------------------------------------------------------------------------
# P3: incoming on z is outgoing on the transposed pair grid
# ----------------------------------------------------------------------------
def test_transpose_identity():
    B, N, D, C = 2, 7, 16, 16
    z = _rand_z(B, N, D, seed=16)
    tm = np.ones(N, np.float32)
    tm[3] = 0
    mask = np.broadcast_to(np.outer(tm, np.ones(N, np.float32)), (B, N, N)).copy()  # non-symmetric
    w = _weights(D, C, random_ln=True)
    zt = np.ascontiguousarray(z.transpose(0, 2, 1, 3))
    mt = np.ascontiguousarray(mask.transpose(0, 2, 1))
    r_in = oracle.trimul_full(z, mask, w, "incoming", dumps=True)
    r_out = oracle.trimul_full(zt, mt, w, "outgoing", dumps=True)
    np.testing.assert_array_equal(r_in["o"], r_out["o"])
    w0 = w.replace(g_out=np.zeros_like(w.g_out))  # output gate = 1/2 everywhere
    np.testing.assert_array_equal(oracle.trimul_full(z, mask, w0, "incoming"),
                                  oracle.trimul_full(zt, mt, w0, "outgoing"))


# ----------------------------------------------------------------------------
# P4: permutation equivariance
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_permutation_equivariance(direction):
    B, N, D, C = 1, 8, 16, 8
    z = _rand_z(B, N, D, seed=17)
    tm = np.ones(N, np.float32)
    tm[[1, 6]] = 0
    mask = np.outer(tm, tm)[None].copy()
    w = _weights(D, C, random_ln=True)
    pi = np.random.default_rng(3).permutation(N)
    zp = z[:, pi][:, :, pi].copy()
    mp = mask[:, pi][:, :, pi].copy()
    out = oracle.trimul_full(z, mask, w, direction)
    outp = oracle.trimul_full(zp, mp, w, direction)
    np.testing.assert_allclose(outp, out[:, pi][:, :, pi], rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------
# P5: the mask
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_mask_compaction_and_garbage(direction):
    B, N, D, C = 1, 9, 16, 8
    z = _rand_z(B, N, D, seed=18)
    tm = np.ones(N, np.float32)
    dead = [2, 7, 8]
    tm[dead] = 0
    mask = np.outer(tm, tm)[None].copy()
    w = _weights(D, C, random_ln=True)
    out = oracle.trimul_full(z, mask, w, direction)
    keep = np.nonzero(tm)[0]
    # (i) deleting the masked tokens leaves the kept outputs bitwise unchanged
    zk = z[:, keep][:, :, keep].copy()
    outk = oracle.trimul_full(zk, None, w, direction)
    np.testing.assert_array_equal(outk, out[:, keep][:, :, keep])
    # (ii) garbage at masked pairs changes nothing on kept pairs
    zg = z.copy()
    junk = _rand_z(B, N, D, seed=19, scale=50.0)
    sel = mask == 0
    zg[sel] = junk[sel]
    outg = oracle.trimul_full(zg, mask, w, direction)
    np.testing.assert_array_equal(outg[:, keep][:, :, keep], out[:, keep][:, :, keep])
    # (iii) with beta_out = 0, every pair that touches a masked token outputs exactly 0
    w0 = w.replace(ln_out_b=np.zeros_like(w.ln_out_b))
    out0 = oracle.trimul_full(z, mask, w0, direction)
    assert (out0[0][dead, :] == 0).all() and (out0[0][:, dead] == 0).all()


# ----------------------------------------------------------------------------
# Grid mode agrees with full mode (same arithmetic order: bitwise)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_grid_equals_full(direction):
    B, N, D, C = 2, 12, 32, 16
    z = _rand_z(B, N, D, seed=20)
    tm = np.ones(N, np.float32)
    tm[10:] = 0
    mask = np.broadcast_to(np.outer(tm, tm), (B, N, N)).copy()
    w = _weights(D, C, random_ln=True)
    full = oracle.trimul_full(z, mask, w, direction, dumps=True)
    I, J = [0, 3, 11], [1, 2, 9, 10]
    for b in range(B):
        zA, mA, zB, mB, zG = oracle.gather_grid(z, mask, b, I, J, direction)
        out, o = oracle.trimul_grid(N, w, zA, mA, zB, mB, zG, want_o=True)
        np.testing.assert_array_equal(out, full["out"][b][np.ix_(I, J)])
        np.testing.assert_array_equal(o, full["o"][b][np.ix_(I, J)])
    # and the torch-tensor gather path gives the same
    zt, mt = torch.as_tensor(z), torch.as_tensor(mask)
    a1 = oracle.gather_grid(zt, mt, 1, I, J, direction)
    a2 = oracle.gather_grid(z, mask, 1, I, J, direction)
    for u, v in zip(a1, a2):
        np.testing.assert_array_equal(u, v)


# ----------------------------------------------------------------------------
# P1: end to end against a composition of library routines on tiny inputs
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("direction", ["outgoing", "incoming"])
def test_tiny_end_to_end_library_composition(direction):
    B, N, D, C = 2, 5, 8, 4
    z = _rand_z(B, N, D, seed=21)
    tm = np.array([1, 1, 0, 1, 1], np.float32)
    mask = np.broadcast_to(np.outer(tm, tm), (B, N, N)).copy()
    w = _weights(D, C, random_ln=True)
    T = lambda a: torch.as_tensor(np.asarray(a, np.float64))
    zt = T(z)
    x = torch.nn.functional.layer_norm(zt, (D,), T(w.ln_in_w), T(w.ln_in_b), w.eps)
    p, g = x @ T(w.p_in).T, x @ T(w.g_in).T
    m = T(mask)[..., None]
    a = m * p[..., :C] * torch.sigmoid(g[..., :C])
    b = m * p[..., C:] * torch.sigmoid(g[..., C:])
    A, Bc = a.permute(0, 3, 1, 2), b.permute(0, 3, 1, 2)  # [B, C, N, N]
    o = A @ Bc.transpose(-1, -2) if direction == "outgoing" else A.transpose(-1, -2) @ Bc
    o = o.permute(0, 2, 3, 1)
    y = torch.nn.functional.layer_norm(o, (C,), T(w.ln_out_w), T(w.ln_out_b), w.eps)
    ref = (y @ T(w.p_out).T) * torch.sigmoid(x @ T(w.g_out).T)
    np.testing.assert_allclose(oracle.trimul_full(z, mask, w, direction), ref.numpy(),
                               rtol=1e-11, atol=1e-12)


def test_rejects_bad_arguments():
    w = _weights(16, 8)
    with pytest.raises(ValueError):
        oracle.trimul_full(_rand_z(1, 3, 16), None, w, "sideways")
    with pytest.raises(ValueError):
        oracle.trimul_full(_rand_z(1, 3, 16), np.ones((1, 3, 4), np.float32), w, 0)


def test_output_stage_matches_full_mode():
    """The stand-alone output stage reproduces full mode from the same o (values exact in float)."""
    B, N, D, C = 1, 5, 32, 16
    z = _rand_z(B, N, D, seed=22)
    w = _weights(D, C, random_ln=True)
    r = oracle.trimul_full(z, None, w, "outgoing", dumps=True)
    o32 = r["o"].astype(np.float32)
    out = oracle.output_stage(z, o32, w)
    ref = _ln_lib(o32.astype(np.float64), w.ln_out_w, w.ln_out_b, w.eps)
    ref = (ref @ w.p_out.astype(np.float64).T) * expit(r["x"] @ w.g_out.astype(np.float64).T)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
