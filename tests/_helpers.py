"""Shared helpers of the GPU tests: seeded inputs on the device, the oracle
check (full or sampled grid) and the normalised error metric."""
import sys

import numpy as np
import torch

import oracle
from triangle_multiplication_amd import inputs


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref):
    """max |got - ref| / max |ref| over all elements."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def workload_inputs(wl, device="cuda", random_ln=False):
    """z, pair mask (or None) on the device, and the host weights of a workload."""
    dev = torch.device(device)
    if wl.N <= 1024:
        z = inputs.make_z(wl.B, wl.N, wl.D, wl.dtype, var=wl.z_var, device="cpu").to(dev)
    else:
        z = inputs.make_z(wl.B, wl.N, wl.D, wl.dtype, var=wl.z_var, device=dev)
    tm = wl.token_mask()
    mask = None if tm is None else inputs.pair_mask(tm, wl.B, wl.dtype, device=dev)
    w = inputs.make_weights(wl.D, wl.C, wl.dtype, random_ln=random_ln)
    return z, mask, w


def oracle_check(z, mask, w, direction, out, full=True, n_sample=64, extra=()):
    """Normalised max error of ``out`` (device tensor) against the oracle.

    full: every output (oracle full mode).  Otherwise a seeded grid of
    n_sample rows x n_sample columns per batch element (oracle grid mode).
    """
    B, N = int(z.shape[0]), int(z.shape[1])
    if full:
        ref = oracle.trimul_full(z.float().cpu().numpy(), None if mask is None else mask.float().cpu().numpy(),
                                 w, direction)
        return rel_err(out.float().cpu().numpy(), ref)
    worst_num, worst_den = 0.0, 0.0
    for b in range(B):
        I, J = inputs.sample_grid(N, n_sample, extra=extra)
        zA, mA, zB, mB, zG = oracle.gather_grid(z, mask, b, I, J, direction)
        ref = oracle.trimul_grid(N, w, zA, mA, zB, mB, zG)
        Ii = torch.as_tensor(I, device=out.device)
        Jj = torch.as_tensor(J, device=out.device)
        got = out[b].index_select(0, Ii).index_select(1, Jj).float().cpu().numpy()
        worst_num = max(worst_num, float(np.abs(got - ref).max()))
        worst_den = max(worst_den, float(np.abs(ref).max()))
    return worst_num / (worst_den if worst_den > 0 else 1.0)


def _to_ab_storage(x, dtype):
    """Plain [B, C, N, N] (row, k) tensor -> the stage buffers' storage
    (include/trimul_internal.h): bf16 K-blocked [B, C, Kp/32, N, 32] with the
    k >= N padding filled with NaN (never read), fp32 unchanged."""
    if dtype != "bf16":
        return x.contiguous()
    B, C, N, _ = x.shape
    kp = (N + 31) // 32 * 32
    xp = torch.full((B, C, N, kp), float("nan"), dtype=x.dtype, device=x.device)
    xp[..., :N] = x
    return xp.view(B, C, N, kp // 32, 32).permute(0, 1, 3, 2, 4).contiguous()


def _from_ab_storage(x, dtype):
    """Inverse of _to_ab_storage: storage -> plain [B, C, N, N]."""
    if dtype != "bf16":
        return x
    B, C, nb, N, _ = x.shape
    return x.permute(0, 1, 3, 2, 4).reshape(B, C, N, nb * 32)[..., :N]


def _exact_contract_reference(a, b, rows=None, chans=None):
    """RNE-rounded exact integer sums sum_k a[c,i,k] b[c,j,k] in float64 on the device."""
    A = a if chans is None else a[:, chans]
    Bm = b if chans is None else b[:, chans]
    if rows is not None:
        A = A[:, :, rows]
    ref = torch.matmul(A.double(), Bm.double().transpose(-1, -2).contiguous())
    return ref
