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
