"""ctypes marshalling for the C oracle (test infrastructure only).

No arithmetic of the method is done here: arrays are checked for shape, made
contiguous float32 (inputs) or allocated float64 (outputs) and handed to
``trimul_oracle.c``.  ``gather_grid`` only indexes z and the mask to collect
the vectors the grid mode reads.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "trimul_oracle.c")
_LIB = os.path.join(_HERE, "liborc_trimul.so")
_lib = None


def lib_path():
    return _LIB


def build(force=True):
    """Compile the oracle with gcc -O2 -fopenmp (plain IEEE double, no fast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # TRIMUL_ORACLE_LIB lets the mutation test point the pins at a
        # deliberately broken build of this same source.
        path = os.environ.get("TRIMUL_ORACLE_LIB")
        if not path:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            path = _LIB
        lib = ctypes.CDLL(path)
        fp = ctypes.POINTER(ctypes.c_float)
        dp = ctypes.POINTER(ctypes.c_double)
        ci = ctypes.c_int
        lib.orc_trimul_full.argtypes = [ci, ci, ci, ci, ci, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp,
                                        ctypes.c_double, dp, dp, dp, dp, dp]
        lib.orc_trimul_full.restype = ci
        lib.orc_trimul_grid.argtypes = [ci, ci, ci, ci, ci, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp,
                                        fp, fp, fp, ctypes.c_double, dp, dp, dp]
        lib.orc_trimul_grid.restype = ci
        lib.orc_output_stage.argtypes = [ctypes.c_int64, ci, ci, fp, fp, fp, fp, fp, fp, fp, fp,
                                         ctypes.c_double, dp]
        lib.orc_output_stage.restype = ci
        lib.orc_max_threads.argtypes = []
        lib.orc_max_threads.restype = ci
        _lib = lib
    return _lib


def max_threads():
    return int(_load().orc_max_threads())


def _f32(a, shape=None):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    if shape is not None and tuple(a.shape) != tuple(shape):
        raise ValueError("expected shape %s, got %s" % (tuple(shape), tuple(a.shape)))
    return a


def _fp(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _dp(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _weights(w, D, C):
    return [
        _f32(w.ln_in_w, (D,)), _f32(w.ln_in_b, (D,)),
        _f32(w.p_in, (2 * C, D)), _f32(w.g_in, (2 * C, D)),
        _f32(w.ln_out_w, (C,)), _f32(w.ln_out_b, (C,)),
        _f32(w.p_out, (D, C)), _f32(w.g_out, (D, D)),
    ]


def _to_np(t):
    if hasattr(t, "detach"):
        t = t.detach().to("cpu")
        import torch  # only for dtype conversion of tensors handed in
        t = t.to(torch.float32).numpy()
    return t


def trimul_full(z, mask, w, direction, dumps=False):
    """Every output of TriMul for z [B,N,N,D] (float values), mask [B,N,N] or None.

    direction: 0/"outgoing" or 1/"incoming".  Returns out [B,N,N,D] float64, or a
    dict with out and the stage dumps x, a, b (pair layout a_bijc) and o when
    ``dumps`` is true.
    """
    lib = _load()
    z = _f32(_to_np(z))
    B, N, N2, D = z.shape
    assert N == N2
    C = int(np.asarray(w.ln_out_w).shape[0])
    m = None if mask is None else _f32(_to_np(mask), (B, N, N))
    d = _dir(direction)
    W = _weights(w, D, C)
    out = np.empty((B, N, N, D), np.float64)
    x = a = b = o = None
    if dumps:
        x = np.empty((B, N, N, D), np.float64)
        a = np.empty((B, N, N, C), np.float64)
        b = np.empty((B, N, N, C), np.float64)
        o = np.empty((B, N, N, C), np.float64)
    rc = lib.orc_trimul_full(B, N, D, C, d, _fp(z), _fp(m), *[_fp(t) for t in W],
                             float(w.eps), _dp(out), _dp(x), _dp(a), _dp(b), _dp(o))
    if rc != 0:
        raise RuntimeError("orc_trimul_full failed (%d)" % rc)
    if dumps:
        return {"out": out, "x": x, "a": a, "b": b, "o": o}
    return out


def _dir(direction):
    if direction in (0, "outgoing"):
        return 0
    if direction in (1, "incoming"):
        return 1
    raise ValueError("direction must be outgoing/0 or incoming/1")


def gather_grid(z, mask, bidx, I, J, direction):
    """Collect the z vectors and mask values the grid mode reads, for batch bidx.

    z may be a numpy array or a torch tensor (on any device); only the needed
    slices are copied to the host.  Returns (zA, mA, zB, mB, zG) as float32
    numpy arrays (mA, mB None when mask is None).
    """
    d = _dir(direction)
    I = [int(i) for i in I]
    J = [int(j) for j in J]
    is_torch = hasattr(z, "detach")
    if is_torch:
        import torch
        dev = z.device
        Ii = torch.tensor(I, device=dev, dtype=torch.long)
        Jj = torch.tensor(J, device=dev, dtype=torch.long)
        zb = z[bidx]
        if d == 0:
            zA, zB = zb.index_select(0, Ii), zb.index_select(0, Jj)
        else:
            zA = zb.index_select(1, Ii).transpose(0, 1)
            zB = zb.index_select(1, Jj).transpose(0, 1)
        zG = zb.index_select(0, Ii).index_select(1, Jj)
        mA = mB = None
        if mask is not None:
            mb = mask[bidx]
            if d == 0:
                mA, mB = mb.index_select(0, Ii), mb.index_select(0, Jj)
            else:
                mA = mb.index_select(1, Ii).transpose(0, 1)
                mB = mb.index_select(1, Jj).transpose(0, 1)
        conv = lambda t: None if t is None else _f32(t.contiguous().to(torch.float32).cpu().numpy())
        return conv(zA), conv(mA), conv(zB), conv(mB), conv(zG)
    z = np.asarray(z)
    zb = z[bidx]
    if d == 0:
        zA, zB = zb[I], zb[J]
    else:
        zA, zB = zb[:, I].transpose(1, 0, 2), zb[:, J].transpose(1, 0, 2)
    zG = zb[np.ix_(I, J)]
    mA = mB = None
    if mask is not None:
        mb = np.asarray(mask)[bidx]
        if d == 0:
            mA, mB = mb[I], mb[J]
        else:
            mA, mB = mb[:, I].T, mb[:, J].T
    conv = lambda t: None if t is None else _f32(t)
    return conv(zA), conv(mA), conv(zB), conv(mB), conv(zG)


def trimul_grid(N, w, zA, mA, zB, mB, zG, want_o=False, want_times=False):
    """Outputs at an I x J grid of one batch element from gathered inputs.

    Returns out [ni,nj,D] float64 (plus o [ni,nj,C] and/or the per-stage wall
    seconds {projection, contraction, output} when requested).
    """
    lib = _load()
    zA = _f32(zA)
    zB = _f32(zB)
    zG = _f32(zG)
    ni, n1, D = zA.shape
    nj = zB.shape[0]
    assert n1 == N and zB.shape == (nj, N, D) and zG.shape == (ni, nj, D)
    C = int(np.asarray(w.ln_out_w).shape[0])
    mA = None if mA is None else _f32(mA, (ni, N))
    mB = None if mB is None else _f32(mB, (nj, N))
    W = _weights(w, D, C)
    out = np.empty((ni, nj, D), np.float64)
    o = np.empty((ni, nj, C), np.float64) if want_o else None
    t = np.zeros(3, np.float64)
    rc = lib.orc_trimul_grid(N, D, C, ni, nj, _fp(zA), _fp(mA), _fp(zB), _fp(mB), _fp(zG),
                             *[_fp(x) for x in W], float(w.eps), _dp(out), _dp(o), _dp(t))
    if rc != 0:
        raise RuntimeError("orc_trimul_grid failed (%d)" % rc)
    res = [out]
    if want_o:
        res.append(o)
    if want_times:
        res.append(t)
    return res[0] if len(res) == 1 else tuple(res)


def output_stage(z, o, w):
    """Output stage alone for pairs: z [..., D] and o [..., C] (same leading shape).

    Returns out [..., D] float64.
    """
    lib = _load()
    z = _f32(_to_np(z))
    o = _f32(_to_np(o))
    D, C = z.shape[-1], o.shape[-1]
    lead = z.shape[:-1]
    assert o.shape[:-1] == lead
    P = int(np.prod(lead)) if len(lead) else 1
    W = _weights(w, D, C)
    out = np.empty(lead + (D,), np.float64)
    Wp = [_fp(t) for t in W]
    rc = lib.orc_output_stage(P, D, C, _fp(z), _fp(o), Wp[0], Wp[1], Wp[4], Wp[5], Wp[6], Wp[7],
                              float(w.eps), _dp(out))
    if rc != 0:
        raise RuntimeError("orc_output_stage failed (%d)" % rc)
    return out
