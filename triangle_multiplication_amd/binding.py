"""Thin ctypes binding of libtrimul (``include/trimul.h``).

Argument marshalling only: torch tensors become device pointers, the current
torch stream becomes the hipStream_t, and status codes become exceptions.
Every step of the computation runs in the library's HIP kernels.  Importing
this module loads ``libtrimul.so`` and raises if it has not been built; there
is no fallback.
"""
import ctypes
import os

import numpy as np
# torch must be loaded first: its HIP runtime (libamdhip64, SONAME .so.7) is the
# one libtrimul binds to.  Loading libtrimul first would pull in a second copy
# of the runtime from /opt/rocm, which then finds no device.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtrimul.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libtrimul.so is not built (expected at %s); run "
                      "`python -c 'import __graft_entry__ as g; g.build()'`" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)

TRIMUL_OK, TRIMUL_ERR_INVALID_ARG, TRIMUL_ERR_UNSUPPORTED, TRIMUL_ERR_ARCH, \
    TRIMUL_ERR_WORKSPACE, TRIMUL_ERR_HIP = range(6)
TRIMUL_BF16, TRIMUL_FP32 = 0, 1
TRIMUL_OUTGOING, TRIMUL_INCOMING = 0, 1
DTYPES = {"bf16": TRIMUL_BF16, "fp32": TRIMUL_FP32}
DIRECTIONS = {"outgoing": TRIMUL_OUTGOING, "incoming": TRIMUL_INCOMING,
              0: TRIMUL_OUTGOING, 1: TRIMUL_INCOMING}

EXPORTED = ["trimul_create", "trimul_destroy", "trimul_workspace_size", "trimul_workspace_query",
            "trimul_workspace_size_lean", "trimul_fwd", "trimul_fwd_noalloc", "trimul_tune", "trimul_check_arch",
            "trimul_status_string", "trimul_last_error",
            "trimul_internal_project", "trimul_internal_mask_ranges", "trimul_internal_contract",
            "trimul_internal_output", "trimul_internal_set_plan", "trimul_internal_get_plan",
            "trimul_internal_plan_candidates", "trimul_internal_cache_store",
            "trimul_internal_cache_lookup", "trimul_internal_cache_path",
            "trimul_internal_peak_mfma", "trimul_internal_peak_stream"]


class trimul_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.POINTER(ctypes.c_float)) for n in
                ("norm_in_weight", "norm_in_bias", "p_in", "g_in", "norm_out_weight",
                 "norm_out_bias", "p_out", "g_out")] + [("eps", ctypes.c_float)]


_vp, _ci, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_lib.trimul_create.argtypes = [_ci, _ci, _ci, ctypes.POINTER(trimul_weights), ctypes.POINTER(_vp)]
_lib.trimul_create.restype = _ci
_lib.trimul_destroy.argtypes = [_vp]
_lib.trimul_destroy.restype = None
_lib.trimul_workspace_size.argtypes = [_vp, _ci, _ci, ctypes.POINTER(_sz)]
_lib.trimul_workspace_size.restype = _ci
_lib.trimul_workspace_query.argtypes = [_ci, _ci, _ci, _ci, _ci, ctypes.POINTER(_sz)]
_lib.trimul_workspace_query.restype = _ci
_lib.trimul_workspace_size_lean.argtypes = [_vp, _ci, _ci, ctypes.POINTER(_sz)]
_lib.trimul_workspace_size_lean.restype = _ci
_lib.trimul_fwd.argtypes = [_vp, _vp, _vp, _ci, _ci, _ci, _vp, _vp, _sz, _vp]
_lib.trimul_fwd.restype = _ci
_lib.trimul_fwd_noalloc.argtypes = [_vp, _vp, _vp, _ci, _ci, _ci, _vp, _vp]
_lib.trimul_fwd_noalloc.restype = _ci
NOALLOC_MAX_BYTES = 128 << 20   # TRIMUL_NOALLOC_MAX_BYTES in include/trimul.h
_lib.trimul_tune.argtypes = [_vp, _vp, _vp, _ci, _ci, _ci, _vp, _vp, _sz, _vp]
_lib.trimul_tune.restype = _ci
_lib.trimul_check_arch.argtypes = [ctypes.c_char_p]
_lib.trimul_check_arch.restype = _ci
_lib.trimul_status_string.argtypes = [_ci]
_lib.trimul_status_string.restype = ctypes.c_char_p
_lib.trimul_last_error.argtypes = []
_lib.trimul_last_error.restype = ctypes.c_char_p
_lib.trimul_internal_project.argtypes = [_vp, _vp, _vp, _ci, _ci, _ci, _vp, _vp, _vp]
_lib.trimul_internal_project.restype = _ci
_lib.trimul_internal_mask_ranges.argtypes = [_vp, _vp, _ci, _ci, _ci, _vp, _vp]
_lib.trimul_internal_mask_ranges.restype = _ci
_lib.trimul_internal_contract.argtypes = [_vp, _vp, _vp, _vp, _ci, _ci, _ci, _vp, _vp]
_lib.trimul_internal_contract.restype = _ci
_lib.trimul_internal_output.argtypes = [_vp, _vp, _vp, _ci, _ci, _vp, _vp]
_lib.trimul_internal_output.restype = _ci
_ip = ctypes.POINTER(_ci)
_lib.trimul_internal_set_plan.argtypes = [_vp, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _ci]
_lib.trimul_internal_set_plan.restype = _ci
_lib.trimul_internal_get_plan.argtypes = [_vp, _ci, _ci, _ci, _ci, _ip, _ip, _ip, _ip]
_lib.trimul_internal_get_plan.restype = _ci
_lib.trimul_internal_plan_candidates.argtypes = [_ip, _ip, _ip, _ip, _ci]
_lib.trimul_internal_plan_candidates.restype = _ci
_lib.trimul_internal_cache_store.argtypes = [ctypes.c_char_p, ctypes.c_char_p] + [_ci] * 11 + [ctypes.c_double]
_lib.trimul_internal_cache_store.restype = _ci
_lib.trimul_internal_cache_lookup.argtypes = [ctypes.c_char_p, ctypes.c_char_p] + [_ci] * 7 + [_ip, _ip, _ip, _ip]
_lib.trimul_internal_cache_lookup.restype = _ci
_lib.trimul_internal_cache_path.argtypes = [ctypes.c_char_p, _ci]
_lib.trimul_internal_cache_path.restype = _ci
_lib.trimul_internal_peak_mfma.argtypes = [_vp, _ci, _ci, _ci, _vp, _vp]
_lib.trimul_internal_peak_mfma.restype = _ci
_lib.trimul_internal_peak_stream.argtypes = [_vp, _vp, _vp, _vp, _sz, _ci, _ci, _ci, _vp]
_lib.trimul_internal_peak_stream.restype = _ci


class TriMulError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        super().__init__("%s: %s" % (trimul_status_string(status), message))


def trimul_status_string(status):
    return _lib.trimul_status_string(int(status)).decode()


def trimul_last_error():
    return _lib.trimul_last_error().decode()


def _check(status):
    if status != TRIMUL_OK:
        raise TriMulError(status, trimul_last_error())


def trimul_check_arch(name):
    """Raise TriMulError unless ``name`` is a gfx950 architecture string."""
    _check(_lib.trimul_check_arch(name.encode() if name is not None else None))


def trimul_workspace_query(D, C, dtype, B, N):
    n = _sz(0)
    _check(_lib.trimul_workspace_query(D, C, DTYPES.get(dtype, dtype), B, N, ctypes.byref(n)))
    return n.value


def _f32p(a, keep):
    a = np.ascontiguousarray(np.asarray(a, np.float32))
    keep.append(a)
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def trimul_create(weights, dtype="bf16"):
    """Create a handle from host fp32 weights (a TriMulWeights-like object)."""
    keep = []
    w = trimul_weights(_f32p(weights.ln_in_w, keep), _f32p(weights.ln_in_b, keep),
                       _f32p(weights.p_in, keep), _f32p(weights.g_in, keep),
                       _f32p(weights.ln_out_w, keep), _f32p(weights.ln_out_b, keep),
                       _f32p(weights.p_out, keep), _f32p(weights.g_out, keep),
                       float(weights.eps))
    D, C = int(np.asarray(weights.ln_in_w).shape[0]), int(np.asarray(weights.ln_out_w).shape[0])
    h = _vp()
    _check(_lib.trimul_create(D, C, DTYPES.get(dtype, dtype), ctypes.byref(w), ctypes.byref(h)))
    return h


def trimul_destroy(h):
    _lib.trimul_destroy(h)


def trimul_workspace_size(h, B, N):
    n = _sz(0)
    _check(_lib.trimul_workspace_size(h, B, N, ctypes.byref(n)))
    return n.value


def trimul_workspace_size_lean(h, B, N):
    n = _sz(0)
    _check(_lib.trimul_workspace_size_lean(h, B, N, ctypes.byref(n)))
    return n.value


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def trimul_fwd(h, z, mask, direction, out, workspace, stream=None):
    """Enqueue the forward pass on ``stream`` (default: torch's current stream)."""
    B, N = int(z.shape[0]), int(z.shape[1])
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.trimul_fwd(h, _ptr(z), _ptr(mask), B, N, DIRECTIONS.get(direction, direction), _ptr(out),
                           _ptr(workspace), ws_bytes, _stream(stream)))


def trimul_fwd_noalloc(h, z, mask, direction, out, stream=None):
    """trimul_fwd with the library's static scratch array as the workspace."""
    B, N = int(z.shape[0]), int(z.shape[1])
    _check(_lib.trimul_fwd_noalloc(h, _ptr(z), _ptr(mask), B, N, DIRECTIONS.get(direction, direction),
                                   _ptr(out), _stream(stream)))


def trimul_tune(h, z, mask, direction, out, workspace, stream=None):
    """Time every candidate plan on these inputs, record the fastest, leave the
    result in ``out`` (blocking)."""
    B, N = int(z.shape[0]), int(z.shape[1])
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.trimul_tune(h, _ptr(z), _ptr(mask), B, N, DIRECTIONS.get(direction, direction), _ptr(out),
                            _ptr(workspace), ws_bytes, _stream(stream)))


def trimul_internal_mask_ranges(h, mask, direction, table, stream=None):
    B, N = int(mask.shape[0]), int(mask.shape[1])
    _check(_lib.trimul_internal_mask_ranges(h, _ptr(mask), B, N, DIRECTIONS.get(direction, direction),
                                            _ptr(table), _stream(stream)))


def mask_table_ints(B, N):
    """int32 length of the mask table (include/trimul_internal.h): ranges
    [B][T][2], a 4-int header, pair lists [B][T*T], T = ceil(N/256)."""
    T = (N + 255) // 256
    return 2 * B * T + 4 + B * T * T


def table_parts(table, B, N):
    """Views (ranges [B][T][2], header [4], pairs [B][T*T]) of a mask table."""
    T = (N + 255) // 256
    r = table[:2 * B * T].view(B, T, 2)
    hdr = table[2 * B * T:2 * B * T + 4]
    pairs = table[2 * B * T + 4:2 * B * T + 4 + B * T * T].view(B, T * T)
    return r, hdr, pairs


def trimul_internal_set_plan(h, B, N, direction, masked, plan):
    """Record plan = (k1_variant, k2_order, k2_gm, k2_tile) for the call shape."""
    k1, order, gm, tile = plan
    _check(_lib.trimul_internal_set_plan(h, B, N, DIRECTIONS.get(direction, direction), int(bool(masked)),
                                         k1, order, gm, tile))


def trimul_internal_get_plan(h, B, N, direction, masked):
    """(k1_variant, k2_order, k2_gm, k2_tile) that trimul_fwd uses for the call shape."""
    v, o, g, t = _ci(0), _ci(0), _ci(0), _ci(0)
    _check(_lib.trimul_internal_get_plan(h, B, N, DIRECTIONS.get(direction, direction), int(bool(masked)),
                                         ctypes.byref(v), ctypes.byref(o), ctypes.byref(g), ctypes.byref(t)))
    return v.value, o.value, g.value, t.value


def plan_candidates():
    n = _lib.trimul_internal_plan_candidates(None, None, None, None, 0)
    v, o, g, t = (_ci * n)(), (_ci * n)(), (_ci * n)(), (_ci * n)()
    _lib.trimul_internal_plan_candidates(v, o, g, t, n)
    return [(v[i], o[i], g[i], t[i]) for i in range(n)]


def cache_store(path, device, D, C, dtype, B, N, direction, masked, plan, ms):
    k1, order, gm, tile = plan
    _check(_lib.trimul_internal_cache_store(path.encode(), device.encode(), D, C, DTYPES.get(dtype, dtype), B, N,
                                            DIRECTIONS.get(direction, direction), int(bool(masked)),
                                            k1, order, gm, tile, float(ms)))


def cache_lookup(path, device, D, C, dtype, B, N, direction, masked):
    """(k1_variant, k2_order, k2_gm, k2_tile) recorded for the key, None if
    absent; raises OSError if the file cannot be read."""
    v, o, g, t = _ci(0), _ci(0), _ci(0), _ci(0)
    r = _lib.trimul_internal_cache_lookup(path.encode(), device.encode(), D, C, DTYPES.get(dtype, dtype), B, N,
                                          DIRECTIONS.get(direction, direction), int(bool(masked)),
                                          ctypes.byref(v), ctypes.byref(o), ctypes.byref(g), ctypes.byref(t))
    if r < 0:
        raise OSError("plan cache %s cannot be read" % path)
    return (v.value, o.value, g.value, t.value) if r else None


def cache_path():
    n = _lib.trimul_internal_cache_path(None, 0)
    buf = ctypes.create_string_buffer(n + 1)
    _lib.trimul_internal_cache_path(buf, n + 1)
    return buf.value.decode()


def trimul_internal_project(h, z, mask, direction, a_cm, b_cm, stream=None):
    B, N = int(z.shape[0]), int(z.shape[1])
    _check(_lib.trimul_internal_project(h, _ptr(z), _ptr(mask), B, N, DIRECTIONS.get(direction, direction),
                                        _ptr(a_cm), _ptr(b_cm), _stream(stream)))


def ab_storage_shape(dtype, B, C, N):
    """Tensor shape of the stage buffers a_cm, b_cm (include/trimul_internal.h):
    bf16 is K-blocked, [B][C][Kp/32][N][32] with Kp = N rounded up to 32;
    fp32 is plain [B][C][N][N]."""
    if dtype == "bf16":
        return (B, C, (N + 31) // 32, N, 32)
    return (B, C, N, N)


def trimul_internal_contract(h, a_cm, b_cm, o, table=None, direction="outgoing", stream=None):
    B, N = int(o.shape[0]), int(o.shape[2])
    _check(_lib.trimul_internal_contract(h, _ptr(a_cm), _ptr(b_cm), _ptr(table), B, N,
                                         DIRECTIONS.get(direction, direction), _ptr(o), _stream(stream)))


def trimul_internal_output(h, z, o, out, stream=None):
    B, N = int(z.shape[0]), int(z.shape[1])
    _check(_lib.trimul_internal_output(h, _ptr(z), _ptr(o), B, N, _ptr(out), _stream(stream)))


def trimul_internal_peak_mfma(seed, blocks, iters, sink, shape=0, stream=None):
    """MFMA-only loop (shape 0: 16x16x32, 1: 32x32x16 bf16 MFMAs): seed is 4096
    bytes of bf16 operands, sink a float32 tensor of at least blocks * 256
    elements; 4 * 262144 * iters * blocks FLOP."""
    if seed.numel() * seed.element_size() < 4096:
        raise ValueError("seed must hold 4096 bytes")
    if sink.dtype.itemsize != 4 or sink.numel() < blocks * 256:
        raise ValueError("sink must hold blocks * 256 float32 values")
    _check(_lib.trimul_internal_peak_mfma(_ptr(seed), int(blocks), int(iters), int(shape), _ptr(sink),
                                          _stream(stream)))


def trimul_internal_peak_stream(src0, dst0, src1=None, dst1=None, nontemporal=False, stream=None):
    """Stream 16-byte chunks: dst0 (and dst1) = src0 (xor src1); all given
    tensors must have the byte size of src0, a multiple of 16."""
    nbytes = src0.numel() * src0.element_size()
    for t in (dst0, src1, dst1):
        if t is not None and t.numel() * t.element_size() != nbytes:
            raise ValueError("stream buffers must have equal byte sizes")
    if nbytes % 16:
        raise ValueError("stream buffers must be a multiple of 16 bytes")
    _check(_lib.trimul_internal_peak_stream(_ptr(src0), _ptr(src1), _ptr(dst0), _ptr(dst1), nbytes // 16,
                                            2 if src1 is not None else 1, 2 if dst1 is not None else 1,
                                            1 if nontemporal else 0, _stream(stream)))


class TriMul:
    """One layer on the current device: owns a handle and a cached workspace.

    ``forward(z, mask, direction)`` returns a new [B, N, N, D] tensor (or fills
    ``out``).  Tensors must be contiguous, on the device the handle was created
    on, in the handle's dtype.  Calls through one TriMul object share its cached
    workspace, so they must not overlap in time on different streams; for
    concurrent calls, pass each its own workspace to ``trimul_fwd`` (the handle
    itself is read-only after create).
    """

    # Device type every tensor argument must live on.
    device_type = "cuda"

    def __init__(self, weights, dtype="bf16"):
        import torch
        self.dtype = dtype
        self.tdtype = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
        self.D = int(np.asarray(weights.ln_in_w).shape[0])
        self.C = int(np.asarray(weights.ln_out_w).shape[0])
        self.h = trimul_create(weights, dtype)
        self._ws = None

    def workspace(self, B, N, device):
        import torch
        need = trimul_workspace_size(self.h, B, N)
        if self._ws is None or self._ws.numel() < need or self._ws.device != device:
            self._ws = None
            self._ws = torch.empty(need, dtype=torch.uint8, device=device)
        return self._ws

    def _check_tensor(self, t, name, shape, device=None):
        """Raise ValueError unless t is a contiguous tensor of the handle's dtype
        with exactly ``shape``, on this layer's device type (and on ``device``
        if given).  The kernels index every tensor as dense row-major with the
        sizes the shape implies, so anything else must be refused here."""
        if (t.dtype != self.tdtype or not t.is_contiguous() or t.device.type != self.device_type
                or tuple(t.shape) != tuple(shape) or (device is not None and t.device != device)):
            raise ValueError("%s must be a contiguous %s %s tensor of shape %s%s; got %s %s on %s%s"
                             % (name, self.tdtype, self.device_type, tuple(shape),
                                "" if device is None else " on " + str(device), t.dtype,
                                tuple(t.shape), t.device, "" if t.is_contiguous() else " (strided)"))

    def forward(self, z, mask=None, direction="outgoing", out=None, stream=None):
        import torch
        if z.dim() != 4:
            raise ValueError("z must be [B, N, N, D]; got shape %s" % (tuple(z.shape),))
        B, N = int(z.shape[0]), int(z.shape[1])
        self._check_tensor(z, "z", (B, N, N, self.D))
        if mask is not None:
            self._check_tensor(mask, "mask", (B, N, N), z.device)
        if out is not None:
            self._check_tensor(out, "out", (B, N, N, self.D), z.device)
        else:
            out = torch.empty_like(z)
        ws = self.workspace(B, N, z.device)
        trimul_fwd(self.h, z, mask, direction, out, ws, stream)
        return out

    __call__ = forward

    def project(self, z, mask=None, direction="outgoing"):
        import torch
        B, N = int(z.shape[0]), int(z.shape[1])
        self._check_tensor(z, "z", (B, N, N, self.D))
        if mask is not None:
            self._check_tensor(mask, "mask", (B, N, N), z.device)
        a = torch.empty(ab_storage_shape(self.dtype, B, self.C, N), dtype=self.tdtype, device=z.device)
        b = torch.empty_like(a)
        trimul_internal_project(self.h, z, mask, direction, a, b)
        return a, b

    def contract(self, a_cm, b_cm, table=None, direction="outgoing"):
        import torch
        B, N = int(a_cm.shape[0]), int(a_cm.shape[-2])
        shape = ab_storage_shape(self.dtype, B, self.C, N)
        self._check_tensor(a_cm, "a_cm", shape)
        self._check_tensor(b_cm, "b_cm", shape, a_cm.device)
        if table is not None and (table.dtype != torch.int32 or not table.is_contiguous()
                                  or tuple(table.shape) != (mask_table_ints(B, N),)
                                  or table.device != a_cm.device):
            raise ValueError("table must be a contiguous int32 tensor of %d elements on %s"
                             % (mask_table_ints(B, N), a_cm.device))
        o = torch.empty((B, self.C, N, N), dtype=self.tdtype, device=a_cm.device)
        trimul_internal_contract(self.h, a_cm, b_cm, o, table, direction)
        return o

    def mask_ranges(self, mask, direction="outgoing"):
        """The mask table with its ranges filled (include/trimul_internal.h)."""
        import torch
        B, N = int(mask.shape[0]), int(mask.shape[1])
        self._check_tensor(mask, "mask", (B, N, N))
        t = torch.zeros(mask_table_ints(B, N), dtype=torch.int32, device=mask.device)
        trimul_internal_mask_ranges(self.h, mask, direction, t)
        return t

    def tune(self, z, mask=None, direction="outgoing", out=None, stream=None):
        """trimul_tune on these inputs; returns the output tensor."""
        import torch
        B, N = int(z.shape[0]), int(z.shape[1])
        self._check_tensor(z, "z", (B, N, N, self.D))
        if mask is not None:
            self._check_tensor(mask, "mask", (B, N, N), z.device)
        if out is not None:
            self._check_tensor(out, "out", (B, N, N, self.D), z.device)
        else:
            out = torch.empty_like(z)
        ws = self.workspace(B, N, z.device)
        trimul_tune(self.h, z, mask, direction, out, ws, stream)
        return out

    def output(self, z, o):
        import torch
        B, N = int(z.shape[0]), int(z.shape[1])
        self._check_tensor(z, "z", (B, N, N, self.D))
        self._check_tensor(o, "o", (B, self.C, N, N), z.device)
        out = torch.empty_like(z)
        trimul_internal_output(self.h, z, o, out)
        return out

    def close(self):
        if getattr(self, "h", None):
            trimul_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
