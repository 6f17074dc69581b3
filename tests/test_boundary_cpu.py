"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point the headers declare, and rejects bad arguments with the
documented status codes before touching a device."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

from triangle_multiplication_amd import binding as tb
from triangle_multiplication_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(trimul_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert "trimul_fwd" in names and "trimul_create" in names and "trimul_destroy" in names
    lib = ctypes.CDLL(tb.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), "libtrimul does not export " + n
    assert set(names) == set(tb.EXPORTED)


def test_status_strings():
    for code, name in enumerate(["TRIMUL_OK", "TRIMUL_ERR_INVALID_ARG", "TRIMUL_ERR_UNSUPPORTED",
                                 "TRIMUL_ERR_ARCH", "TRIMUL_ERR_WORKSPACE", "TRIMUL_ERR_HIP"]):
        assert tb.trimul_status_string(code) == name
    assert tb.trimul_status_string(99) == "TRIMUL_ERR_UNKNOWN"


@pytest.mark.parametrize("name", ["gfx950", "gfx950:sramecc+:xnack-", "gfx950:xnack+"])
def test_arch_gate_accepts_gfx950(name):
    tb.trimul_check_arch(name)


@pytest.mark.parametrize("name", ["gfx942", "gfx942:sramecc+:xnack-", "gfx90a", "gfx9500", "gfx95", ""])
def test_arch_gate_refuses_others(name):
    with pytest.raises(tb.TriMulError) as e:
        tb.trimul_check_arch(name)
    assert e.value.status == tb.TRIMUL_ERR_ARCH
    assert "requires gfx950" in str(e.value) and ("got " + name) in str(e.value)


def test_arch_gate_null():
    with pytest.raises(tb.TriMulError) as e:
        tb.trimul_check_arch(None)
    assert e.value.status == tb.TRIMUL_ERR_INVALID_ARG


def test_workspace_query_sizes():
    # a and b: B*C*N*Kp elements (bf16: Kp = N rounded up to 32; fp32: Kp = N),
    # o: B*C*N*N elements, the mask table (int32);
    # each rounded up to 256 bytes
    def r256(x):
        return (x + 255) // 256 * 256

    def rt(B, N):   # the mask table: ranges [B][T][2], 4-int header, pair lists [B][T*T]
        T = (N + 255) // 256
        return r256(4 * (2 * B * T + 4 + B * T * T))
    assert tb.trimul_workspace_query(256, 256, "bf16", 1, 4096) == 3 * 256 * 4096 * 4096 * 2 + rt(1, 4096)
    assert tb.trimul_workspace_query(32, 32, "fp32", 1, 64) == 3 * 32 * 64 * 64 * 4 + rt(1, 64)
    n = tb.trimul_workspace_query(32, 64, "bf16", 3, 8)
    assert n == 2 * r256(3 * 64 * 8 * 32 * 2) + r256(3 * 64 * 8 * 8 * 2) + rt(3, 8)
    n = tb.trimul_workspace_query(64, 32, "bf16", 2, 200)
    assert n == 2 * r256(2 * 32 * 200 * 224 * 2) + r256(2 * 32 * 200 * 200 * 2) + rt(2, 200)
    n = tb.trimul_workspace_query(64, 32, "fp32", 2, 200)
    assert n == 3 * r256(2 * 32 * 200 * 200 * 4) + rt(2, 200)
    assert tb.trimul_workspace_query(128, 128, "bf16", 1, 8192) == 3 * 128 * 8192 ** 2 * 2 + rt(1, 8192)


def test_ab_storage_shape():
    assert tb.ab_storage_shape("bf16", 2, 64, 200) == (2, 64, 7, 200, 32)
    assert tb.ab_storage_shape("bf16", 1, 32, 4096) == (1, 32, 128, 4096, 32)
    assert tb.ab_storage_shape("fp32", 2, 64, 200) == (2, 64, 200, 200)


@pytest.mark.parametrize("D,C", [(48, 32), (32, 0), (288, 32), (32, 300), (16, 16)])
def test_workspace_query_unsupported_widths(D, C):
    with pytest.raises(tb.TriMulError) as e:
        tb.trimul_workspace_query(D, C, "bf16", 1, 64)
    assert e.value.status == tb.TRIMUL_ERR_UNSUPPORTED


def test_workspace_query_bad_dtype_and_sizes():
    with pytest.raises(tb.TriMulError) as e:
        tb.trimul_workspace_query(32, 32, 7, 1, 64)
    assert e.value.status == tb.TRIMUL_ERR_INVALID_ARG
    with pytest.raises(tb.TriMulError) as e:
        tb.trimul_workspace_query(32, 32, "bf16", 0, 64)
    assert e.value.status == tb.TRIMUL_ERR_INVALID_ARG


def test_create_rejects_bad_widths_before_any_device_call():
    w = inputs.make_weights(48, 32)
    with pytest.raises(tb.TriMulError) as e:
        tb.trimul_create(w)
    assert e.value.status == tb.TRIMUL_ERR_UNSUPPORTED and "D=48" in str(e.value)


def test_create_rejects_bad_eps():
    w = inputs.make_weights(32, 32).replace(eps=0.0)
    with pytest.raises(tb.TriMulError) as e:
        tb.trimul_create(w)
    assert e.value.status == tb.TRIMUL_ERR_INVALID_ARG and "eps" in str(e.value)


def test_create_null_weight_pointer():
    lib = ctypes.CDLL(tb.LIB_PATH)
    lib.trimul_create.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.POINTER(tb.trimul_weights), ctypes.POINTER(ctypes.c_void_p)]
    w = tb.trimul_weights()  # all NULL
    w.eps = 1e-5
    h = ctypes.c_void_p()
    assert lib.trimul_create(32, 32, 0, ctypes.byref(w), ctypes.byref(h)) == tb.TRIMUL_ERR_INVALID_ARG
    assert "norm_in_weight" in tb.trimul_last_error()
    assert lib.trimul_create(32, 32, 0, None, ctypes.byref(h)) == tb.TRIMUL_ERR_INVALID_ARG
    assert lib.trimul_create(32, 32, 0, ctypes.byref(w), None) == tb.TRIMUL_ERR_INVALID_ARG


def test_fwd_null_handle():
    lib = ctypes.CDLL(tb.LIB_PATH)
    lib.trimul_fwd.argtypes = tb._lib.trimul_fwd.argtypes
    rc = lib.trimul_fwd(None, None, None, 1, 64, 0, None, None, 0, None)
    assert rc == tb.TRIMUL_ERR_INVALID_ARG and "handle" in tb.trimul_last_error()


def test_destroy_accepts_null():
    tb.trimul_destroy(None)


def test_create_without_device_reports_hip_error():
    """On a host with no GPU the first device query fails cleanly (no crash)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    w = inputs.make_weights(32, 32)
    with pytest.raises(tb.TriMulError) as e:
        tb.trimul_create(w)
    assert e.value.status == tb.TRIMUL_ERR_HIP


def test_product_path_does_not_reference_the_oracle():
    """Nothing under the package may import or load the oracle."""
    pkg = os.path.join(ROOT, "triangle_multiplication_amd")
    for f in glob.glob(os.path.join(pkg, "**", "*"), recursive=True):
        if os.path.isfile(f) and f.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
            text = open(f).read()
            assert "import oracle" not in text and "from oracle" not in text, f
            assert "orc_" not in text and "liborc" not in text, f


def _unbound_layer(D=32, C=32, dtype="bf16"):
    """A TriMul whose tensors live on the CPU and that has no handle: any call
    that got past the Python checks would reach the C library with a NULL
    handle and raise TriMulError, so a ValueError proves the check came first."""
    import torch
    layer = tb.TriMul.__new__(tb.TriMul)
    layer.dtype, layer.tdtype = dtype, {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    layer.D, layer.C, layer.h, layer._ws = D, C, None, None
    layer.device_type = "cpu"
    return layer


@pytest.mark.parametrize("bad", ["shape", "dtype", "strided", "small"])
def test_forward_rejects_bad_out_before_enqueueing(bad):
    import torch
    layer = _unbound_layer()
    z = torch.zeros((1, 8, 8, 32), dtype=torch.bfloat16)
    out = {"shape": torch.empty((1, 8, 8, 64), dtype=torch.bfloat16),
           "dtype": torch.empty((1, 8, 8, 32), dtype=torch.float32),
           "strided": torch.empty((1, 8, 8, 64), dtype=torch.bfloat16)[..., ::2],
           "small": torch.empty((1, 8, 4, 32), dtype=torch.bfloat16)}[bad]
    with pytest.raises(ValueError) as e:
        layer.forward(z, None, "outgoing", out=out)
    assert "out must be" in str(e.value)


def test_forward_checks_reach_the_library_when_arguments_are_good():
    import torch
    layer = _unbound_layer()
    z = torch.zeros((1, 8, 8, 32), dtype=torch.bfloat16)
    with pytest.raises(tb.TriMulError) as e:   # NULL handle: the C side refuses it
        layer.forward(z, None, "outgoing", out=torch.empty_like(z))
    assert e.value.status == tb.TRIMUL_ERR_INVALID_ARG


def test_stage_helpers_check_shapes():
    import torch
    layer = _unbound_layer(32, 64)
    good = torch.zeros(tb.ab_storage_shape("bf16", 1, 64, 16), dtype=torch.bfloat16)
    with pytest.raises(ValueError) as e:
        layer.contract(good, torch.zeros((1, 64, 16, 16), dtype=torch.bfloat16))
    assert "b_cm" in str(e.value)
    z = torch.zeros((1, 16, 16, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError) as e:
        layer.output(z, torch.zeros((1, 32, 16, 16), dtype=torch.bfloat16))
    assert "o must be" in str(e.value)
    with pytest.raises(ValueError) as e:
        layer.project(z, torch.zeros((1, 16, 8), dtype=torch.bfloat16))
    assert "mask" in str(e.value)


def _vp(x):
    return ctypes.c_void_p(x)


@pytest.mark.parametrize("reads,writes", [(0, 1), (2, 2), (1, 0), (3, 1), (1, 3)])
def test_peak_stream_rejects_unknown_modes(reads, writes):
    st = tb._lib.trimul_internal_peak_stream(_vp(256), _vp(256), _vp(512), _vp(512), 4, reads, writes, 0, None)
    assert st == tb.TRIMUL_ERR_INVALID_ARG
    assert "(reads, writes)" in tb.trimul_last_error()


def test_peak_stream_checks_pointers_and_size():
    lib = tb._lib
    assert lib.trimul_internal_peak_stream(None, None, _vp(512), None, 4, 1, 1, 0, None) == tb.TRIMUL_ERR_INVALID_ARG
    assert lib.trimul_internal_peak_stream(_vp(256), None, _vp(512), None, 4, 2, 1, 0, None) == tb.TRIMUL_ERR_INVALID_ARG
    assert lib.trimul_internal_peak_stream(_vp(256), None, _vp(512), None, 4, 1, 2, 0, None) == tb.TRIMUL_ERR_INVALID_ARG
    assert lib.trimul_internal_peak_stream(_vp(256), None, _vp(520), None, 4, 1, 1, 0, None) == tb.TRIMUL_ERR_INVALID_ARG
    assert "aligned" in tb.trimul_last_error()
    assert lib.trimul_internal_peak_stream(_vp(256), None, _vp(512), None, 0, 1, 1, 0, None) == tb.TRIMUL_ERR_INVALID_ARG


def test_peak_mfma_checks_arguments():
    lib = tb._lib
    assert lib.trimul_internal_peak_mfma(None, 1, 1, 0, _vp(256), None) == tb.TRIMUL_ERR_INVALID_ARG
    assert lib.trimul_internal_peak_mfma(_vp(256), 0, 1, 0, _vp(256), None) == tb.TRIMUL_ERR_INVALID_ARG
    assert lib.trimul_internal_peak_mfma(_vp(256), 1, 0, 0, _vp(256), None) == tb.TRIMUL_ERR_INVALID_ARG
    assert lib.trimul_internal_peak_mfma(_vp(256), 1, 1, 2, _vp(256), None) == tb.TRIMUL_ERR_INVALID_ARG
    assert "shape" in tb.trimul_last_error()
    assert lib.trimul_internal_peak_mfma(_vp(264), 1, 1, 0, _vp(256), None) == tb.TRIMUL_ERR_INVALID_ARG
    assert "aligned" in tb.trimul_last_error()
