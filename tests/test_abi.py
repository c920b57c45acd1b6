"""The C ABI without a GPU: the library loads, exports every declared symbol, and its host
logic (status codes, padding, the power-of-4 test, the dense RHT, argument validation)
behaves as include/convrot.h states.  No test here enqueues device work: every call either
is host-only or fails validation before any launch."""
import os
import re

import numpy as np
import pytest

import rotation_w4a4_quantized_convrot_amd as cr
from rotation_w4a4_quantized_convrot_amd import _lib
from oracle import convrot_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "convrot.h")


def _declared():
    text = open(HEADER).read()
    return re.findall(r"CONVROT_API\s+[\w\s\*]+?\b(convrot_\w+)\s*\(", text)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libconvrot.so not built")
    return _lib.load_library()


def test_header_declares_the_abi():
    names = _declared()
    for required in ("convrot_make_rht", "convrot_rotate_quant_act", "convrot_quant_weight",
                     "convrot_w4a4_linear", "convrot_w4a4_gemm"):
        assert required in names
    assert sorted(names) == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {_lib.LIB_PATH}").read()
    exported = set(re.findall(r"\b(convrot_\w+)\b", out))
    assert exported == set(_declared())          # nothing else leaks out of the library


def test_status_strings(lib):
    for st in range(0, -10, -1):
        assert cr.convrot_status_string(st) not in ("", "unknown status")
    assert cr.convrot_status_string(-99) == "unknown status"
    assert cr.convrot_version() >= 100


def test_power_of_four_matches_oracle(lib):
    for line in open(os.path.join(ROOT, "tests", "golden", "power_of_four.txt")):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        verdict, expr = line.split(None, 1)
        value = eval(expr, {"__builtins__": {}})
        if not (-2 ** 63 <= value < 2 ** 63):
            continue
        assert cr.convrot_is_power_of_4(value) == (verdict == "accept") == O.is_power_of_four(value)


def test_padded_k(lib):
    for K in (1, 15, 16, 17, 3072, 3100, 12288, 15360):
        for g in (4, 16, 64, 256, 1024):
            assert cr.convrot_padded_k(K, g) == O.padded_k(K, g)
    with pytest.raises(ValueError, match="Regular Hadamard size must be a power of 4, got 8"):
        cr.convrot_padded_k(100, 8)
    with pytest.raises(cr.ConvRotError):
        cr.convrot_padded_k(0, 16)


@pytest.mark.parametrize("g", [4, 16, 64, 256, 1024])
def test_make_rht_matches_oracle_kronecker(lib, g):
    """The library's closed form equals the oracle's Kronecker construction."""
    h = cr.convrot_make_rht(g).numpy()
    assert np.array_equal(h.astype(np.float64), O.regular_hadamard(g))
    hn = cr.convrot_make_rht(g, normalized=True).numpy().astype(np.float64)
    assert np.array_equal(hn, O.regular_hadamard(g) / np.sqrt(g))


def test_make_rht_errors(lib):
    import ctypes
    buf = (ctypes.c_float * 64)()
    assert lib.convrot_make_rht(8, ctypes.addressof(buf), 0) == _lib.CONVROT_ERR_GROUP
    assert lib.convrot_make_rht(16, None, 0) == _lib.CONVROT_ERR_NULL
    assert lib.convrot_make_rht(4 ** 7, ctypes.addressof(buf), 0) == _lib.CONVROT_ERR_UNSUPPORTED


def test_workspace_bytes(lib):
    assert cr.convrot_w4a4_workspace_bytes(4608, 3072, 256) == 4608 * 1536 + 18432
    assert cr.convrot_w4a4_workspace_bytes(3, 17, 16) == 256 + 256
    assert cr.convrot_w4a4_workspace_bytes(10, 100, 8) == 0
    assert cr.convrot_w4a4_workspace_bytes(-1, 100, 16) == 0


# Fake device addresses: validation must reject these calls before any launch.
A16 = 0x10000
MIS = 0x10001


def _rq(lib, x=A16, dt=1, M=4, K=64, ldx=64, g=16, q=A16, s=A16, rot=None):
    return lib.convrot_rotate_quant_act(x, dt, M, K, ldx, g, q, s, rot, None)


def test_rotate_quant_validation(lib):
    E = _lib
    assert _rq(lib, g=8) == E.CONVROT_ERR_GROUP
    assert _rq(lib, g=2 ** 58) == E.CONVROT_ERR_UNSUPPORTED
    assert _rq(lib, g=4) == E.CONVROT_ERR_UNSUPPORTED
    assert _rq(lib, g=4096) == E.CONVROT_ERR_UNSUPPORTED
    assert _rq(lib, dt=7) == E.CONVROT_ERR_DTYPE
    assert _rq(lib, M=-1) == E.CONVROT_ERR_SHAPE
    assert _rq(lib, K=0) == E.CONVROT_ERR_SHAPE
    assert _rq(lib, ldx=63) == E.CONVROT_ERR_SHAPE
    assert _rq(lib, K=65537, ldx=65537, g=1024) == E.CONVROT_ERR_UNSUPPORTED
    assert _rq(lib, K=61441, ldx=61441, g=1024) == E.CONVROT_ERR_UNSUPPORTED
    assert _rq(lib, dt=0, K=32769, ldx=32769, g=1024) == E.CONVROT_ERR_UNSUPPORTED
    assert _rq(lib, K=16385, ldx=16385, g=16) == E.CONVROT_ERR_UNSUPPORTED
    assert _rq(lib, K=32769, ldx=32769, g=256) == E.CONVROT_ERR_UNSUPPORTED
    assert _rq(lib, K=32769, ldx=32769, g=64) == E.CONVROT_ERR_UNSUPPORTED
    assert _rq(lib, x=None) == E.CONVROT_ERR_NULL
    assert _rq(lib, q=None) == E.CONVROT_ERR_NULL
    assert _rq(lib, s=None) == E.CONVROT_ERR_NULL
    assert _rq(lib, x=MIS) == E.CONVROT_ERR_ALIGN
    assert _rq(lib, q=A16 + 8) == E.CONVROT_ERR_ALIGN
    assert _rq(lib, s=A16 + 2) == E.CONVROT_ERR_ALIGN
    assert _rq(lib, rot=A16 + 4) == E.CONVROT_ERR_ALIGN
    assert _rq(lib, M=0, x=None, q=None, s=None) == E.CONVROT_OK      # empty input: no-op
    assert lib.convrot_quant_weight(A16, 1, 4, 64, 8, A16, A16, None) == E.CONVROT_ERR_GROUP
    assert lib.convrot_quant_weight(A16, 1, 4, 64, 16, None, A16, None) == E.CONVROT_ERR_NULL


def _gemm(lib, xq=A16, xs=A16, wq=A16, ws=A16, b=None, M=4, N=4, Kp=64, y=A16, acc=None):
    return lib.convrot_w4a4_gemm(xq, xs, wq, ws, b, M, N, Kp, y, acc, None)


def test_gemm_validation(lib):
    E = _lib
    assert _gemm(lib, Kp=24) == E.CONVROT_ERR_SHAPE
    assert _gemm(lib, Kp=0) == E.CONVROT_ERR_SHAPE
    assert _gemm(lib, M=-1) == E.CONVROT_ERR_SHAPE
    assert _gemm(lib, Kp=65536 + 16) == E.CONVROT_ERR_UNSUPPORTED
    assert _gemm(lib, xq=None) == E.CONVROT_ERR_NULL
    assert _gemm(lib, y=None) == E.CONVROT_ERR_NULL
    assert _gemm(lib, wq=A16 + 8) == E.CONVROT_ERR_ALIGN
    assert _gemm(lib, y=A16 + 2) == E.CONVROT_ERR_ALIGN
    assert _gemm(lib, b=MIS) == E.CONVROT_ERR_ALIGN
    assert _gemm(lib, acc=A16 + 4) == E.CONVROT_ERR_ALIGN
    assert _gemm(lib, M=0, xq=None, y=None) == E.CONVROT_OK
    assert _gemm(lib, N=0, wq=None, y=None) == E.CONVROT_OK


def _lin(lib, x=A16, dt=1, M=4, K=64, g=16, wq=A16, ws=A16, N=4, b=None, y=A16, wsp=A16 * 16,
         nbytes=1 << 20):
    return lib.convrot_w4a4_linear(x, dt, M, K, g, wq, ws, N, b, y, wsp, nbytes, None)


def test_linear_validation(lib):
    E = _lib
    assert _lin(lib, g=32) == E.CONVROT_ERR_GROUP
    assert _lin(lib, g=4) == E.CONVROT_ERR_UNSUPPORTED
    assert _lin(lib, dt=3) == E.CONVROT_ERR_DTYPE
    assert _lin(lib, N=-2) == E.CONVROT_ERR_SHAPE
    assert _lin(lib, wsp=None) == E.CONVROT_ERR_NULL
    assert _lin(lib, wsp=A16 * 16 + 16) == E.CONVROT_ERR_ALIGN
    assert _lin(lib, nbytes=cr.convrot_w4a4_workspace_bytes(4, 64, 16) - 1) == E.CONVROT_ERR_WORKSPACE
    assert _lin(lib, ws=A16 + 1) == E.CONVROT_ERR_ALIGN
    assert _lin(lib, M=0, x=None, wsp=None) == E.CONVROT_OK


def test_python_binding_rejects_cpu_tensors(lib):
    import torch
    with pytest.raises(ValueError, match="GPU"):
        cr.convrot_rotate_quant_act(torch.zeros((2, 16), dtype=torch.bfloat16), 16)
    with pytest.raises(ValueError, match="power of 4, got 8"):
        cr.convrot_rotate_quant_act(torch.zeros((2, 16), dtype=torch.bfloat16), 8)


def test_w8a8_workspace_bytes(lib):
    assert cr.convrot_w8a8_workspace_bytes(4608, 3072, 256) == 4608 * 3072 + 18432
    assert cr.convrot_w8a8_workspace_bytes(3, 17, 16) == 256 + 256
    assert cr.convrot_w8a8_workspace_bytes(10, 100, 8) == 0
    assert cr.convrot_w8a8_workspace_bytes(-1, 100, 16) == 0


def test_int8_entry_points_validate(lib):
    E = _lib
    rq = lambda **k: lib.convrot_rotate_quant_act_i8(  # noqa: E731
        k.get("x", A16), k.get("dt", 1), k.get("M", 4), k.get("K", 64), k.get("ldx", k.get("K", 64)),
        k.get("g", 16), k.get("q", A16), k.get("s", A16), k.get("rot"), None)
    assert rq(g=8) == E.CONVROT_ERR_GROUP
    assert rq(g=4096) == E.CONVROT_ERR_UNSUPPORTED
    assert rq(dt=5) == E.CONVROT_ERR_DTYPE
    assert rq(K=64, ldx=63) == E.CONVROT_ERR_SHAPE
    # int8 codes take twice the register room: g = 1024 bf16 rows stop at K' = 53248
    assert rq(K=53249, g=1024) == E.CONVROT_ERR_UNSUPPORTED
    assert rq(K=32769, g=1024, dt=0) == E.CONVROT_ERR_UNSUPPORTED
    assert rq(K=28673, g=1024, dt=0) == E.CONVROT_ERR_UNSUPPORTED
    assert rq(K=30721, g=256, dt=0) == E.CONVROT_ERR_UNSUPPORTED
    assert rq(K=30721, g=64, dt=0) == E.CONVROT_ERR_UNSUPPORTED
    assert rq(q=None) == E.CONVROT_ERR_NULL
    assert rq(q=A16 + 8) == E.CONVROT_ERR_ALIGN
    assert rq(M=0, x=None, q=None, s=None) == E.CONVROT_OK
    assert lib.convrot_quant_weight_i8(A16, 1, 4, 64, 32, A16, A16, None) == E.CONVROT_ERR_GROUP
    gm = lambda **k: lib.convrot_w8a8_gemm(  # noqa: E731
        k.get("xq", A16), A16, A16, A16, k.get("b"), k.get("M", 4), 4, k.get("Kp", 64),
        k.get("y", A16), k.get("acc"), None)
    assert gm(Kp=40) == E.CONVROT_ERR_SHAPE
    assert gm(Kp=65536 + 16) == E.CONVROT_ERR_UNSUPPORTED
    assert gm(xq=None) == E.CONVROT_ERR_NULL
    assert gm(xq=A16 + 8) == E.CONVROT_ERR_ALIGN
    assert gm(b=MIS) == E.CONVROT_ERR_ALIGN
    assert gm(M=0, xq=None, y=None) == E.CONVROT_OK
    ln = lambda **k: lib.convrot_w8a8_linear(  # noqa: E731
        A16, 1, k.get("M", 4), 64, k.get("g", 16), A16, A16, 4, None, A16, k.get("wsp", A16 * 16),
        k.get("nbytes", 1 << 20), None)
    assert ln(g=32) == E.CONVROT_ERR_GROUP
    assert ln(wsp=None) == E.CONVROT_ERR_NULL
    assert ln(wsp=A16 * 16 + 16) == E.CONVROT_ERR_ALIGN
    assert ln(nbytes=cr.convrot_w8a8_workspace_bytes(4, 64, 16) - 1) == E.CONVROT_ERR_WORKSPACE
    assert ln(M=0, wsp=None) == E.CONVROT_OK


def test_modules_allocate_each_formats_buffers(lib):
    """Host-side shapes and dtypes of the three linear modules' weight buffers (CPU tensors)."""
    K, N, g = 3100, 200, 256
    kp = O.padded_k(K, g)
    m4 = cr.ConvLinear4bit(K, N, g)
    assert tuple(m4.weight_packed.shape) == (N, kp // 2)
    assert str(m4.weight_packed.dtype) == "torch.uint8"
    assert tuple(m4.weight_scale.shape) == (N,) and str(m4.weight_scale.dtype) == "torch.float32"
    m8 = cr.ConvLinear8bit(K, N, g)
    assert tuple(m8.weight_packed.shape) == (N, kp) and str(m8.weight_packed.dtype) == "torch.int8"
    assert tuple(m8.weight_scale.shape) == (N,)
    mf = cr.ConvLinearFP4(K, N, g)
    assert tuple(mf.weight_packed.shape) == (N, kp // 2)
    assert tuple(mf.weight_scale.shape) == (N, 4 * (-(-kp // 128)))
    assert str(mf.weight_scale.dtype) == "torch.uint8"


def test_noalloc_linear_validates_before_touching_the_device(lib):
    """The no-allocation entry point checks its arguments, and that the problem fits its fixed
    scratch array, before any HIP call (these run without a GPU)."""
    E = _lib
    call = lambda **k: lib.convrot_w4a4_linear_noalloc(  # noqa: E731
        k.get("x", A16), k.get("dt", 1), k.get("M", 4), k.get("K", 64), k.get("g", 16),
        k.get("wq", A16), k.get("ws", A16), k.get("N", 4), k.get("b"), k.get("y", A16), None)
    assert call(g=8) == E.CONVROT_ERR_GROUP
    assert call(g=4096) == E.CONVROT_ERR_UNSUPPORTED
    assert call(dt=7) == E.CONVROT_ERR_DTYPE
    assert call(M=-1) == E.CONVROT_ERR_SHAPE
    assert call(x=None) == E.CONVROT_ERR_NULL
    assert call(M=0, x=None, y=None) == E.CONVROT_OK
    # K = 3072, g = 256: 1536 code bytes + 4 scale bytes per row (each part 256-byte rounded)
    limit = _lib.CONVROT_NOALLOC_SCRATCH_BYTES
    fits = max(m for m in range(49000, 49300)
               if cr.convrot_w4a4_workspace_bytes(m, 3072, 256) <= limit)
    assert fits == 49024
    assert call(M=fits + 1, K=3072, g=256) == E.CONVROT_ERR_SCRATCH
    assert "no-allocation" in cr.convrot_status_string(E.CONVROT_ERR_SCRATCH)


def test_fused_linear_validates_before_launch(lib):
    """convrot_w4a4_linear_fused refuses what its single kernel does not implement, before
    any device call (no GPU needed)."""
    E = _lib
    call = lambda **k: lib.convrot_w4a4_linear_fused(  # noqa: E731
        k.get("x", A16), k.get("dt", 1), k.get("M", 4), k.get("K", 3072), k.get("g", 256),
        k.get("wq", A16), k.get("ws", A16), k.get("N", 4), k.get("b"), k.get("y", A16),
        k.get("wsp", A16 * 16), k.get("nbytes", 1 << 20), k.get("status", A16), None)
    assert call(g=8) == E.CONVROT_ERR_GROUP
    assert call(g=64) == E.CONVROT_ERR_UNSUPPORTED         # window sizes 256 and 1024 only
    assert call(dt=0) == E.CONVROT_ERR_UNSUPPORTED         # bf16 rows only
    assert call(K=3071) == E.CONVROT_ERR_UNSUPPORTED       # odd rows are not dword aligned
    assert call(K=17000) == E.CONVROT_ERR_UNSUPPORTED      # a row beyond eight waves
    assert call(status=None) == E.CONVROT_ERR_NULL
    assert call(wsp=A16 * 16 + 16) == E.CONVROT_ERR_ALIGN
    assert call(nbytes=cr.convrot_w4a4_workspace_bytes(4, 3072, 256) - 1) == E.CONVROT_ERR_WORKSPACE
    assert call(M=0, x=None, y=None) == E.CONVROT_OK


def test_calibration_library_exports():
    """libconvrot_calib.so (built with the layer's library) exports its calls, and the
    launcher rejects bad arguments before touching the device."""
    import ctypes
    from rotation_w4a4_quantized_convrot_amd import calibration as C
    if not os.path.exists(C.CALIB_PATH):
        pytest.skip("libconvrot_calib.so not built")
    lib = C.load()
    assert lib.convrot_calib_ops_per_inst(0) == 2 * 32 * 32 * 32
    assert lib.convrot_calib_ops_per_inst(1) == 2 * 32 * 32 * 64
    assert lib.convrot_calib_ops_per_inst(2) == 2 * 16 * 16 * 128
    assert lib.convrot_calib_ops_per_inst(3) == lib.convrot_calib_ops_per_inst(4) == 2 * 32 ** 3
    assert lib.convrot_calib_ops_per_inst(5) == 0
    assert lib.convrot_calib_chains() >= 1
    bad = [(0, 0, 256, 1), (0, 1, 100, 1), (0, 1, 2048, 1), (0, 1, 256, -1), (5, 1, 256, 1),
           (-1, 1, 256, 1)]
    for kind, grid, block, iters in bad:
        assert lib.convrot_calib_mfma(kind, grid, block, iters, ctypes.c_void_p(16),
                                      ctypes.c_void_p(16), None) != 0
    assert lib.convrot_calib_mfma(0, 1, 256, 1, None, ctypes.c_void_p(16), None) != 0
