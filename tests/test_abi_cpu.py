"""C ABI checks that need no GPU: the library loads, exports every entry
point include/mosaicq.h declares, and rejects bad arguments before any HIP
call (status codes only; nothing is computed)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "bit_gemm_amd", "libmosaicq.so")
HEADER = os.path.join(ROOT, "include", "mosaicq.h")


@pytest.fixture(scope="module")
def lib():
    assert os.path.exists(LIB), "libmosaicq.so is not built (python -m bit_gemm_amd.build)"
    from bit_gemm_amd import mosaicq
    return mosaicq.lib


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mq_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(
        ["mq_pack", "mq_linear", "mq_linear_with", "mq_linear_noalloc", "mq_residual_add", "mq_stream_read", "mq_packed_info", "mq_export_canonical",
         "mq_export_tiled", "mq_pack_blocks", "mq_block_count", "mq_export_blocks", "mq_smooth_weights",
         "mq_smooth_activations", "mq_quantize_activations", "mq_linear_a4", "mq_decode_a4", "mq_concat", "mq_linear_group",
         "mq_free", "mq_status_string"])


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    # nothing else leaks out of the library
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert exported == declared_functions()


def test_status_strings(lib):
    from bit_gemm_amd import mosaicq
    for code, name in mosaicq.STATUS.items():
        assert mosaicq.mq_status_string(code) == name
    assert mosaicq.mq_status_string(12345) == "MQ_ERR_UNKNOWN"


FAKE = ctypes.c_void_p(1 << 20)          # aligned, never dereferenced by validation


def _pack(lib, W=FAKE, N=32, K=256, G=128, rho=0.1, out=True):
    h = ctypes.c_void_p()
    return lib.mq_pack(W, N, K, G, rho, None, ctypes.byref(h) if out else None)


@pytest.mark.parametrize("kw,code", [
    (dict(W=None), -1), (dict(out=False), -1), (dict(N=0), -1), (dict(K=-128), -1),
    (dict(rho=-0.01), -1), (dict(rho=1.5), -1), (dict(rho=math.nan), -1),
    (dict(G=48), -2), (dict(G=256), -2), (dict(K=96, G=64), -1),
    (dict(K=65536 + 128), -2), (dict(N=(1 << 31) // 4096 + 1, K=4096), -2),
    (dict(W=ctypes.c_void_p((1 << 20) + 2)), -1),
])
def test_pack_argument_validation(lib, kw, code):
    assert _pack(lib, **kw) == code


def _pack_blocks(lib, W=FAKE, N=32, K=256, G=128, frac=0.1, h=FAKE, out=True):
    hd = ctypes.c_void_p()
    return lib.mq_pack_blocks(W, N, K, G, frac, h, None, ctypes.byref(hd) if out else None)


@pytest.mark.parametrize("kw,code", [
    (dict(W=None), -1), (dict(h=None), -1), (dict(out=False), -1), (dict(N=0), -1),
    (dict(frac=-0.1), -1), (dict(frac=1.01), -1), (dict(frac=math.nan), -1),
    (dict(G=48), -2), (dict(K=96, G=64), -1), (dict(K=65536 + 128), -2),
    (dict(h=ctypes.c_void_p((1 << 20) + 2)), -1), (dict(W=ctypes.c_void_p((1 << 20) + 8)), -1),
])
def test_pack_blocks_argument_validation(lib, kw, code):
    assert _pack_blocks(lib, **kw) == code


def test_smooth_argument_validation(lib):
    assert lib.mq_smooth_weights(None, 4, 8, FAKE, FAKE, FAKE, None) == -1
    assert lib.mq_smooth_weights(FAKE, 0, 8, FAKE, FAKE, FAKE, None) == -1
    assert lib.mq_smooth_weights(FAKE, 4, 8, ctypes.c_void_p((1 << 20) + 2), FAKE, FAKE, None) == -1
    assert lib.mq_smooth_weights(FAKE, (1 << 31) // 8, 8, FAKE, FAKE, FAKE, None) == -2
    assert lib.mq_smooth_activations(FAKE, 4, 8, None, FAKE, None) == -1
    assert lib.mq_smooth_activations(FAKE, 4, -8, FAKE, FAKE, None) == -1
    assert lib.mq_smooth_activations(ctypes.c_void_p((1 << 20) + 1), 4, 8, FAKE, FAKE, None) == -1


def test_pack_without_a_device_reports_device_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _pack(lib) == -5


def test_bad_handles_are_rejected(lib):
    from bit_gemm_amd import mosaicq
    bogus = ctypes.c_void_p(0xDEADBEE0)
    assert lib.mq_linear(FAKE, 1, None, FAKE, None) == -6
    assert lib.mq_linear(FAKE, 1, bogus, FAKE, None) == -6
    assert lib.mq_linear_with(FAKE, 1, bogus, FAKE, None, mosaicq.KERNEL_GEMV) == -6
    assert lib.mq_linear_noalloc(FAKE, 1, bogus, FAKE, None) == -6
    assert lib.mq_residual_add(FAKE, 1, bogus, FAKE, None) == -6
    n = ctypes.c_int64()
    assert lib.mq_packed_info(bogus, ctypes.byref(n), None, None, None, None) == -6
    assert lib.mq_export_canonical(bogus, None, None, None, None, None, None, None) == -6
    assert lib.mq_export_tiled(bogus, None, None, None, None) == -6
    assert lib.mq_block_count(bogus, ctypes.byref(n)) == -6
    assert lib.mq_export_blocks(bogus, None, None, None, None) == -6
    assert lib.mq_decode_a4(FAKE, 1, bogus, FAKE, None) == -6
    out = ctypes.c_void_p()
    arr = (ctypes.c_void_p * 2)(bogus, bogus)
    assert lib.mq_concat(arr, 2, None, ctypes.byref(out)) == -6
    assert out.value is None
    assert lib.mq_concat(None, 2, None, ctypes.byref(out)) == -1
    assert lib.mq_concat(arr, 0, None, ctypes.byref(out)) == -1
    assert lib.mq_concat(arr, 2, None, None) == -1
    xs = (ctypes.c_void_p * 2)(FAKE, FAKE)
    assert lib.mq_linear_group(xs, 16, arr, xs, 2, None) == -6
    assert lib.mq_linear_group(None, 16, arr, xs, 2, None) == -1
    assert lib.mq_linear_group(xs, 16, arr, None, 2, None) == -1
    assert lib.mq_linear_group(xs, 16, None, xs, 2, None) == -1
    assert lib.mq_linear_group(xs, 16, arr, xs, 0, None) == -1
    assert lib.mq_linear_group(xs, 0, arr, xs, 2, None) == -1
    lib.mq_free(None)        # accepted
    lib.mq_free(bogus)       # unknown handle: ignored, no crash


def test_quantize_activations_validation(lib):
    f = lib.mq_quantize_activations
    mis = ctypes.c_void_p((1 << 20) + 8)
    assert f(None, 4, 256, 128, FAKE, FAKE, None) == -1
    assert f(FAKE, 0, 256, 128, FAKE, FAKE, None) == -1
    assert f(FAKE, 4, 256, 96, FAKE, FAKE, None) == -1          # G not supported
    assert f(FAKE, 4, 192, 128, FAKE, FAKE, None) == -1         # K % G != 0
    assert f(FAKE, 4, 131072, 128, FAKE, FAKE, None) == -1      # K > 65536
    assert f(mis, 4, 256, 128, FAKE, FAKE, None) == -1          # X not 16-byte aligned
    assert f(FAKE, 4, 256, 128, mis, FAKE, None) == -1          # codes not 16-byte aligned
    assert f(FAKE, 4, 256, 128, FAKE, ctypes.c_void_p((1 << 20) + 2), None) == -1
    assert f(FAKE, 1 << 20, 4096, 128, FAKE, FAKE, None) == -2  # M * Kp >= 2^31


def test_linear_a4_validation(lib):
    f = lib.mq_linear_a4
    assert f(FAKE, FAKE, 4, None, FAKE, None) == -6              # no handle
    assert f(FAKE, FAKE, 4, FAKE, FAKE, None) == -6              # not a live handle


def test_stream_read_validation(lib):
    f = lib.mq_stream_read
    assert f(None, 1024, 4, FAKE, None) == -1
    assert f(FAKE, 0, 4, FAKE, None) == -1
    assert f(FAKE, 1000, 4, FAKE, None) == -1                       # not a multiple of 16
    assert f(FAKE, 1024, 0, FAKE, None) == -1
    assert f(ctypes.c_void_p((1 << 20) + 8), 1024, 4, FAKE, None) == -1
    assert f(FAKE, 1024, 4, ctypes.c_void_p((1 << 20) + 2), None) == -1
    assert f(FAKE, 16 * 256 * 16 + 16, 1, FAKE, None) == -1      # more than 16 loads per thread


def test_linear_group_binding_checks_arguments(lib):
    import torch
    from bit_gemm_amd import mosaicq
    with pytest.raises(ValueError):
        mosaicq.mq_linear_group([], [])                      # no layer
    with pytest.raises(ValueError):
        mosaicq.mq_linear_group([torch.zeros(1)], [None, None])   # one input per layer
    with pytest.raises(TypeError):
        mosaicq.mq_linear_group([1], [None])                 # not a tensor
    with pytest.raises(TypeError):
        mosaicq.mq_linear_group([torch.zeros((2, 64), dtype=torch.float16)], [None])   # host memory
