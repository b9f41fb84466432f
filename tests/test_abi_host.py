"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point include/moe_ffn.h declares, and rejects bad arguments before
touching the device."""
import ctypes as C
import os

import pytest

from helpers import public_header_symbols

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ffn.h")


@pytest.fixture(scope="module")
def B():
    from mixture_experts_ffn_gemm_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from mixture_experts_ffn_gemm_amd import build
        build.build()
    return binding


def test_header_declares_the_expected_entry_points(B):
    syms = public_header_symbols(HEADER)
    assert set(syms) == set(B.EXPORTED)


def test_library_exports_every_header_symbol(B):
    L = B.lib()
    for s in public_header_symbols(HEADER):
        assert hasattr(L, s), s


def test_status_strings(B):
    assert B.status_str(0) == "ok"
    assert B.status_str(-3) == "workspace too small"
    assert B.status_str(12345) == "unknown status"


@pytest.mark.parametrize("dims,rc", [
    ((0, 8, 2, 256, 0, 0), -1),          # d = 0
    ((100, 8, 2, 256, 0, 0), -2),        # d not a multiple of 32
    ((128, 8, 9, 256, 0, 0), -1),        # top_k > E
    ((128, 300, 2, 256, 0, 0), -2),      # E > 256
    ((128, 64, 17, 256, 0, 0), -2),      # top_k > 16
    ((128, 8, 2, 250, 0, 0), -2),        # ffn not a multiple of 32
    ((128, 8, 2, 256, 0, 2), -1),        # norm flag not 0/1
])
def test_weights_create_rejects_bad_dims_before_any_device_call(B, dims, rc):
    h = C.c_void_p(1234)
    dm = B.moe_ffn_dims(*dims)
    got = B.lib().moe_ffn_weights_create(C.byref(dm), 8, None, 16, 16, 16, None, None, None, None,
                                         None, C.byref(h))
    assert got == rc
    assert h.value is None


def test_weights_create_rejects_null_and_partial_shared(B):
    h = C.c_void_p()
    dm = B.moe_ffn_dims(128, 8, 2, 256, 0, 0)
    assert B.lib().moe_ffn_weights_create(C.byref(dm), None, None, 16, 16, 16, None, None, None, None,
                                          None, C.byref(h)) == -1
    # shared pointers without a shared expert
    assert B.lib().moe_ffn_weights_create(C.byref(dm), 8, None, 16, 16, 16, 16, None, None, None,
                                          None, C.byref(h)) == -1
    dm2 = B.moe_ffn_dims(128, 8, 2, 256, 64, 0)
    assert B.lib().moe_ffn_weights_create(C.byref(dm2), 8, None, 16, 16, 16, 16, 16, None, 16,
                                          None, C.byref(h)) == -1
    assert B.lib().moe_ffn_weights_create(C.byref(dm), 8, None, 16, 16, 16, None, None, None, None,
                                          None, None) == -1


def test_weights_create_fmt_rejects_formats_and_kquant_shapes_before_any_device_call(B):
    h = C.c_void_p(1234)
    L = B.lib()

    def create(dims, fmt, sh=None):
        dm = B.moe_ffn_dims(*dims)
        return L.moe_ffn_weights_create_fmt(C.byref(dm), fmt, 8, None, 16, 16, 16, sh, sh, sh, sh, None,
                                            C.byref(h))
    assert create((256, 8, 2, 256, 0, 0), 3) == -1             # unknown format
    assert create((256, 8, 2, 256, 0, 0), -1) == -1
    assert create((128, 8, 2, 256, 0, 0), B.FMT_Q4_K) == -2    # d not a multiple of 256
    assert create((256, 8, 2, 128, 0, 0), B.FMT_Q4_K) == -2    # ffn not a multiple of 256
    assert create((256, 8, 2, 256, 64, 0), B.FMT_Q4_K, 16) == -2   # shared ffn not a multiple of 256
    assert create((0, 8, 2, 256, 0, 0), B.FMT_Q4_K) == -1      # the common dims checks still apply
    assert create((128, 8, 2, 256, 0, 0), B.FMT_Q3_K) == -2    # Q3_K: multiples of 256 as well
    assert create((256, 8, 2, 256, 32, 0), B.FMT_Q3_K, 16) == -2
    assert h.value is None


def test_stage_entry_points_validate_on_the_host(B):
    L = B.lib()
    assert L.moe_ffn_combine(None, 16, None, 4, 2, 128, 32, None) == -1
    assert L.moe_ffn_combine(16, 16, None, 4, 0, 128, 4096, None) == -1      # k = 0
    assert L.moe_ffn_combine(16, 16, None, 4, 17, 128, 4096, None) == -1     # k > 16
    assert L.moe_ffn_combine(16, 16, None, 4, 2, 130, 4096, None) == -2      # d % 4
    assert L.moe_ffn_combine(16, 16, None, 4, 2, 128, 16, None) == -1        # out overlaps partial
    assert L.moe_ffn_quantize(16, 33, 64, 128, None) == -2
    assert L.moe_ffn_quantize(None, 32, 64, 128, None) == -1
    assert L.moe_ffn_quantize(16, -32, 64, 128, None) == -1
    assert L.moe_ffn_residual_rmsnorm(16, None, 16, 4, 8, 1e-5, None) == -1   # xn overlaps h
    assert L.moe_ffn_residual_rmsnorm(16, None, 4096, 4, 8, -1.0, None) == -1
    n = C.c_size_t()
    assert L.moe_ffn_workspace_size(None, 16, C.byref(n)) == -1
    dm = B.moe_ffn_dims()
    assert L.moe_ffn_weights_dims(None, C.byref(dm)) == -1
    assert L.moe_ffn_prefill(None, 16, 4, 32, 64, 1 << 20, None, None) == -1
    assert L.moe_ffn_prefill_residual(None, 16, 4, 32, 16, 1e-5, 64, 1 << 20, None, None) == -1
    assert L.moe_ffn_decode(None, 16, 9, 32, 64, 1 << 20, None, None) == -1
    assert L.moe_ffn_decode(None, 16, 0, 32, 64, 1 << 20, None, None) == -1
    assert L.moe_ffn_decode_profiled(None, 16, 1, 32, 64, 1 << 20, None, None, None) == -1   # no events
    ev = (C.c_void_p * 5)(*([None] * 5))
    assert L.moe_ffn_decode_profiled(None, 16, 1, 32, 64, 1 << 20, None, None, ev) == -1     # null events
    assert L.moe_ffn_weights_destroy(None) == 0


@pytest.mark.parametrize("dims", [
    (2048, 64, 8, 1024, 0, 0),      # OLMoE-shaped layer
    (128, 8, 2, 256, 0, 0),         # tiny
    (2048, 256, 8, 512, 512, 1),    # 35B-A3B-shaped layer with a shared expert
    (160, 16, 3, 96, 64, 0),
    (128, 256, 16, 64, 32, 0),
])
def test_workspace_size_never_shrinks_with_max_tokens(B, dims):
    """A workspace sized once for max_tokens must serve every call with fewer
    tokens (prefill or decode), so the size is non-decreasing in max_tokens."""
    dm = B.moe_ffn_dims(*dims)
    sizes = [B.moe_ffn_workspace_size_for_dims(dm, n) for n in range(0, 70)]
    sizes += [B.moe_ffn_workspace_size_for_dims(dm, n) for n in (127, 128, 129, 511, 512, 513, 2048, 4096)]
    assert all(a <= b for a, b in zip(sizes, sizes[1:])), sizes
    assert sizes[0] > 0


def test_workspace_size_for_dims_validates(B):
    n = C.c_size_t()
    L = B.lib()
    assert L.moe_ffn_workspace_size_for_dims(None, 16, C.byref(n)) == -1
    dm = B.moe_ffn_dims(100, 8, 2, 256, 0, 0)
    assert L.moe_ffn_workspace_size_for_dims(C.byref(dm), 16, C.byref(n)) == -2
    dm = B.moe_ffn_dims(128, 8, 2, 256, 0, 0)
    assert L.moe_ffn_workspace_size_for_dims(C.byref(dm), -1, C.byref(n)) == -1
    assert L.moe_ffn_workspace_size_for_dims(C.byref(dm), 16, None) == -1


def test_probe_library_exports_its_header_and_validates(B):
    """libmoe_probe.so (the calibration kernels of the benchmark) exports what
    include/moe_probe.h declares and rejects bad arguments on the host."""
    from mixture_experts_ffn_gemm_amd import build
    syms = public_header_symbols(os.path.join(ROOT, "include", "moe_probe.h"), prefix="moe_probe_")
    assert syms == ["moe_probe_copy", "moe_probe_int8_mfma"]
    P = C.CDLL(build.PROBE_LIB)
    for s in syms:
        assert hasattr(P, s), s
    P.moe_probe_int8_mfma.argtypes = [C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]
    P.moe_probe_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    assert P.moe_probe_int8_mfma(0, 4, 64, None) == -1
    assert P.moe_probe_int8_mfma(10, 0, 64, None) == -1
    assert P.moe_probe_int8_mfma(10, 4, None, None) == -1
    assert P.moe_probe_copy(None, 64, 64, None) == -1
    assert P.moe_probe_copy(64, 128, 24, None) == -1      # not a multiple of 16
    assert P.moe_probe_copy(64, 96, 64, None) == -1       # overlapping
    assert P.moe_probe_copy(64, 4096, 0, None) == 0       # nothing to do


def test_chunked_prefill_validates_on_the_host(B):
    L = B.lib()
    assert L.moe_ffn_prefill_chunked(None, 16, 4, 2, 0, 32, 64, 1 << 20, None) == -1   # no handle
    assert L.moe_ffn_prefill_chunked(16, 16, 4, 0, 0, 32, 64, 1 << 20, None) == -1     # chunk 0
    assert L.moe_ffn_prefill_chunked(16, 16, 4, 2, 2, 32, 64, 1 << 20, None) == -1     # unknown flag
    assert L.moe_ffn_prefill_chunked(16, 16, -1, 2, 0, 32, 64, 1 << 20, None) == -1    # negative n


@pytest.mark.parametrize("dims, limit", [
    ((2048, 64, 8, 1024, 0, 0), 2026),      # OLMoE-shaped layer
    ((2048, 256, 8, 512, 512, 1), 1748),    # 35B-A3B-shaped layer with a shared expert
])
def test_static_scratch_token_limits_match_the_header(B, dims, limit):
    """The header states how many tokens the no-allocation entry point takes
    at these two shapes: exactly the largest batch whose workspace fits."""
    dm = B.moe_ffn_dims(*dims)
    assert B.moe_ffn_workspace_size_for_dims(dm, limit) <= B.STATIC_SCRATCH_BYTES
    assert B.moe_ffn_workspace_size_for_dims(dm, limit + 1) > B.STATIC_SCRATCH_BYTES
    header = open(os.path.join(os.path.dirname(__file__), "..", "include", "moe_ffn.h")).read()
    assert f"{limit} tokens" in header or f"above {limit}" in header
