"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

The library must load without a device, export every function the header
declares, and reject every invalid argument before touching HIP.

With BITNET_TEST_HOST_LIB set (tests/test_abi_sanitized.py does this in a
child process), the same checks run against a host-only build of the ABI
(abi.cpp with recording launcher stubs, under AddressSanitizer and
UndefinedBehaviorSanitizer), and the dispatch tests at the end check which
launchers valid calls reach.
"""

import ctypes
import os

import pytest

from bit_activation_linear_amd import _lib

FAKE = 0x10000  # a 16-B aligned non-null address; never dereferenced on these paths
HOST_LIB = os.environ.get("BITNET_TEST_HOST_LIB")


@pytest.fixture(scope="module")
def lib():
    if not HOST_LIB:
        return _lib.load()
    host = ctypes.CDLL(HOST_LIB)
    for name, (res, args) in _lib.SIGNATURES.items():
        fn = getattr(host, name)
        fn.restype = res
        fn.argtypes = args
    host.bitnet_stub_calls.restype = ctypes.c_char_p
    _lib._lib = host  # _lib.call goes to the host build in this (child) process
    return host


def test_exports_every_declared_symbol(lib):
    declared = _lib.header_declared_functions()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding lacks a signature for {name}"
    assert set(_lib.SIGNATURES) == set(declared)


def test_version_and_empty_error(lib):
    assert lib.bitnet_abi_version() == 4


def test_workspace_sizes(lib):
    # codes M*K bytes + scales 4*M bytes, each rounded up to 256 B
    # with the transform, K <= 256 keeps a token row in one wave: fused, no workspace
    assert lib.bitnet_forward_workspace_bytes(4, 256, 256, 4, 1) == 0
    assert lib.bitnet_forward_workspace_bytes(4, 512, 256, 4, 1) == 2048 + 2 * 256
    assert lib.bitnet_forward_workspace_bytes(2048, 8192, 2048, 4, 1) == 2048 * 8192 + 2 * 8192
    assert lib.bitnet_forward_workspace_bytes(0, 64, 8, 8, 0) == 0
    assert lib.bitnet_forward_workspace_bytes(4, 100, 8, 8, 0) == 0  # invalid K
    assert lib.bitnet_ternarize_workspace_bytes(14336, 4096) >= 8 * 1024
    # decode without the transform and a small batch: one fused kernel, no workspace
    assert lib.bitnet_forward_workspace_bytes(1, 2560, 6912, 8, 0) == 0
    assert lib.bitnet_forward_workspace_bytes(16, 1024, 64, 4, 0) == 0
    # with the transform the same shape needs codes + scales
    assert lib.bitnet_forward_workspace_bytes(1, 2048, 6912, 8, 1) == 2048 + 2 * 256
    # decode with long rows or the transform: codes + scales
    assert lib.bitnet_forward_workspace_bytes(16, 16384, 4096, 4, 1) == 16 * 16384 + 2 * 256
    assert lib.bitnet_forward_workspace_bytes(1, 8192, 4096, 8, 0) == 8192 + 2 * 256


def _fwd(lib, x=FAKE, xt=_lib.BF16, M=4, K=512, Wp=FAKE, N=256, alpha=FAKE, bits=4, had=1,
         y=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return lib.bitnet_hbitlinear_forward(x, xt, M, K, Wp, N, alpha, bits, had, y, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=None), _lib.ERR_INVALID_ARG),
    (dict(Wp=None), _lib.ERR_INVALID_ARG),
    (dict(alpha=None), _lib.ERR_INVALID_ARG),
    (dict(y=None), _lib.ERR_INVALID_ARG),
    (dict(ws=None), _lib.ERR_INVALID_ARG),
    (dict(ws_bytes=10), _lib.ERR_INVALID_ARG),
    (dict(M=-1), _lib.ERR_INVALID_ARG),
    (dict(N=-3), _lib.ERR_INVALID_ARG),
    (dict(bits=6), _lib.ERR_BAD_BITS),
    (dict(bits=0), _lib.ERR_BAD_BITS),
    (dict(K=192, had=1), _lib.ERR_NOT_POW2),
    (dict(K=100), _lib.ERR_ALIGN),
    (dict(K=0), _lib.ERR_ALIGN),
    (dict(K=65536), _lib.ERR_UNSUPPORTED),
    (dict(K=32768 + 64, had=0), _lib.ERR_UNSUPPORTED),
    (dict(xt=7), _lib.ERR_UNSUPPORTED),
    (dict(x=FAKE + 2), _lib.ERR_ALIGN),
    (dict(Wp=FAKE + 8), _lib.ERR_ALIGN),
    (dict(ws=FAKE + 4), _lib.ERR_ALIGN),
    (dict(y=FAKE + 1), _lib.ERR_ALIGN),
])
def test_forward_validation(lib, kwargs, status):
    assert _fwd(lib, **kwargs) == status
    assert lib.bitnet_last_error() != b""


def test_forward_workspace_may_be_null_when_fused(lib):
    # the fused decode shape needs no workspace; a missing one is not an error
    # (the call then reaches the launch, so only the validation is checked
    # here: an invalid bits value still wins)
    assert _fwd(lib, M=1, K=2560, N=6912, bits=6, had=0, ws=None, ws_bytes=0) == _lib.ERR_BAD_BITS
    assert _fwd(lib, M=1, K=2560, N=6912, bits=8, had=0, ws=None, ws_bytes=0,
                x=None) == _lib.ERR_INVALID_ARG
    # non-fused shapes without workspace
    assert _fwd(lib, M=1, K=2048, N=6912, bits=8, had=1, ws=None, ws_bytes=0) == _lib.ERR_INVALID_ARG
    assert _fwd(lib, M=64, K=2560, N=6912, bits=8, had=0, ws=None, ws_bytes=0) == _lib.ERR_INVALID_ARG


def test_forward_empty_is_noop(lib):
    # M = 0 / N = 0 return OK without launching (pointers are not touched).
    assert _fwd(lib, M=0, x=None, y=None, ws=None) == _lib.OK
    assert _fwd(lib, N=0, Wp=None, y=None, ws=None) == _lib.OK
    assert lib.bitnet_last_error() == b""


def test_ternarize_validation(lib):
    f = lib.bitnet_ternarize_weights
    assert f(None, 4, 64, FAKE, FAKE, FAKE, 1 << 20, None) == _lib.ERR_INVALID_ARG
    assert f(FAKE, 4, 60, FAKE, FAKE, FAKE, 1 << 20, None) == _lib.ERR_ALIGN
    assert f(FAKE, 0, 64, FAKE, FAKE, FAKE, 1 << 20, None) == _lib.ERR_INVALID_ARG
    assert f(FAKE, 4, 64, FAKE, FAKE, FAKE, 8, None) == _lib.ERR_INVALID_ARG
    assert f(FAKE, 4, 64, FAKE, FAKE + 2, FAKE, 1 << 20, None) == _lib.ERR_ALIGN


def test_pack_validation(lib):
    f = lib.bitnet_pack_2bit
    assert f(None, 4, 64, FAKE, None) == _lib.ERR_INVALID_ARG
    assert f(FAKE, 4, 96, FAKE, None) == _lib.ERR_ALIGN
    assert f(FAKE, 0, 64, None, None) == _lib.OK


def test_stage_entry_points_validation(lib):
    q = lib.bitnet_quantize_activations
    assert q(FAKE, _lib.F32, 2, 64, 5, 0, FAKE, FAKE, None, None) == _lib.ERR_BAD_BITS
    assert q(FAKE, _lib.F32, 2, 320, 8, 1, FAKE, FAKE, None, None) == _lib.ERR_NOT_POW2
    assert q(None, _lib.F32, 2, 64, 8, 0, FAKE, FAKE, None, None) == _lib.ERR_INVALID_ARG
    assert q(FAKE, _lib.F32, 2, 64, 8, 0, FAKE, FAKE, FAKE + 2, None) == _lib.ERR_ALIGN
    g = lib.bitnet_ternary_gemm_i32
    assert g(FAKE, 2, 70, FAKE, 3, FAKE, None) == _lib.ERR_ALIGN
    assert g(None, 2, 64, FAKE, 3, FAKE, None) == _lib.ERR_INVALID_ARG
    assert g(FAKE, 0, 64, FAKE, 3, None, None) == _lib.OK
    assert g(FAKE, 2, 65536, FAKE, 3, FAKE, None) == _lib.ERR_UNSUPPORTED
    assert g(FAKE + 8, 2, 64, FAKE, 3, FAKE, None) == _lib.ERR_ALIGN
    d = lib.bitnet_ternary_linear_dequant
    assert d(FAKE, FAKE, None, 2, 64, FAKE, 3, FAKE, 3, FAKE, None) == _lib.ERR_BAD_BITS
    assert d(FAKE, None, None, 2, 64, FAKE, 3, FAKE, 8, FAKE, None) == _lib.ERR_INVALID_ARG
    assert d(FAKE, FAKE, FAKE + 2, 2, 64, FAKE, 3, FAKE, 8, FAKE, None) == _lib.ERR_ALIGN


def test_binding_raises_typed_error(lib):
    with pytest.raises(_lib.BitNetError) as ei:
        _lib.call("bitnet_pack_2bit", None, 4, 64, FAKE, None)
    assert ei.value.status == _lib.ERR_INVALID_ARG
    assert "null pointer" in str(ei.value)


def test_last_error_is_per_thread(lib):
    import threading
    assert lib.bitnet_pack_2bit(None, 4, 64, FAKE, None) == _lib.ERR_INVALID_ARG
    seen = {}

    def other():
        seen["msg"] = lib.bitnet_last_error()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] == b""
    assert lib.bitnet_last_error() != b""


def _fwd_pro(lib, x=FAKE, up=FAKE, xt=_lib.BF16, M=4, K=256, rms=1, g=FAKE, eps=1e-7, Wp=FAKE,
             N=256, alpha=FAKE, bits=4, had=1, y=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return lib.bitnet_hbitlinear_forward_prologue(x, up, xt, M, K, rms, g, eps, Wp, N, alpha, bits,
                                                  had, y, ws, ws_bytes, None)


def test_prologue_workspace_sizes(lib):
    # always the two-launch path: codes + scales, even where the plain forward fuses
    assert lib.bitnet_forward_prologue_workspace_bytes(1, 2560, 6912, 8, 0) == 2560 + 2 * 256
    assert lib.bitnet_forward_prologue_workspace_bytes(2048, 8192, 2048, 4, 1) == 2048 * 8192 + 2 * 8192
    assert lib.bitnet_forward_prologue_workspace_bytes(0, 64, 8, 8, 0) == 0
    assert lib.bitnet_forward_prologue_workspace_bytes(4, 100, 8, 8, 0) == 0


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=None), _lib.ERR_INVALID_ARG),
    (dict(ws=None), _lib.ERR_INVALID_ARG),
    (dict(ws_bytes=100), _lib.ERR_INVALID_ARG),
    (dict(rms=2), _lib.ERR_INVALID_ARG),
    (dict(eps=0.0), _lib.ERR_INVALID_ARG),
    (dict(eps=-1e-7), _lib.ERR_INVALID_ARG),
    (dict(eps=float("inf")), _lib.ERR_INVALID_ARG),
    (dict(eps=float("nan")), _lib.ERR_INVALID_ARG),
    (dict(up=FAKE + 4), _lib.ERR_ALIGN),
    (dict(g=FAKE + 8), _lib.ERR_ALIGN),
    (dict(bits=3), _lib.ERR_BAD_BITS),
    (dict(K=192, had=1), _lib.ERR_NOT_POW2),
    (dict(K=100), _lib.ERR_ALIGN),
])
def test_prologue_forward_validation(lib, kwargs, status):
    assert _fwd_pro(lib, **kwargs) == status
    assert lib.bitnet_last_error() != b""


def test_prologue_optional_parts_and_noop(lib):
    # no RMSNorm: eps and the weight pointer are not inspected
    assert _fwd_pro(lib, rms=0, eps=0.0, g=FAKE + 8, x=None) == _lib.ERR_INVALID_ARG
    assert b"null pointer" in lib.bitnet_last_error()
    # M = 0 / N = 0 are no-ops
    assert _fwd_pro(lib, M=0, x=None, up=None, y=None, ws=None) == _lib.OK
    assert _fwd_pro(lib, N=0, Wp=None, y=None, ws=None) == _lib.OK
    q = lib.bitnet_quantize_activations_prologue
    assert q(FAKE, None, _lib.F32, 2, 64, 1, None, 0.0, 8, 0, FAKE, FAKE, None) == _lib.ERR_INVALID_ARG
    assert q(FAKE, FAKE + 2, _lib.F32, 2, 64, 0, None, 1e-7, 8, 0, FAKE, FAKE, None) == _lib.ERR_ALIGN
    assert q(None, None, _lib.F32, 0, 64, 1, None, 1e-7, 8, 0, None, None, None) == _lib.OK


@pytest.mark.parametrize("args,status", [
    (dict(R=-1), _lib.ERR_INVALID_ARG),
    (dict(bits=2), _lib.ERR_BAD_BITS),
    (dict(bits=16), _lib.ERR_BAD_BITS),
    (dict(D=12), _lib.ERR_ALIGN),
    (dict(D=0), _lib.ERR_ALIGN),
    (dict(D=520), _lib.ERR_UNSUPPORTED),
    (dict(S=0), _lib.ERR_INVALID_ARG),
    (dict(R=10, S=4), _lib.ERR_INVALID_ARG),
    (dict(dt=5), _lib.ERR_UNSUPPORTED),
    (dict(kv=None), _lib.ERR_INVALID_ARG),
    (dict(codes=FAKE + 4), _lib.ERR_ALIGN),
    (dict(kv=FAKE + 2), _lib.ERR_ALIGN),
])
def test_kv_quantize_validation(lib, args, status):
    a = dict(kv=FAKE, dt=_lib.BF16, R=16, D=128, S=8, bits=3, codes=FAKE, scales=FAKE)
    a.update(args)
    assert lib.bitnet_kv_quantize(a["kv"], a["dt"], a["R"], a["D"], a["S"], a["bits"], a["codes"],
                                  a["scales"], None) == status
    assert lib.bitnet_last_error() != b""


def test_kv_quantize_empty_is_noop(lib):
    assert lib.bitnet_kv_quantize(None, _lib.BF16, 0, 64, 4, 4, None, None, None) == _lib.OK


@pytest.mark.parametrize("args,status", [
    (dict(bits=8), _lib.ERR_BAD_BITS),        # packing is for 3 and 4 bits
    (dict(bits=2), _lib.ERR_BAD_BITS),
    (dict(bits=3, D=40), _lib.ERR_ALIGN),     # 3-bit rows must be whole 32-bit words
    (dict(bits=4, D=12), _lib.ERR_ALIGN),
    (dict(bits=4, D=520), _lib.ERR_UNSUPPORTED),
    (dict(R=10, S=4), _lib.ERR_INVALID_ARG),
    (dict(bos=None), _lib.ERR_INVALID_ARG),
    (dict(packed=None), _lib.ERR_INVALID_ARG),
    (dict(packed=FAKE + 2), _lib.ERR_ALIGN),
    (dict(bos=FAKE + 4), _lib.ERR_ALIGN),
    (dict(kv=FAKE + 8), _lib.ERR_ALIGN),
])
def test_kv_quantize_packed_validation(lib, args, status):
    a = dict(kv=FAKE, dt=_lib.BF16, R=16, D=128, S=8, bits=3, packed=FAKE, bos=FAKE, scales=FAKE)
    a.update(args)
    assert lib.bitnet_kv_quantize_packed(a["kv"], a["dt"], a["R"], a["D"], a["S"], a["bits"],
                                         a["packed"], a["bos"], a["scales"], None) == status
    assert lib.bitnet_last_error() != b""


def test_kv_quantize_packed_empty_is_noop(lib):
    assert lib.bitnet_kv_quantize_packed(None, _lib.BF16, 0, 64, 4, 4, None, None, None,
                                         None) == _lib.OK


def test_backward_workspace_sizes(lib):
    # dx: t^T in bf16 (K*N*2); an fp32 dy adds its two bf16 halves (2*M*N*2)
    assert lib.bitnet_backward_workspace_bytes(128, 256, 192, _lib.BF16, 1, 0) == 256 * 192 * 2
    assert lib.bitnet_backward_workspace_bytes(128, 256, 192, _lib.F32, 1, 0) == \
        256 * 192 * 2 + 2 * 128 * 192 * 2
    # dw: hi/lo of dy*s/c transposed (2*N*Mp*2) + codes transposed (K*Mp*2), Mp = M padded to 64
    assert lib.bitnet_backward_workspace_bytes(100, 256, 192, _lib.BF16, 0, 1) == \
        2 * 192 * 128 * 2 + 256 * 128 * 2
    # both: the two parts share the bytes
    dx_part = 256 * 192 * 2 + 2 * 100 * 192 * 2        # every part a multiple of 256 here
    dw_part = 2 * 192 * 128 * 2 + 256 * 128 * 2
    assert lib.bitnet_backward_workspace_bytes(100, 256, 192, _lib.F32, 1, 1) == max(dx_part, dw_part)
    assert lib.bitnet_backward_workspace_bytes(100, 256, 192, _lib.BF16, 1, 1) == dw_part
    assert lib.bitnet_backward_workspace_bytes(4, 100, 64, _lib.BF16, 1, 1) == 0  # invalid K
    assert lib.bitnet_backward_workspace_bytes(4, 128, 96, _lib.BF16, 1, 1) == 0  # invalid N


def _bwd(lib, dy=FAKE, dt=_lib.BF16, M=128, N=192, codes=FAKE, scales=FAKE, K=256, Wp=FAKE,
         alpha=FAKE, bits=8, had=1, dx=FAKE, dw=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return lib.bitnet_hbitlinear_backward(dy, dt, M, N, codes, scales, K, Wp, alpha, bits, had, dx,
                                          dw, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dy=None), _lib.ERR_INVALID_ARG),
    (dict(codes=None), _lib.ERR_INVALID_ARG),
    (dict(scales=None), _lib.ERR_INVALID_ARG),
    (dict(Wp=None), _lib.ERR_INVALID_ARG),
    (dict(alpha=None), _lib.ERR_INVALID_ARG),
    (dict(ws=None), _lib.ERR_INVALID_ARG),
    (dict(ws_bytes=100), _lib.ERR_INVALID_ARG),
    (dict(M=-1), _lib.ERR_INVALID_ARG),
    (dict(had=2), _lib.ERR_INVALID_ARG),
    (dict(bits=3), _lib.ERR_BAD_BITS),
    (dict(K=100), _lib.ERR_ALIGN),
    (dict(N=100), _lib.ERR_ALIGN),
    (dict(K=192, had=1), _lib.ERR_NOT_POW2),
    (dict(K=65536, had=1), _lib.ERR_NOT_POW2),
    (dict(M=1 << 22), _lib.ERR_UNSUPPORTED),
    (dict(dt=9), _lib.ERR_UNSUPPORTED),
    (dict(dy=FAKE + 2), _lib.ERR_ALIGN),
    (dict(codes=FAKE + 8), _lib.ERR_ALIGN),
    (dict(ws=FAKE + 16), _lib.ERR_ALIGN),
    (dict(dx=FAKE + 1), _lib.ERR_ALIGN),
])
def test_backward_validation(lib, kwargs, status):
    assert _bwd(lib, **kwargs) == status
    assert lib.bitnet_last_error() != b""


def test_backward_optional_outputs(lib):
    # neither gradient wanted: nothing to do, nothing read
    assert _bwd(lib, dx=None, dw=None, dy=None, ws=None) == _lib.OK
    # dx only: codes and scales are not needed; dw only: the weights are not
    assert _bwd(lib, dw=None, codes=None, scales=None, Wp=None) == _lib.ERR_INVALID_ARG
    assert _bwd(lib, dx=None, Wp=None, alpha=None, codes=None) == _lib.ERR_INVALID_ARG
    # no tokens and no weight gradient: dx has no elements
    assert _bwd(lib, M=0, dw=None, dy=None, ws=None) == _lib.OK


def test_tl2_sizes_and_validation(lib):
    # 80 bytes per column and 384-weight block (5 bits per 3 weights)
    assert lib.bitnet_tl2_bytes(6912, 2560) == 6912 * (6 * 80 + 64)   # a last block of 3 groups
    assert lib.bitnet_tl2_bytes(3, 384) == 3 * 80
    assert lib.bitnet_tl2_bytes(2, 448) == 2 * (80 + 32)             # ... of 1 group
    assert lib.bitnet_tl2_bytes(1, 16384) == 42 * 80 + 64
    assert lib.bitnet_tl2_bytes(3, 100) == 0            # K not a multiple of 64
    assert lib.bitnet_tl2_bytes(0, 64) == 0
    p = lib.bitnet_pack_tl2
    assert p(None, 4, 64, FAKE, None) == _lib.ERR_INVALID_ARG
    assert p(FAKE, 4, 96, FAKE, None) == _lib.ERR_ALIGN
    assert p(FAKE, 4, 64, FAKE + 8, None) == _lib.ERR_ALIGN
    assert p(FAKE, 0, 64, None, None) == _lib.OK
    f = lib.bitnet_hbitlinear_forward_tl2
    assert f(FAKE, _lib.BF16, 2, 256, FAKE, 16, FAKE, 8, FAKE, None) == _lib.ERR_UNSUPPORTED
    assert f(FAKE, _lib.BF16, 1, 4672, FAKE, 16, FAKE, 8, FAKE, None) == _lib.ERR_UNSUPPORTED
    assert f(FAKE, _lib.BF16, 1, 256, FAKE, 16, FAKE, 5, FAKE, None) == _lib.ERR_BAD_BITS
    assert f(FAKE, _lib.BF16, 1, 100, FAKE, 16, FAKE, 8, FAKE, None) == _lib.ERR_ALIGN
    assert f(None, _lib.BF16, 1, 256, FAKE, 16, FAKE, 8, FAKE, None) == _lib.ERR_INVALID_ARG
    assert f(None, _lib.BF16, 0, 256, None, 16, None, 8, None, None) == _lib.OK


def test_tl2_batched_sizes_and_validation(lib):
    w = lib.bitnet_tl2_forward_workspace_bytes
    assert w(1, 2560) == 0                               # one token: the single-token kernel
    assert w(1, 4672) == 5120 + 2 * 256                  # K past it: 4992 codes, 256-B rounded
    assert w(16, 16384) == 16 * 16512 + 2 * 256          # 43 blocks of 384 codes per row
    assert w(17, 64) == 0 and w(4, 100) == 0 and w(0, 64) == 0
    f = lib.bitnet_hbitlinear_forward_tl2_batched
    args = lambda M=4, K=512, x=FAKE, ws=FAKE, ws_bytes=1 << 30, bits=8: (
        x, _lib.BF16, M, K, FAKE, 16, FAKE, bits, FAKE, ws, ws_bytes, None)
    assert f(*args(M=17)) == _lib.ERR_UNSUPPORTED
    assert f(*args(bits=5)) == _lib.ERR_BAD_BITS
    assert f(*args(K=100)) == _lib.ERR_ALIGN
    assert f(*args(x=None)) == _lib.ERR_INVALID_ARG
    assert f(*args(ws=None, ws_bytes=0)) == _lib.ERR_INVALID_ARG
    assert f(*args(ws_bytes=w(4, 512) - 1)) == _lib.ERR_INVALID_ARG
    assert f(*args(ws=FAKE + 8)) == _lib.ERR_ALIGN
    assert f(*args(M=0, x=None, ws=None, ws_bytes=0)) == _lib.OK


def _stages(lib, stages, M=4, K=512, N=256, bits=4, had=1, x=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return lib.bitnet_hbitlinear_forward_stages(x, _lib.BF16, M, K, FAKE, N, FAKE, bits, had, FAKE,
                                                ws, ws_bytes, stages, None)


def test_forward_stages_validation(lib):
    assert _stages(lib, 0) == _lib.ERR_INVALID_ARG
    assert _stages(lib, 4) == _lib.ERR_INVALID_ARG
    assert _stages(lib, 1, bits=5) == _lib.ERR_BAD_BITS
    assert _stages(lib, 2, x=None) == _lib.ERR_INVALID_ARG
    assert _stages(lib, 1, ws=None, ws_bytes=0) == _lib.ERR_INVALID_ARG
    # a shape the forward runs as one fused kernel has no separate stages
    assert _stages(lib, 1, M=1, K=2560, N=6912, bits=8, had=0) == _lib.ERR_UNSUPPORTED
    assert b"fused" in lib.bitnet_last_error()
    assert _stages(lib, 2, M=0) == _lib.OK


def test_stream_read_validation(lib):
    f = lib.bitnet_stream_read
    assert f(None, 1024, FAKE, None) == _lib.ERR_INVALID_ARG
    assert f(FAKE, 1024, None, None) == _lib.ERR_INVALID_ARG
    assert f(FAKE + 8, 1024, FAKE, None) == _lib.ERR_ALIGN
    assert f(FAKE, 1000, FAKE, None) == _lib.ERR_ALIGN
    assert f(None, 0, None, None) == _lib.OK


# Every entry point that launches work, with arguments that pass validation:
# with an injected launch error each must report BITNET_ERR_HIP, name itself
# and the HIP code in bitnet_last_error(), and launch nothing (the hook is
# taken before any HIP call, so no device is needed).
LAUNCHING_CALLS = {
    "bitnet_ternarize_weights": (FAKE, 4, 64, FAKE, FAKE, FAKE, 1 << 20, None),
    "bitnet_pack_2bit": (FAKE, 4, 64, FAKE, None),
    "bitnet_hbitlinear_forward": (FAKE, _lib.BF16, 4, 512, FAKE, 256, FAKE, 4, 1, FAKE, FAKE,
                                  1 << 30, None),
    "bitnet_hbitlinear_forward_stages": (FAKE, _lib.BF16, 4, 512, FAKE, 256, FAKE, 4, 1, FAKE,
                                         FAKE, 1 << 30, 1, None),
    "bitnet_quantize_activations": (FAKE, _lib.F32, 2, 64, 8, 0, FAKE, FAKE, None, None),
    "bitnet_ternary_gemm_i32": (FAKE, 2, 64, FAKE, 3, FAKE, None),
    "bitnet_ternary_linear_dequant": (FAKE, FAKE, None, 2, 64, FAKE, 3, FAKE, 8, FAKE, None),
    "bitnet_hbitlinear_forward_prologue": (FAKE, FAKE, _lib.BF16, 4, 256, 1, FAKE, 1e-7, FAKE, 256,
                                           FAKE, 4, 1, FAKE, FAKE, 1 << 30, None),
    "bitnet_quantize_activations_prologue": (FAKE, None, _lib.F32, 2, 64, 1, None, 1e-7, 8, 0,
                                             FAKE, FAKE, None),
    "bitnet_kv_quantize": (FAKE, _lib.BF16, 16, 128, 8, 3, FAKE, FAKE, None),
    "bitnet_kv_quantize_packed": (FAKE, _lib.BF16, 16, 128, 8, 3, FAKE, FAKE, FAKE, None),
    "bitnet_pack_tl2": (FAKE, 4, 64, FAKE, None),
    "bitnet_hbitlinear_forward_tl2": (FAKE, _lib.BF16, 1, 256, FAKE, 16, FAKE, 8, FAKE, None),
    "bitnet_hbitlinear_forward_tl2_batched": (FAKE, _lib.BF16, 4, 512, FAKE, 16, FAKE, 8, FAKE,
                                              FAKE, 1 << 30, None),
    "bitnet_hbitlinear_backward": (FAKE, _lib.BF16, 128, 192, FAKE, FAKE, 256, FAKE, FAKE, 8, 1,
                                   FAKE, FAKE, FAKE, 1 << 30, None),
    "bitnet_stream_read": (FAKE, 1024, FAKE, None),
    "bitnet_hbitlinear_forward_noalloc": (FAKE, _lib.BF16, 4, 512, FAKE, 256, FAKE, 4, 1, FAKE,
                                          None),
}

HIP_ERROR_OUT_OF_MEMORY = 2  # hipErrorOutOfMemory


@pytest.mark.parametrize("name", sorted(LAUNCHING_CALLS))
def test_injected_launch_error_is_reported(lib, name):
    lib.bitnet_test_fail_next_launch(HIP_ERROR_OUT_OF_MEMORY)
    assert getattr(lib, name)(*LAUNCHING_CALLS[name]) == _lib.ERR_HIP
    msg = lib.bitnet_last_error().decode()
    assert name in msg and "HIP error 2" in msg, msg
    with pytest.raises(_lib.BitNetError) as ei:
        lib.bitnet_test_fail_next_launch(HIP_ERROR_OUT_OF_MEMORY)
        _lib.call(name, *LAUNCHING_CALLS[name])
    assert ei.value.status == _lib.ERR_HIP


def test_injected_error_is_taken_once_and_not_by_failed_validation(lib):
    lib.bitnet_test_fail_next_launch(HIP_ERROR_OUT_OF_MEMORY)
    # an argument error comes first and leaves the injected error pending
    assert lib.bitnet_pack_2bit(None, 4, 64, FAKE, None) == _lib.ERR_INVALID_ARG
    assert lib.bitnet_pack_2bit(FAKE, 4, 64, FAKE, None) == _lib.ERR_HIP
    # cleared: a no-op call succeeds and clears the message
    lib.bitnet_test_fail_next_launch(HIP_ERROR_OUT_OF_MEMORY)
    lib.bitnet_test_fail_next_launch(0)
    assert lib.bitnet_pack_2bit(FAKE, 0, 64, None, None) == _lib.OK
    assert lib.bitnet_last_error() == b""


def test_every_launching_entry_point_is_covered():
    """Every declared entry point that returns a status and takes a stream is
    in the injected-error table."""
    with open(_lib.HEADER_PATH) as f:
        text = f.read()
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    launching = set(re.findall(r"bitnet_status\s+(bitnet_[a-z0-9_]+)\s*\([^;]*hipStream_t", text))
    assert launching == set(LAUNCHING_CALLS)


# ---- dispatch, on the host build only (its launchers record their names) ----
stub_only = pytest.mark.skipif(not HOST_LIB, reason="needs the host-only sanitizer build")


def _calls(lib, fn, *args):
    lib.bitnet_stub_reset()
    assert fn(*args) == _lib.OK, lib.bitnet_last_error()
    return lib.bitnet_stub_calls().decode().split()


@stub_only
@pytest.mark.parametrize("M,K,N,bits,had,want", [
    (1, 2560, 6912, 8, 0, ["fused_decode"]),                    # single-token decode
    (4, 256, 256, 4, 1, ["fused_decode"]),                      # transform fused for K <= 256
    (16, 16384, 4096, 4, 1, ["quantize_nibbles", "matmul_nibbles"]),
    (16, 16384, 4096, 8, 1, ["quantize", "matmul"]),
    (2048, 8192, 2048, 4, 1, ["quantize_fp8_pairs", "matmul_fp8_pairs"]),  # bf16, transform, 4-bit
    (2048, 8192, 2048, 8, 1, ["quantize", "matmul"]),           # prefill: never nibble codes
    (8192, 8192, 8192, 4, 1, ["quantize", "matmul"]),           # 1024 tiles of 256: int8 codes
    (2048, 1024, 2048, 4, 1, ["quantize_fp8_pairs", "matmul_fp8_pairs"]),  # the butterfly kernel
    (2048, 1024, 2048, 4, 0, ["quantize", "matmul"]),           # no transform: int8 codes
    (3, 192, 40, 4, 0, ["fused_decode"]),
])
def test_forward_dispatch(lib, M, K, N, bits, had, want):
    need = lib.bitnet_forward_workspace_bytes(M, K, N, bits, had)
    ws = ctypes.create_string_buffer(max(need, 16) + 256)
    ws_addr = (ctypes.addressof(ws) + 255) // 256 * 256
    got = _calls(lib, lib.bitnet_hbitlinear_forward, FAKE, _lib.BF16, M, K, FAKE, N, FAKE, bits,
                 had, FAKE, ws_addr if need else None, need, None)
    assert got == want
    if need:
        q = _calls(lib, lib.bitnet_hbitlinear_forward_stages, FAKE, _lib.BF16, M, K, FAKE, N, FAKE,
                   bits, had, FAKE, ws_addr, need, _lib.STAGE_QUANTIZE, None)
        p = _calls(lib, lib.bitnet_hbitlinear_forward_stages, FAKE, _lib.BF16, M, K, FAKE, N, FAKE,
                   bits, had, FAKE, ws_addr, need, _lib.STAGE_PRODUCT, None)
        assert q + p == want


@stub_only
def test_other_dispatch(lib):
    ws = ctypes.create_string_buffer(1 << 16)
    a = (ctypes.addressof(ws) + 255) // 256 * 256
    tl2 = lib.bitnet_hbitlinear_forward_tl2_batched
    assert _calls(lib, tl2, FAKE, _lib.BF16, 1, 2560, FAKE, 64, FAKE, 8, FAKE, None, 0,
                  None) == ["tl2_decode"]
    assert _calls(lib, tl2, FAKE, _lib.BF16, 4, 512, FAKE, 64, FAKE, 4, FAKE, a, 1 << 14,
                  None) == ["quantize_tl2_order", "tl2_gemv"]
    assert _calls(lib, lib.bitnet_ternarize_weights, FAKE, 4, 64, FAKE, FAKE, a, 1 << 14,
                  None) == ["absmean_partial", "ternarize_pack"]
    assert _calls(lib, lib.bitnet_ternary_gemm_i32, FAKE, 2, 64, FAKE, 3, FAKE, None) == ["matmul_i32"]
    assert _calls(lib, lib.bitnet_kv_quantize, FAKE, _lib.BF16, 16, 128, 8, 4, FAKE, FAKE,
                  None) == ["kv_quantize"]
    assert _calls(lib, lib.bitnet_kv_quantize_packed, FAKE, _lib.BF16, 16, 128, 8, 4, FAKE, FAKE,
                  FAKE, None) == ["kv_quantize_packed"]
    # backward with an fp32 dy: dx from split halves and the transform, then dw
    bws = lib.bitnet_backward_workspace_bytes(128, 256, 192, _lib.F32, 1, 1)
    big = ctypes.create_string_buffer(bws + 256)
    b = (ctypes.addressof(big) + 255) // 256 * 256
    assert _calls(lib, lib.bitnet_hbitlinear_backward, FAKE, _lib.F32, 128, 192, FAKE, FAKE, 256,
                  FAKE, FAKE, 8, 1, FAKE, FAKE, b, bws, None) == [
        "expand_transpose", "split_rows", "bf16_gemm_nt", "fwht_f32", "scale_transpose_split",
        "codes_transpose", "bf16_gemm_nt"]


def test_noalloc_validation(lib):
    f = lib.bitnet_hbitlinear_forward_noalloc
    # a batch whose workspace exceeds the fixed scratch is refused up front
    assert f(FAKE, _lib.BF16, 8192, 16384, FAKE, 64, FAKE, 8, 0, FAKE, None) == _lib.ERR_UNSUPPORTED
    assert b"scratch" in lib.bitnet_last_error()
    # the limit is the workspace the forward needs: codes M * K plus 8 B of
    # scales and row sums per token (each part rounded up to 256 B)
    M, K = 65536 - 512, 1024
    assert lib.bitnet_forward_workspace_bytes(M, K, 64, 8, 0) <= _lib.NOALLOC_SCRATCH_BYTES
    assert lib.bitnet_forward_workspace_bytes(M + 256, K, 64, 8, 0) > _lib.NOALLOC_SCRATCH_BYTES
    assert f(FAKE, _lib.BF16, M + 256, K, FAKE, 64, FAKE, 8, 0, FAKE, None) == _lib.ERR_UNSUPPORTED
    lib.bitnet_test_fail_next_launch(HIP_ERROR_OUT_OF_MEMORY)  # stop before any launch
    assert f(FAKE, _lib.BF16, M, K, FAKE, 64, FAKE, 8, 0, FAKE, None) == _lib.ERR_HIP
    # the other checks are the forward's
    assert f(None, _lib.BF16, 4, 512, FAKE, 256, FAKE, 4, 1, FAKE, None) == _lib.ERR_INVALID_ARG
    assert f(FAKE, _lib.BF16, 4, 512, FAKE, 256, FAKE, 5, 1, FAKE, None) == _lib.ERR_BAD_BITS
    assert f(FAKE, _lib.BF16, 4, 192, FAKE, 256, FAKE, 4, 1, FAKE, None) == _lib.ERR_NOT_POW2
    assert f(FAKE + 2, _lib.BF16, 4, 512, FAKE, 256, FAKE, 4, 1, FAKE, None) == _lib.ERR_ALIGN
    assert f(None, _lib.BF16, 0, 512, None, 256, None, 4, 1, None, None) == _lib.OK


@stub_only
def test_noalloc_dispatch(lib):
    f = lib.bitnet_hbitlinear_forward_noalloc
    assert _calls(lib, f, FAKE, _lib.BF16, 64, 1024, FAKE, 256, FAKE, 8, 1, FAKE,
                  None) == ["noalloc_scratch", "quantize", "matmul"]
    # a fused shape needs no scratch and does not look it up
    assert _calls(lib, f, FAKE, _lib.BF16, 1, 2560, FAKE, 6912, FAKE, 8, 0, FAKE,
                  None) == ["fused_decode"]
