"""Parity of the forward with its input prologue (RMSNorm, SwiGLU product)
on MI355X, through the C ABI, against the CPU oracle.

Engine page: HBitLinear.forward step 1 (nn.RMSNorm) and BitNetV2FFN.forward
(silu(gate) * up feeding the H-BitLinear down projection). Same acceptance
rules as the plain forward: codes bit-exact up to +-1 flips inside the 1e-4
rounding band, int32 products exact on the GPU's codes, y to 1e-3.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import bit_activation_linear_amd as bl
from bit_activation_linear_amd import workloads
from parity_util import (assert_codes_match, assert_packed_match, assert_y_close, assert_y_in_band,
                         assert_y_with_flips, decode_packed)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _to_dev(x_np, x_dtype):
    if x_dtype == "bf16":
        return torch.from_numpy(x_np.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(x_np).to(DEV)


def _run(M, K, N, bits, had, x_dtype, swiglu, rms, gamma, seed):
    _say(f"prologue case M={M} K={K} N={N} bits={bits} hadamard={had} x={x_dtype} "
         f"swiglu={swiglu} rms={rms} gamma={gamma} seed={seed}")
    case = workloads.make_case(M, K, N, x_dtype=x_dtype, n_out=max(1, K // 100), factor=20.0,
                               seed=seed)
    rng = np.random.default_rng(seed + 1000)
    up_np = None
    if swiglu:
        # the up projection, same dtype and shape as the gate projection x
        upc = workloads.make_case(M, K, 1, x_dtype=x_dtype, seed=seed + 1)
        up_np = upc["x"]
    g_np = (rng.standard_normal(K) * 0.3 + 1.0).astype(np.float32) if gamma else None

    x = _to_dev(case["x"], x_dtype)
    up = _to_dev(up_np, x_dtype) if swiglu else None
    g = torch.from_numpy(g_np).to(DEV) if gamma else None
    W = torch.from_numpy(case["W"]).to(DEV)
    Wp, alpha = bl.ternarize_weights(W)
    codes, scales = bl.quantize_activations_prologue(x, bits, had, up=up, rmsnorm=rms, norm_weight=g)
    y = bl.hbitlinear_forward_prologue(x, Wp, alpha, bits, had, up=up, rmsnorm=rms, norm_weight=g)
    y2 = bl.ternary_linear_dequant(codes, scales, Wp, alpha, bits)
    torch.cuda.synchronize()

    t_ref, a_ref, p_w = oracle.ternarize(case["W"])
    assert_packed_match(Wp.cpu().numpy(), t_ref, p_w)
    ref = oracle.forward_prologue(case["x"], x_dtype, t_ref, a_ref, bits, had, up=up_np, rms=rms,
                                  norm_weight=None if g_np is None else g_np.astype(np.float64))
    q_gpu = codes.cpu().numpy()
    assert_codes_match(q_gpu, ref["q"], ref["p"])
    np.testing.assert_allclose(scales.cpu().numpy(), ref["s"], rtol=1e-5)
    # the staged product on the inspected codes; a flip inside the rounding
    # band is allowed its bounded effect on y
    assert_y_with_flips(y2.cpu().numpy(), q_gpu, decode_packed(Wp.cpu().numpy()), ref["q"], t_ref,
                        ref["s"], a_ref, bits, ref["y64"])
    # The forward is those two stages, bit for bit, except for the decode
    # shapes it runs as one fused kernel: there the statistic and the sum of
    # squares are reduced in another order, so an ulp of a scale can move a
    # code on a rounding boundary. That forward is compared with the oracle
    # directly, each code in the rounding band allowed its bounded effect.
    if bl.forward_workspace_bytes(M, K, N, bits, had) == 0:
        assert_y_in_band(y.cpu().numpy(), decode_packed(Wp.cpu().numpy()), ref["q"], ref["p"],
                         t_ref, ref["s"], a_ref, bits, ref["y64"])
    else:
        np.testing.assert_array_equal(y.cpu().numpy(), y2.cpu().numpy())


@pytest.mark.parametrize("M,K,N,bits,had,xdt,swiglu,rms,gamma", [
    (4, 256, 256, 4, 1, "fp32", True, True, True),       # single layer, whole prologue
    (2, 128, 50, 8, 1, "bf16", True, True, True),        # fused with the transform
    (1, 256, 64, 4, 1, "fp32", False, True, False),      # fused with the transform, one row
    (1, 2560, 300, 8, 0, "bf16", False, True, True),     # decode row, RMSNorm only: one-wave kernel
    (1, 1088, 77, 4, 0, "fp32", False, True, True),      # one-wave kernel, int4, partial super-block
    (1, 64, 33, 8, 0, "bf16", False, True, False),       # one-wave kernel, a single 64-weight block
    (1, 4096, 40, 4, 0, "bf16", False, True, True),      # one-wave kernel, sixteen super-blocks
    (16, 16384, 96, 4, 1, "bf16", True, True, False),    # batched decode, long rows
    (300, 1024, 260, 8, 1, "bf16", False, True, False),  # prefill tile, unit-weight norm
    (129, 8192, 130, 4, 1, "bf16", True, True, True),    # Wdown-style prefill (fp8-pair product)
    (100, 512, 64, 4, 1, "fp32", True, True, True),      # fp8 pairs, 8 elements per thread
    (40, 2048, 96, 4, 1, "bf16", False, True, True),     # fp8 pairs, few rows, 16 elements per thread
    (64, 4096, 200, 8, 0, "fp32", True, False, False),   # SwiGLU product only
    (3, 64, 17, 4, 0, "bf16", True, True, True),         # smallest K, ragged N (fused decode)
    (4, 4096, 90, 4, 0, "bf16", True, True, True),       # fused decode kernel, whole prologue
    (16, 1024, 48, 8, 0, "fp32", True, False, False),    # fused decode kernel, SwiGLU only
    (1, 2048, 200, 8, 0, "bf16", False, True, False),    # fused decode kernel, unit-weight norm
    (2, 2048, 70, 4, 0, "bf16", True, True, True),       # fused decode kernel, two rows, whole prologue
    (1, 4096, 64, 8, 0, "fp32", True, True, True),       # fused decode kernel, fp32, longest fused row
])
def test_prologue_parity(M, K, N, bits, had, xdt, swiglu, rms, gamma):
    _run(M, K, N, bits, had, xdt, swiglu, rms, gamma, seed=M + K + N + 7 * bits + had)


def test_prologue_without_parts_matches_plain_forward():
    """No SwiGLU and no RMSNorm: the prologue path computes exactly the plain
    forward's codes and scales (a prologue with both parts off runs the plain
    quantizer) and the same output."""
    case = workloads.make_case(40, 2048, 70, x_dtype="bf16", n_out=20, factor=30.0, seed=9)
    x = _to_dev(case["x"], "bf16")
    Wp, alpha = bl.ternarize_weights(torch.from_numpy(case["W"]).to(DEV))
    for bits, had in [(8, 0), (4, 1)]:
        c0, s0 = bl.quantize_activations(x, bits, had)
        c1, s1 = bl.quantize_activations_prologue(x, bits, had, rmsnorm=False)
        y0 = bl.hbitlinear_forward(x, Wp, alpha, bits, had)
        y1 = bl.hbitlinear_forward_prologue(x, Wp, alpha, bits, had, rmsnorm=False)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(c0.cpu().numpy(), c1.cpu().numpy())
        np.testing.assert_array_equal(s0.cpu().numpy(), s1.cpu().numpy())
        np.testing.assert_array_equal(y0.cpu().numpy(), y1.cpu().numpy())


def test_prologue_zero_rows():
    """A zero gate row gives a zero SwiGLU row: RMSNorm keeps it zero
    (rms = sqrt(eps)), codes 0, scale eps, output row 0."""
    M, K, N = 4, 512, 33
    x = torch.zeros((M, K), dtype=torch.float32, device=DEV)
    x[1] = torch.linspace(-3, 3, K, device=DEV)
    up = torch.ones((M, K), dtype=torch.float32, device=DEV)
    W = torch.randn((N, K), generator=torch.Generator().manual_seed(0)).to(DEV) * 0.02
    Wp, alpha = bl.ternarize_weights(W)
    for bits, had in [(8, 0), (4, 1)]:
        codes, scales = bl.quantize_activations_prologue(x, bits, had, up=up, rmsnorm=True)
        y = bl.hbitlinear_forward_prologue(x, Wp, alpha, bits, had, up=up, rmsnorm=True)
        torch.cuda.synchronize()
        c = codes.cpu().numpy()
        assert np.all(c[[0, 2, 3]] == 0) and np.any(c[1] != 0)
        s = scales.cpu().numpy()
        np.testing.assert_allclose(s[[0, 2, 3]], 1e-7, rtol=1e-6)
        assert np.all(y.cpu().numpy()[[0, 2, 3]] == 0.0)


def test_module_wrapper_whole_layer():
    """HBitLinear(rmsnorm=True) runs the engine page's whole HBitLinear.forward;
    forward(x, up=...) the FFN's down projection of silu(x) * up."""
    case = workloads.make_case(9, 512, 70, x_dtype="fp32", n_out=5, factor=40.0, seed=13)
    up_np = workloads.make_case(9, 512, 1, x_dtype="fp32", seed=14)["x"]
    g_np = (np.random.default_rng(15).standard_normal(512) * 0.2 + 1.0).astype(np.float32)
    layer = bl.HBitLinear(torch.from_numpy(case["W"]).to(DEV), bits=4, hadamard=True, rmsnorm=True,
                          norm_weight=torch.from_numpy(g_np).to(DEV))
    x = torch.from_numpy(case["x"]).to(DEV)
    y1 = layer(x)
    y2 = layer(x, up=torch.from_numpy(up_np).to(DEV))
    torch.cuda.synchronize()
    t, a, _ = oracle.ternarize(case["W"])
    r1 = oracle.forward_prologue(case["x"], "fp32", t, a, 4, 1, rms=True, norm_weight=g_np)
    r2 = oracle.forward_prologue(case["x"], "fp32", t, a, 4, 1, up=up_np, rms=True, norm_weight=g_np)
    assert_y_close(y1.cpu().numpy(), r1["y64"])
    assert_y_close(y2.cpu().numpy(), r2["y64"])
