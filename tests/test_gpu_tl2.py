"""TL2 weight code (edge page, module docstring item 2 and class
SignedUnsignedWeightPacker) on the GPU, through the C ABI.

* bitnet_pack_tl2 re-encodes the 2-bit weights; its bytes must equal the
  oracle's TL2 encoding of the same ternary weights, bit for bit.
* bitnet_hbitlinear_forward_tl2 is the single-token decode forward on those
  bytes, and bitnet_hbitlinear_forward_tl2_batched the forward of up to 16
  tokens (the same kernel for one token of K <= 4608). It takes the same quantization steps as the 2-bit single-token
  kernel: with int8 (absmax, order-free) its output must equal the 2-bit
  forward's bit for bit; with int4 the absmean sums in another order, and a
  code on a rounding boundary may move. Both are compared with the fp64
  oracle at the forward's tolerance, each code in the rounding band allowed
  its bounded effect on the output.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import bit_activation_linear_amd as bl
from bit_activation_linear_amd import workloads
from parity_util import assert_y_close, assert_y_in_band

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev_x(x_np, x_dtype):
    if x_dtype == "bf16":
        return torch.from_numpy(x_np.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(x_np).to(DEV)


@pytest.mark.parametrize("N,K", [(16, 64), (37, 384), (5, 448), (64, 2560), (3, 4608), (2, 8192),
                                 (130, 1152), (7, 320)])
def test_pack_tl2_matches_oracle(N, K):
    _say(f"pack_tl2 N={N} K={K}")
    rng = np.random.default_rng(N * 7 + K)
    t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    t[0, : min(K, 90)] = 0                        # an all-zero stretch (index 0, sign 0)
    Wp = bl.pack_2bit(torch.from_numpy(t).to(DEV))
    Wt = bl.pack_tl2(Wp)
    torch.cuda.synchronize()
    assert Wt.numel() == bl.tl2_bytes(N, K) == oracle.tl2.packed_bytes(N, K)
    np.testing.assert_array_equal(Wt.cpu().numpy().reshape(N, -1), oracle.tl2.pack(t))


@pytest.mark.parametrize("K,N,bits,xdt", [
    (64, 16, 8, "bf16"),       # one partial block of one group, one super-block
    (320, 24, 8, "fp32"),      # a partial block of four groups
    (384, 50, 8, "fp32"),      # one whole block, ragged N
    (640, 33, 4, "bf16"),
    (2560, 200, 8, "bf16"),    # the headline's K: 7 blocks, the 8th padding
    (2560, 77, 4, "fp32"),
    (4096, 64, 8, "fp32"),
    (4608, 48, 4, "bf16"),     # the largest K: six whole super-blocks
])
def test_forward_tl2(K, N, bits, xdt):
    _say(f"forward_tl2 K={K} N={N} bits={bits} x={xdt}")
    case = workloads.make_case(1, K, N, x_dtype=xdt, n_out=max(1, K // 100), factor=30.0,
                               seed=K + N + bits)
    x = _dev_x(case["x"], xdt)
    W = torch.from_numpy(case["W"]).to(DEV)
    Wp, alpha = bl.ternarize_weights(W)
    Wt = bl.pack_tl2(Wp)
    y_tl2 = bl.hbitlinear_forward_tl2(x, Wt, alpha, bits)
    y_2b = bl.hbitlinear_forward(x, Wp, alpha, bits, 0)
    torch.cuda.synchronize()
    t_ref, a_ref, _ = oracle.ternarize(case["W"])
    ref = oracle.forward(case["x"], xdt, t_ref, a_ref, bits, 0)
    # the TL2 kernel's codes are not visible: compared with the oracle, each
    # code in the rounding band allowed its bounded effect on y
    assert_y_in_band(y_tl2.cpu().numpy(), t_ref, ref["q"], ref["p"], t_ref, ref["s"], a_ref, bits,
                     ref["y64"])
    if bits == 8:
        np.testing.assert_array_equal(y_tl2.cpu().numpy(), y_2b.cpu().numpy())


def test_forward_tl2_headline_full_size():
    wl = workloads.WORKLOADS["decode_int8_m1_k2560_n6912"]
    case = workloads.make_workload("decode_int8_m1_k2560_n6912", seed=0)
    x = _dev_x(case["x"], wl.x_dtype)
    W = torch.from_numpy(case["W"]).to(DEV)
    Wp, alpha = bl.ternarize_weights(W)
    Wt = bl.pack_tl2(Wp)
    y_tl2 = bl.hbitlinear_forward_tl2(x, Wt, alpha, wl.bits)
    y_2b = bl.hbitlinear_forward(x, Wp, alpha, wl.bits, 0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y_tl2.cpu().numpy(), y_2b.cpu().numpy())
    t_ref, a_ref, _ = oracle.ternarize(case["W"])
    ref = oracle.forward(case["x"], wl.x_dtype, t_ref, a_ref, wl.bits, 0)
    assert_y_close(y_tl2.cpu().numpy(), ref["y64"], what="TL2 headline vs oracle")
    # 1.67 bits per weight, the last block holding the three groups it reaches
    assert Wt.numel() == 6912 * (6 * 80 + 64)


@pytest.mark.parametrize("M,K,N,bits,xdt", [
    (2, 256, 40, 8, "bf16"),       # two tokens, one partial block (three groups)
    (5, 448, 40, 8, "bf16"),       # a last block of one group
    (4, 640, 33, 4, "fp32"),       # a partial second block, ragged N
    (1, 8192, 50, 8, "bf16"),      # one token past the single-token kernel's K
    (7, 4608, 100, 8, "fp32"),
    (16, 16384, 64, 4, "bf16"),    # the batched decode's K: 43 blocks, the last one partial
    (13, 32768, 30, 4, "bf16"),    # the longest row
])
def test_forward_tl2_batched(M, K, N, bits, xdt):
    """The batched TL2 forward (edge page, TL2KernelEdge.compute_gemv on x [B, K]):
    its codes are the public quantizer's, stored in the product's order, so
    its output equals the 2-bit product of those codes bit for bit, and the
    oracle's at the forward's tolerance."""
    _say(f"forward_tl2 batched M={M} K={K} N={N} bits={bits} x={xdt}")
    case = workloads.make_case(M, K, N, x_dtype=xdt, n_out=max(1, K // 100), factor=30.0,
                               seed=M + K + N + bits)
    x = _dev_x(case["x"], xdt)
    W = torch.from_numpy(case["W"]).to(DEV)
    Wp, alpha = bl.ternarize_weights(W)
    Wt = bl.pack_tl2(Wp)
    y_tl2 = bl.hbitlinear_forward_tl2(x, Wt, alpha, bits)
    rowsum = torch.empty((M,), dtype=torch.int32, device=DEV)
    codes, scales = bl.quantize_activations(x, bits, 0, rowsum=rowsum)
    y_2b = bl.ternary_linear_dequant(codes, scales, Wp, alpha, bits, rowsum=rowsum)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y_tl2.cpu().numpy(), y_2b.cpu().numpy())
    t_ref, a_ref, _ = oracle.ternarize(case["W"])
    ref = oracle.forward(case["x"], xdt, t_ref, a_ref, bits, 0)
    assert_y_in_band(y_tl2.cpu().numpy(), t_ref, ref["q"], ref["p"], t_ref, ref["s"], a_ref, bits,
                     ref["y64"])


def test_forward_tl2_batched_decode_full_size():
    """The batched-decode shape (M=16, K=16384, N=4096) on TL2 weights, int4,
    without the transform: 1.672 bits per weight (42 blocks of 80 bytes and a
    last block of three groups)."""
    M, K, N = 16, 16384, 4096
    case = workloads.make_case(M, K, N, x_dtype="bf16", dist="student_t3", n_out=100, factor=30.0,
                               seed=11)
    x = _dev_x(case["x"], "bf16")
    W = torch.from_numpy(case["W"]).to(DEV)
    Wp, alpha = bl.ternarize_weights(W)
    Wt = bl.pack_tl2(Wp)
    assert Wt.numel() == N * (42 * 80 + 64)
    y_tl2 = bl.hbitlinear_forward_tl2(x, Wt, alpha, 4)
    rowsum = torch.empty((M,), dtype=torch.int32, device=DEV)
    codes, scales = bl.quantize_activations(x, 4, 0, rowsum=rowsum)
    y_2b = bl.ternary_linear_dequant(codes, scales, Wp, alpha, 4, rowsum=rowsum)
    torch.cuda.synchronize()
    del W
    np.testing.assert_array_equal(y_tl2.cpu().numpy(), y_2b.cpu().numpy())
    t_ref, a_ref, _ = oracle.ternarize(case["W"])
    ref = oracle.forward(case["x"], "bf16", t_ref, a_ref, 4, 0)
    assert_y_in_band(y_tl2.cpu().numpy(), t_ref, ref["q"], ref["p"], t_ref, ref["s"], a_ref, 4,
                     ref["y64"])


def test_forward_tl2_limits():
    x = torch.zeros((17, 256), dtype=torch.bfloat16, device=DEV)
    Wt = torch.zeros((16, bl.tl2_bytes(16, 256) // 16), dtype=torch.uint8, device=DEV)
    alpha = torch.ones((1,), dtype=torch.float32, device=DEV)
    with pytest.raises(bl.BitNetError):
        bl.hbitlinear_forward_tl2(x, Wt, alpha, 8)                      # 17 tokens
    y = bl.hbitlinear_forward_tl2(torch.zeros((0, 256), dtype=torch.bfloat16, device=DEV), Wt,
                                  alpha, 8)
    assert y.shape == (0, 16)
