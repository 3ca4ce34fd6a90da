"""Parity of the low-bit KV-cache quantizer on MI355X with the CPU oracle.

Engine page: module docstring item 5 (Section 3.1) and
BitNetV2Attention._quantize_kv_head. Codes bit-exact up to +-1 flips inside
the 1e-4 rounding band; scales to fp32 rounding of the statistic.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import bit_activation_linear_amd as bl
from bit_activation_linear_amd import workloads
from parity_util import assert_codes_match

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _kv(B, H, S, D, x_dtype, seed):
    case = workloads.make_case(B * H * S, D, 1, x_dtype=x_dtype, n_out=max(1, D // 32), factor=8.0,
                               seed=seed)
    x = case["x"]
    if x_dtype == "bf16":
        dev = torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        dev = torch.from_numpy(x).to(DEV)
    return x, dev.view(B, H, S, D)


@pytest.mark.parametrize("B,H,S,D,xdt", [
    (1, 2, 5, 64, "bf16"),
    (2, 8, 33, 128, "bf16"),
    (1, 4, 7, 96, "fp32"),      # G = 16 lanes per token, 12 of them loaded
    (1, 1, 1, 8, "fp32"),       # a single BOS token of 8 elements
    (3, 2, 4, 512, "bf16"),     # the largest head dimension
    (1, 32, 1024, 128, "bf16"),  # a 1024-token cache of 32 heads
])
@pytest.mark.parametrize("bits", [3, 4, 8])
def test_kv_quantize_parity(B, H, S, D, xdt, bits):
    print(f"kv case B={B} H={H} S={S} D={D} x={xdt} bits={bits}", flush=True)
    sys.stdout.flush()
    x_np, kv = _kv(B, H, S, D, xdt, seed=B * 1000 + H * 100 + S + D + bits)
    codes, scales = bl.kv_quantize(kv, bits)
    torch.cuda.synchronize()
    ref_in = oracle.widen_input(x_np, xdt).reshape(B, H, S, D)
    q, s, p = oracle.kv_quantize(ref_in, bits)
    assert_codes_match(codes.cpu().numpy(), q, p)
    np.testing.assert_allclose(scales.cpu().numpy(), s, rtol=2e-6)
    c = codes.cpu().numpy()
    assert c[..., 0, :].min() >= -128
    if S > 1:
        lo, hi = {3: (-4, 3), 4: (-8, 7), 8: (-128, 127)}[bits]
        assert c[..., 1:, :].min() >= lo and c[..., 1:, :].max() <= hi


@pytest.mark.parametrize("B,H,S,D,xdt,bits", [
    (1, 32, 4096, 128, "bf16", 3),   # the timed cache
    (1, 33, 4001, 128, "bf16", 4),   # a ragged last workgroup
    (2, 32, 4099, 64, "bf16", 8),
    (1, 128, 4097, 32, "fp32", 3),
])
def test_kv_quantize_parity_large(B, H, S, D, xdt, bits):
    print(f"kv large case B={B} H={H} S={S} D={D} x={xdt} bits={bits}", flush=True)
    x_np, kv = _kv(B, H, S, D, xdt, seed=7 + S + D + bits)
    codes, scales = bl.kv_quantize(kv, bits)
    torch.cuda.synchronize()
    ref_in = oracle.widen_input(x_np, xdt).reshape(B, H, S, D)
    q, s, p = oracle.kv_quantize(ref_in, bits)
    assert_codes_match(codes.cpu().numpy(), q, p)
    np.testing.assert_allclose(scales.cpu().numpy(), s, rtol=2e-6)


@pytest.mark.parametrize("B,H,S,D,xdt,bits", [
    (1, 2, 5, 64, "bf16", 4),
    (1, 2, 5, 64, "bf16", 3),
    (2, 8, 33, 128, "bf16", 3),
    (1, 4, 7, 96, "fp32", 3),     # G = 16 lanes, three groups of four store
    (1, 4, 7, 40, "fp32", 4),     # five lanes of a row
    (1, 1, 1, 32, "bf16", 3),     # only a BOS token: its packed row is zero
    (3, 2, 4, 512, "bf16", 4),
    (1, 32, 4096, 128, "bf16", 3),  # the timed cache
    (1, 33, 4001, 128, "bf16", 4),  # a ragged last workgroup
])
def test_kv_quantize_packed_parity(B, H, S, D, xdt, bits):
    """Packed storage: the bytes are the oracle's packing of the unpacked
    entry point's codes (same kernel arithmetic), those codes match the
    oracle's, and the BOS codes and scales are the unpacked call's."""
    print(f"kv packed case B={B} H={H} S={S} D={D} x={xdt} bits={bits}", flush=True)
    x_np, kv = _kv(B, H, S, D, xdt, seed=11 + B + H + S + D + bits)
    packed, bos, scales = bl.kv_quantize_packed(kv, bits)
    codes, scales_u = bl.kv_quantize(kv, bits)
    torch.cuda.synchronize()
    c = codes.cpu().numpy()
    ref_in = oracle.widen_input(x_np, xdt).reshape(B, H, S, D)
    q, s, p = oracle.kv_quantize(ref_in, bits)
    assert_codes_match(c, q, p)
    np.testing.assert_array_equal(scales.cpu().numpy(), scales_u.cpu().numpy())
    np.testing.assert_array_equal(bos.cpu().numpy(), c[:, :, 0, :])
    rest = c.copy()
    rest[:, :, 0, :] = 0  # BOS rows are zero in the packed array
    want = oracle.kv_pack(rest.reshape(-1, D), bits).reshape(B, H, S, D * bits // 8)
    np.testing.assert_array_equal(packed.cpu().numpy(), want)
    assert packed.numel() * 8 == B * H * S * D * bits
