"""Pins of the oracle's input prologue (RMSNorm, SwiGLU product) — CPU only.

Engine page: HBitLinear.forward step 1 (nn.RMSNorm(in_features, eps)) and
BitNetV2FFN.forward (F.silu(gate) * up feeding the H-BitLinear down projection).
Each test ties the oracle to something other than its own formula: hand-derived
values, exact identities, or torch's independent implementations.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from bit_activation_linear_amd import workloads


def test_silu_hand_values_and_identity():
    # silu(0) = 0; silu(1) = 1 / (1 + 1/e); silu(-1) = -1 / (1 + e)
    e = math.e
    np.testing.assert_allclose(oracle.silu([0.0, 1.0, -1.0]), [0.0, 1.0 / (1.0 + 1.0 / e), -1.0 / (1.0 + e)],
                               rtol=1e-15, atol=0)
    # x*sig(x) - (-x)*sig(-x) = x (sig(x) + sig(-x) = 1)
    x = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=1e-13, atol=1e-13)
    # large arguments: silu(x) -> x, silu(-x) -> 0
    np.testing.assert_allclose(oracle.silu([40.0]), [40.0], rtol=1e-15)
    assert abs(oracle.silu([-40.0])[0]) < 1e-15


def test_silu_matches_torch():
    rng = np.random.default_rng(3)
    g = rng.standard_normal(4096) * 4
    ref = torch.nn.functional.silu(torch.from_numpy(g)).numpy()
    np.testing.assert_allclose(oracle.silu(g), ref, rtol=1e-14, atol=1e-15)


def test_swiglu_is_product():
    g = np.array([0.0, 1.0, -2.0, 3.5])
    u = np.array([5.0, -2.0, 4.0, 0.0])
    np.testing.assert_allclose(oracle.swiglu(g, u), oracle.silu(g) * u, rtol=0, atol=0)
    assert oracle.swiglu(g, u)[0] == 0.0 and oracle.swiglu(g, u)[3] == 0.0


def test_rmsnorm_hand_values():
    # [3, 4]: mean square 12.5, rms = sqrt(12.5 + eps)
    r = math.sqrt(12.5 + 1e-7)
    np.testing.assert_allclose(oracle.rmsnorm(np.array([[3.0, 4.0]])), [[3.0 / r, 4.0 / r]], rtol=1e-15)
    # constant row c: every element becomes c / sqrt(c^2 + eps)
    np.testing.assert_allclose(oracle.rmsnorm(np.full((1, 8), -2.0)), np.full((1, 8), -2.0 / math.sqrt(4.0 + 1e-7)),
                               rtol=1e-15)
    # zero row stays zero
    assert np.all(oracle.rmsnorm(np.zeros((2, 16))) == 0.0)


@pytest.mark.parametrize("K", [64, 1000, 4096])
def test_rmsnorm_matches_torch(K):
    rng = np.random.default_rng(K)
    u = rng.standard_normal((5, K)) * 3
    w = rng.standard_normal(K)
    m = torch.nn.RMSNorm(K, eps=1e-7, dtype=torch.float64)
    with torch.no_grad():
        m.weight.copy_(torch.from_numpy(w))
        ref = m(torch.from_numpy(u)).numpy()
    np.testing.assert_allclose(oracle.rmsnorm(u, w, 1e-7), ref, rtol=1e-13, atol=1e-14)


def test_rmsnorm_properties():
    rng = np.random.default_rng(7)
    u = rng.standard_normal((4, 2048)) * 50
    out = oracle.rmsnorm(u)
    np.testing.assert_allclose(np.mean(out * out, axis=-1), 1.0, rtol=1e-9)
    np.testing.assert_allclose(oracle.rmsnorm(u * 123.0), out, rtol=1e-9)


def test_prologue_reduces_to_forward():
    case = workloads.make_case(3, 256, 64, x_dtype="bf16", n_out=4, factor=50.0, seed=11)
    t, alpha, _ = oracle.ternarize(case["W"])
    for bits, had in [(8, 0), (4, 1)]:
        a = oracle.forward(case["x"], "bf16", t, alpha, bits, had)
        b = oracle.forward_prologue(case["x"], "bf16", t, alpha, bits, had)
        np.testing.assert_array_equal(a["q"], b["q"])
        np.testing.assert_array_equal(a["y64"], b["y64"])


def test_prologue_matches_torch_module_chain():
    """silu(gate) * up -> nn.RMSNorm -> the engine page's fake-quant route
    (F.linear of the dequantized codes and alpha * t), all in torch fp64."""
    rng = np.random.default_rng(5)
    M, K, N = 3, 128, 40
    gate = rng.standard_normal((M, K)).astype(np.float32) * 2
    up = rng.standard_normal((M, K)).astype(np.float32)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    gamma = rng.standard_normal(K) * 0.5 + 1.0
    t, alpha, _ = oracle.ternarize(W)
    for bits, had in [(8, 0), (4, 1), (8, 1)]:
        r = oracle.forward_prologue(gate, "fp32", t, alpha, bits, had, up=up, rms=True, norm_weight=gamma)
        g64 = torch.from_numpy(gate.astype(np.float64))
        u64 = torch.from_numpy(up.astype(np.float64))
        inter = torch.nn.functional.silu(g64) * u64
        norm = torch.nn.RMSNorm(K, eps=1e-7, dtype=torch.float64)
        with torch.no_grad():
            norm.weight.copy_(torch.from_numpy(gamma))
            xn = norm(inter)
        xn_np = xn.detach().numpy()
        xr = oracle.fwht_dense(xn_np) if had else xn_np
        # fake-quant route: per-token absmax/absmean, round, clip, rescale
        if bits == 8:
            s = np.max(np.abs(xr), axis=-1, keepdims=True) + 1e-7
            xq = np.clip(np.rint(127.0 * xr / s), -128, 127) * s / 127.0
        else:
            s = np.mean(np.abs(xr), axis=-1, keepdims=True) + 1e-7
            xq = np.clip(np.rint(math.sqrt(7.0) * xr / s), -8, 7) * s / math.sqrt(7.0)
        y_ref = torch.nn.functional.linear(torch.from_numpy(xq), torch.from_numpy(t * alpha)).numpy()
        np.testing.assert_allclose(r["y64"], y_ref, rtol=1e-10, atol=1e-12)


def test_rmsnorm_leaves_codes_scale_invariant():
    """Per-token quantization is invariant to a positive row scale (up to
    eps), so RMSNorm with unit weight changes the scales, not the codes."""
    case = workloads.make_case(4, 512, 8, x_dtype="fp32", n_out=4, factor=50.0, seed=2)
    t, alpha, _ = oracle.ternarize(case["W"])
    a = oracle.forward(case["x"], "fp32", t, alpha, 8, 1)
    b = oracle.forward_prologue(case["x"], "fp32", t, alpha, 8, 1, rms=True)
    far = oracle.quant_boundary_distance(a["p"]) > 1e-4
    np.testing.assert_array_equal(a["q"][far], b["q"][far])
    x64 = oracle.widen_input(case["x"], "fp32")
    rms = np.sqrt(np.mean(x64 * x64, axis=-1) + 1e-7)
    np.testing.assert_allclose(b["s"], (a["s"] - 1e-7) / rms + 1e-7, rtol=1e-12)
