"""Pins of the oracle's H-BitLinear backward — CPU only.

Engine page: Eq. 8 (HadamardTransformFunction.backward applies the transform
to the gradient) and the straight-through estimators of the weight and
activation quantizers (their backward passes return the incoming gradient).
Each pin reaches the gradients by a route other than the oracle's formula:
torch autograd through the STE forward, the adjoint identity of the
linearised layer, H * H = I, a hand-worked case and brute-force loops.
"""

import math

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle


def _case(M, K, N, bits, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    t, alpha, _ = oracle.ternarize(W)
    dy = rng.standard_normal((M, N))
    return x, W, t, alpha, dy


class _Ste(torch.autograd.Function):
    """Forward returns the quantized value, backward the gradient unchanged
    (the engine page's STE autograd functions)."""

    @staticmethod
    def forward(ctx, x, xq):
        return xq.clone()

    @staticmethod
    def backward(ctx, g):
        return g.clone(), None


@pytest.mark.parametrize("bits,hadamard", [(8, 0), (8, 1), (4, 1), (4, 0)])
def test_backward_matches_torch_autograd(bits, hadamard):
    M, K, N = 6, 32, 24
    x, W, t, alpha, dy = _case(M, K, N, bits, seed=10 + bits + hadamard)
    xr = oracle.fwht(x) if hadamard else x
    q, s, _ = oracle.quantize_activations(xr, bits)
    c = oracle.INT8_SCALE if bits == 8 else oracle.INT4_SCALE

    # torch fp64 autograd: dense normalized Hadamard matmul (scipy's matrix),
    # STE on activations and weights, then F.linear.
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W.astype(np.float64), requires_grad=True)
    if hadamard:
        Hm = torch.tensor(scipy.linalg.hadamard(K) / math.sqrt(K), dtype=torch.float64)
        xr_t = xt @ Hm.T
    else:
        xr_t = xt
    xq_val = torch.tensor(q.astype(np.float64) * (s[:, None] / c))
    wq_val = torch.tensor(alpha * t.astype(np.float64))
    y = torch.nn.functional.linear(_Ste.apply(xr_t, xq_val), _Ste.apply(Wt, wq_val))
    y.backward(torch.tensor(dy))

    dx, dw = oracle.backward(dy, q, s, t, alpha, bits, hadamard)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw, Wt.grad.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("hadamard", [0, 1])
def test_backward_is_the_adjoint_of_the_linearised_layer(hadamard):
    """Under the STE the layer is linear in x (x -> H x . w_q^T) and in the
    weights (w -> x_q . w^T); the gradients are the adjoints:
    <dy, L(v)> = <dx, v> for every v."""
    M, K, N = 5, 64, 40
    x, W, t, alpha, dy = _case(M, K, N, 8, seed=3 + hadamard)
    xr = oracle.fwht(x) if hadamard else x
    q, s, _ = oracle.quantize_activations(xr, 8)
    dx, dw = oracle.backward(dy, q, s, t, alpha, 8, hadamard)
    rng = np.random.default_rng(99)
    v = rng.standard_normal((M, K))
    Lv = (oracle.fwht(v) if hadamard else v) @ (alpha * t.astype(np.float64)).T
    assert abs(np.sum(dy * Lv) - np.sum(dx * v)) <= 1e-10 * np.sum(np.abs(dy * Lv))
    V = rng.standard_normal((N, K))
    xq = q.astype(np.float64) * (s[:, None] / 127.0)
    LV = xq @ V.T
    assert abs(np.sum(dy * LV) - np.sum(dw * V)) <= 1e-10 * np.sum(np.abs(dy * LV))


def test_eq8_transform_of_the_gradient():
    """dx with the transform is H applied to dx without it, and H undoes
    itself (H * H = I)."""
    x, W, t, alpha, dy = _case(4, 128, 16, 4, seed=5)
    q, s, _ = oracle.quantize_activations(oracle.fwht(x), 4)
    dx_h, dw_h = oracle.backward(dy, q, s, t, alpha, 4, 1)
    dx_0, dw_0 = oracle.backward(dy, q, s, t, alpha, 4, 0)
    np.testing.assert_allclose(dx_h, oracle.fwht(dx_0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.fwht(dx_h), dx_0, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(dw_h, dw_0)  # the weight gradient does not see H


def test_hand_worked_case():
    # M = N = 1, K = 2, t = [1, -1], alpha = 0.5, dy = [[2]], codes q = [127, -64]
    # with s = 3 (int8, c = 127): x_q = [3, -64 * 3 / 127].
    # dL/dx_r = alpha * dy * t = [1, -1]; with H_2 = [[1, 1], [1, -1]] / sqrt2:
    # dx = [0, 2 / sqrt2] = [0, sqrt2]; without the transform dx = [1, -1].
    # dw = dy^T x_q = [6, -384 / 127].
    t = np.array([[1, -1]], dtype=np.int8)
    q = np.array([[127, -64]], dtype=np.int8)
    s = np.array([3.0])
    dy = np.array([[2.0]])
    dx, dw = oracle.backward(dy, q, s, t, 0.5, 8, 1)
    np.testing.assert_allclose(dx, [[0.0, math.sqrt(2.0)]], atol=1e-15)
    np.testing.assert_allclose(dw, [[6.0, -384.0 / 127.0]], rtol=1e-15)
    dx0, _ = oracle.backward(dy, q, s, t, 0.5, 8, 0)
    np.testing.assert_allclose(dx0, [[1.0, -1.0]], rtol=1e-15)


def test_brute_force_loops():
    M, K, N = 3, 8, 5
    x, W, t, alpha, dy = _case(M, K, N, 4, seed=8)
    q, s, _ = oracle.quantize_activations(x, 4)
    dx, dw = oracle.backward(dy, q, s, t, alpha, 4, 0)
    c = math.sqrt(7.0)
    for m in range(M):
        for k in range(K):
            ref = sum(float(dy[m, n]) * alpha * int(t[n, k]) for n in range(N))
            assert abs(dx[m, k] - ref) <= 1e-12
    for n in range(N):
        for k in range(K):
            ref = sum(float(dy[m, n]) * int(q[m, k]) * float(s[m]) / c for m in range(M))
            assert abs(dw[n, k] - ref) <= 1e-12
