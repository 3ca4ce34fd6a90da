"""Parity of the H-BitLinear backward (through the C ABI) with the CPU oracle.

Engine page: Eq. 8 (the transform's gradient is the transform of the
gradient) and the STE backward of the quantizers. Both sides take the same
inputs: dy, and the oracle's own codes, scales, ternary weights and alpha
(the scales and alpha rounded to the fp32 the library stores). Tolerance:
relative Frobenius error 1e-4 on dx and dw. The arithmetic behind it: every
MFMA product is exact (bf16 dy or its hi/lo parts times t or q), the sums
are fp32 (relative error ~1e-7 per term), and the hi/lo split of
dy * s / c leaves a relative residual below 2^-17 per element; dropping the
lo part (2^-9) or any term would exceed the bound.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import bit_activation_linear_amd as bl
from bit_activation_linear_amd import workloads
from parity_util import rel_frobenius

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
GRAD_TOL = 1e-4


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(M, K, N, bits, had, dy_dtype, seed, dy_scale=1e-3):
    case = workloads.make_case(M, K, N, x_dtype="bf16", n_out=max(1, K // 100), factor=20.0,
                               seed=seed)
    t, alpha, _ = oracle.ternarize(case["W"])
    x64 = oracle.widen_input(case["x"], "bf16")
    q, s, _ = oracle.quantize_activations(oracle.fwht(x64) if had else x64, bits)
    s32 = s.astype(np.float32)
    a32 = np.float32(alpha)
    rng = np.random.default_rng(seed + 77)
    dy32 = (rng.standard_normal((M, N)) * dy_scale).astype(np.float32)
    if dy_dtype == "bf16":
        dy_bits = workloads.fp32_to_bf16_bits(dy32)
        dy64 = workloads.bf16_bits_to_fp32(dy_bits).astype(np.float64)
        dy_dev = torch.from_numpy(dy_bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        dy64 = dy32.astype(np.float64)
        dy_dev = torch.from_numpy(dy32).to(DEV)
    dev = dict(dy=dy_dev, codes=torch.from_numpy(q).to(DEV), scales=torch.from_numpy(s32).to(DEV),
               Wp=torch.from_numpy(oracle.pack_2bit(t)).to(DEV),
               alpha=torch.tensor([a32], device=DEV))
    ref = dict(dy=dy64, q=q, s=s32.astype(np.float64), t=t, alpha=float(a32))
    return dev, ref


def _gpu_backward(dev, bits, had, want_dx=True, want_dw=True):
    return bl.hbitlinear_backward(dev["dy"], dev["codes"], dev["scales"], dev["Wp"], dev["alpha"],
                                  bits, had, want_dx=want_dx, want_dw=want_dw)


@pytest.mark.parametrize("M,K,N,bits,had,dyt", [
    (1, 64, 64, 8, 0, "bf16"),         # one token, one tile
    (3, 128, 64, 4, 1, "fp32"),        # fp32 gradient: two bf16 parts
    (100, 256, 192, 8, 1, "bf16"),     # ragged rows in both products
    (300, 512, 320, 4, 1, "fp32"),     # several tiles in every direction, ragged
    (257, 1024, 576, 8, 0, "bf16"),
    (64, 2048, 256, 4, 1, "bf16"),
    (600, 320, 704, 8, 0, "fp32"),     # K not a power of two (no transform)
    (520, 4096, 128, 4, 1, "bf16"),    # long rows through the transform
])
def test_backward_parity(M, K, N, bits, had, dyt):
    _say(f"backward case M={M} K={K} N={N} bits={bits} hadamard={had} dy={dyt}")
    dev, ref = _inputs(M, K, N, bits, had, dyt, seed=M + K + N + bits)
    dx, dw = _gpu_backward(dev, bits, had)
    torch.cuda.synchronize()
    dx_ref, dw_ref = oracle.backward(ref["dy"], ref["q"], ref["s"], ref["t"], ref["alpha"], bits, had)
    ex = rel_frobenius(dx.cpu().numpy(), dx_ref)
    ew = rel_frobenius(dw.cpu().numpy(), dw_ref)
    _say(f"  rel-Frobenius dx {ex:.2e} dw {ew:.2e}")
    assert ex <= GRAD_TOL and ew <= GRAD_TOL


@pytest.mark.parametrize("key", ["prefill_int4_hadamard_m2048_k8192_n2048",
                                 "prefill_int8_m8192_k4096_n14336"])
def test_backward_full_size_sampled(key):
    """The two prefill workloads at full size (the shapes the bench times),
    checked on sampled rows of dx and of dw."""
    wl = workloads.WORKLOADS[key]
    M, K, N, bits, had = wl.M, wl.K, wl.N, wl.bits, wl.hadamard
    _say(f"backward workload {key}")
    dev, ref = _inputs(M, K, N, bits, had, "bf16", seed=21)
    dx, dw = _gpu_backward(dev, bits, had)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 30, replace=False)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 30, replace=False)]))
    dx_ref, _ = oracle.backward(ref["dy"][rows], ref["q"][rows], ref["s"][rows], ref["t"],
                                ref["alpha"], bits, had)
    _, dw_ref = oracle.backward(ref["dy"][:, cols], ref["q"], ref["s"], ref["t"][cols],
                                ref["alpha"], bits, had)
    ex = rel_frobenius(dx.cpu().numpy()[rows], dx_ref)
    ew = rel_frobenius(dw.cpu().numpy()[cols], dw_ref)
    _say(f"  rel-Frobenius dx {ex:.2e} dw {ew:.2e}")
    assert ex <= GRAD_TOL and ew <= GRAD_TOL


def test_backward_single_gradients_match_both():
    dev, _ = _inputs(130, 512, 192, 4, 1, "bf16", seed=3)
    dx, dw = _gpu_backward(dev, 4, 1)
    dx1, none_w = _gpu_backward(dev, 4, 1, want_dw=False)
    none_x, dw1 = _gpu_backward(dev, 4, 1, want_dx=False)
    torch.cuda.synchronize()
    assert none_w is None and none_x is None
    assert torch.equal(dx, dx1) and torch.equal(dw, dw1)


def test_backward_deterministic():
    dev, _ = _inputs(200, 1024, 320, 8, 0, "fp32", seed=4)
    a = _gpu_backward(dev, 8, 0)
    b = _gpu_backward(dev, 8, 0)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_backward_degenerate_sizes():
    # no tokens: dw = dy^T x_q is a sum over nothing, exactly zero
    dev, _ = _inputs(4, 256, 128, 8, 1, "bf16", seed=6)
    empty = {k: (v[:0].contiguous() if k in ("dy", "codes", "scales") else v) for k, v in dev.items()}
    dx, dw = _gpu_backward(empty, 8, 1)
    torch.cuda.synchronize()
    assert dx.shape == (0, 256) and dw.shape == (128, 256)
    assert torch.count_nonzero(dw).item() == 0
    # a zero gradient gives zero gradients
    zero = dict(dev)
    zero["dy"] = torch.zeros_like(dev["dy"])
    dx, dw = _gpu_backward(zero, 8, 1)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dx).item() == 0 and torch.count_nonzero(dw).item() == 0
