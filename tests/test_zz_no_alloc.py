"""The forward entry point that allocates nothing
(bitnet_hbitlinear_forward_noalloc), through the C ABI on MI355X.

Its workspace is the library's fixed device array, shared by every call on a
GPU and holding the last call's contents: each call must still give exactly
the output of bitnet_hbitlinear_forward (same kernels, caller's workspace),
bit for bit, including a smaller call right after a larger one, and the
first call's output must meet the oracle at the forward's tolerance.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import bit_activation_linear_amd as bl
from bit_activation_linear_amd import _lib, workloads
from parity_util import assert_y_with_flips, decode_packed

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(M, K, N, x_dtype, seed):
    case = workloads.make_case(M, K, N, x_dtype=x_dtype, n_out=max(1, K // 100), factor=30.0,
                               seed=seed)
    if x_dtype == "bf16":
        x = torch.from_numpy(case["x"].view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        x = torch.from_numpy(case["x"]).to(DEV)
    Wp, alpha = bl.ternarize_weights(torch.from_numpy(case["W"]).to(DEV))
    return case, x, Wp, alpha


@pytest.mark.parametrize("big,small", [
    # (M, K, N, bits, hadamard, x dtype): the prefill path, then a smaller prefill
    ((300, 4096, 260, 4, 1, "bf16"), (40, 1024, 70, 4, 1, "bf16")),
    # batched decode with nibble codes, then a smaller two-launch decode
    ((16, 16384, 200, 4, 1, "bf16"), (3, 2048, 90, 8, 1, "fp32")),
    # int8 prefill without the transform, then a fused single-kernel decode
    ((129, 2560, 300, 8, 0, "bf16"), (1, 2560, 120, 8, 0, "bf16")),
])
def test_noalloc_matches_forward_on_consecutive_calls(big, small):
    outs = []
    for i, (M, K, N, bits, had, xdt) in enumerate((big, small)):
        _say(f"noalloc call {i}: M={M} K={K} N={N} bits={bits} hadamard={had} x={xdt}")
        case, x, Wp, alpha = _case(M, K, N, xdt, seed=M + K + N)
        y_ref = bl.hbitlinear_forward(x, Wp, alpha, bits, had)
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        bl.hbitlinear_forward_noalloc(x, Wp, alpha, bits, had, out=y)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy(), y_ref.cpu().numpy())
        outs.append((case, y.cpu().numpy(), Wp.cpu().numpy(), bits, had, xdt))
    # the first call against the oracle as well
    case, y, wp, bits, had, xdt = outs[0]
    t_ref, a_ref, _ = oracle.ternarize(case["W"])
    ref = oracle.forward(case["x"], xdt, t_ref, a_ref, bits, had)
    x = torch.from_numpy(case["x"].view(np.int16) if xdt == "bf16" else case["x"]).to(DEV)
    if xdt == "bf16":
        x = x.view(torch.bfloat16)
    codes, _ = bl.quantize_activations(x, bits, had)
    torch.cuda.synchronize()
    assert_y_with_flips(y, codes.cpu().numpy(), decode_packed(wp), ref["q"], t_ref, ref["s"],
                        a_ref, bits, ref["y64"])


def test_noalloc_rejects_a_batch_beyond_the_scratch():
    _say("noalloc: beyond the scratch")
    M, K, N = 8192, 16384, 64
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    Wp = torch.full((N, K // 4), 0x55, dtype=torch.uint8, device=DEV)
    alpha = torch.ones((1,), dtype=torch.float32, device=DEV)
    y = torch.zeros((M, N), dtype=torch.float32, device=DEV)
    assert bl.forward_workspace_bytes(M, K, N, 8, 0) > _lib.NOALLOC_SCRATCH_BYTES
    with pytest.raises(bl.BitNetError) as ei:
        bl.hbitlinear_forward_noalloc(x, Wp, alpha, 8, 0, out=y)
    assert ei.value.status == _lib.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0
