"""Parity of the HIP path (through the C ABI) with the CPU oracle on MI355X.

Small cases span several tiles with ragged M, N and K tails and both kernel
shapes (M <= 16 streams the weights, M > 16 runs the prefill tile); the five
measured workloads run at full size in the launch configuration the bench
times, compared in full where the oracle is quick and on sampled rows
otherwise.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import bit_activation_linear_amd as bl
from bit_activation_linear_amd import workloads
from parity_util import (EPILOGUE_TOL, assert_codes_match, assert_packed_match, assert_y_close,
                         assert_y_in_band, assert_y_with_flips, decode_packed)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _to_dev_x(x_np, x_dtype):
    if x_dtype == "bf16":
        return torch.from_numpy(x_np.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(x_np).to(DEV)


def _run_case(M, K, N, bits, had, x_dtype, seed, dist="normal", n_out=0, factor=1.0):
    _say(f"case M={M} K={K} N={N} bits={bits} hadamard={had} x={x_dtype} seed={seed}")
    case = workloads.make_case(M, K, N, x_dtype=x_dtype, dist=dist, n_out=n_out, factor=factor,
                               seed=seed)
    x = _to_dev_x(case["x"], x_dtype)
    W = torch.from_numpy(case["W"]).to(DEV)

    Wp, alpha = bl.ternarize_weights(W)
    rowsum = torch.empty((M,), dtype=torch.int32, device=DEV)
    codes, scales = bl.quantize_activations(x, bits, had, rowsum=rowsum)
    y = bl.hbitlinear_forward(x, Wp, alpha, bits, had)
    y2 = bl.ternary_linear_dequant(codes, scales, Wp, alpha, bits)
    y3 = bl.ternary_linear_dequant(codes, scales, Wp, alpha, bits, rowsum=rowsum)
    torch.cuda.synchronize()
    # the quantizer's code sums are exact, and the product given them is the
    # product that sums the codes itself, bit for bit
    np.testing.assert_array_equal(rowsum.cpu().numpy(), codes.cpu().numpy().astype(np.int64).sum(1))
    np.testing.assert_array_equal(y3.cpu().numpy(), y2.cpu().numpy())

    t_ref, a_ref, p_w = oracle.ternarize(case["W"])
    assert_packed_match(Wp.cpu().numpy(), t_ref, p_w)
    assert abs(alpha.item() - a_ref) <= 1e-6 * a_ref

    ref = oracle.forward(case["x"], x_dtype, t_ref, a_ref, bits, had)
    q_gpu = codes.cpu().numpy()
    assert_codes_match(q_gpu, ref["q"], ref["p"])
    np.testing.assert_allclose(scales.cpu().numpy(), ref["s"], rtol=2e-6)

    # The product stages on the oracle's own codes, weights, scales and alpha:
    # int32 accumulators bit-exact, the dequantized output to fp32 rounding.
    q_ref_d = torch.from_numpy(ref["q"]).to(DEV)
    Wp_ref = torch.from_numpy(oracle.pack_2bit(t_ref)).to(DEV)
    s32 = ref["s"].astype(np.float32)
    a32 = np.float32(a_ref)
    acc_ref_gpu = bl.ternary_gemm_i32(q_ref_d, Wp_ref)
    y_ep = bl.ternary_linear_dequant(q_ref_d, torch.from_numpy(s32).to(DEV), Wp_ref,
                                     torch.tensor([a32], device=DEV), bits)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc_ref_gpu.cpu().numpy(), ref["acc"])
    assert_y_close(y_ep.cpu().numpy(),
                   oracle.dequantize(ref["acc"], float(a32), s32.astype(np.float64), bits),
                   what="epilogue on the oracle's codes", tol=EPILOGUE_TOL)

    # End to end on the GPU's own codes and weights; a flip inside the
    # rounding band is allowed its bounded effect on y.
    assert_y_with_flips(y2.cpu().numpy(), q_gpu, decode_packed(Wp.cpu().numpy()), ref["q"], t_ref,
                        ref["s"], a_ref, bits, ref["y64"])
    # The forward is the two stages back to back, bit for bit, except where it
    # runs as one fused kernel with int4: the absmean is then summed in another
    # order, so an ulp of the scale can move a code that sits on a rounding
    # boundary. That forward is compared with the oracle directly, each code
    # in the rounding band allowed its bounded effect on y.
    fused = bl.forward_workspace_bytes(M, K, N, bits, had) == 0
    if fused and bits == 4:
        assert_y_in_band(y.cpu().numpy(), decode_packed(Wp.cpu().numpy()), ref["q"], ref["p"],
                         t_ref, ref["s"], a_ref, bits, ref["y64"])
    else:
        np.testing.assert_array_equal(y.cpu().numpy(), y2.cpu().numpy())


# M <= 16: weight-streaming shape ------------------------------------------
@pytest.mark.parametrize("M,K,N,bits,had,xdt", [
    (1, 64, 1, 8, 0, "bf16"),
    (1, 2560, 200, 8, 0, "bf16"),
    (3, 320, 47, 4, 0, "fp32"),
    (16, 1024, 130, 4, 1, "bf16"),
    (1, 64, 40, 8, 1, "bf16"),         # fused with the transform (K <= 256): one wave per token row
    (3, 128, 77, 4, 1, "fp32"),
    (16, 256, 100, 8, 1, "bf16"),
    (5, 256, 33, 4, 1, "bf16"),
    (7, 4096, 33, 8, 1, "fp32"),
    (12, 8192, 40, 4, 1, "bf16"),      # transform, 16 elements per thread for a few long rows
    (16, 16384, 130, 8, 1, "fp32"),    # transform, 32 elements per thread, int8 codes
    (3, 8192, 77, 8, 1, "bf16"),
    (1, 16384, 40, 4, 1, "bf16"),      # one long row with the transform, nibble codes
    (16, 8192, 16, 4, 1, "bf16"),      # a single column tile
    (5, 16384, 300, 4, 1, "fp32"),
    (16, 512, 70, 4, 1, "bf16"),       # nibble codes, shortest row they take with the transform
    (16, 4352, 50, 4, 0, "bf16"),      # nibble codes without the transform, 17 super-blocks
    (13, 1280, 33, 4, 0, "fp32"),      # nibble codes, fp32 input, ragged M
    (16, 16384, 64, 4, 1, "bf16"),
    (2, 192, 31, 8, 0, "bf16"),
    (5, 32768, 40, 8, 0, "fp32"),
    (1, 32768, 100, 8, 0, "bf16"),     # eight rounds of super-blocks per wave
    (2, 8192, 70, 4, 0, "bf16"),       # two rounds, not fused
    (4, 4096, 90, 4, 0, "bf16"),       # fused, int4
    (16, 1024, 48, 4, 0, "fp32"),      # fused, full 16 rows
    (16, 4096, 150, 8, 0, "bf16"),     # not fused (M*K too big), 4 column tiles
    (9, 2048, 33, 4, 1, "fp32"),
    (2, 2048, 100, 4, 0, "bf16"),      # multi-wave fused kernel, two rows
    (4, 1024, 70, 8, 0, "fp32"),       # multi-wave fused kernel, four rows
    (1, 4096, 50, 4, 0, "fp32"),       # one-wave kernel (single token), sixteen super-blocks
    (1, 1344, 77, 8, 0, "bf16"),       # one-wave kernel, 21 blocks: a partial last super-block
    (1, 2624, 90, 8, 0, "fp32"),       # one-wave kernel, fp32 input, one block in the last super-block
    (3, 1344, 40, 8, 0, "bf16"),       # multi-wave fused kernel, partial last super-block
    (4, 32768, 70, 4, 1, "bf16"),      # nibble codes by pairs of super-blocks, two rounds per wave
    (16, 24576, 33, 4, 0, "bf16"),     # pairs, three per wave: a second round half live
    (7, 9728, 45, 4, 0, "fp32"),       # pairs, 19 of them over 16 waves
])
def test_parity_decode_shapes(M, K, N, bits, had, xdt):
    _run_case(M, K, N, bits, had, xdt, seed=M * 7 + K + N, n_out=max(1, K // 100), factor=30.0)


# M > 16: prefill tile ------------------------------------------------------
@pytest.mark.parametrize("M,K,N,bits,had,xdt", [
    (17, 64, 33, 8, 0, "bf16"),
    (129, 192, 257, 4, 0, "bf16"),
    (300, 1024, 260, 8, 1, "bf16"),
    (256, 256, 256, 4, 1, "fp32"),
    (130, 2560, 129, 8, 0, "bf16"),
    (40, 32768, 16, 4, 1, "bf16"),
    (513, 4096, 384, 4, 1, "bf16"),
    (80, 2048, 96, 4, 1, "bf16"),      # transform with 16 elements per thread
    (70, 16384, 64, 8, 1, "bf16"),     # transform with 512 threads per row
    (66, 32768, 16, 4, 1, "fp32"),     # transform with 1024 threads per row
])
def test_parity_prefill_shapes(M, K, N, bits, had, xdt):
    _run_case(M, K, N, bits, had, xdt, seed=M + K * 3 + N, n_out=max(1, K // 200), factor=50.0)


def test_parity_student_t_inputs():
    _run_case(16, 2048, 96, 4, 1, "bf16", seed=5, dist="student_t3")
    _run_case(64, 2048, 96, 4, 1, "bf16", seed=6, dist="student_t3")


# Full-size workloads ------------------------------------------------------
SAMPLE_ROWS = 96


@pytest.mark.parametrize("key", workloads.WORKLOAD_ORDER)
def test_parity_full_workload(key):
    wl = workloads.WORKLOADS[key]
    _say(f"workload {key}")
    case = workloads.make_workload(key, seed=0)
    x = _to_dev_x(case["x"], wl.x_dtype)
    W = torch.from_numpy(case["W"]).to(DEV)
    Wp, alpha = bl.ternarize_weights(W)
    y = bl.hbitlinear_forward(x, Wp, alpha, wl.bits, wl.hadamard)
    codes, scales = bl.quantize_activations(x, wl.bits, wl.hadamard)
    torch.cuda.synchronize()
    del W

    t_ref, a_ref, p_w = oracle.ternarize(case["W"])
    assert_packed_match(Wp.cpu().numpy(), t_ref, p_w)
    assert abs(alpha.item() - a_ref) <= 1e-6 * a_ref
    del p_w

    x64 = oracle.widen_input(case["x"], wl.x_dtype)
    xr = oracle.fwht(x64) if wl.hadamard else x64
    q_ref, s_ref, p_ref = oracle.quantize_activations(xr, wl.bits)
    del xr, x64
    q_gpu = codes.cpu().numpy()
    assert_codes_match(q_gpu, q_ref, p_ref)
    np.testing.assert_allclose(scales.cpu().numpy(), s_ref, rtol=2e-6)
    del p_ref

    if wl.M <= SAMPLE_ROWS:
        rows = np.arange(wl.M)
    else:
        rng = np.random.default_rng(1)
        rows = np.unique(np.concatenate([[0, wl.M - 1], rng.choice(wl.M, SAMPLE_ROWS - 2, replace=False)]))
    acc_ref, y_ref = oracle.forward_from_codes(q_ref[rows], s_ref[rows], t_ref, a_ref, wl.bits)
    assert_y_close(y.cpu().numpy()[rows], y_ref)
    # exact integer product of the oracle's codes and weights on the sampled rows
    acc = bl.ternary_gemm_i32(torch.from_numpy(np.ascontiguousarray(q_ref[rows])).to(DEV),
                              torch.from_numpy(oracle.pack_2bit(t_ref)).to(DEV))
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_ref)


# Many tiles per CU --------------------------------------------------------
# Large products where the forward has the quantizer's row sums run one
# workgroup per CU that walks its tiles with one stage pipeline across tile
# boundaries, storing each tile's outputs while the next one is fetched and
# multiplied; other shapes fall back to the per-tile kernel. The forward is
# compared bit for bit with the per-tile product of the same codes (which
# sums the codes itself), and on sampled rows with the oracle.
@pytest.mark.parametrize("M,K,N,bits,had", [
    (8293, 512, 8228, 8, 0),    # ragged rows and columns, 4-5 tiles per workgroup, 4 stages each
    (4200, 640, 16384, 4, 0),   # 5 stages per tile
    (4100, 1024, 16384, 4, 1),  # transform, 8 stages per tile
    (8200, 576, 8196, 8, 0),    # K not a multiple of 128: per-tile kernel
    (8200, 512, 8190, 4, 0),    # N not a multiple of 4: per-tile kernel
])
def test_parity_many_tiles(M, K, N, bits, had):
    _say(f"many tiles M={M} K={K} N={N} bits={bits} hadamard={had}")
    case = workloads.make_case(M, K, N, x_dtype="bf16", n_out=max(1, K // 100), factor=20.0,
                               seed=M + N)
    x = _to_dev_x(case["x"], "bf16")
    W = torch.from_numpy(case["W"]).to(DEV)
    Wp, alpha = bl.ternarize_weights(W)
    y = bl.hbitlinear_forward(x, Wp, alpha, bits, had)
    rowsum = torch.empty((M,), dtype=torch.int32, device=DEV)
    codes, scales = bl.quantize_activations(x, bits, had, rowsum=rowsum)
    y2 = bl.ternary_linear_dequant(codes, scales, Wp, alpha, bits)
    y3 = bl.ternary_linear_dequant(codes, scales, Wp, alpha, bits, rowsum=rowsum)
    torch.cuda.synchronize()
    del W
    y_np = y.cpu().numpy()
    np.testing.assert_array_equal(y_np, y2.cpu().numpy())
    np.testing.assert_array_equal(y3.cpu().numpy(), y_np)
    np.testing.assert_array_equal(rowsum.cpu().numpy(), codes.cpu().numpy().astype(np.int64).sum(1))
    del y2, y3

    t_ref, a_ref, _ = oracle.ternarize(case["W"])
    x64 = oracle.widen_input(case["x"], "bf16")
    q_ref, s_ref, p_ref = oracle.quantize_activations(oracle.fwht(x64) if had else x64, bits)
    assert_codes_match(codes.cpu().numpy(), q_ref, p_ref)
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([[0, M - 1], np.arange(M - (M % 256), M)[:8],
                                     rng.choice(M, 40, replace=False)]))
    _, y_ref = oracle.forward_from_codes(q_ref[rows], s_ref[rows], t_ref, a_ref, bits)
    assert_y_close(y_np[rows], y_ref)


# FP8 pairs -----------------------------------------------------------------
# 4-bit codes with the transform reach the 128x128 tile product as fp8 E4M3
# bytes in the order of the fp4 weight fields, one fp8 x fp4 MFMA per
# 64-weight block with fp32 sums (exact: half-integers below 2^19). Both
# transform kernels write them: the matrix-core one (bf16, K >= 2048) and the
# butterfly one (8, 16 or 32 elements per thread). The forward must equal, bit
# for bit, the int8-code product of the public quantizer's codes with their
# row sums, and the oracle.
@pytest.mark.parametrize("M,K,N,xdt", [
    (17, 2048, 40, "bf16"),       # one row past the decode batch, one ragged tile
    (300, 4096, 260, "bf16"),     # ragged rows and columns
    (129, 32768, 130, "bf16"),    # the longest row
    (1000, 2048, 2048, "bf16"),   # many tiles, eight stages each
    (2100, 16384, 64, "bf16"),    # a partial tile row at the bottom
    (17, 64, 40, "fp32"),         # the shortest row: butterflies, 8 elements per thread
    (100, 1024, 130, "fp32"),     # 16 elements per thread
    (40, 4096, 96, "fp32"),       # few rows: 16 elements per thread
    (300, 512, 200, "bf16"),      # bf16 below 2048: butterflies
    (70, 16384, 64, "fp32"),      # 32 elements per thread
])
def test_fp8_pair_forward_exact(M, K, N, xdt):
    _say(f"fp8 pairs M={M} K={K} N={N} x={xdt}")
    case = workloads.make_case(M, K, N, x_dtype=xdt, n_out=max(1, K // 100), factor=30.0,
                               seed=M + K + N)
    x = _to_dev_x(case["x"], xdt)
    W = torch.from_numpy(case["W"]).to(DEV)
    Wp, alpha = bl.ternarize_weights(W)
    y = bl.hbitlinear_forward(x, Wp, alpha, 4, 1)
    rowsum = torch.empty((M,), dtype=torch.int32, device=DEV)
    codes, scales = bl.quantize_activations(x, 4, 1, rowsum=rowsum)
    y2 = bl.ternary_linear_dequant(codes, scales, Wp, alpha, 4, rowsum=rowsum)
    torch.cuda.synchronize()
    del W
    y_np = y.cpu().numpy()
    np.testing.assert_array_equal(y_np, y2.cpu().numpy())
    del y2
    t_ref, a_ref, _ = oracle.ternarize(case["W"])
    x64 = oracle.widen_input(case["x"], xdt)
    q_ref, s_ref, p_ref = oracle.quantize_activations(oracle.fwht(x64), 4)
    assert_codes_match(codes.cpu().numpy(), q_ref, p_ref)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 40), replace=False)]))
    _, y_ref = oracle.forward_from_codes(q_ref[rows], s_ref[rows], t_ref, a_ref, 4)
    assert_y_close(y_np[rows], y_ref)


# Edge and degenerate cases ------------------------------------------------
def test_zero_weights_give_zero_output():
    _say("zero weights")
    x = torch.randn(5, 256, device=DEV)
    W = torch.zeros(40, 256, device=DEV)
    Wp, alpha = bl.ternarize_weights(W)
    y = bl.hbitlinear_forward(x, Wp, alpha, 4, 1)
    torch.cuda.synchronize()
    assert alpha.item() == 0.0
    assert np.all(Wp.cpu().numpy() == 0x55)
    assert torch.count_nonzero(y).item() == 0


def test_zero_rows_and_constant_weights():
    _say("zero rows, constant weights")
    x = torch.randn(20, 128, device=DEV)
    x[3] = 0
    x[17] = 0
    W = torch.full((24, 128), -0.25, device=DEV)
    Wp, alpha = bl.ternarize_weights(W)
    codes, scales = bl.quantize_activations(x, 8, 1)
    y = bl.hbitlinear_forward(x, Wp, alpha, 8, 1)
    torch.cuda.synchronize()
    assert alpha.item() == pytest.approx(0.25)
    assert np.all(decode_packed(Wp.cpu().numpy()) == -1)
    assert torch.count_nonzero(codes[3]).item() == 0 and torch.count_nonzero(y[17]).item() == 0
    assert scales[3].item() == pytest.approx(1e-7)


@pytest.mark.parametrize("K,last_only,rms", [(2560, False, False), (1344, True, False),
                                              (1344, True, True), (2560, False, True)])
def test_single_token_statistic_edges(K, last_only, rms):
    """The one-wave kernel on a zero token (statistic 0: s = eps, every code
    0, y = 0) and on a token whose only non-zero value is its last element,
    inside a partial last super-block (lanes past K must not enter the max):
    bit for bit the two-stage forward, codes as the oracle's."""
    _say(f"single-token statistic edges K={K} last_only={last_only} rms={rms}")
    N = 70
    rng = np.random.default_rng(K + 7)
    W = torch.from_numpy((rng.standard_normal((N, K)) * 0.02).astype(np.float32)).to(DEV)
    Wp, alpha = bl.ternarize_weights(W)
    x_np = np.zeros((1, K), dtype=np.float32)
    if last_only:
        x_np[0, K - 1] = -3.0
    x = torch.from_numpy(x_np).to(DEV).to(torch.bfloat16)
    if rms:
        y = bl.hbitlinear_forward_prologue(x, Wp, alpha, 8, 0, rmsnorm=True)
        torch.cuda.synchronize()
        assert torch.isfinite(y).all()
        if not last_only:
            assert torch.count_nonzero(y).item() == 0
            return
        t_ref, a_ref, _ = oracle.ternarize(W.cpu().numpy())
        ref = oracle.forward_prologue(x_np, "fp32", t_ref, a_ref, 8, 0, rms=True)
        assert_y_close(y.cpu().numpy(), ref["y64"], what="RMSNorm single token, one value",
                       tol=1e-3)
        return
    y = bl.hbitlinear_forward(x, Wp, alpha, 8, 0)
    codes, scales = bl.quantize_activations(x, 8, 0)
    y2 = bl.ternary_linear_dequant(codes, scales, Wp, alpha, 8)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), y2.cpu().numpy())
    q_ref, _, _ = oracle.quantize_activations(x_np.astype(np.float64), 8)
    q = codes.cpu().numpy()
    np.testing.assert_array_equal(q, q_ref)
    if last_only:
        assert q[0, K - 1] == -127 and np.count_nonzero(q) == 1
    else:
        assert np.count_nonzero(q) == 0 and torch.count_nonzero(y).item() == 0


def test_empty_batch_is_noop():
    _say("empty batch")
    W = torch.randn(8, 64, device=DEV) * 0.02
    Wp, alpha = bl.ternarize_weights(W)
    x = torch.empty(0, 64, device=DEV)
    y = bl.hbitlinear_forward(x, Wp, alpha, 8, 0)
    torch.cuda.synchronize()
    assert y.shape == (0, 8)


def test_pack_2bit_matches_oracle():
    _say("pack_2bit")
    rng = np.random.default_rng(3)
    t = rng.integers(-1, 2, size=(77, 640)).astype(np.int8)
    Wp = bl.pack_2bit(torch.from_numpy(t).to(DEV))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(Wp.cpu().numpy(), oracle.pack_2bit(t))


def test_integer_extremes_exact():
    _say("integer extremes")
    K = 32768
    q = np.full((18, K), 127, dtype=np.int8)
    q[1] = -128
    q[5, ::3] = -128
    t = np.ones((33, K), dtype=np.int8)
    t[2] = -1
    t[7, ::2] = 0
    codes = torch.from_numpy(q).to(DEV)
    Wp = bl.pack_2bit(torch.from_numpy(t).to(DEV))
    for m in (18, 2):  # prefill tile and the streaming shape
        acc = bl.ternary_gemm_i32(codes[:m].contiguous(), Wp)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc.cpu().numpy(), oracle.ternary_matmul_i64(q[:m], t))


def test_bitwise_deterministic():
    _say("determinism")
    case = workloads.make_case(300, 4096, 200, x_dtype="bf16", n_out=20, factor=20.0, seed=9)
    x = _to_dev_x(case["x"], "bf16")
    W = torch.from_numpy(case["W"]).to(DEV)
    outs = []
    for _ in range(2):
        Wp, alpha = bl.ternarize_weights(W)
        y = bl.hbitlinear_forward(x, Wp, alpha, 4, 1)
        torch.cuda.synchronize()
        outs.append((Wp.cpu().numpy(), alpha.item(), y.cpu().numpy()))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    assert outs[0][1] == outs[1][1]
    np.testing.assert_array_equal(outs[0][2], outs[1][2])


@pytest.mark.parametrize("M,K,N,bits,had", [
    (1, 2560, 700, 8, 0),      # one fused kernel
    (16, 16384, 300, 4, 1),    # transform + streaming product
    (200, 1024, 300, 4, 1),    # prefill tile
    (200, 2048, 300, 4, 1),    # prefill tile on fp8 pairs
])
def test_graph_replay_matches_eager(M, K, N, bits, had):
    _say(f"graph replay M={M} K={K} N={N}")
    case = workloads.make_case(M, K, N, x_dtype="bf16", n_out=8, factor=30.0, seed=M + N)
    x = _to_dev_x(case["x"], "bf16")
    Wp, alpha = bl.ternarize_weights(torch.from_numpy(case["W"]).to(DEV))
    need = bl.forward_workspace_bytes(M, K, N, bits, had)
    ws = torch.empty((need,), dtype=torch.uint8, device=DEV) if need else None
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    bl.hbitlinear_forward(x, Wp, alpha, bits, had, out=y, workspace=ws)
    torch.cuda.synchronize()
    eager = y.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            bl.hbitlinear_forward(x, Wp, alpha, bits, had, out=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(4):
        y.fill_(float("nan"))
        # unrelated eager work between replays
        junk = torch.randn(64, 64, device=DEV) @ torch.randn(64, 64, device=DEV)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy(), eager.cpu().numpy())
        del junk


def test_module_wrapper():
    _say("HBitLinear wrapper")
    case = workloads.make_case(9, 512, 70, x_dtype="fp32", n_out=5, factor=40.0, seed=12)
    layer = bl.HBitLinear(torch.from_numpy(case["W"]).to(DEV), bits=4, hadamard=True)
    y = layer(torch.from_numpy(case["x"]).to(DEV))
    torch.cuda.synchronize()
    t, a, _ = oracle.ternarize(case["W"])
    ref = oracle.forward(case["x"], "fp32", t, a, 4, 1)
    assert_y_close(y.cpu().numpy(), ref["y64"])


@pytest.mark.parametrize("M,K,N,bits,had", [
    (16, 16384, 130, 4, 1),    # nibble codes between the stages
    (200, 1024, 300, 8, 0),    # prefill tile
    (5, 2048, 77, 8, 1),       # transform kernel + weight-streaming product
])
def test_forward_stages_compose_to_the_forward(M, K, N, bits, had):
    """The quantization stage then the product stage, on one workspace, give
    the forward's output bit for bit; a fused shape refuses a lone stage."""
    _say(f"stages M={M} K={K} N={N} bits={bits} hadamard={had}")
    case = workloads.make_case(M, K, N, x_dtype="bf16", n_out=8, factor=30.0, seed=M + K)
    x = _to_dev_x(case["x"], "bf16")
    Wp, alpha = bl.ternarize_weights(torch.from_numpy(case["W"]).to(DEV))
    ws = torch.empty((bl.forward_workspace_bytes(M, K, N, bits, had),), dtype=torch.uint8,
                     device=DEV)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    bl.hbitlinear_forward_stages(x, Wp, alpha, bits, had, 1, out=y, workspace=ws)
    bl.hbitlinear_forward_stages(x, Wp, alpha, bits, had, 2, out=y, workspace=ws)
    y_ref = bl.hbitlinear_forward(x, Wp, alpha, bits, had)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), y_ref.cpu().numpy())
    xs = _to_dev_x(workloads.make_case(1, 2560, 16, x_dtype="bf16", seed=1)["x"], "bf16")
    Wps = torch.full((16, 640), 0x55, dtype=torch.uint8, device=DEV)
    with pytest.raises(bl.BitNetError):
        bl.hbitlinear_forward_stages(xs, Wps, alpha, 8, 0, 1, out=torch.empty((1, 16), device=DEV),
                                     workspace=torch.empty((16,), dtype=torch.uint8, device=DEV))


def test_stream_read_reads_without_writing():
    _say("stream read")
    buf = torch.zeros((3 * 2 ** 20 + 4096,), dtype=torch.uint8, device=DEV)
    sink = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    bl.stream_read(buf, sink)
    torch.cuda.synchronize()
    assert sink.item() == 7  # zero data never matches the sink's constant
    with pytest.raises(ValueError):
        bl.stream_read(buf, torch.zeros((2,), dtype=torch.int32, device=DEV))


def test_binding_rejects_wrong_outputs():
    _say("binding output checks")
    x = torch.zeros((4, 256), dtype=torch.float32, device=DEV)
    Wp = torch.full((32, 64), 0x55, dtype=torch.uint8, device=DEV)
    alpha = torch.ones((1,), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        bl.hbitlinear_forward(x, Wp, alpha, 8, 1, out=torch.empty((4, 31), device=DEV))
    with pytest.raises(TypeError):
        bl.hbitlinear_forward(x, Wp, alpha, 8, 1,
                              out=torch.empty((4, 32), dtype=torch.float16, device=DEV))
    with pytest.raises(ValueError):
        bl.hbitlinear_forward(x, Wp, alpha, 8, 1, out=torch.empty((4, 32)))
    with pytest.raises(ValueError):
        bl.quantize_activations(x, 8, 1, codes=torch.empty((4, 128), dtype=torch.int8, device=DEV))
    with pytest.raises(ValueError):
        bl.ternarize_weights(torch.zeros((32, 256), device=DEV),
                             out=torch.empty((32, 32), dtype=torch.uint8, device=DEV))
    kv = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        bl.kv_quantize(kv, 4, codes=torch.empty((1, 2, 8, 32), dtype=torch.int8, device=DEV))
    with pytest.raises(ValueError):
        bl.kv_quantize(kv, 4, scales=torch.empty((1, 2, 8)))
    with pytest.raises(ValueError):
        bl.kv_quantize_packed(kv, 3, packed=torch.empty((1, 2, 8, 64), dtype=torch.uint8,
                                                        device=DEV))
    with pytest.raises(TypeError):
        bl.kv_quantize_packed(kv, 4, bos_codes=torch.empty((1, 2, 64), dtype=torch.uint8,
                                                           device=DEV))

