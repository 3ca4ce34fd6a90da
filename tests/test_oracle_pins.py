"""Pins of the CPU oracle to things other than itself (CPU only).

Every oracle function is checked against at least one of: a hand-derived
worked value (tests/golden), a closed form, a library routine that computes a
special case (scipy.linalg.hadamard, torch's per-channel quantizer, torch's
bf16 conversion), brute force on tiny inputs, or an invariant that a plausible
mistake (dropped term, wrong sign or index, transposed operand, wrong
constant) would break.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.stats
import torch

import oracle
from bit_activation_linear_amd import workloads


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- FWHT ----

@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64])
def test_hadamard_closed_form_matches_scipy(n):
    # scipy.linalg.hadamard builds the unnormalised Sylvester matrix.
    H = oracle.hadamard_matrix(n)
    np.testing.assert_array_equal(H * math.sqrt(n), scipy.linalg.hadamard(n).astype(np.float64))


def _sylvester_by_recursion(m):
    # The page's recursion, unrolled by explicit block assembly.
    H = np.array([[1.0]])
    for _ in range(m):
        H = np.block([[H, H], [H, -H]]) / math.sqrt(2.0)
    return H


@pytest.mark.parametrize("m", range(0, 7))
def test_hadamard_closed_form_matches_recursion(m):
    np.testing.assert_allclose(oracle.hadamard_matrix(2 ** m), _sylvester_by_recursion(m),
                               rtol=0, atol=1e-15)


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32, 64, 128, 1024])
def test_fwht_butterflies_equal_dense_definition(n):
    rng = np.random.default_rng(n)
    x = rng.standard_normal((5, n))
    ref = x @ (scipy.linalg.hadamard(n) / math.sqrt(n))
    np.testing.assert_allclose(oracle.fwht(x), ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.fwht_dense(x), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [2, 8, 64, 256])
def test_hadamard_symmetric_and_involutory(n):
    H = oracle.hadamard_matrix(n)
    np.testing.assert_array_equal(H, H.T)
    np.testing.assert_allclose(H @ H, np.eye(n), rtol=0, atol=1e-13)


def test_fwht_parseval_and_twice_is_identity():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 4096)) * 3.0
    y = oracle.fwht(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_allclose(oracle.fwht(y), x, rtol=0, atol=1e-12)


def test_fwht_golden(golden_dir):
    g = _load(golden_dir, "fwht_small.json")
    for case in g["cases"]:
        np.testing.assert_allclose(oracle.fwht(np.array(case["x"])), np.array(case["y"]),
                                   rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("n", [0, 3, 6, 12, 100])
def test_fwht_rejects_non_power_of_two(n):
    with pytest.raises(ValueError):
        oracle.fwht(np.zeros((1, n)))


def test_fwht_spreads_outlier_channels():
    # The engine page's outlier profiler: the transform lowers the peak and the
    # excess kurtosis of activations with a few large channels.
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 2048))
    x[:, rng.choice(2048, 10, replace=False)] *= 50.0
    y = oracle.fwht(x)

    def kurt(a):
        a = a.ravel()
        return scipy.stats.kurtosis(a, fisher=True, bias=True)

    assert np.abs(y).max() < np.abs(x).max() / 4
    assert abs(kurt(y)) < abs(kurt(x))


# ---------------------------------------------------------- ternarize ----

def test_ternarize_golden(golden_dir):
    g = _load(golden_dir, "ternarize_small.json")
    W = np.array(g["W"], dtype=np.float32)
    t, alpha, p = oracle.ternarize(W)
    assert abs(alpha - g["alpha"]) < g["alpha_tol"]
    np.testing.assert_array_equal(t, np.array(g["t"], dtype=np.int8))


def test_ternarize_statistics_of_gaussian_weights():
    # For W ~ N(0, sigma^2): E|W| = sigma sqrt(2/pi); a weight rounds to 0 iff
    # |W| < alpha/2, so the zero fraction is 2 Phi(sqrt(2/pi)/2) - 1 = 0.3101.
    rng = np.random.default_rng(5)
    sigma = 0.02
    W = (rng.standard_normal((512, 1024)) * sigma).astype(np.float32)
    t, alpha, _ = oracle.ternarize(W)
    assert abs(alpha - sigma * math.sqrt(2 / math.pi)) < 3e-3 * alpha
    zero_frac = np.mean(t == 0)
    expect = 2 * scipy.stats.norm.cdf(0.5 * math.sqrt(2 / math.pi)) - 1
    assert abs(zero_frac - expect) < 3e-3
    assert set(np.unique(t)) == {-1, 0, 1}
    # +1 and -1 are equally likely
    assert abs(np.mean(t == 1) - np.mean(t == -1)) < 5e-3


def test_ternarize_special_cases():
    for c in (0.7, -0.003, 5.0):
        t, alpha, _ = oracle.ternarize(np.full((3, 8), c, dtype=np.float32))
        assert alpha == pytest.approx(abs(np.float32(c)), rel=1e-12)
        assert np.all(t == np.sign(c))
    t, alpha, _ = oracle.ternarize(np.zeros((2, 64), dtype=np.float32))
    assert alpha == 0.0 and np.all(t == 0)
    # one big weight among zeros: alpha = big/n, big/alpha = n -> clipped to 1
    W = np.zeros((1, 64), dtype=np.float32)
    W[0, 5] = -2.0
    t, alpha, p = oracle.ternarize(W)
    assert alpha == pytest.approx(2.0 / 64)
    assert t[0, 5] == -1 and np.count_nonzero(t) == 1


# ------------------------------------------------------------- pack ----

def test_pack_golden(golden_dir):
    g = _load(golden_dir, "pack_small.json")
    t = np.zeros((len(g["rows"]), 64), dtype=np.int8)
    for r, row in enumerate(g["rows"]):
        for k, v in row["set"].items():
            t[r, int(k)] = v
    packed = oracle.pack_2bit(t)
    np.testing.assert_array_equal(packed, np.array([row["bytes"] for row in g["rows"]], dtype=np.uint8))


def test_pack_roundtrip_and_no_code_three():
    rng = np.random.default_rng(7)
    t = rng.integers(-1, 2, size=(33, 64 * 7)).astype(np.int8)
    packed = oracle.pack_2bit(t)
    assert packed.shape == (33, 64 * 7 // 4)
    np.testing.assert_array_equal(oracle.unpack_2bit(packed), t)
    for j in range(4):
        assert not np.any(((packed >> (2 * j)) & 3) == 3)


def test_pack_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.pack_2bit(np.zeros((2, 60), dtype=np.int8))
    with pytest.raises(ValueError):
        oracle.pack_2bit(np.full((2, 64), 2, dtype=np.int8))


# ------------------------------------------------------- act quant ----

def test_act_quant_golden(golden_dir):
    g = _load(golden_dir, "act_quant_small.json")
    for case in g["cases"]:
        q, s, p = oracle.quantize_activations(np.array([case["x"]]), case["bits"])
        np.testing.assert_array_equal(q[0], np.array(case["q"], dtype=np.int8))
        assert s[0] == pytest.approx(case["s"], rel=1e-15)


def test_int8_codes_match_torch_per_channel_quantizer():
    # A symmetric per-row int8 quantizer with scale s/127 is torch's
    # quantize_per_channel (fp32, round half to even). Away from .5 boundaries
    # the codes must agree exactly.
    rng = np.random.default_rng(11)
    x = rng.standard_normal((16, 512)).astype(np.float32)
    x[:, :3] *= 40
    q, s, p = oracle.quantize_activations(x.astype(np.float64), 8)
    scales = torch.tensor(s / 127.0, dtype=torch.float64)
    tq = torch.quantize_per_channel(torch.from_numpy(x), scales, torch.zeros(16, dtype=torch.int64),
                                    0, torch.qint8).int_repr().numpy()
    safe = oracle.quant_boundary_distance(p) > 1e-4
    np.testing.assert_array_equal(q[safe], tq[safe])


def test_int8_invariants():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((32, 300)) * rng.uniform(0.01, 100, size=(32, 1))
    q, s, p = oracle.quantize_activations(x, 8)
    am = np.argmax(np.abs(x), axis=1)
    np.testing.assert_array_equal(np.abs(q[np.arange(32), am]), 127)
    assert q.min() >= -127 and q.max() <= 127
    np.testing.assert_allclose(s, np.abs(x).max(axis=1) + oracle.EPS, rtol=1e-15)
    # scale invariance up to eps: codes of 4x equal the codes of x off-boundary
    q4, _, _ = oracle.quantize_activations(4.0 * x, 8)
    safe = oracle.quant_boundary_distance(p) > 1e-4
    np.testing.assert_array_equal(q4[safe], q[safe])


def test_int4_invariants():
    rng = np.random.default_rng(17)
    x = rng.standard_normal((32, 256))
    x[:, 7] *= 80
    q, s, p = oracle.quantize_activations(x, 4)
    assert q.min() == -8 or q.max() == 7
    assert q.min() >= -8 and q.max() <= 7
    np.testing.assert_allclose(s, np.abs(x).mean(axis=1) + oracle.EPS, rtol=1e-13)
    # on a Gaussian row absmean*sqrt7 scaling maps x to roughly N(0, 7*pi/2)
    g = rng.standard_normal((4, 1 << 16))
    qg, _, _ = oracle.quantize_activations(g, 4)
    assert abs(np.mean(qg == 0) - (2 * scipy.stats.norm.cdf(0.5 / math.sqrt(7 * math.pi / 2)) - 1)) < 0.01


def test_zero_row_quantizes_to_zero():
    for bits in (4, 8):
        q, s, p = oracle.quantize_activations(np.zeros((2, 64)), bits)
        assert np.all(q == 0)
        np.testing.assert_array_equal(s, [oracle.EPS, oracle.EPS])


def test_quant_boundary_distance_hand_values():
    """Distance of a pre-round value from the nearest rounding boundary
    (k + 1/2) of RoundClip ([engine] Eq. 1, 5, 6): values worked by hand."""
    p = np.array([2.5, 2.0, -1.49, -2.5, 126.99995, 0.0, 0.25, -0.75, 7.5001])
    want = np.array([0.0, 0.5, 0.01, 0.0, 0.49995, 0.5, 0.25, 0.25, 0.0001])
    np.testing.assert_allclose(oracle.quant_boundary_distance(p), want, rtol=0, atol=1e-9)


def test_quant_boundary_distance_is_the_rounding_margin():
    """d(p) is exactly how far p can move before rint(p) changes: every shift
    below d keeps the rounded value, a shift just beyond d (towards the
    boundary) changes it. A slip such as |p - rint(p)| (the distance to the
    integer, 1/2 - d) fails this."""
    rng = np.random.default_rng(41)
    p = rng.uniform(-130, 130, 20000)
    d = oracle.quant_boundary_distance(p)
    assert np.all((d >= 0) & (d <= 0.5))
    toward = np.sign(p - np.rint(p))  # direction of the nearer boundary
    toward[toward == 0] = 1.0
    keep = d > 1e-9
    inside = p + 0.999 * d * toward
    beyond = p + (d + 1e-7) * toward
    np.testing.assert_array_equal(np.rint(inside[keep]), np.rint(p[keep]))
    assert np.all(np.rint(beyond[keep & (d < 0.4999)]) != np.rint(p[keep & (d < 0.4999)]))


def test_in_band_rule_accepts_band_flips_and_rejects_others():
    """The GPU parity rule for forwards whose codes are not visible: a +-1
    code flip at a position inside the 1e-4 band is absorbed by its bounded
    effect on y; the same flip at a position outside the band is not (the
    mistake is planted in an oracle result, on the CPU)."""
    from parity_util import assert_y_in_band

    rng = np.random.default_rng(43)
    M, K, N = 3, 128, 24
    x = rng.standard_normal((M, K))
    W = rng.standard_normal((N, K)) * 0.02
    t, a, _ = oracle.ternarize(W)
    q, s, p = oracle.quantize_activations(x, 4)
    # place one value of row 1 exactly on a rounding boundary's band
    k_band = 5
    p = p.copy()
    p[1, k_band] = np.floor(p[1, k_band]) + 0.5 + 3e-5
    y_ref = oracle.dequantize(oracle.ternary_matmul_i64(q, t), a, s, 4)
    assert_y_in_band(y_ref, t, q, p, t, s, a, 4, y_ref)
    # one flipped code moves its output row well past 1e-3 of ||y|| here;
    # flipped inside the band it is allowed, outside it is not
    def flipped(k):
        q2 = q.astype(np.int64).copy()
        q2[1, k] += 1
        return oracle.dequantize(oracle.ternary_matmul_i64(q2, t), a, s, 4)
    y_in = flipped(k_band)
    assert_y_in_band(y_in, t, q, p, t, s, a, 4, y_ref)
    k_out = 9
    assert oracle.quant_boundary_distance(p[1, k_out]) > 1e-4
    y_out = flipped(k_out)
    assert np.linalg.norm(y_out - y_ref) > 1e-3 * np.linalg.norm(y_ref)
    with pytest.raises(AssertionError):
        assert_y_in_band(y_out, t, q, p, t, s, a, 4, y_ref)


def test_quant_rejects_bad_bits():
    with pytest.raises(ValueError):
        oracle.quantize_activations(np.zeros((1, 4)), 6)


# ---------------------------------------------------- integer product ----

def test_ternary_matmul_brute_force():
    rng = np.random.default_rng(19)
    q = rng.integers(-128, 128, size=(5, 37)).astype(np.int8)
    t = rng.integers(-1, 2, size=(6, 37)).astype(np.int8)
    acc = oracle.ternary_matmul_i64(q, t)
    brute = np.zeros((5, 6), dtype=np.int64)
    for m in range(5):
        for n in range(6):
            total = 0
            for k in range(37):
                total += int(q[m, k]) * int(t[n, k])
            brute[m, n] = total
    np.testing.assert_array_equal(acc, brute)


def test_ternary_matmul_extremes_exact():
    K = 1 << 15
    q = np.full((2, K), 127, dtype=np.int8)
    q[1] = -128
    t = np.ones((3, K), dtype=np.int8)
    t[1] = -1
    t[2, ::2] = 0
    acc = oracle.ternary_matmul_i64(q, t)
    np.testing.assert_array_equal(acc, [[127 * K, -127 * K, 127 * K // 2],
                                        [-128 * K, 128 * K, -128 * K // 2]])


# ------------------------------------------------------- full forward ----

@pytest.mark.parametrize("bits,hadamard", [(4, 1), (8, 1), (4, 0), (8, 0)])
def test_forward_integer_route_equals_fake_quant_route(bits, hadamard):
    # The engine page computes F.linear(Q_act(x_r), alpha * t) on dequantized
    # floats; the oracle multiplies integer codes and rescales afterwards. The
    # two must agree to rounding.
    case = workloads.make_case(6, 256, 40, x_dtype="bf16", n_out=3, factor=30.0, seed=23)
    t, alpha, _ = oracle.ternarize(case["W"])
    out = oracle.forward(case["x"], "bf16", t, alpha, bits, hadamard)
    xq = torch.from_numpy(out["q"].astype(np.float64) * (out["s"][:, None] / (127.0 if bits == 8 else math.sqrt(7))))
    wq = torch.from_numpy(t.astype(np.float64) * alpha)
    y_fake = torch.nn.functional.linear(xq, wq).numpy()
    np.testing.assert_allclose(out["y64"], y_fake, rtol=1e-12, atol=1e-12 * np.abs(y_fake).max())


def test_forward_int8_no_hadamard_is_b158_bitlinear():
    # Special case: bits=8, no Hadamard is the b1.58 BitLinear of the blog page
    # without its RMSNorm (integer product, then * w_scale * x_scale / Qb), with
    # Qb = 127 and eps = 1e-7 as on the engine page. The blog rescales with the
    # statistic itself rather than stat + eps: a relative change of eps/gamma.
    case = workloads.make_case(4, 128, 24, x_dtype="fp32", n_out=2, factor=10.0, seed=29)
    t, alpha, _ = oracle.ternarize(case["W"])
    out = oracle.forward(case["x"], "fp32", t, alpha, 8, 0)
    x = torch.from_numpy(case["x"].astype(np.float64))
    w = torch.from_numpy(case["W"].astype(np.float64))
    w_scale = w.abs().mean()
    w_q = torch.clamp(torch.round(w / (w_scale + 1e-7)), -1, 1)
    gamma = x.abs().max(dim=-1, keepdim=True).values
    x_q = torch.clamp(torch.round(x * 127 / (gamma + 1e-7)), -128, 127)
    y_blog = torch.nn.functional.linear(x_q, w_q) * (w_scale * gamma) / 127
    np.testing.assert_allclose(out["y64"], y_blog.numpy(), rtol=1e-6, atol=1e-9)


def test_forward_zero_weights_and_zero_rows():
    x = np.zeros((3, 64), dtype=np.float32)
    x[1] = np.linspace(-1, 1, 64, dtype=np.float32)
    t, alpha, _ = oracle.ternarize(np.zeros((5, 64), dtype=np.float32))
    out = oracle.forward(x, "fp32", t, alpha, 4, 1)
    assert np.all(out["y"] == 0)
    t2 = np.ones((5, 64), dtype=np.int8)
    out2 = oracle.forward(x, "fp32", t2, 0.5, 8, 0)
    assert np.all(out2["y"][0] == 0) and np.all(out2["y"][2] == 0)
    assert np.all(out2["q"][0] == 0)


def test_widen_bf16_matches_torch():
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x0001, 0x7F7F, 0x8000, 0x4049], dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.widen_input(bits, "bf16"), ref)


def test_generator_bf16_rounding_matches_torch():
    rng = np.random.default_rng(31)
    x = (rng.standard_normal(100000) * 10).astype(np.float32)
    ours = workloads.fp32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_test_side_decoder_agrees_with_the_oracle():
    """The GPU parity tests decode packed weights with their own decoder
    (no GPU output is ever passed to the oracle); it must read the layout
    the oracle packs."""
    from parity_util import decode_packed

    rng = np.random.default_rng(12)
    t = rng.integers(-1, 2, size=(9, 320)).astype(np.int8)
    np.testing.assert_array_equal(decode_packed(oracle.pack_2bit(t)), t)
