"""Comparison rules between the HIP path and the CPU oracle.

Acceptance (stated for this library):
  - packed weights and activation codes are bit-exact, except +-1 flips where
    the oracle's pre-rounding value lies within 1e-4 of a .5 boundary (the
    two sides compute that value in different precisions);
  - int32 accumulators are bit-exact on identical codes;
  - the fp32 output has relative Frobenius error <= 1e-3.
"""

import numpy as np

import oracle

BAND = 1e-4
Y_TOL = 1e-3


def assert_codes_match(q_gpu, q_ref, p_ref, what="codes"):
    q_gpu = np.asarray(q_gpu).astype(np.int32)
    q_ref = np.asarray(q_ref).astype(np.int32)
    assert q_gpu.shape == q_ref.shape, (q_gpu.shape, q_ref.shape)
    diff = q_gpu - q_ref
    bad = diff != 0
    n_bad = int(bad.sum())
    if n_bad:
        dist = oracle.quant_boundary_distance(np.asarray(p_ref)[bad])
        ok = (np.abs(diff[bad]) == 1) & (dist < BAND)
        if not np.all(ok):
            idx = np.argwhere(bad)[~ok][:5]
            raise AssertionError(
                f"{what}: {int((~ok).sum())} mismatches outside the rounding band, first at "
                f"{idx.tolist()}: gpu={q_gpu[tuple(idx[0])]} ref={q_ref[tuple(idx[0])]} "
                f"p={np.asarray(p_ref)[tuple(idx[0])]!r}")
    return n_bad


def decode_packed(wp):
    """Ternary weights of a packed [N, K/4] array, decoded on the test side
    from the library's block-64 layout (byte b of the 16-byte block g holds
    the weights 64 g + 16 j + b in bit pair j, as code t + 1). Kept apart
    from the oracle so that no GPU output is ever an oracle input."""
    wp = np.asarray(wp, dtype=np.uint8)
    N, KB = wp.shape
    blocks = wp.reshape(N, KB // 16, 16)
    t = np.empty((N, KB // 16, 4, 16), dtype=np.int8)
    for j in range(4):
        t[:, :, j, :] = ((blocks >> (2 * j)) & 3).astype(np.int8) - 1
    return t.reshape(N, KB * 4)


def assert_packed_match(wp_gpu, t_ref, p_ref):
    wp_gpu = np.asarray(wp_gpu)
    # no field may hold the unused code 3
    for j in range(4):
        assert not np.any(((wp_gpu >> (2 * j)) & 3) == 3)
    t_gpu = decode_packed(wp_gpu)
    n_flips = assert_codes_match(t_gpu, t_ref, p_ref, what="ternary weights")
    if n_flips == 0:
        np.testing.assert_array_equal(wp_gpu, oracle.pack_2bit(t_ref))
    return n_flips


def rel_frobenius(a, ref):
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(a - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def assert_y_close(y_gpu, y_ref, what="y", tol=Y_TOL):
    err = rel_frobenius(y_gpu, y_ref)
    assert err <= tol, f"{what}: relative Frobenius error {err:.3e} > {tol}"
    return err


# The epilogue alone (int32 acc -> fp32 y) differs from the fp64 oracle only
# by fp32 rounding of alpha * s / c and of the final product.
EPILOGUE_TOL = 1e-5


def assert_y_with_flips(y_gpu, q_gpu, t_gpu, q_ref, t_ref, s_ref, alpha, bits, y_ref):
    """End-to-end output check. Without code or weight flips: relative
    Frobenius error <= 1e-3 against the oracle. A +-1 flip allowed by the
    rounding band moves y[m, n] by at most alpha * s_m / c per flipped code
    (times |t|) or flipped weight (times |q|); that allowance is taken off
    each element's error and the rest must meet the same 1e-3."""
    q_gpu = np.asarray(q_gpu, dtype=np.float64)
    t_gpu = np.asarray(t_gpu, dtype=np.float64)
    q_ref = np.asarray(q_ref, dtype=np.float64)
    t_ref = np.asarray(t_ref, dtype=np.float64)
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    dq = np.abs(q_gpu - q_ref)
    dt = np.abs(t_gpu - t_ref)
    if not dq.any() and not dt.any():
        return assert_y_close(y_gpu, y_ref)
    c = oracle.INT8_SCALE if bits == 8 else oracle.INT4_SCALE
    allowance = (dq @ np.abs(t_gpu).T + np.abs(q_ref) @ dt.T) * (alpha * np.asarray(s_ref)[:, None] / c)
    excess = np.maximum(np.abs(y_gpu - y_ref) - allowance * (1 + 1e-6), 0.0)
    err = float(np.linalg.norm(excess) / max(np.linalg.norm(y_ref), 1e-300))
    assert err <= Y_TOL, f"y: error beyond the flip allowance {err:.3e} > {Y_TOL}"
    return err


def assert_y_in_band(y_gpu, t_gpu, q_ref, p_ref, t_ref, s_ref, alpha, bits, y_ref):
    """End-to-end check of a forward whose codes are not visible (the fused
    single-kernel decode, the TL2 decode): its codes may differ from the
    oracle's only by the +-1 flips the rounding band allows, i.e. at the
    positions whose oracle pre-round value lies within 1e-4 of a .5 boundary.
    Each such position may move y[m, n] by alpha * s_m / c * |t[n, k]|, and
    each weight flip by alpha * s_m / c * |q[m, k]|; that allowance is taken
    off each element's error and the rest must meet the 1e-3 rule. With no
    position in the band this is the plain relative Frobenius check."""
    t_gpu = np.asarray(t_gpu, dtype=np.float64)
    t_ref = np.asarray(t_ref, dtype=np.float64)
    q_ref = np.asarray(q_ref, dtype=np.float64)
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    in_band = (oracle.quant_boundary_distance(p_ref) < BAND).astype(np.float64)
    dt = np.abs(t_gpu - t_ref)
    if not in_band.any() and not dt.any():
        return assert_y_close(y_gpu, y_ref)
    c = oracle.INT8_SCALE if bits == 8 else oracle.INT4_SCALE
    allowance = (in_band @ np.abs(t_gpu).T + np.abs(q_ref) @ dt.T) * \
        (alpha * np.asarray(s_ref)[:, None] / c)
    excess = np.maximum(np.abs(y_gpu - y_ref) - allowance * (1 + 1e-6), 0.0)
    err = float(np.linalg.norm(excess) / max(np.linalg.norm(y_ref), 1e-300))
    assert err <= Y_TOL, f"y: error beyond the rounding-band allowance {err:.3e} > {Y_TOL}"
    return err
