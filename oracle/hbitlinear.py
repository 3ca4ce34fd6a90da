"""fp64 NumPy oracle of the H-BitLinear forward and backward — TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the bench's CPU-baseline leg may call this.
Nothing here is used by, or uses, the HIP library.

Sources (the pages the method is taken from):
  [engine]  Quillan-Ronin "bitnet_v2_engine.py" page: a PyTorch restatement of
            BitNet v2 (arXiv 2504.18415). Its module docstring lists Eq. 1-8;
            functions fast_hadamard_transform, quantize_weight_ternary,
            quantize_act_int8, quantize_act_int4 and class HBitLinear.
  [edge]    Quillan-Ronin "bitnet_cpp_edge.py" page: bitnet.cpp kernel
            simulation (arXiv 2502.11880), Table 1 taxonomy, I2_S kernel.
  [blog]    youngju.dev "BitNet 论文解析" page: BitLinear_b158 code block.

Precision: every floating-point step is fp64 (the pages compute in fp32; the
fp64 oracle plus a +-1 code-flip band of 1e-4 around .5 rounding boundaries is
the acceptance rule of this library).
"""

from __future__ import annotations

import math

import numpy as np

# [engine] every quantizer and HBitLinear default to eps = 1e-7. The edge and
# blog pages use 1e-5; the engine page is the only one that defines
# H-BitLinear and the sqrt(7) int4 scale, so its value is taken.
EPS = 1e-7
# [engine] Eq. 5: int8 absmax scale 127, clip [-128, 127].
INT8_SCALE = 127.0
# [engine] Eq. 6: int4 absmean scale sqrt(7), clip [-8, 7].
INT4_SCALE = math.sqrt(7.0)

_QUANT = {8: (INT8_SCALE, -128, 127), 4: (INT4_SCALE, -8, 7)}


def _is_pow2(n: int) -> bool:
    return n > 0 and (n & (n - 1)) == 0


def widen_input(x: np.ndarray, x_dtype: str) -> np.ndarray:
    """Exact widening of the layer input to fp64.

    bf16 inputs arrive as uint16 bit patterns; a bf16 value is the fp32 value
    whose upper 16 bits are those bits and whose lower 16 bits are zero."""
    if x_dtype == "fp32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if x_dtype == "bf16":
        u32 = np.asarray(x, dtype=np.uint16).astype(np.uint32) * np.uint32(65536)
        return u32.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown input dtype {x_dtype!r}")


# ---------------------------------------------------------------------------
# Hadamard transform — [engine] module docstring item 2 (Eq. 3, 4, 7) and
# fast_hadamard_transform.
# ---------------------------------------------------------------------------

def hadamard_matrix(n: int) -> np.ndarray:
    """Orthonormal Sylvester-Hadamard matrix H_n in closed form.

    Unrolling the recursion H_m = (1/sqrt 2) [[H_{m-1}, H_{m-1}], [H_{m-1}, -H_{m-1}]],
    H_0 = [1] ([engine] Eq. 3-4) gives H[i, j] = (-1)^popcount(i & j) / sqrt(n)."""
    if not _is_pow2(n):
        raise ValueError(f"Hadamard dimension {n} must be a power of 2")
    i = np.arange(n, dtype=np.int64)
    anded = i[:, None] & i[None, :]
    parity = np.zeros_like(anded)
    while np.any(anded):
        parity ^= anded & 1
        anded >>= 1
    return np.where(parity == 1, -1.0, 1.0) / math.sqrt(n)


def fwht_dense(x: np.ndarray) -> np.ndarray:
    """The definition written out: x_r = x H along the last axis (H = H^T)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    return x @ hadamard_matrix(n)


def fwht(x: np.ndarray) -> np.ndarray:
    """Fast Walsh-Hadamard transform along the last axis, fp64.

    [engine] Eq. 3-4 define H_m recursively as (1/sqrt 2) [[H, H], [H, -H]]
    over H_{m-1}, i.e. H_n is the Kronecker product of log2(n) copies of the
    2x2 factor (1/sqrt 2) [[1, 1], [1, -1]], one per bit of the index. The
    factor of bit b mixes each pair of elements whose indices differ only in
    bit b: with i the index whose bit b is clear and j = i XOR 2^b,
    (x_i, x_j) -> ((x_i + x_j)/sqrt 2, (x_i - x_j)/sqrt 2). Applying the
    factors for b = 0, 1, ..., log2(n) - 1 is the O(n log n) fast transform
    of fast_hadamard_transform (which rejects a non-power-of-2 length and
    casts the result back to the input dtype; here it stays fp64, with no
    intermediate rounding)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    if not _is_pow2(n):
        raise ValueError(f"Hadamard transform dimension {n} must be a power of 2")
    lead = x.shape[:-1]
    y = x.reshape(-1, n).copy()
    r = 1.0 / math.sqrt(2.0)
    index = np.arange(n)
    bit = 1
    while bit < n:
        i = index[(index & bit) == 0]   # bit b clear
        j = i ^ bit                     # the partner: bit b set
        u = y[:, i]
        v = y[:, j]
        y[:, i] = (u + v) * r
        y[:, j] = (u - v) * r
        bit <<= 1
    return y.reshape(*lead, n)


# ---------------------------------------------------------------------------
# Ternary weights — [engine] docstring item 3, Eq. 1-2, quantize_weight_ternary.
# ---------------------------------------------------------------------------

def absmean_alpha(W: np.ndarray) -> float:
    """alpha = mean(|W|) over the whole tensor ([engine] Eq. 2, per-tensor)."""
    W = np.asarray(W, dtype=np.float64)
    return float(np.sum(np.abs(W)) / W.size)


def ternarize(W: np.ndarray, eps: float = EPS):
    """t = RoundClip(W / (alpha + eps), -1, 1) ([engine] Eq. 1).

    Returns (t int8 [N, K], alpha, p) where p = W / (alpha + eps) is the
    pre-rounding value (kept for the rounding-boundary rule). RoundClip rounds
    half to even, as torch.round does."""
    W64 = np.asarray(W, dtype=np.float32).astype(np.float64)
    alpha = absmean_alpha(W64)
    p = W64 / (alpha + eps)
    t = np.clip(np.rint(p), -1.0, 1.0).astype(np.int8)
    return t, alpha, p


# ---------------------------------------------------------------------------
# 2-bit packing (4 weights per byte, 2 bits per weight as in the edge page's
# I2_S format, Table 1). The code value t + 1 in {0, 1, 2} follows the blog
# page's LUT simulation (w -> w + 1). The placement of weights inside a block
# is this library's contract, not the pages':
#   K is cut into blocks of 64 weights; block g of row n is bytes 16g..16g+15
#   of that row; byte b of a block holds the weights at block offsets
#   b, 16 + b, 32 + b, 48 + b in bit pairs 0-1, 2-3, 4-5, 6-7.
# ---------------------------------------------------------------------------

BLOCK = 64


def pack_2bit(t: np.ndarray) -> np.ndarray:
    t = np.asarray(t)
    N, K = t.shape
    if K % BLOCK:
        raise ValueError(f"K={K} must be a multiple of {BLOCK}")
    if t.size and (t.min() < -1 or t.max() > 1):
        raise ValueError("ternary values must lie in {-1, 0, 1}")
    code = (t.astype(np.int16) + 1).astype(np.uint8)
    # axis 2 = which quarter of the block (bit pair), axis 3 = byte in block
    quarters = code.reshape(N, K // BLOCK, 4, BLOCK // 4)
    packed = np.zeros((N, K // BLOCK, BLOCK // 4), dtype=np.uint8)
    for j in range(4):
        packed |= quarters[:, :, j, :] << np.uint8(2 * j)
    return packed.reshape(N, K // 4)


def unpack_2bit(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    N, KB = packed.shape
    K = KB * 4
    if K % BLOCK:
        raise ValueError(f"K={K} must be a multiple of {BLOCK}")
    blocks = packed.reshape(N, K // BLOCK, BLOCK // 4)
    out = np.empty((N, K // BLOCK, 4, BLOCK // 4), dtype=np.int8)
    for j in range(4):
        out[:, :, j, :] = ((blocks >> np.uint8(2 * j)) & np.uint8(3)).astype(np.int8) - 1
    return out.reshape(N, K)


# ---------------------------------------------------------------------------
# Activation quantization — [engine] Eq. 5 (quantize_act_int8) and Eq. 6
# (quantize_act_int4), per token along the last axis.
# ---------------------------------------------------------------------------

def quantize_activations(x: np.ndarray, bits: int, eps: float = EPS):
    """Per-token quantization.

    bits=8: s = max|x| + eps, q = RoundClip(127 x / s, -128, 127)   (Eq. 5)
    bits=4: s = mean|x| + eps, q = RoundClip(sqrt7 x / s, -8, 7)     (Eq. 6)
    Returns (q int8 [M, K], s fp64 [M], p fp64 [M, K] pre-rounding)."""
    if bits not in _QUANT:
        raise ValueError(f"bits must be 4 or 8, got {bits}")
    c, lo, hi = _QUANT[bits]
    x = np.asarray(x, dtype=np.float64)
    if bits == 8:
        stat = np.max(np.abs(x), axis=-1, keepdims=True)
    else:
        stat = np.mean(np.abs(x), axis=-1, keepdims=True)
    s = stat + eps
    p = (c / s) * x
    q = np.clip(np.rint(p), lo, hi).astype(np.int8)
    return q, s[..., 0], p


def quant_boundary_distance(p: np.ndarray) -> np.ndarray:
    """Distance of each pre-rounding value from the nearest .5 boundary."""
    p = np.asarray(p, dtype=np.float64)
    return np.abs(p - (np.floor(p) + 0.5))


# ---------------------------------------------------------------------------
# Integer product and dequantization — [engine] HBitLinear.forward ends in
# F.linear(x_q, w_q); the blog's BitLinear_b158 computes the same product on
# the integer codes and rescales by (w_scale * x_scale) / Qb afterwards.
# ---------------------------------------------------------------------------

def ternary_matmul_i64(q: np.ndarray, t: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k q[m, k] * t[n, k], exact.

    Computed as an fp64 matrix product of integer-valued arrays; every partial
    sum is an integer below 2^53 (|q| <= 128, |t| <= 1, K <= 2^40), so the
    product is exact."""
    q = np.asarray(q)
    t = np.asarray(t)
    if q.shape[1] != t.shape[1]:
        raise ValueError("inner dimensions differ")
    if q.shape[1] >= 2 ** 40:
        raise ValueError("K too large for an exact fp64 product")
    acc = q.astype(np.float64) @ t.astype(np.float64).T
    return np.rint(acc).astype(np.int64)


def dequantize(acc: np.ndarray, alpha: float, s: np.ndarray, bits: int) -> np.ndarray:
    """y = acc * alpha * s / c (c = 127 or sqrt 7), fp64.

    [engine] the quantizers return (s / c) * q with s = stat + eps, and the
    weight quantizer returns alpha * t; by linearity of F.linear the output is
    acc * alpha * s / c."""
    c = _QUANT[bits][0]
    return np.asarray(acc, dtype=np.float64) * (alpha * np.asarray(s, dtype=np.float64)[:, None] / c)


def forward_from_codes(q, s, t, alpha, bits):
    acc = ternary_matmul_i64(q, t)
    y64 = dequantize(acc, alpha, s, bits)
    return acc, y64


def forward(x: np.ndarray, x_dtype: str, t: np.ndarray, alpha: float, bits: int,
            hadamard: int, eps: float = EPS) -> dict:
    """H-BitLinear forward from already-ternarized weights.

    [engine] HBitLinear.forward minus its RMSNorm prologue: x_r = FWHT(x) if
    hadamard, then per-token quantization, then the ternary product and the
    dequantization. Returns a dict with y (fp32), y64, acc, q, s, p."""
    x64 = widen_input(x, x_dtype)
    xr = fwht(x64) if hadamard else x64
    q, s, p = quantize_activations(xr, bits, eps)
    acc, y64 = forward_from_codes(q, s, t, alpha, bits)
    return {"y": y64.astype(np.float32), "y64": y64, "acc": acc, "q": q, "s": s, "p": p, "xr": xr}


# ---------------------------------------------------------------------------
# Prologue of the layer input — [engine] HBitLinear.forward step 1
# (nn.RMSNorm(in_features, eps)) and BitNetV2FFN.forward (Swish(gate) * up,
# the input of the H-BitLinear down projection).
# ---------------------------------------------------------------------------

def silu(g: np.ndarray) -> np.ndarray:
    """Swish / SiLU, g * sigmoid(g) = g / (1 + e^-g) (the FFN's F.silu)."""
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """[engine] BitNetV2FFN.forward: F.silu(gate_proj(x)) * up_proj(x)."""
    return silu(gate) * np.asarray(up, dtype=np.float64)


def rmsnorm(u: np.ndarray, weight=None, eps: float = EPS) -> np.ndarray:
    """[engine] HBitLinear.forward step 1, nn.RMSNorm: per row,
    u / sqrt(mean(u^2) + eps), times the elementwise weight (ones when None,
    the module's initial value)."""
    u = np.asarray(u, dtype=np.float64)
    r = np.sqrt(np.mean(u * u, axis=-1, keepdims=True) + eps)
    out = u / r
    if weight is not None:
        out = out * np.asarray(weight, dtype=np.float64)
    return out


def forward_prologue(x: np.ndarray, x_dtype: str, t: np.ndarray, alpha: float, bits: int,
                     hadamard: int, up=None, rms: bool = False, norm_weight=None,
                     norm_eps: float = EPS, eps: float = EPS) -> dict:
    """The whole [engine] HBitLinear.forward with its input prologue: the
    layer input is u = silu(x) * up when `up` is given (x is then the gate
    projection), else x; RMSNorm when `rms`; then the transform, the
    per-token quantization, the ternary product and the dequantization."""
    u = widen_input(x, x_dtype)
    if up is not None:
        u = swiglu(u, widen_input(up, x_dtype))
    if rms:
        u = rmsnorm(u, norm_weight, norm_eps)
    xr = fwht(u) if hadamard else u
    q, s, p = quantize_activations(xr, bits, eps)
    acc, y64 = forward_from_codes(q, s, t, alpha, bits)
    return {"y": y64.astype(np.float32), "y64": y64, "acc": acc, "q": q, "s": s, "p": p, "xr": xr,
            "u": u}


# ---------------------------------------------------------------------------
# Low-bit KV cache — [engine] module docstring item 5 (Section 3.1, Tables 2
# and 3) and BitNetV2Attention._quantize_kv_head: post-RoPE keys/values
# [B, H, S, D] quantized per token along the head dimension, the BOS token
# (s = 0) always with the 8-bit absmax quantizer.
# ---------------------------------------------------------------------------

# bits -> (scale constant c, clip lo, clip hi, statistic); the 3-bit branch is
# absmax with scale 3 and clip [-4, 3] (the page's own formula for it).
_KV = {8: (127.0, -128, 127, "absmax"), 4: (math.sqrt(7.0), -8, 7, "absmean"),
       3: (3.0, -4, 3, "absmax")}


def kv_code_params(bits: int, token: int):
    """(c, lo, hi, statistic) used for token index `token` of a head."""
    return _KV[8] if token == 0 else _KV[bits]


def kv_quantize(kv: np.ndarray, bits: int, eps: float = EPS):
    """Codes q, scales s (s = stat + eps, so x ~ q * s / c) and pre-round p of
    a [..., S, D] key or value tensor. Token 0 of every head uses the int8
    absmax quantizer, the others `bits` (3, 4 or 8)."""
    if bits not in _KV:
        raise ValueError("KV cache bits must be 3, 4 or 8")
    x = np.asarray(kv, dtype=np.float64)
    S = x.shape[-2]
    q = np.empty(x.shape, dtype=np.int8)
    s = np.empty(x.shape[:-1], dtype=np.float64)
    p = np.empty(x.shape, dtype=np.float64)
    for tok in range(S):
        c, lo, hi, stat = kv_code_params(bits, tok)
        row = x[..., tok, :]
        st = np.max(np.abs(row), axis=-1) if stat == "absmax" else np.mean(np.abs(row), axis=-1)
        st = st + eps
        pr = c * row / st[..., None]
        q[..., tok, :] = np.clip(np.rint(pr), lo, hi).astype(np.int8)
        s[..., tok] = st
        p[..., tok, :] = pr
    return q, s, p


def kv_dequantize(q: np.ndarray, s: np.ndarray, bits: int) -> np.ndarray:
    """x_hat = q * s / c with each token's own constant c."""
    q = np.asarray(q, dtype=np.float64)
    out = np.empty(q.shape, dtype=np.float64)
    for tok in range(q.shape[-2]):
        c = kv_code_params(bits, tok)[0]
        out[..., tok, :] = q[..., tok, :] * np.asarray(s)[..., tok, None] / c
    return out


# Packed storage of the low-bit KV codes. The engine page keeps the
# fake-quantized tensor; storing the b-bit codes b bits apiece is this
# library's layout, not the page's. Codes are b-bit two's complement
# ([-8, 7] at 4 bits, [-4, 3] at 3 bits), laid out as one little-endian bit
# stream per token row: code k of the row occupies bits b k .. b k + b - 1
# (bit i of the stream is bit i % 8 of byte i // 8). At 4 bits that is two
# codes per byte, code 2 i in the low nibble of byte i; at 3 bits, eight codes
# per three bytes.

def kv_pack(q: np.ndarray, bits: int) -> np.ndarray:
    """uint8 [R, D * bits / 8] packing of the codes q [R, D] (bits 3 or 4)."""
    if bits not in (3, 4):
        raise ValueError("packed KV codes are 3 or 4 bits wide")
    q = np.asarray(q, dtype=np.int64)
    R, D = q.shape
    if (D * bits) % 8:
        raise ValueError("a packed row must be a whole number of bytes")
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    if q.size and (q.min() < lo or q.max() > hi):
        raise ValueError(f"codes outside the {bits}-bit range")
    out = np.zeros((R, D * bits // 8), dtype=np.uint8)
    field = q & ((1 << bits) - 1)  # two's complement in b bits
    for k in range(D):
        for b in range(bits):
            pos = bits * k + b
            out[:, pos // 8] |= (((field[:, k] >> b) & 1) << (pos % 8)).astype(np.uint8)
    return out


def kv_unpack(packed: np.ndarray, bits: int, D: int) -> np.ndarray:
    """int8 codes [R, D] of a kv_pack'ed array (sign-extended from b bits)."""
    if bits not in (3, 4):
        raise ValueError("packed KV codes are 3 or 4 bits wide")
    packed = np.asarray(packed, dtype=np.int64)
    R = packed.shape[0]
    field = np.zeros((R, D), dtype=np.int64)
    for k in range(D):
        for b in range(bits):
            pos = bits * k + b
            field[:, k] |= ((packed[:, pos // 8] >> (pos % 8)) & 1) << b
    return np.where(field >= (1 << (bits - 1)), field - (1 << bits), field).astype(np.int8)


# ---------------------------------------------------------------------------
# Backward — [engine] Eq. 8 (HadamardTransformFunction: the gradient of the
# transform is the transform of the gradient, H being symmetric and
# orthonormal) and the straight-through estimators of WeightQuantTernarySTE,
# ActQuantINT8STE and ActQuantINT4STE, whose backward passes hand the
# incoming gradient through unchanged. HBitLinear.forward ends in
# F.linear(x_q, w_q) with x_q = (s / c) q and w_q = alpha t.
# ---------------------------------------------------------------------------

def backward(dy: np.ndarray, q: np.ndarray, s: np.ndarray, t: np.ndarray, alpha: float,
             bits: int, hadamard: int):
    """Gradients of the H-BitLinear forward under the engine page's STE rules.

    dy [M, N] is dL/dy; q [M, K], s [M] the per-token codes and scales the
    forward quantized with; t [N, K] the ternary weights and alpha their
    scale. Returns (dx [M, K], dw [N, K]), fp64:
      dL/dx_q = dy . w_q              F.linear's input gradient
      dL/dx_r = dL/dx_q               activation quantizer STE
      dx      = H dL/dx_r (hadamard)  Eq. 8; else dL/dx_r
      dL/dw_q = dy^T . x_q            F.linear's weight gradient
      dw      = dL/dw_q               ternarizer STE (latent weights)
    dx is the gradient with respect to the transform's input (the layer input
    after its RMSNorm)."""
    dy = np.asarray(dy, dtype=np.float64)
    c = _QUANT[bits][0]
    w_q = float(alpha) * np.asarray(t, dtype=np.float64)
    x_q = np.asarray(q, dtype=np.float64) * (np.asarray(s, dtype=np.float64)[:, None] / c)
    d_xr = dy @ w_q
    dx = fwht(d_xr) if hadamard else d_xr
    dw = dy.T @ x_q
    return dx, dw
