"""Seeded synthetic inputs for the H-BitLinear forward.

This module only draws random numbers and stores them in the input formats the
layer accepts (fp32, or bf16 bits with round-to-nearest-even). It holds none of
the method's arithmetic: no Hadamard transform, no quantizer, no packing. Both
the HIP path and the CPU oracle are fed from here, and nothing else is shared
between them.

Workload shapes follow the five H-BitLinear cases this library is measured on:
activations are N(0,1) rows (Student-t with 3 degrees of freedom for the
batched-decode case) with a few outlier channels scaled up, the same channels
for every token; latent weights are N(0, 0.02) in fp32, the init scale the
bitnet.cpp simulation page and the BitNet b1.58 blog page both use for
BitLinear weights.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str            # short name used by tests and the bench
    M: int              # tokens
    K: int              # in_features (the Hadamard/quantization axis)
    N: int              # out_features
    bits: int           # 4 or 8
    hadamard: int       # 1: online FWHT before quantization
    x_dtype: str        # "fp32" or "bf16"
    x_dist: str         # "normal" or "student_t3"
    n_out: int          # number of outlier channels
    factor: float       # multiplier applied to the outlier channels
    w_std: float = 0.02
    description: str = ""


# The five measured cases. Outlier counts are the stated fractions of K
# rounded to the nearest integer (1% of 2560 -> 26, 0.5% of 8192 -> 41,
# 1% of 4096 -> 41).
WORKLOADS = {
    "int4_hadamard_m4_k256_n256": Workload(
        "int4_hadamard_m4_k256_n256", 4, 256, 256, 4, 1, "fp32", "normal", 4, 50.0,
        description="single H-BitLinear, int4 + Hadamard, fp32 X, 4 of 256 channels x50"),
    "decode_int8_m1_k2560_n6912": Workload(
        "decode_int8_m1_k2560_n6912", 1, 2560, 6912, 8, 0, "bf16", "normal", 26, 30.0,
        description="decode GEMV, int8 absmax, no Hadamard, 1% channels x30"),
    "prefill_int4_hadamard_m2048_k8192_n2048": Workload(
        "prefill_int4_hadamard_m2048_k8192_n2048", 2048, 8192, 2048, 4, 1, "bf16", "normal", 41, 50.0,
        description="Wdown-style prefill, int4 absmean + Hadamard, 0.5% channels x50"),
    "decode_int4_hadamard_m16_k16384_n4096": Workload(
        "decode_int4_hadamard_m16_k16384_n4096", 16, 16384, 4096, 4, 1, "bf16", "student_t3", 0, 1.0,
        description="batched decode, int4 + Hadamard, Student-t(3) activations"),
    "prefill_int8_m8192_k4096_n14336": Workload(
        "prefill_int8_m8192_k4096_n14336", 8192, 4096, 14336, 8, 0, "bf16", "normal", 41, 20.0,
        description="large prefill, int8 absmax, no Hadamard, 1% channels x20, on-device ternarize+pack"),
}

WORKLOAD_ORDER = list(WORKLOADS)


def fp32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Store fp32 values as bf16 bit patterns, rounding to nearest even.

    Inputs are finite (the generators never produce NaN/Inf)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_fp32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (a format change only)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_activations(rng: np.random.Generator, M: int, K: int, dist: str, n_out: int,
                     factor: float, x_dtype: str) -> tuple[np.ndarray, np.ndarray]:
    """Draw X [M, K]; returns (x, outlier_channel_indices).

    x is float32, or uint16 bf16 bit patterns when x_dtype == "bf16"."""
    if dist == "normal":
        x = rng.standard_normal((M, K))
    elif dist == "student_t3":
        x = rng.standard_t(3, (M, K))
    else:
        raise ValueError(f"unknown activation distribution {dist!r}")
    idx = np.zeros(0, dtype=np.int64)
    if n_out > 0:
        idx = rng.choice(K, n_out, replace=False)
        x[:, idx] *= factor
    if x_dtype == "fp32":
        return np.ascontiguousarray(x.astype(np.float32)), idx
    if x_dtype == "bf16":
        return fp32_to_bf16_bits(x.astype(np.float32)), idx
    raise ValueError(f"unknown activation dtype {x_dtype!r}")


def make_weights(rng: np.random.Generator, N: int, K: int, std: float = 0.02) -> np.ndarray:
    """Latent fp32 weights [N, K] (out_features x in_features, K contiguous)."""
    w = rng.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(std)
    return w


def make_case(M: int, K: int, N: int, *, x_dtype: str = "bf16", dist: str = "normal",
              n_out: int = 0, factor: float = 1.0, w_std: float = 0.02,
              seed: int = 0) -> dict:
    """Draw order: X, then the outlier channels, then W (one PCG64 stream)."""
    rng = np.random.default_rng(seed)
    x, idx = make_activations(rng, M, K, dist, n_out, factor, x_dtype)
    w = make_weights(rng, N, K, w_std)
    return {"x": x, "x_dtype": x_dtype, "W": w, "outliers": idx}


def make_workload(key: str, seed: int = 0, M: Optional[int] = None) -> dict:
    """Inputs of one named workload. M overrides the token count (same recipe)."""
    wl = WORKLOADS[key]
    case = make_case(wl.M if M is None else M, wl.K, wl.N, x_dtype=wl.x_dtype, dist=wl.x_dist,
                     n_out=wl.n_out, factor=wl.factor, w_std=wl.w_std, seed=seed)
    case["workload"] = wl
    return case
