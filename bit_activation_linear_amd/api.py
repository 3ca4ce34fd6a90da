"""Torch-facing binding of the H-BitLinear library.

PyTorch provides device memory and the current HIP stream; each function
checks dtype, device and contiguity, allocates outputs/workspace with torch,
and hands raw pointers to the C ABI. All arithmetic happens in the library's
HIP kernels.

Names follow the BitNet v2 engine page (Quillan-Ronin bitnet_v2_engine.py):
HBitLinear, quantize_weight_ternary (here: ternarize_weights, which also
packs), and the per-token activation quantizers of Eq. 5-6.
"""

from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib


def _stream_ptr(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _require(t: torch.Tensor, name: str, dtypes, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_out(t: torch.Tensor, name: str, dtype, shape, device) -> None:
    """A caller-supplied output: the C ABI only sees its address, so its
    dtype, shape, device and contiguity are checked here (a tensor that is too
    small or of the wrong type would be written past its end)."""
    _require(t, name, (dtype,), len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _check_workspace(ws: torch.Tensor, need: int, device) -> None:
    _require(ws, "workspace", (torch.uint8,), 1)
    if ws.device != device:
        raise ValueError(f"workspace must be on {device}, got {ws.device}")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {need} are required")


def _same_device(device, **tensors) -> None:
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} must be on {device}, got {t.device}")


def _x_dtype(x: torch.Tensor) -> int:
    return _lib.BF16 if x.dtype == torch.bfloat16 else _lib.F32


def ternarize_weights(W: torch.Tensor, out: Optional[torch.Tensor] = None,
                      alpha: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Absmean-ternarize fp32 W [N, K] and pack it (block-64, 2 bits per weight).

    Returns (Wpacked uint8 [N, K/4], alpha fp32 [1] on the device)."""
    _require(W, "W", (torch.float32,), 2)
    N, K = W.shape
    if out is None:
        out = torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
    _check_out(out, "out", torch.uint8, (N, K // 4), W.device)
    if alpha is None:
        alpha = torch.empty((1,), dtype=torch.float32, device=W.device)
    _check_out(alpha, "alpha", torch.float32, (1,), W.device)
    ws_bytes = _lib.load().bitnet_ternarize_workspace_bytes(N, K)
    if workspace is None:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=W.device)
    _check_workspace(workspace, ws_bytes, W.device)
    _lib.call("bitnet_ternarize_weights", W.data_ptr(), N, K, out.data_ptr(), alpha.data_ptr(),
              workspace.data_ptr(), workspace.numel(), _stream_ptr(W))
    return out, alpha


def pack_2bit(T: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Pack ternary int8 T [N, K] into the block-64 2-bit layout."""
    _require(T, "T", (torch.int8,), 2)
    N, K = T.shape
    if out is None:
        out = torch.empty((N, K // 4), dtype=torch.uint8, device=T.device)
    _check_out(out, "out", torch.uint8, (N, K // 4), T.device)
    _lib.call("bitnet_pack_2bit", T.data_ptr(), N, K, out.data_ptr(), _stream_ptr(T))
    return out


def tl2_bytes(N: int, K: int) -> int:
    """Bytes of the TL2 (1.67 bits per weight) encoding of [N, K] weights."""
    return int(_lib.load().bitnet_tl2_bytes(N, K))


def pack_tl2(Wpacked: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """TL2 encoding uint8 [N, tl2_bytes(N, K) / N] of 2-bit packed weights [N, K/4]."""
    _require(Wpacked, "Wpacked", (torch.uint8,), 2)
    N, K = Wpacked.shape[0], Wpacked.shape[1] * 4
    nbytes = tl2_bytes(N, K)
    if out is None:
        out = torch.empty((N, nbytes // max(N, 1)), dtype=torch.uint8, device=Wpacked.device)
    _check_out(out, "out", torch.uint8, (N, nbytes // max(N, 1)), Wpacked.device)
    _lib.call("bitnet_pack_tl2", Wpacked.data_ptr(), N, K, out.data_ptr(), _stream_ptr(Wpacked))
    return out


def tl2_forward_workspace_bytes(M: int, K: int) -> int:
    return int(_lib.load().bitnet_tl2_forward_workspace_bytes(M, K))


def hbitlinear_forward_tl2(x: torch.Tensor, Wtl2: torch.Tensor, alpha: torch.Tensor, bits: int,
                           out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y fp32 [M, N] (M <= 16): the forward (no transform) on TL2 weights."""
    _require(x, "x", (torch.float32, torch.bfloat16), 2)
    _require(Wtl2, "Wtl2", (torch.uint8,), 2)
    _require(alpha, "alpha", (torch.float32,), 1)
    M, K = x.shape
    N = Wtl2.shape[0]
    if Wtl2.numel() != tl2_bytes(N, K):
        raise ValueError("Wtl2 does not hold the TL2 encoding of [N, K] weights")
    _same_device(x.device, Wtl2=Wtl2, alpha=alpha)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check_out(out, "out", torch.float32, (M, N), x.device)
    need = tl2_forward_workspace_bytes(M, K)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
    if workspace is not None:
        _check_workspace(workspace, need, x.device)
    ws_ptr, ws_len = (workspace.data_ptr(), workspace.numel()) if workspace is not None else (None, 0)
    _lib.call("bitnet_hbitlinear_forward_tl2_batched", x.data_ptr(), _x_dtype(x), M, K,
              Wtl2.data_ptr(), N, alpha.data_ptr(), int(bits), out.data_ptr(), ws_ptr, ws_len,
              _stream_ptr(x))
    return out


def forward_workspace_bytes(M: int, K: int, N: int, bits: int, hadamard: int) -> int:
    return int(_lib.load().bitnet_forward_workspace_bytes(M, K, N, bits, int(hadamard)))


def hbitlinear_forward(x: torch.Tensor, Wpacked: torch.Tensor, alpha: torch.Tensor, bits: int,
                       hadamard: int, out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y fp32 [M, N] = H-BitLinear forward of x [M, K] (fp32 or bf16)."""
    _require(x, "x", (torch.float32, torch.bfloat16), 2)
    _require(Wpacked, "Wpacked", (torch.uint8,), 2)
    _require(alpha, "alpha", (torch.float32,), 1)
    M, K = x.shape
    N = Wpacked.shape[0]
    if Wpacked.shape[1] * 4 != K:
        raise ValueError(f"Wpacked has {Wpacked.shape[1]} bytes per row, expected K/4 = {K // 4}")
    _same_device(x.device, Wpacked=Wpacked, alpha=alpha)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check_out(out, "out", torch.float32, (M, N), x.device)
    need = forward_workspace_bytes(M, K, N, bits, hadamard)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
    if workspace is not None:
        _check_workspace(workspace, need, x.device)
    ws_ptr, ws_len = (workspace.data_ptr(), workspace.numel()) if workspace is not None else (None, 0)
    _lib.call("bitnet_hbitlinear_forward", x.data_ptr(), _x_dtype(x), M, K, Wpacked.data_ptr(), N,
              alpha.data_ptr(), int(bits), int(hadamard), out.data_ptr(), ws_ptr, ws_len,
              _stream_ptr(x))
    return out


def hbitlinear_forward_stages(x: torch.Tensor, Wpacked: torch.Tensor, alpha: torch.Tensor,
                              bits: int, hadamard: int, stages: int, out: torch.Tensor,
                              workspace: torch.Tensor) -> torch.Tensor:
    """One stage of the forward on its own kernels and workspace format:
    stages = 1 writes the transform + quantization stage's results into
    `workspace`, 2 reads them and writes `out`, 3 is the whole forward."""
    _require(x, "x", (torch.float32, torch.bfloat16), 2)
    _require(Wpacked, "Wpacked", (torch.uint8,), 2)
    _require(alpha, "alpha", (torch.float32,), 1)
    M, K = x.shape
    N = Wpacked.shape[0]
    if Wpacked.shape[1] * 4 != K:
        raise ValueError(f"Wpacked has {Wpacked.shape[1]} bytes per row, expected K/4 = {K // 4}")
    _same_device(x.device, Wpacked=Wpacked, alpha=alpha)
    _check_out(out, "out", torch.float32, (M, N), x.device)
    need = forward_workspace_bytes(M, K, N, bits, hadamard)
    _check_workspace(workspace, need, x.device)
    _lib.call("bitnet_hbitlinear_forward_stages", x.data_ptr(), _x_dtype(x), M, K,
              Wpacked.data_ptr(), N, alpha.data_ptr(), int(bits), int(hadamard), out.data_ptr(),
              workspace.data_ptr(), workspace.numel(), int(stages), _stream_ptr(x))
    return out


def hbitlinear_forward_noalloc(x: torch.Tensor, Wpacked: torch.Tensor, alpha: torch.Tensor,
                               bits: int, hadamard: int, out: torch.Tensor) -> torch.Tensor:
    """The forward into the caller's `out` (fp32 [M, N]) with the library's
    fixed device scratch as its workspace: the library allocates nothing.
    Calls that overlap in time on one GPU race on that scratch."""
    _require(x, "x", (torch.float32, torch.bfloat16), 2)
    _require(Wpacked, "Wpacked", (torch.uint8,), 2)
    _require(alpha, "alpha", (torch.float32,), 1)
    M, K = x.shape
    N = Wpacked.shape[0]
    if Wpacked.shape[1] * 4 != K:
        raise ValueError(f"Wpacked has {Wpacked.shape[1]} bytes per row, expected K/4 = {K // 4}")
    _same_device(x.device, Wpacked=Wpacked, alpha=alpha)
    _check_out(out, "out", torch.float32, (M, N), x.device)
    _lib.call("bitnet_hbitlinear_forward_noalloc", x.data_ptr(), _x_dtype(x), M, K,
              Wpacked.data_ptr(), N, alpha.data_ptr(), int(bits), int(hadamard), out.data_ptr(),
              _stream_ptr(x))
    return out


def stream_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Plain read of every byte of `buf` (contiguous, numel * itemsize a
    multiple of 16) with no arithmetic: the streaming-read ceiling that the
    forward's weight stream is measured against. `sink`: int32 [1]."""
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous tensor on a HIP device")
    _check_out(sink, "sink", torch.int32, (1,), buf.device)
    _lib.call("bitnet_stream_read", buf.data_ptr(), buf.numel() * buf.element_size(),
              sink.data_ptr(), _stream_ptr(buf))


def quantize_activations(x: torch.Tensor, bits: int, hadamard: int,
                         codes: Optional[torch.Tensor] = None,
                         scales: Optional[torch.Tensor] = None,
                         rowsum: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(codes int8 [M, K], scales fp32 [M]) of the transform + quantization
    stage; `rowsum` (int32 [M]), when given, receives each token's code sum."""
    _require(x, "x", (torch.float32, torch.bfloat16), 2)
    M, K = x.shape
    if codes is None:
        codes = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check_out(codes, "codes", torch.int8, (M, K), x.device)
    _check_out(scales, "scales", torch.float32, (M,), x.device)
    if rowsum is not None:
        _check_out(rowsum, "rowsum", torch.int32, (M,), x.device)
    _lib.call("bitnet_quantize_activations", x.data_ptr(), _x_dtype(x), M, K, int(bits),
              int(hadamard), codes.data_ptr(), scales.data_ptr(),
              rowsum.data_ptr() if rowsum is not None else None, _stream_ptr(x))
    return codes, scales


def _prologue_args(x: torch.Tensor, up: Optional[torch.Tensor], rmsnorm: bool,
                   norm_weight: Optional[torch.Tensor]):
    if up is not None:
        _check_out(up, "up", x.dtype, tuple(x.shape), x.device)
    if norm_weight is not None:
        _check_out(norm_weight, "norm_weight", torch.float32, (x.shape[1],), x.device)
    return (up.data_ptr() if up is not None else None, int(bool(rmsnorm)),
            norm_weight.data_ptr() if (rmsnorm and norm_weight is not None) else None)


def forward_prologue_workspace_bytes(M: int, K: int, N: int, bits: int, hadamard: int) -> int:
    return int(_lib.load().bitnet_forward_prologue_workspace_bytes(M, K, N, bits, int(hadamard)))


def hbitlinear_forward_prologue(x: torch.Tensor, Wpacked: torch.Tensor, alpha: torch.Tensor,
                                bits: int, hadamard: int, up: Optional[torch.Tensor] = None,
                                rmsnorm: bool = True, norm_weight: Optional[torch.Tensor] = None,
                                norm_eps: float = 1e-7, out: Optional[torch.Tensor] = None,
                                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The engine page's whole HBitLinear.forward: y = H-BitLinear of
    RMSNorm(u) (when rmsnorm), with u = silu(x) * up when `up` is given (the
    FFN's down projection: x is the gate projection) and u = x otherwise."""
    _require(x, "x", (torch.float32, torch.bfloat16), 2)
    _require(Wpacked, "Wpacked", (torch.uint8,), 2)
    _require(alpha, "alpha", (torch.float32,), 1)
    M, K = x.shape
    N = Wpacked.shape[0]
    if Wpacked.shape[1] * 4 != K:
        raise ValueError(f"Wpacked has {Wpacked.shape[1]} bytes per row, expected K/4 = {K // 4}")
    up_ptr, rms, g_ptr = _prologue_args(x, up, rmsnorm, norm_weight)
    _same_device(x.device, Wpacked=Wpacked, alpha=alpha)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check_out(out, "out", torch.float32, (M, N), x.device)
    need = forward_prologue_workspace_bytes(M, K, N, bits, hadamard)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    _check_workspace(workspace, need, x.device)
    _lib.call("bitnet_hbitlinear_forward_prologue", x.data_ptr(), up_ptr, _x_dtype(x), M, K, rms,
              g_ptr, float(norm_eps), Wpacked.data_ptr(), N, alpha.data_ptr(), int(bits),
              int(hadamard), out.data_ptr(), workspace.data_ptr(), workspace.numel(),
              _stream_ptr(x))
    return out


def quantize_activations_prologue(x: torch.Tensor, bits: int, hadamard: int,
                                  up: Optional[torch.Tensor] = None, rmsnorm: bool = True,
                                  norm_weight: Optional[torch.Tensor] = None,
                                  norm_eps: float = 1e-7) -> Tuple[torch.Tensor, torch.Tensor]:
    """(codes, scales) of the prologue + transform + quantization stage."""
    _require(x, "x", (torch.float32, torch.bfloat16), 2)
    M, K = x.shape
    up_ptr, rms, g_ptr = _prologue_args(x, up, rmsnorm, norm_weight)
    codes = torch.empty((M, K), dtype=torch.int8, device=x.device)
    scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    _lib.call("bitnet_quantize_activations_prologue", x.data_ptr(), up_ptr, _x_dtype(x), M, K, rms,
              g_ptr, float(norm_eps), int(bits), int(hadamard), codes.data_ptr(),
              scales.data_ptr(), _stream_ptr(x))
    return codes, scales


def kv_quantize(kv: torch.Tensor, bits: int, codes: Optional[torch.Tensor] = None,
                scales: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Low-bit KV cache (engine page, BitNetV2Attention._quantize_kv_head):
    kv [B, H, S, D] (fp32 or bf16, contiguous) -> (codes int8 [B, H, S, D],
    scales fp32 [B, H, S]); token 0 of every head with the int8 absmax rule,
    the others with `bits` in {3, 4, 8}."""
    _require(kv, "kv", (torch.float32, torch.bfloat16), 4)
    B, H, S, D = kv.shape
    if codes is None:
        codes = torch.empty(kv.shape, dtype=torch.int8, device=kv.device)
    if scales is None:
        scales = torch.empty((B, H, S), dtype=torch.float32, device=kv.device)
    _check_out(codes, "codes", torch.int8, tuple(kv.shape), kv.device)
    _check_out(scales, "scales", torch.float32, (B, H, S), kv.device)
    _lib.call("bitnet_kv_quantize", kv.data_ptr(), _x_dtype(kv), B * H * S, D, S, int(bits),
              codes.data_ptr(), scales.data_ptr(), _stream_ptr(kv))
    return codes, scales


def kv_quantize_packed(kv: torch.Tensor, bits: int, packed: Optional[torch.Tensor] = None,
                       bos_codes: Optional[torch.Tensor] = None,
                       scales: Optional[torch.Tensor] = None
                       ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """kv_quantize with the 3- or 4-bit codes stored `bits` bits apiece:
    kv [B, H, S, D] -> (packed uint8 [B, H, S, D * bits / 8], one little-endian
    bit stream per token with the BOS rows zero; bos_codes int8 [B, H, D],
    the BOS tokens' int8 codes; scales fp32 [B, H, S])."""
    _require(kv, "kv", (torch.float32, torch.bfloat16), 4)
    B, H, S, D = kv.shape
    if bits not in (3, 4) or (D * bits) % 8:
        raise ValueError("packed KV codes are 3 or 4 bits wide and fill whole bytes")
    row = D * bits // 8
    if packed is None:
        packed = torch.empty((B, H, S, row), dtype=torch.uint8, device=kv.device)
    if bos_codes is None:
        bos_codes = torch.empty((B, H, D), dtype=torch.int8, device=kv.device)
    if scales is None:
        scales = torch.empty((B, H, S), dtype=torch.float32, device=kv.device)
    _check_out(packed, "packed", torch.uint8, (B, H, S, row), kv.device)
    _check_out(bos_codes, "bos_codes", torch.int8, (B, H, D), kv.device)
    _check_out(scales, "scales", torch.float32, (B, H, S), kv.device)
    _lib.call("bitnet_kv_quantize_packed", kv.data_ptr(), _x_dtype(kv), B * H * S, D, S,
              int(bits), packed.data_ptr(), bos_codes.data_ptr(), scales.data_ptr(),
              _stream_ptr(kv))
    return packed, bos_codes, scales


def backward_workspace_bytes(M: int, K: int, N: int, dy_dtype: torch.dtype, want_dx: bool = True,
                             want_dw: bool = True) -> int:
    code = _lib.BF16 if dy_dtype == torch.bfloat16 else _lib.F32
    return int(_lib.load().bitnet_backward_workspace_bytes(M, K, N, code, int(want_dx),
                                                           int(want_dw)))


def hbitlinear_backward(dy: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                        Wpacked: torch.Tensor, alpha: torch.Tensor, bits: int, hadamard: int,
                        want_dx: bool = True, want_dw: bool = True,
                        dx: Optional[torch.Tensor] = None, dw: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None):
    """Gradients of the H-BitLinear forward (engine page Eq. 8 and the STE
    quantizer gradients): dx fp32 [M, K] with respect to the transform's input
    and dw fp32 [N, K] of the latent weights, from dy [M, N] (bf16 or fp32)
    and the forward's codes / scales (bitnet quantize_activations). Returns
    (dx or None, dw or None)."""
    _require(dy, "dy", (torch.float32, torch.bfloat16), 2)
    _require(codes, "codes", (torch.int8,), 2)
    _require(scales, "scales", (torch.float32,), 1)
    _require(Wpacked, "Wpacked", (torch.uint8,), 2)
    _require(alpha, "alpha", (torch.float32,), 1)
    M, N = dy.shape
    K = codes.shape[1]
    if codes.shape[0] != M or scales.shape[0] != M:
        raise ValueError("codes and scales must have one row per row of dy")
    if Wpacked.shape[0] != N or Wpacked.shape[1] * 4 != K:
        raise ValueError(f"Wpacked must be [N, K/4] = [{N}, {K // 4}], got {tuple(Wpacked.shape)}")
    _same_device(dy.device, codes=codes, scales=scales, Wpacked=Wpacked, alpha=alpha)
    if want_dx and dx is None:
        dx = torch.empty((M, K), dtype=torch.float32, device=dy.device)
    if want_dw and dw is None:
        dw = torch.empty((N, K), dtype=torch.float32, device=dy.device)
    if want_dx:
        _check_out(dx, "dx", torch.float32, (M, K), dy.device)
    if want_dw:
        _check_out(dw, "dw", torch.float32, (N, K), dy.device)
    need = backward_workspace_bytes(M, K, N, dy.dtype, want_dx, want_dw)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dy.device)
    if workspace is not None:
        _check_workspace(workspace, need, dy.device)
    ws_ptr, ws_len = (workspace.data_ptr(), workspace.numel()) if workspace is not None else (None, 0)
    _lib.call("bitnet_hbitlinear_backward", dy.data_ptr(), _x_dtype(dy), M, N, codes.data_ptr(),
              scales.data_ptr(), K, Wpacked.data_ptr(), alpha.data_ptr(), int(bits), int(hadamard),
              dx.data_ptr() if want_dx else None, dw.data_ptr() if want_dw else None, ws_ptr,
              ws_len, _stream_ptr(dy))
    return (dx if want_dx else None), (dw if want_dw else None)


def ternary_gemm_i32(codes: torch.Tensor, Wpacked: torch.Tensor,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """acc int32 [M, N] = codes . t^T (exact)."""
    _require(codes, "codes", (torch.int8,), 2)
    _require(Wpacked, "Wpacked", (torch.uint8,), 2)
    M, K = codes.shape
    N = Wpacked.shape[0]
    if Wpacked.shape[1] * 4 != K:
        raise ValueError("Wpacked row length does not match K/4")
    _same_device(codes.device, Wpacked=Wpacked)
    if out is None:
        out = torch.empty((M, N), dtype=torch.int32, device=codes.device)
    _check_out(out, "out", torch.int32, (M, N), codes.device)
    _lib.call("bitnet_ternary_gemm_i32", codes.data_ptr(), M, K, Wpacked.data_ptr(), N,
              out.data_ptr(), _stream_ptr(codes))
    return out


def ternary_linear_dequant(codes: torch.Tensor, scales: torch.Tensor, Wpacked: torch.Tensor,
                           alpha: torch.Tensor, bits: int, out: Optional[torch.Tensor] = None,
                           rowsum: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y fp32 [M, N] = (codes . t^T) * alpha * scales / c. `rowsum`: the
    codes' per-token sums from quantize_activations, or None."""
    _require(codes, "codes", (torch.int8,), 2)
    _require(scales, "scales", (torch.float32,), 1)
    _require(Wpacked, "Wpacked", (torch.uint8,), 2)
    _require(alpha, "alpha", (torch.float32,), 1)
    M, K = codes.shape
    N = Wpacked.shape[0]
    if Wpacked.shape[1] * 4 != K:
        raise ValueError("Wpacked row length does not match K/4")
    if scales.shape[0] != M:
        raise ValueError("scales must have one entry per token")
    _same_device(codes.device, scales=scales, Wpacked=Wpacked, alpha=alpha)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=codes.device)
    _check_out(out, "out", torch.float32, (M, N), codes.device)
    if rowsum is not None:
        _check_out(rowsum, "rowsum", torch.int32, (M,), codes.device)
    _lib.call("bitnet_ternary_linear_dequant", codes.data_ptr(), scales.data_ptr(),
              rowsum.data_ptr() if rowsum is not None else None, M, K, Wpacked.data_ptr(), N,
              alpha.data_ptr(), int(bits), out.data_ptr(), _stream_ptr(codes))
    return out


class HBitLinear:
    """Prepared H-BitLinear layer: weights ternarized and packed once on the
    device, then forward(x) many times (the prepare-once / forward-many split
    of the bitnet.cpp simulation page's edge linear layer).

    With rmsnorm=True the engine page's whole HBitLinear.forward runs,
    RMSNorm (weight `norm_weight`, ones when None, and `norm_eps`) included;
    forward(x, up=...) then also takes the FFN's SwiGLU product silu(x) * up
    as the input. With rmsnorm=False (the default) x is taken to be the
    normalized input."""

    def __init__(self, weight: torch.Tensor, bits: int = 4, hadamard: bool = True,
                 rmsnorm: bool = False, norm_weight: Optional[torch.Tensor] = None,
                 norm_eps: float = 1e-7):
        if bits not in (4, 8):
            raise ValueError("bits must be 4 or 8")
        K = weight.shape[1]
        if hadamard and (K & (K - 1)) != 0:
            raise ValueError(f"H-BitLinear in_features ({K}) must be a power of 2")
        self.bits = bits
        self.hadamard = int(bool(hadamard))
        self.in_features = K
        self.out_features = weight.shape[0]
        self.Wpacked, self.alpha = ternarize_weights(weight.contiguous())
        self.rmsnorm = bool(rmsnorm)
        self.norm_weight = norm_weight
        self.norm_eps = float(norm_eps)
        self._ws = None

    def forward(self, x: torch.Tensor, up: Optional[torch.Tensor] = None) -> torch.Tensor:
        M = x.shape[0]
        if self.rmsnorm or up is not None:
            need = forward_prologue_workspace_bytes(M, self.in_features, self.out_features,
                                                    self.bits, self.hadamard)
            if self._ws is None or self._ws.numel() < need or self._ws.device != x.device:
                self._ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
            return hbitlinear_forward_prologue(x, self.Wpacked, self.alpha, self.bits,
                                               self.hadamard, up=up, rmsnorm=self.rmsnorm,
                                               norm_weight=self.norm_weight,
                                               norm_eps=self.norm_eps, workspace=self._ws)
        need = forward_workspace_bytes(M, self.in_features, self.out_features, self.bits,
                                       self.hadamard)
        if need > 0 and (self._ws is None or self._ws.numel() < need or self._ws.device != x.device):
            self._ws = torch.empty((need,), dtype=torch.uint8, device=x.device)
        return hbitlinear_forward(x, self.Wpacked, self.alpha, self.bits, self.hadamard,
                                  workspace=self._ws if need > 0 else None)

    __call__ = forward
