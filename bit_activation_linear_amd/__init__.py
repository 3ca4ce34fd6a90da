"""H-BitLinear forward and backward (BitNet v2) on AMD MI355X.

The compute path is the HIP library libbitnet_mi355x.so (C ABI in
include/bitnet_mi355x.h); this package is its thin torch binding. Importing
the package does not load the library; the first call does, and fails loudly
if it has not been built.
"""

from .api import (  # noqa: F401
    HBitLinear,
    backward_workspace_bytes,
    forward_prologue_workspace_bytes,
    forward_workspace_bytes,
    hbitlinear_backward,
    hbitlinear_forward,
    hbitlinear_forward_noalloc,
    hbitlinear_forward_prologue,
    hbitlinear_forward_stages,
    hbitlinear_forward_tl2,
    kv_quantize,
    kv_quantize_packed,
    pack_2bit,
    pack_tl2,
    quantize_activations,
    quantize_activations_prologue,
    stream_read,
    ternarize_weights,
    ternary_gemm_i32,
    ternary_linear_dequant,
    tl2_bytes,
    tl2_forward_workspace_bytes,
)
from ._lib import BitNetError  # noqa: F401
