"""CPU oracle for the H-BitLinear forward and backward passes — TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 NumPy restatement of what the method computes, written
from the pages (see the citations on each function). It is the yardstick the
HIP path is checked against and is not part of the product: only the test
suite, the smoke check and the bench's CPU-baseline leg may import it. It
shares no code with the HIP library and imports nothing from it.

Pins (tests/test_oracle_pins.py) tie every function to something other than
itself: the closed-form/Sylvester Hadamard matrix and scipy.linalg.hadamard,
orthogonality, hand-derived worked values under tests/golden/, brute-force
integer products and the fake-quant route of the BitNet v2 engine page.

Parity status per function (mirrors the design notes):
  fwht                 pinned (closed form, scipy.linalg.hadamard, H*H=I)
  absmean_alpha        pinned (hand values, closed-form statistics)
  ternarize            pinned (hand values, sign special cases)
  pack_2bit/unpack     pinned (hand-built bytes, round trip); the byte layout
                       itself is a contract of this library, not of the pages
  quantize_activations pinned (hand values, torch per-channel quantizer)
  ternary_matmul_i64   pinned (int64 brute force)
  dequantize / forward pinned (fake-quant route of the engine page)
  silu / swiglu        pinned (closed-form special values, torch.nn.functional.silu)
  rmsnorm              pinned (torch.nn.RMSNorm, unit mean square, scale invariance)
  forward_prologue     pinned (reduces to forward; torch module chain on small shapes)
  kv_quantize          pinned (hand values per branch, reduction to the pinned
                       activation quantizers, 3-bit range and error bounds)
  kv_pack / kv_unpack  pinned (hand-built bytes at 3 and 4 bits, round trips,
                       numpy's own bit packing of the same stream); the bit
                       layout is a contract of this library, not of the pages
  backward             pinned (torch autograd through the STE forward, adjoint
                       identities, Eq. 8 via H*H = I, hand values, brute force)
  tl2 (module)         pinned (tests/test_oracle_tl2.py: the mirror table against
                       all 27 states, the index's closed form, round trips, hand
                       built bytes, 5/3 bits per weight)
"""

from .hbitlinear import (  # noqa: F401
    EPS,
    INT4_SCALE,
    INT8_SCALE,
    absmean_alpha,
    backward,
    dequantize,
    forward,
    forward_from_codes,
    forward_prologue,
    fwht,
    fwht_dense,
    hadamard_matrix,
    kv_code_params,
    kv_dequantize,
    kv_pack,
    kv_quantize,
    kv_unpack,
    pack_2bit,
    quant_boundary_distance,
    quantize_activations,
    rmsnorm,
    silu,
    swiglu,
    ternarize,
    ternary_matmul_i64,
    unpack_2bit,
    widen_input,
)

from . import tl2  # noqa: F401,E402
