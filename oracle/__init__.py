"""CPU oracle for the int4 group-quantized MoE SwitchGLU layer — TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the HIP path is checked
against.  Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
it; the product path (the C-ABI library and its Python binding) never does, and the two
share no code: no kernels, headers, helpers, tables or constant generators.  The only
thing both sides use is the seeded input generator module ``synth``, which holds no
arithmetic of the method.

Precision policy
----------------
* Matmuls, LoRA deltas, activations and routing weights are evaluated in float64 from the
  exact dequantized weights (``scale * q + bias`` is exact in float64 for fp16 scale/bias
  and integer codes, and for bf16 ones checked per matrix), so the oracle is the definition
  of the layer up to float64 rounding; integer dot products are exact (int64).
* Where a floating-point value *decides an integer* (a quantized code, a scale that later
  decides codes), the oracle takes that decision in float32, the precision of the kernel,
  with every operation spelled out in IEEE float32 (numpy float32 arrays, no contraction).
* Outputs that the method stores in fp16 are rounded once, round-to-nearest-even.

Modules
-------
``affine``      group-wise affine quantize / pack / unpack / dequantize (4- and 8-bit; group
                64 or 32; fp16 or bf16 scale and bias).
``moe``         quantized linear, LoRA delta, router + top-K, experts, shared expert, layer,
                layer stack.
``supergroup``  mixed ternary / 4-bit super-group quantizer, packing, the weight-only GEMM
                and the 8-bit-activation integer path.
``prerouter``   the prerouter head's forward (the next layer's predicted routing).

Every function here is pinned by a CPU test that does not take its expected value from the
function itself (closed forms, hand-worked values, exact integer arithmetic, brute force,
library routines, or the same function written another way).  The pages print no worked
value of a whole layer, so the layer's composition is pinned through its parts: the shared
expert and its gate by hand-worked constant-matrix examples and torch modules with the
adapters merged in (``tests/test_oracle_shared_expert.py``), the routed part by the dense
SwiGLU, identical-expert and per-pair recomputation identities.
"""
from . import affine, moe, prerouter, supergroup  # noqa: F401
