"""CPU oracle for absorbed MLA decode over a quantized latent KV cache.

This package is TEST INFRASTRUCTURE. Only the test suite, the package smoke
check and the CPU-baseline leg of the benchmark may import or run it. The
product path (the HIP library and its Python binding) never calls into it,
and it never calls into the product path: the two share no code.

It is written for a reader to check by eye against the pages it follows:

* "Absorbed MLA Cache Optimization on DeepSeek-V2-Lite" (technical report,
  English and Chinese versions): the cache stores the 512-d latent plus the
  64-d RoPE key per token and projects at compute time (section 2.1, the
  AbsorbedMLACache store/get sketch); per-channel INT8 in 32 blocks, k_pe INT8
  in 8 blocks, asymmetric INT4 in 32 blocks (section 3.2 / 4.2 tables);
  per-token byte and capacity arithmetic (sections 1.2, 2.2, 4.3).
* "DeepSeek的MLA技术" (juejin tutorial): K_i = C·W_i^upK, V_i = C·W_i^upV
  (MLA mechanism, step 2), per-head softmax(Q K^T / sqrt(d)) V (the
  MLAttention and MLAttentionWithCache code), the toy numeric example
  (angle 3), and the INT8 snippet (optimization 3, quantization).

Modules:
  quant       fp32-exact quantizers and fp64 dequantizers (parity is bit-exact
              on codes, scales and zero-points, so these fix the definition)
  attention   fp64 absorbed decode and the naive expanded decode it must equal
  accounting  per-token byte and capacity arithmetic
"""

from . import accounting, attention, quant  # noqa: F401
