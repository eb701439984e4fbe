"""CPU oracle for group-wise asymmetric W4A16 (int4 weight, 16-bit activation) GEMM
and for the one-time repack of AWQ-packed weights into the GPU tile layout.

This package is TEST INFRASTRUCTURE, not product code. Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it. The HIP library
never calls it, and it shares no code, header, table or helper with the HIP
library: everything here is written from the method's definition.

Everything is plain NumPy. Floating-point work is done in float64, where every
step of the method is exact except the final sum over K.

Sources (pages, by title and section):
  * "Carga de capas cuantizadas: AWQ / GPTQ / Marlin / fp8" (vLLM architecture
    note), section "Flujo de datos": shapes of qweight int32 [K, N/8], qzeros
    int32 [K/G, N/8] and scales [K/G, N], packed along the output dimension with
    pack factor 8; section "Motivación de diseño": AWQ's order of the codes in a
    word is not the ascending one, so vLLM reorders them once after loading;
    section "Límites y fallos": group_size = -1 means one group spanning all of K.
  * vllm-omni commit "Add cpu_int4, an asymmetric 4-bit weight path for vLLM's
    CPU backend": the method is asymmetric, group-wise, 4-bit weights with
    16-bit activations.
  * The statement of the problem this library implements: dequant(w) = (q - z) * s
    per 128-element K-group, AWQ nibble slots holding columns in the interleaved
    order 0,2,4,6,1,3,5,7.

Modules:
  numerics     16-bit float bit patterns -> float64 (definitions of fp16 / bf16)
  awq          pack_awq / unpack_awq: the AWQ int32 nibble packing
  gptq         GPTQ-standard packing: codes along K, zero points along N, standard order
  tile_layout  repack / decode: the GPU tile layout, written from its spec
  gemm         dequant / gemm / tolerance check
  embedding    tied-embedding gather: dequantised columns of the head weight
  w4a8         fp8 (E4M3) activations: the format, per-row quantisation, the
               activation operand order, the W4A8 product
"""

from . import numerics, awq, gptq, tile_layout, gemm, embedding, w4a8  # noqa: F401
