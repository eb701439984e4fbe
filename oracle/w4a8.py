"""W4A8: the int4 weights of the W4A16 layer with fp8 (E4M3) activations, written
from the definitions.

Test infrastructure only (see the package docstring).

Sources:
  * vLLM note "Carga de capas cuantizadas: AWQ / GPTQ / Marlin / fp8", section
    "Límites y fallos": when the activation type of the int4 Marlin kernel is
    float8_e4m3fn, the weights get a one-time fp8 pre-processing after loading and
    the scales are multiplied by 512.
  * vllm-omni commit "Add cpu_int4, an asymmetric 4-bit weight path for vLLM's CPU
    backend": a W4A8 path (4-bit weights, 8-bit activations) is named beside the
    W4A16 one as the adjacent variant.
  * The E4M3 format itself (OCP 8-bit floating point specification, "fn" variant):
    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
    S.1111.111 is NaN, the largest finite value is 448 (0x7E), exponent field 0
    gives the subnormals m * 2^-9.

Readings (the pages name the activation type and the factor 512, nothing more):
  * activations are quantised dynamically, one scale per row (token): the row's
    scale is a = max_k |x[m, k]| / 448 in float32, its codes e = RNE_e4m3(x / a)
    with the quotient taken in float32; a row of zeros takes a = 1 (all codes 0);
  * the product is y[m, n] = a[m] * sum_k dec(e[m, k]) * (q[k, n] - z[g, n]) * s[g, n]
    (+ bias), exact in float64 up to the sum over K, rounded once to the output
    dtype by the kernel;
  * the factor 512: a 4-bit code q placed in the low nibble of an E4M3 byte reads
    as q * 2^-9 exactly (exponent field 0 or 1, mantissa the low 3 bits), so a
    product formed on such bytes carries 2^-9, which 512 = 2^9 undoes.

The operand order of the quantised activations (`operand_order`) is the layout the
GPU kernels read; it is defined here from its written statement, not shared.
"""

import numpy as np

from .gemm import dequant
from .numerics import half_bits_to_f64

E4M3_MAX = 448.0
ROWS_PER_BLOCK = 128
# Operand order inside each 128-element block of a row: byte 32 h + 8 i + j holds
# element 32 i + 8 h + ROW_OF_BYTE[j] (lane group h, 32-row step i, byte j).
ROW_OF_BYTE = (0, 4, 1, 5, 2, 6, 3, 7)


def e4m3_decode(codes):
    """uint8 E4M3 codes -> float64 values (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode_rne(values):
    """float64 values -> nearest E4M3 code, ties to even mantissa.

    Values of magnitude 464 or more (past the midpoint between 448 and the next
    binade) and NaN are outside what the quantiser produces and raise ValueError.
    """
    v = np.asarray(values, dtype=np.float64)
    if np.any(~np.isfinite(v)) or np.any(np.abs(v) >= 464.0):
        raise ValueError("value outside the E4M3 range")
    sign = np.where(np.signbit(v), 0x80, 0)
    a = np.abs(v)
    # subnormal range: multiples of 2^-9 (a result of 8 is the smallest normal, code 8)
    sub_code = np.rint(a * 512.0)
    # normal range: a = sig * 2^E, sig in [1, 2); 3 mantissa bits, RNE
    frac, exp = np.frexp(np.where(a > 0, a, 1.0))     # a = frac * 2^exp, frac in [0.5, 1)
    E = exp - 1
    mant = np.rint((2.0 * frac - 1.0) * 8.0)
    carry = mant == 8.0
    E = np.where(carry, E + 1, E)
    mant = np.where(carry, 0.0, mant)
    norm_code = ((E + 7) << 3) | mant.astype(np.int64)
    code = np.where(a < 2.0 ** -6, sub_code.astype(np.int64), norm_code)
    return (code | sign).astype(np.uint8)


def quantize_rows(x_bits, dtype):
    """16-bit activations [M, K] -> (codes uint8 [M, K] in element order, scale float32 [M])."""
    X = half_bits_to_f64(x_bits, dtype).astype(np.float32)     # exact
    amax = np.max(np.abs(X), axis=1) if X.shape[1] else np.zeros(X.shape[0], np.float32)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    quotient = (X / scale[:, None]).astype(np.float32)          # float32, correctly rounded
    return e4m3_encode_rne(quotient.astype(np.float64)), scale


def block_sums(codes):
    """sum of the decoded codes over each 128-element block of a row: float64 [M, K/128]."""
    M, K = codes.shape
    return e4m3_decode(codes).reshape(M, K // ROWS_PER_BLOCK, ROWS_PER_BLOCK).sum(axis=2)


def operand_order(codes):
    """Element-order codes [M, K] -> operand-order bytes [M, K] (see ROW_OF_BYTE)."""
    M, K = codes.shape
    src = codes.reshape(M, K // ROWS_PER_BLOCK, 4, 4, 8)        # [m, kb, i, h, row e]
    src = src[:, :, :, :, list(ROW_OF_BYTE)]                    # byte j <- row ROW_OF_BYTE[j]
    return np.ascontiguousarray(src.transpose(0, 1, 3, 2, 4)).reshape(M, K)   # [m, kb, h, i, j]


def element_order(ops):
    """Inverse of operand_order."""
    M, K = ops.shape
    src = ops.reshape(M, K // ROWS_PER_BLOCK, 4, 4, 8).transpose(0, 1, 3, 2, 4)   # [m, kb, i, h, j]
    out = np.empty_like(src)
    out[:, :, :, :, list(ROW_OF_BYTE)] = src
    return np.ascontiguousarray(out).reshape(M, K)


def w4a8_reference(codes, scale, Q, Z, scale_bits, dtype, group_size, bias_bits=None):
    """codes uint8 [M, K] (element order), scale [M]; Q [K, N], Z [K/G, N] codes,
    scale_bits [K/G, N] -> y float64 [M, N] (unrounded)."""
    A = e4m3_decode(codes)
    W = dequant(Q, Z, half_bits_to_f64(scale_bits, dtype), group_size)
    Y = np.asarray(scale, dtype=np.float64)[:, None] * (A @ W)
    if bias_bits is not None:
        Y = Y + half_bits_to_f64(bias_bits, dtype)[None, :]
    return Y


def w4a8_layer(x_bits, qweight, qzeros, scale_bits, dtype, group_size, bias_bits=None):
    """The whole W4A8 layer from 16-bit activations and the AWQ checkpoint tensors."""
    from .awq import unpack_awq
    codes, scale = quantize_rows(x_bits, dtype)
    return w4a8_reference(codes, scale, unpack_awq(qweight), unpack_awq(qzeros), scale_bits, dtype,
                          group_size, bias_bits)
