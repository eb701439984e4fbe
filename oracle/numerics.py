"""Decoding of 16-bit floating-point bit patterns into float64.

Test infrastructure only (see the package docstring).

The activations and the per-group scales of a W4A16 layer are fp16 or bf16
("params_dtype" of the scales in the vLLM note "Carga de capas cuantizadas",
section "Flujo de datos"; bf16 activations in the vllm-omni cpu_int4 commit).
The oracle keeps them as raw uint16 bit patterns and turns them into float64
by definition:
  * bf16 is the upper half of an IEEE-754 binary32 word, so the value is the
    binary32 word (bits << 16);
  * fp16 is IEEE-754 binary16, which NumPy's float16 implements.
"""

import numpy as np

FP16 = "fp16"
BF16 = "bf16"
DTYPES = (FP16, BF16)


def half_bits_to_f64(bits, dtype):
    """uint16 bit patterns -> float64 values (exact: both formats embed in float64)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == FP16:
        return bits.view(np.float16).astype(np.float64)
    raise ValueError(f"unknown 16-bit dtype {dtype!r}")


def f64_to_half_bits_rne(values, dtype):
    """float64 -> nearest 16-bit value, ties to even, returned as uint16 bits.

    Used by the tests to state the exactly-rounded output that a kernel must
    produce in the special cases where the GEMM result is exact. bf16 rounding is
    done from the float64 value itself (not via float32), by locating the two
    neighbouring bf16 values and picking the nearer one, even mantissa on a tie.
    """
    v = np.asarray(values, dtype=np.float64)
    if dtype == FP16:
        return v.astype(np.float16).view(np.uint16)
    if dtype != BF16:
        raise ValueError(f"unknown 16-bit dtype {dtype!r}")
    out = np.empty(v.shape, dtype=np.uint16)
    flat_v = v.reshape(-1)
    flat_o = out.reshape(-1)
    for idx, x in enumerate(flat_v):
        if x == 0.0:
            flat_o[idx] = 0x8000 if np.signbit(x) else 0
            continue
        # truncation toward zero in float32, then in bf16: a lower neighbour
        lo32 = np.float32(x)
        if abs(float(lo32)) > abs(x):
            lo32 = np.nextafter(lo32, np.float32(0.0))
        lo_bits = int(np.array(lo32).view(np.uint32)) >> 16
        lo = float(half_bits_to_f64(np.uint16(lo_bits), BF16))
        hi = float(half_bits_to_f64(np.uint16(lo_bits + 1), BF16))  # next magnitude up
        if abs(x - lo) < abs(hi - x):
            pick = lo_bits
        elif abs(x - lo) > abs(hi - x):
            pick = lo_bits + 1
        else:
            pick = lo_bits if (lo_bits & 1) == 0 else lo_bits + 1
        flat_o[idx] = pick
    return out
