"""Dequantisation and the W4A16 product, written from their definitions.

Test infrastructure only (see the package docstring).

Definitions:
  * group of row k of the weight is g = k div G, groups contiguous along K
    (vLLM note "Carga de capas cuantizadas", "Flujo de datos": num_groups =
    input_size // group_size, scales and qzeros have one row per group);
    group_size = -1 means a single group of all K rows ("Límites y fallos");
  * dequant: W[k, n] = (Q[k, n] - Z[g, n]) * S[g, n] with integer codes Q, Z in
    0..15 and S the 16-bit scale (problem statement; asymmetric, group-wise per
    the vllm-omni cpu_int4 commit "Add cpu_int4 ...");
  * product: Y[m, n] = sum_k X[m, k] * W[k, n]  (y = x . dequant(W), X is [M, K]).

Everything is float64. Each W[k, n] is exact in float64 (|q - z| <= 15 times a
16-bit scale), each product X*W is exact, so the only rounding is in the sum
over K, done by NumPy's float64 matmul: relative error around 1e-16 * K.
"""

import numpy as np

from .numerics import half_bits_to_f64


def resolve_group_size(K, group_size):
    G = K if group_size == -1 else int(group_size)
    if G <= 0 or K % G != 0:
        raise ValueError(f"group_size {group_size} does not divide K={K}")
    return G


def dequant(Q, Z, S, group_size):
    """Q uint8 [K, N], Z uint8 [K/G, N], S float64 [K/G, N] -> W float64 [K, N]."""
    Q = np.asarray(Q)
    K, N = Q.shape
    G = resolve_group_size(K, group_size)
    if Z.shape != (K // G, N) or S.shape != (K // G, N):
        raise ValueError("zeros/scales must be [K/G, N]")
    group_of_row = np.arange(K) // G
    return (Q.astype(np.float64) - Z[group_of_row].astype(np.float64)) * S[group_of_row]


def gemm(X, W):
    """X float64 [M, K], W float64 [K, N] -> Y float64 [M, N] = X . W (unrounded)."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    if X.ndim != 2 or W.ndim != 2 or X.shape[1] != W.shape[0]:
        raise ValueError("shape mismatch")
    return X @ W


def w4a16_reference(x_bits, qweight, qzeros, scale_bits, dtype, group_size, bias_bits=None):
    """The whole layer from the checkpoint tensors: AWQ words in, float64 Y out.

    x_bits [M, K] and scale_bits [K/G, N] (and bias_bits [N] if given) are uint16
    bit patterns of `dtype`; qweight / qzeros are the AWQ int32 tensors.
    A bias, when present, is added to the exact product (before any rounding).
    """
    from .awq import unpack_awq
    Q = unpack_awq(qweight)
    Z = unpack_awq(qzeros)
    S = half_bits_to_f64(scale_bits, dtype)
    X = half_bits_to_f64(x_bits, dtype)
    Y = gemm(X, dequant(Q, Z, S, group_size))
    if bias_bits is not None:
        Y = Y + half_bits_to_f64(bias_bits, dtype)[None, :]
    return Y


def max_rel_error(y_test, y_ref):
    """max |y_test - y_ref| / max |y_ref| over the whole output tensor."""
    y_test = np.asarray(y_test, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    denom = np.max(np.abs(y_ref)) if y_ref.size else 0.0
    num = np.max(np.abs(y_test - y_ref)) if y_ref.size else 0.0
    if denom == 0.0:
        return 0.0 if num == 0.0 else np.inf
    return num / denom


TOLERANCE = 1e-2   # max |y_gpu - y_ref| <= 1e-2 * max |y_ref|, per output tensor


def within_tolerance(y_test, y_ref, tol=TOLERANCE):
    return max_rel_error(y_test, y_ref) <= tol
