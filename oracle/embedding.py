"""Tied-embedding gather, written from its definition.

Test infrastructure only (see the package docstring).

A model whose input embedding is tied to its output head stores one quantised
matrix for both: the vllm-omni commit "cpu_int4: repack weights in n-blocks, to
bound the load-time peak" lists the 131072 x 2048 embedding as the same matrix as
the output head, and the commit "Add cpu_int4, an asymmetric 4-bit weight path for vLLM's CPU
backend" checks the quantised tied embedding. Stored as the head, W [K, N] with
K hidden and N the vocabulary (y = x . W), the embedding of token t is column t of
dequant(W), one row of K values:

  E[i, k] = (Q[k, t_i] - Z[k div G, t_i]) * S[k div G, t_i]

exact in float64, then rounded once to the 16-bit dtype (nearest, ties to even).
Reading taken where the pages are silent: an id outside [0, N) gives a row of
zeros.

Only the columns asked for are unpacked and dequantised (the whole 131072-column
head in float64 would be 2 GiB), with the same AWQ unpacking and dequantisation as
the GEMM oracle.
"""

import numpy as np

from .awq import unpack_awq
from .gemm import dequant
from .numerics import f64_to_half_bits_rne, half_bits_to_f64


def embedding_f64(ids, qweight, qzeros, scale_bits, dtype, group_size):
    """ids [T] -> float64 [T, K]: exact dequantised columns (zeros for ids out of range)."""
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    K = qweight.shape[0]
    N = qweight.shape[1] * 8
    valid = (ids >= 0) & (ids < N)
    E = np.zeros((ids.size, K), dtype=np.float64)
    if not valid.any():
        return E
    cols = np.unique(ids[valid])
    words = np.unique(cols // 8)                       # AWQ word columns holding them
    Q = unpack_awq(qweight[:, words])                  # [K, 8 * len(words)]
    Z = unpack_awq(qzeros[:, words])
    S = half_bits_to_f64(scale_bits.reshape(scale_bits.shape[0], -1)[:, (words[:, None] * 8 + np.arange(8)).reshape(-1)], dtype)
    W = dequant(Q, Z, S, group_size)                   # [K, 8 * len(words)]
    where = np.searchsorted(words, ids[valid] // 8) * 8 + ids[valid] % 8
    E[valid] = W[:, where].T
    return E


def embedding(ids, qweight, qzeros, scale_bits, dtype, group_size):
    """ids [T] -> uint16 bit patterns [T, K] of `dtype`: each value rounded once."""
    return f64_to_half_bits_rne(embedding_f64(ids, qweight, qzeros, scale_bits, dtype, group_size), dtype)
