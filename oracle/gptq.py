"""GPTQ-standard int32 nibble packing, written from its description.

Test infrastructure only (see the package docstring).

Facts used (vLLM note "Carga de capas cuantizadas", section "Motivación de
diseño"): GPTQ-style packing runs along the input dimension with the standard bit
order (the Marlin kernel accepts only that style, so AWQ checkpoints are converted
to it). Hence:
  * qweight int32 [K/8, N]: word (i, n) carries the codes of rows 8i .. 8i+7 of
    column n, row 8i + j in nibble j (bits 4j..4j+3 from the least significant bit);
  * qzeros int32 [K/G, N/8], packed along the output dimension like AWQ's but in
    the standard order: nibble j of word w holds column 8w + j.
Reading taken where the pages are silent: the stored zero point is z itself, used
in (q - z) * s with no +1 offset.

Words are two's-complement int32 in memory; codes are read from the unsigned view.
"""

import numpy as np


def _check_codes(codes, axis_multiple_of_8):
    codes = np.asarray(codes)
    if codes.ndim != 2 or codes.shape[axis_multiple_of_8] % 8 != 0:
        raise ValueError("codes must be 2-D with a multiple of 8 along the packed axis")
    if codes.size and (codes.min() < 0 or codes.max() > 15):
        raise ValueError("codes must lie in 0..15")
    return codes


def pack_gptq_weight(codes):
    """codes uint8 [K, N] (K % 8 == 0) -> int32 [K/8, N], packed along K."""
    codes = _check_codes(codes, 0)
    K, N = codes.shape
    grouped = codes.astype(np.uint32).reshape(K // 8, 8, N)     # [i, j, n]: row 8i + j
    words = np.zeros((K // 8, N), dtype=np.uint32)
    for j in range(8):
        words |= grouped[:, j, :] << np.uint32(4 * j)
    return words.view(np.int32)


def unpack_gptq_weight(words):
    """int32 [K/8, N] -> codes uint8 [K, N]; the inverse of pack_gptq_weight."""
    w = np.ascontiguousarray(np.asarray(words, dtype=np.int32)).view(np.uint32)
    if w.ndim != 2:
        raise ValueError("packed words must be 2-D")
    I, N = w.shape
    codes = np.zeros((I, 8, N), dtype=np.uint8)
    for j in range(8):
        codes[:, j, :] = ((w >> np.uint32(4 * j)) & np.uint32(0xF)).astype(np.uint8)
    return codes.reshape(8 * I, N)


def pack_gptq_zeros(codes):
    """zero points uint8 [R, N] (N % 8 == 0) -> int32 [R, N/8], packed along N."""
    codes = _check_codes(codes, 1)
    R, N = codes.shape
    grouped = codes.astype(np.uint32).reshape(R, N // 8, 8)     # [g, w, j]: column 8w + j
    words = np.zeros((R, N // 8), dtype=np.uint32)
    for j in range(8):
        words |= grouped[:, :, j] << np.uint32(4 * j)
    return words.view(np.int32)


def unpack_gptq_zeros(words):
    """int32 [R, N/8] -> zero points uint8 [R, N]; the inverse of pack_gptq_zeros."""
    w = np.ascontiguousarray(np.asarray(words, dtype=np.int32)).view(np.uint32)
    if w.ndim != 2:
        raise ValueError("packed words must be 2-D")
    R, J = w.shape
    codes = np.zeros((R, J, 8), dtype=np.uint8)
    for j in range(8):
        codes[:, :, j] = ((w >> np.uint32(4 * j)) & np.uint32(0xF)).astype(np.uint8)
    return codes.reshape(R, 8 * J)
