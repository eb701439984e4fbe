"""AWQ int32 nibble packing, written from its definition.

Test infrastructure only (see the package docstring).

Facts used (vLLM note "Carga de capas cuantizadas", sections "Flujo de datos"
and "Motivación de diseño"):
  * qweight is int32 [K, N/8] and qzeros is int32 [K/G, N/8]: each int32 carries
    8 four-bit codes of 8 consecutive output columns (packed_dim = 1, the output
    dimension, packed_factor = 8);
  * the codes inside an AWQ word are not in ascending column order.
The order itself is that of the problem statement this library implements:
"interleaved order 0,2,4,6,1,3,5,7". Reading taken (the plainest reading of a
packing order): nibble slot s, i.e. bits 4s..4s+3 counted from the least
significant bit, holds column 8j + AWQ_ORDER[s] of word j. Equivalently column
8j + t sits in slot AWQ_SLOT_OF_COLUMN[t].

Words are two's-complement int32 in memory; codes are read from the unsigned
view of the same 32 bits, so the word -1 holds eight 15s.
"""

import numpy as np

AWQ_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)        # column offset held by nibble slot s
AWQ_SLOT_OF_COLUMN = tuple(AWQ_ORDER.index(t) for t in range(8))  # = (0,4,1,5,2,6,3,7)


def pack_awq(codes):
    """codes uint8 [R, C] with values 0..15 (C % 8 == 0) -> int32 [R, C/8]."""
    codes = np.asarray(codes)
    if codes.ndim != 2 or codes.shape[1] % 8 != 0:
        raise ValueError("codes must be 2-D with a multiple of 8 columns")
    if codes.size and (codes.min() < 0 or codes.max() > 15):
        raise ValueError("codes must lie in 0..15")
    R, C = codes.shape
    grouped = codes.astype(np.uint32).reshape(R, C // 8, 8)   # [..., column offset t]
    words = np.zeros((R, C // 8), dtype=np.uint32)
    for s in range(8):
        words |= grouped[:, :, AWQ_ORDER[s]] << np.uint32(4 * s)
    return words.view(np.int32)


def unpack_awq(words):
    """int32 [R, C/8] -> codes uint8 [R, C]; the inverse of pack_awq."""
    w = np.ascontiguousarray(np.asarray(words, dtype=np.int32)).view(np.uint32)
    if w.ndim != 2:
        raise ValueError("packed words must be 2-D")
    R, J = w.shape
    codes = np.zeros((R, J, 8), dtype=np.uint8)
    for s in range(8):
        codes[:, :, AWQ_ORDER[s]] = ((w >> np.uint32(4 * s)) & np.uint32(0xF)).astype(np.uint8)
    return codes.reshape(R, 8 * J)


def unpacked_shape(packed_shape):
    """Shape of the code matrix that unpacking a [R, C/8] int32 tensor produces."""
    R, J = packed_shape
    return (R, 8 * J)
