"""The GPU tile layout of packed W4A16 weights, written from its specification.

Test infrastructure only (see the package docstring). The HIP repack kernel
must produce exactly these bytes; nothing here is shared with it.

The pages describe a one-time reorder after loading (vLLM note "Carga de capas
cuantizadas", "Responsabilidades" and "Flujo de datos": process_weights_after_loading
rewrites qweight into the layout the kernel expects) but the layout is the
kernel's own. This library's layout, version 2, for a K x N weight with group
size G (G = K for group_size = -1; G = 32, 64, or a multiple of 128 dividing K):

  KB = K / 128 row blocks; Np = N rounded up to a multiple of 16, NB = Np / 16
  column blocks. N must be a multiple of 8, the pack factor of the checkpoint
  words (vLLM note, "Flujo de datos": packed_factor 8). When N % 16 == 8 the last
  block's columns N .. Np-1 are padding: code 0 in every row and metadata word 0
  (the vllm-omni commit "cpu_int4: dequantize prefill weights from the tinygemm
  layout, not a copy" reads an N that does not fill the last block as a case to be
  handled, not silently mis-read; here it is handled by whole zero columns).

  Weight plane, bytes [0, K*Np/2):
    block (nb, kb) is 1024 bytes at offset 1024 * (nb * KB + kb); so the whole K
    range of one 16-column block is contiguous.
    Inside a block, lane L in 0..63 owns bytes 16L .. 16L+15 = four little-endian
    uint32 words i = 0..3. Word i of lane L holds column n = 16 nb + (L mod 16)
    and rows k = 128 kb + 32 i + 8 (L div 16) + e for e = 0..7; nibble slot s
    (bits 4s .. 4s+3) holds the code of row e = TILE_ORDER[s].
    TILE_ORDER = (0, 2, 4, 6, 1, 3, 5, 7): slots t and t+4 hold rows 2t and 2t+1.

  Metadata plane, bytes [K*Np/2, K*Np/2 + 4*Np*UW): one word per metadata unit
  of Gu = min(G, 128) rows (a 128-row block, or 1/2 or 1/4 of one for G = 64 or
  32); U = K / Gu units, UW = U rounded up to a multiple of 4:
    uint32 number n * UW + b describes column n over unit b (rows b Gu ..
    b Gu + Gu - 1; so one column's words are contiguous), whose group is
    g = (b Gu) div G:
      bits 0..15  = the 16-bit pattern of S[g, n] (the scale, fp16 or bf16),
      bits 16..19 = Z[g, n] (the zero point, 0..15),
      bits 20..31 = 0;
    words b = U .. UW-1 of every column are 0 (padding).
  For G >= 128 a unit is a row block (UW = KB rounded up to 4).

  Total size: K*Np/2 + 4*Np*UW bytes.

Column blocks are independent (as the n-blocks of the CPU layout are in the
vllm-omni commit "cpu_int4: repack weights in n-blocks, to bound the load-time
peak"): repacking a range of whole column blocks yields exactly the bytes of
that range in both planes.
"""

import numpy as np

TILE_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)
ROWS_PER_BLOCK = 128
COLS_PER_BLOCK = 16
BLOCK_BYTES = 1024
LAYOUT_VERSION = 2


def check_shape(K, N, group_size):
    """Returns G; raises ValueError for shapes this layout does not cover."""
    if K <= 0 or N <= 0:
        raise ValueError("K and N must be positive")
    if K % ROWS_PER_BLOCK != 0:
        raise ValueError("K must be a multiple of 128")
    if N % 8 != 0:
        raise ValueError("N must be a multiple of 8")
    G = K if group_size == -1 else int(group_size)
    if G <= 0 or K % G != 0 or (G % ROWS_PER_BLOCK != 0 and G not in (32, 64)):
        raise ValueError("group size must be -1, 32, 64 or a multiple of 128 dividing K")
    return G


def padded_row_blocks(K):
    KB = K // ROWS_PER_BLOCK
    return (KB + 3) // 4 * 4


def unit_rows(G):
    """Rows described by one metadata word: min(G, 128)."""
    return min(G, ROWS_PER_BLOCK)


def padded_units(K, G):
    """Metadata words per column: K / unit_rows(G) rounded up to a multiple of 4."""
    U = K // unit_rows(G)
    return (U + 3) // 4 * 4


def padded_cols(N):
    return (N + COLS_PER_BLOCK - 1) // COLS_PER_BLOCK * COLS_PER_BLOCK


def packed_bytes(K, N, group_size):
    G = check_shape(K, N, group_size)
    Np = padded_cols(N)
    return K * Np // 2 + 4 * Np * padded_units(K, G)


def repack(Q, Z, scale_bits, group_size):
    """Codes Q uint8 [K, N], zeros Z uint8 [K/G, N], scale bits uint16 [K/G, N]
    -> packed buffer as uint8 [packed_bytes]."""
    Q = np.asarray(Q, dtype=np.uint8)
    K, N = Q.shape
    G = check_shape(K, N, group_size)
    Z = np.asarray(Z, dtype=np.uint8)
    scale_bits = np.asarray(scale_bits, dtype=np.uint16)
    if Z.shape != (K // G, N) or scale_bits.shape != (K // G, N):
        raise ValueError("zeros and scales must be [K/G, N]")
    N_real, N = N, padded_cols(N)
    if N != N_real:       # zero padding columns: code 0, zero point 0, scale bits 0
        pad = ((0, 0), (0, N - N_real))
        Q, Z, scale_bits = np.pad(Q, pad), np.pad(Z, pad), np.pad(scale_bits, pad)
    KB, NB = K // ROWS_PER_BLOCK, N // COLS_PER_BLOCK

    # Name the axes of Q by the layout: k = 128 kb + 32 i + 8 h + e, n = 16 nb + c.
    q = Q.reshape(KB, 4, 4, 8, NB, 16)                  # [kb, i, h, e, nb, c]
    words = np.zeros((NB, KB, 4, 16, 4), dtype=np.uint32)   # [nb, kb, h, c, i]
    for s in range(8):
        codes = q[:, :, :, TILE_ORDER[s], :, :]          # [kb, i, h, nb, c]
        codes = codes.transpose(3, 0, 2, 4, 1)           # [nb, kb, h, c, i]
        words |= codes.astype(np.uint32) << np.uint32(4 * s)
    # lane L = 16 h + c, so [h, c] flattens to L in order
    weight_plane = words.reshape(NB, KB, 64, 4)

    Gu = unit_rows(G)
    U = K // Gu
    group_of_unit = (np.arange(U) * Gu) // G                           # [b]
    s_u = scale_bits[group_of_unit].astype(np.uint32)                  # [b, N]
    z_u = Z[group_of_unit].astype(np.uint32)                           # [b, N]
    meta = np.zeros((N, padded_units(K, G)), dtype=np.uint32)          # [n, b], padding 0
    meta[:, :U] = (s_u | (z_u << np.uint32(16))).T

    out = np.concatenate([
        np.ascontiguousarray(weight_plane).astype("<u4").view(np.uint8).reshape(-1),
        np.ascontiguousarray(meta).astype("<u4").view(np.uint8).reshape(-1),
    ])
    assert out.size == packed_bytes(K, N_real, group_size)
    return out


def repack_loops(Q, Z, scale_bits, group_size):
    """The same layout with one Python loop per field: slow, for tiny shapes only.
    Kept beside the array version so the two statements can be checked against
    each other."""
    Q = np.asarray(Q, dtype=np.uint8)
    K, N = Q.shape
    G = check_shape(K, N, group_size)
    Np = padded_cols(N)
    KB, NB = K // ROWS_PER_BLOCK, Np // COLS_PER_BLOCK
    out = bytearray(packed_bytes(K, N, group_size))
    for nb in range(NB):
        for kb in range(KB):
            base = BLOCK_BYTES * (nb * KB + kb)
            for lane in range(64):
                n = 16 * nb + lane % 16
                if n >= N:
                    continue           # padding column: its bytes stay 0
                for i in range(4):
                    word = 0
                    for s in range(8):
                        k = 128 * kb + 32 * i + 8 * (lane // 16) + TILE_ORDER[s]
                        word |= int(Q[k, n]) << (4 * s)
                    off = base + 16 * lane + 4 * i
                    out[off:off + 4] = word.to_bytes(4, "little")
    meta_base = K * Np // 2
    Gu = min(G, 128)
    UW = padded_units(K, G)
    for n in range(N):                 # padding columns' words stay 0
        for b in range(K // Gu):       # words b >= K / Gu stay 0
            g = (Gu * b) // G
            word = int(scale_bits[g, n]) | (int(Z[g, n]) << 16)
            off = meta_base + 4 * (n * UW + b)
            out[off:off + 4] = word.to_bytes(4, "little")
    return np.frombuffer(bytes(out), dtype=np.uint8)


def decode(packed, K, N, group_size):
    """Inverse of repack: packed bytes -> (Q uint8 [K, N], Z uint8 [K/G, N],
    scale bits uint16 [K/G, N]). Raises ValueError if the buffer is not a valid
    layout (nonzero reserved bits, or row blocks of one group disagreeing)."""
    G = check_shape(K, N, group_size)
    packed = np.asarray(packed, dtype=np.uint8)
    if packed.size != packed_bytes(K, N, group_size):
        raise ValueError("packed buffer has the wrong size")
    N_real, N = N, padded_cols(N)
    KB, NB = K // ROWS_PER_BLOCK, N // COLS_PER_BLOCK
    wbytes = K * N // 2
    words = packed[:wbytes].view("<u4").reshape(NB, KB, 4, 16, 4)     # [nb, kb, h, c, i]
    q = np.zeros((KB, 4, 4, 8, NB, 16), dtype=np.uint8)              # [kb, i, h, e, nb, c]
    for s in range(8):
        codes = ((words >> np.uint32(4 * s)) & np.uint32(0xF)).astype(np.uint8)
        q[:, :, :, TILE_ORDER[s], :, :] = codes.transpose(1, 4, 2, 0, 3)
    Q = q.reshape(K, N)

    U = K // unit_rows(G)
    meta_all = packed[wbytes:].view("<u4").reshape(N, padded_units(K, G))
    if np.any(meta_all[:, U:]):
        raise ValueError("metadata padding is not zero")
    meta = meta_all[:, :U].T                                           # [b, n]
    if np.any(meta >> np.uint32(20)):
        raise ValueError("reserved metadata bits are not zero")
    units_per_group = G // unit_rows(G)
    meta_g = meta.reshape(K // G, units_per_group, N)
    if np.any(meta_g != meta_g[:, :1, :]):
        raise ValueError("units of one group carry different metadata")
    first = meta_g[:, 0, :]
    S = (first & np.uint32(0xFFFF)).astype(np.uint16)
    Z = ((first >> np.uint32(16)) & np.uint32(0xF)).astype(np.uint8)
    if np.any(Q[:, N_real:]) or np.any(meta[:, N_real:]):
        raise ValueError("padding columns are not zero")
    return Q[:, :N_real], Z[:, :N_real], S[:, :N_real]
