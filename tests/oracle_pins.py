"""Pin checks for the CPU oracle, as functions returning True when the oracle
agrees with a fact fixed independently of it (a printed value, a hand-worked
example, a closed form, an invariant, exact arithmetic).

They are plain functions of the oracle's modules so that tests can run them both
against the oracle and against copies of it with a planted mistake, to show that
each plausible mistake trips at least one pin.
"""

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def awq_golden_entries():
    out = []
    for line in _lines("awq_word_pins.txt"):
        kind, rest = line.split(None, 1)
        lhs, rhs = [p.strip() for p in rest.split("->")]
        if kind == "pack":
            out.append(("pack", [int(v) for v in lhs.split()], int(rhs, 16)))
        else:
            out.append(("unpack", int(lhs, 16), [int(v) for v in rhs.split()]))
    return out


def pin_awq_golden(awq):
    for kind, a, b in awq_golden_entries():
        if kind == "pack":
            w = int(awq.pack_awq(np.array([a], dtype=np.uint8))[0, 0].view(np.uint32))
            if w != b:
                return False
        else:
            word = np.array([[a]], dtype=np.uint32).view(np.int32)
            if awq.unpack_awq(word)[0].tolist() != b:
                return False
    return True


def worked_example():
    rows = [line.split() for line in _lines("worked_example_bf16.txt")]
    s = [float(r[1]) for r in rows]
    y = np.array([[float(r[2]) for r in rows], [float(r[3]) for r in rows]])
    qweight = np.empty((128, 2), dtype=np.uint32)
    qweight[0] = [0x75316420, 0xFFFFFFFF]
    qweight[1] = [0x00000000, 0x11111111]
    qweight[2:] = 0x88888888
    qzeros = np.array([[0x33333333, 0x33333333]], dtype=np.uint32)
    scale_bits = (np.array([s], dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = np.zeros((2, 128), dtype=np.float32)
    x[0, 0], x[0, 1] = 1.0, 2.0
    x[1, :] = 1.0
    x_bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    return dict(qweight=qweight.view(np.int32), qzeros=qzeros.view(np.int32),
                scale_bits=scale_bits, x_bits=x_bits, y=y)


def pin_worked_example(gemm_mod):
    ex = worked_example()
    y = gemm_mod.w4a16_reference(ex["x_bits"], ex["qweight"], ex["qzeros"], ex["scale_bits"],
                                 "bf16", 128)
    return y.shape == ex["y"].shape and np.array_equal(y, ex["y"])


def page3_transients():
    return [(r[0], int(r[1]), int(r[2]), int(r[3])) for r in (l.split() for l in _lines("page3_int32_transients.txt"))]


def pin_page3_transients(awq):
    for _, N, K, mib in page3_transients():
        R, C = awq.unpacked_shape((K, N // 8))
        if R * C * 4 != mib * 2**20:
            return False
    return True


def _fraction_reference(x_bits, qweight, qzeros, scale_bits, G):
    """Exact y from the AWQ words with Python integers and Fractions. Codes are
    read per element with the slot-of-column table (the inverse view of the
    packing order), bf16 values decoded with integer arithmetic."""
    slot_of_column = (0, 4, 1, 5, 2, 6, 3, 7)

    def code(words, r, n):
        w = int(words[r, n // 8]) & 0xFFFFFFFF
        return (w >> (4 * slot_of_column[n % 8])) & 0xF

    def bf16(b):
        b = int(b)
        sign = -1 if b & 0x8000 else 1
        e = (b >> 7) & 0xFF
        m = b & 0x7F
        if e == 0:
            return sign * Fraction(m, 2**133)      # 2^-126 * m / 2^7
        return sign * Fraction(128 + m, 128) * (Fraction(2) ** (e - 127))

    M, K = x_bits.shape
    N = qweight.shape[1] * 8
    y = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                g = k // G
                w = (code(qweight, k, n) - code(qzeros, g, n)) * bf16(scale_bits[g, n])
                acc += bf16(x_bits[m, k]) * w
            y[m][n] = acc
    return y


def pin_fraction_bruteforce(gemm_mod, seed=7):
    rng = np.random.default_rng(seed)
    for (M, K, N, G) in [(2, 128, 16, 128), (3, 256, 8, 128), (1, 256, 24, 64)]:
        qweight = rng.integers(0, 2**32, (K, N // 8), dtype=np.uint32).view(np.int32)
        qzeros = rng.integers(0, 2**32, (K // G, N // 8), dtype=np.uint32).view(np.int32)
        s = rng.uniform(0.005, 0.02, (K // G, N)).astype(np.float32)
        scale_bits = (s.view(np.uint32) >> 16).astype(np.uint16)
        x = rng.standard_normal((M, K)).astype(np.float32)
        x_bits = (x.view(np.uint32) >> 16).astype(np.uint16)
        y = gemm_mod.w4a16_reference(x_bits, qweight, qzeros, scale_bits, "bf16", G)
        exact = _fraction_reference(x_bits, qweight, qzeros, scale_bits, G)
        for m in range(M):
            for n in range(N):
                e = float(exact[m][n])
                if abs(y[m, n] - e) > 1e-12 * max(1.0, abs(e)):
                    return False
    return True


def pin_closed_form_constant_codes(gemm_mod, awq):
    """Q = c and Z = z0 everywhere: y[m, n] = (c - z0) * sum_g S[g, n] * sum_{k in g} x[m, k]."""
    rng = np.random.default_rng(11)
    M, K, N, G = 3, 512, 32, 128
    c, z0 = 13, 4
    qweight = awq.pack_awq(np.full((K, N), c, dtype=np.uint8))
    qzeros = awq.pack_awq(np.full((K // G, N), z0, dtype=np.uint8))
    s = rng.uniform(0.005, 0.02, (K // G, N)).astype(np.float32)
    scale_bits = (s.view(np.uint32) >> 16).astype(np.uint16)
    S = (scale_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x_bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    X = (x_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    group_sums = X.reshape(M, K // G, G).sum(axis=2)               # [M, K/G]
    expect = (c - z0) * np.einsum("mg,gn->mn", group_sums, S)
    y = gemm_mod.w4a16_reference(x_bits, qweight, qzeros, scale_bits, "bf16", G)
    return np.allclose(y, expect, rtol=1e-12, atol=1e-12)


def pin_integer_special_case(gemm_mod, awq):
    """S = 1, Z = 0 and integer activations: y = x . Q, an integer matrix product
    computed exactly with int64."""
    rng = np.random.default_rng(5)
    M, K, N, G = 4, 256, 48, 128
    Q = rng.integers(0, 16, (K, N), dtype=np.uint8)
    qweight = awq.pack_awq(Q)
    qzeros = awq.pack_awq(np.zeros((K // G, N), dtype=np.uint8))
    scale_bits = np.full((K // G, N), 0x3F80, dtype=np.uint16)   # bf16 1.0
    xi = rng.integers(-3, 4, (M, K)).astype(np.int64)
    x_bits = (xi.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = gemm_mod.w4a16_reference(x_bits, qweight, qzeros, scale_bits, "bf16", G)
    return np.array_equal(y, (xi @ Q.astype(np.int64)).astype(np.float64))


def pin_zero_point_cancels(gemm_mod, awq):
    """Z equal to the (per group, per column constant) code: every weight is 0, y = 0."""
    rng = np.random.default_rng(3)
    M, K, N, G = 2, 256, 16, 128
    Zc = rng.integers(0, 16, (K // G, N), dtype=np.uint8)
    Q = np.repeat(Zc, G, axis=0)
    s = rng.uniform(0.005, 0.02, (K // G, N)).astype(np.float32)
    scale_bits = (s.view(np.uint32) >> 16).astype(np.uint16)
    x_bits = (rng.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = gemm_mod.w4a16_reference(x_bits, awq.pack_awq(Q), awq.pack_awq(Zc), scale_bits, "bf16", G)
    return np.array_equal(y, np.zeros((M, N)))


def pin_group_index(gemm_mod, awq):
    """Only group g's scale is nonzero: y must equal the contribution of rows in g
    alone, which (Q = 1, Z = 0, scale 1) is the plain sum of x over those rows."""
    rng = np.random.default_rng(9)
    M, K, N, G = 2, 512, 16, 128
    ok = True
    for g in range(K // G):
        scale_bits = np.zeros((K // G, N), dtype=np.uint16)
        scale_bits[g] = 0x3F80
        qweight = awq.pack_awq(np.ones((K, N), dtype=np.uint8))
        qzeros = awq.pack_awq(np.zeros((K // G, N), dtype=np.uint8))
        xi = rng.integers(-4, 5, (M, K)).astype(np.int64)
        x_bits = (xi.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        y = gemm_mod.w4a16_reference(x_bits, qweight, qzeros, scale_bits, "bf16", G)
        expect = np.repeat(xi[:, g * G:(g + 1) * G].sum(axis=1, keepdims=True), N, axis=1)
        ok &= np.array_equal(y, expect.astype(np.float64))
    return bool(ok)


ALL_GEMM_PINS = ("pin_worked_example", "pin_fraction_bruteforce", "pin_closed_form_constant_codes",
                 "pin_integer_special_case", "pin_zero_point_cancels", "pin_group_index")


def run_gemm_pins(gemm_mod, awq):
    res = {}
    res["pin_worked_example"] = pin_worked_example(gemm_mod)
    res["pin_fraction_bruteforce"] = pin_fraction_bruteforce(gemm_mod)
    res["pin_closed_form_constant_codes"] = pin_closed_form_constant_codes(gemm_mod, awq)
    res["pin_integer_special_case"] = pin_integer_special_case(gemm_mod, awq)
    res["pin_zero_point_cancels"] = pin_zero_point_cancels(gemm_mod, awq)
    res["pin_group_index"] = pin_group_index(gemm_mod, awq)
    return res


# ---- tile layout pins: closed-form byte patterns for index-pattern code matrices ----

def layout_index_pattern_cases(K=256, N=48):
    """(description, Q, expected weight-plane check) triples. Each Q is chosen so
    that every byte of the repacked weight plane has a closed-form value."""
    k = np.arange(K)[:, None]
    n = np.arange(N)[None, :]
    KB, NB = K // 128, N // 16
    lane = np.arange(64)

    def expect_by_lane(f):      # byte value of every byte of lane L's 16 bytes
        e = np.repeat(f(lane)[:, None], 16, axis=1).reshape(-1).astype(np.uint8)
        return np.tile(e, NB * KB)

    cases = []
    cases.append(("code = column within block -> lane L all nibbles L mod 16",
                  (n % 16) + 0 * k, expect_by_lane(lambda L: 0x11 * (L % 16))))
    cases.append(("code = (k div 8) mod 4 -> lane L all nibbles L div 16",
                  ((k // 8) % 4) + 0 * n, expect_by_lane(lambda L: 0x11 * (L // 16))))
    w_i = np.array([0x11111111 * i for i in range(4)], dtype="<u4").view(np.uint8)
    cases.append(("code = (k div 32) mod 4 -> word i is 0x11111111 * i",
                  ((k // 32) % 4) + 0 * n, np.tile(w_i, 64 * NB * KB)))
    w_o = np.array([0x75316420], dtype="<u4").view(np.uint8)
    cases.append(("code = k mod 8 -> every word 0x75316420",
                  (k % 8) + 0 * n, np.tile(w_o, 4 * 64 * NB * KB)))
    blk = np.array([0x11 * (kb % 16) for nb in range(NB) for kb in range(KB)], dtype=np.uint8)
    cases.append(("code = row block kb -> block (nb, kb) all bytes 0x11 * kb (nb-major order)",
                  (k // 128) % 16 + 0 * n, np.repeat(blk, 1024)))
    blk = np.array([0x11 * (nb % 16) for nb in range(NB) for kb in range(KB)], dtype=np.uint8)
    cases.append(("code = column block nb -> block (nb, kb) all bytes 0x11 * nb",
                  (n // 16) % 16 + 0 * k, np.repeat(blk, 1024)))
    return [(d, q.astype(np.uint8), e) for d, q, e in cases]


def pin_layout_index_patterns(tile_layout, K=256, N=48, G=128):
    zeros = np.zeros((K // G, N), dtype=np.uint8)
    sbits = np.zeros((K // G, N), dtype=np.uint16)
    for _, Q, expect in layout_index_pattern_cases(K, N):
        out = tile_layout.repack(Q, zeros, sbits, G)
        if not np.array_equal(out[:K * N // 2], expect):
            return False
    return True


def pin_layout_metadata(tile_layout, K=768, N=32, G=256):
    """scale bits = column index, zero = group mod 16: metadata word of (n, kb)
    must be n | ((128 kb div G) mod 16) << 16 at position n * KBP + kb, with the
    padding words of each column zero (K = 768: 6 row blocks, padded to 8)."""
    KG, KB = K // G, K // 128
    KBP = (KB + 3) // 4 * 4
    sbits = np.tile(np.arange(N, dtype=np.uint16), (KG, 1))
    Z = np.repeat((np.arange(KG) % 16).astype(np.uint8)[:, None], N, axis=1)
    out = tile_layout.repack(np.zeros((K, N), np.uint8), Z, sbits, G)
    meta = out[K * N // 2:].view("<u4")
    expect = [(n | ((((128 * kb) // G) % 16) << 16)) if kb < KB else 0
              for n in range(N) for kb in range(KBP)]
    return meta.tolist() == expect


def pin_layout_half_block(tile_layout):
    """N = 24 (a last half block): every real code 15, zero points 5, scale bits
    0x1234 + n. Closed form: block 1 holds columns 16..23 in lanes c < 8 (every word
    0xFFFFFFFF) and zero words in lanes c >= 8; the metadata plane starts at K*32/2
    and columns 24..31 have all-zero words; the buffer is K*32/2 + 4*32*KBP bytes."""
    K, N, G = 256, 24, 128
    KB, KBP = K // 128, 4
    Q = np.full((K, N), 15, dtype=np.uint8)
    Z = np.full((K // G, N), 5, dtype=np.uint8)
    S = np.tile((0x1234 + np.arange(N)).astype(np.uint16), (K // G, 1))
    out = tile_layout.repack(Q, Z, S, G)
    if out.size != K * 32 // 2 + 4 * 32 * KBP:
        return False
    words = out[:K * 32 // 2].view("<u4").reshape(2, KB, 64, 4)          # [nb, kb, lane, i]
    c = np.arange(64) % 16
    if not np.all(words[0] == 0xFFFFFFFF):
        return False
    if not (np.all(words[1][:, c < 8] == 0xFFFFFFFF) and np.all(words[1][:, c >= 8] == 0)):
        return False
    meta = out[K * 32 // 2:].view("<u4").reshape(32, KBP)
    for n in range(32):
        want = [(0x1234 + n) | (5 << 16) if (n < N and kb < KB) else 0 for kb in range(KBP)]
        if meta[n].tolist() != want:
            return False
    return True


def pin_layout_small_groups(tile_layout, G, K=384, N=16):
    """G = 32 or 64: scale bits of group g, column n = (g << 8) | n, zero point
    (3 g) mod 16. Closed form: K / G words per column (a word per G rows), word b
    of column n = ((b << 8) | n) | ((3 b mod 16) << 16), padded with zero words to a
    multiple of 4, the plane after the K*N/2 code bytes; the codes are untouched."""
    U = K // G
    UW = (U + 3) // 4 * 4
    g = np.arange(U)
    S = ((g[:, None] << 8) | np.arange(N)[None, :]).astype(np.uint16)
    Z = np.repeat(((3 * g) % 16).astype(np.uint8)[:, None], N, axis=1)
    Q = (np.arange(K)[:, None] % 16 + np.zeros((1, N), dtype=np.int64)).astype(np.uint8)
    out = tile_layout.repack(Q, Z, S, G)
    if out.size != K * N // 2 + 4 * N * UW:
        return False
    ref128 = tile_layout.repack(Q, np.zeros((K // 128, N), np.uint8), np.zeros((K // 128, N), np.uint16), 128)
    if not np.array_equal(out[:K * N // 2], ref128[:K * N // 2]):
        return False
    meta = out[K * N // 2:].view("<u4").reshape(N, UW)
    for n in range(N):
        want = [((b << 8) | n) | (((3 * b) % 16) << 16) for b in range(U)] + [0] * (UW - U)
        if meta[n].tolist() != want:
            return False
    return True


# ---------------------------------------------------------------- tied embedding

def _bf16_bits_of(v):
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0] >> 16)


def embedding_golden():
    weights, rounding = [], []
    for line in _lines("worked_example_embedding.txt"):
        f = line.split()
        if f[0] == "weights":
            weights.append((int(f[1]), float(f[2]), float(f[3]), float(f[4])))
        else:
            rounding.append((f[1], int(f[2], 16), int(f[3]), int(f[4]), int(f[5], 16)))
    return weights, rounding


def pin_embedding_worked_example(emb):
    """The hand-worked rows: exact values, so their bf16 bits are known."""
    ex = worked_example()
    weights, _ = embedding_golden()
    ids = np.array([w[0] for w in weights])
    got = emb.embedding(ids, ex["qweight"], ex["qzeros"], ex["scale_bits"], "bf16", 128)
    if got.shape != (len(ids), 128):
        return False
    for i, (_, e0, e1, rest) in enumerate(weights):
        want = [_bf16_bits_of(e0), _bf16_bits_of(e1)] + [_bf16_bits_of(rest)] * 126
        if got[i].tolist() != want:
            return False
    return True


def pin_embedding_rounding(emb):
    """(q - z) * s needing a rounding step: hand-rounded results (ties to even)."""
    _, rounding = embedding_golden()
    for dtype, sbits, q, z, want in rounding:
        qweight = np.full((128, 1), q * 0x11111111, dtype=np.uint32).view(np.int32)   # every column code q
        qzeros = np.full((1, 1), z * 0x11111111, dtype=np.uint32).view(np.int32)
        scale_bits = np.full((1, 8), sbits, dtype=np.uint16)
        got = emb.embedding(np.array([0, 5]), qweight, qzeros, scale_bits, dtype, 128)
        if not np.all(got == want):
            return False
    return True


def pin_embedding_matches_gemm(emb, gemm_mod, seed=11):
    """Row t of the embedding is column t of the GEMM oracle's product with the
    identity activation (x = I_K gives y = W exactly), zeros for ids out of range."""
    rng = np.random.default_rng(seed)
    for (K, N, G, dtype) in [(256, 24, 128, "bf16"), (128, 16, 128, "fp16"), (256, 8, -1, "bf16")]:
        GG = K if G == -1 else G
        qweight = rng.integers(0, 2**32, (K, N // 8), dtype=np.uint32).view(np.int32)
        qzeros = rng.integers(0, 2**32, (K // GG, N // 8), dtype=np.uint32).view(np.int32)
        s = rng.uniform(0.005, 0.02, (K // GG, N))
        scale_bits = (s.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16) if dtype == "bf16" \
            else s.astype(np.float16).view(np.uint16)
        one = 0x3F80 if dtype == "bf16" else 0x3C00
        x_bits = np.where(np.eye(K, dtype=bool), one, 0).astype(np.uint16)
        y = gemm_mod.w4a16_reference(x_bits, qweight, qzeros, scale_bits, dtype, G)    # = W
        ids = np.array([N - 1, 0, 3, 3, N, -2, 5])
        e = emb.embedding_f64(ids, qweight, qzeros, scale_bits, dtype, G)
        for i, t in enumerate(ids):
            want = y[:, t] if 0 <= t < N else np.zeros(K)
            if not np.array_equal(e[i], want):
                return False
    return True


def run_embedding_pins(emb, gemm_mod):
    return {"worked example": pin_embedding_worked_example(emb),
            "rounding": pin_embedding_rounding(emb),
            "identity product": pin_embedding_matches_gemm(emb, gemm_mod)}


# ---------------------------------------------------------------- GPTQ-standard packing

def gptq_golden_entries():
    out = []
    for line in _lines("gptq_word_pins.txt"):
        kind, direction, rest = line.split(None, 2)
        lhs, rhs = [p.strip() for p in rest.split("->")]
        if direction == "pack":
            out.append((kind, "pack", [int(v) for v in lhs.split()], int(rhs, 16)))
        else:
            out.append((kind, "unpack", int(lhs, 16), [int(v) for v in rhs.split()]))
    return out


def pin_gptq_golden(gptq):
    """Hand-derived words: weights as one column of 8 rows, zeros as one row of 8 columns."""
    for kind, direction, a, b in gptq_golden_entries():
        if kind == "weight":
            if direction == "pack":
                w = gptq.pack_gptq_weight(np.array(a, dtype=np.uint8).reshape(8, 1))
                if w.shape != (1, 1) or int(w.view(np.uint32)[0, 0]) != b:
                    return False
            else:
                c = gptq.unpack_gptq_weight(np.array([[a]], dtype=np.uint32).view(np.int32))
                if c.shape != (8, 1) or c[:, 0].tolist() != b:
                    return False
        else:
            if direction == "pack":
                w = gptq.pack_gptq_zeros(np.array([a], dtype=np.uint8))
                if w.shape != (1, 1) or int(w.view(np.uint32)[0, 0]) != b:
                    return False
            else:
                c = gptq.unpack_gptq_zeros(np.array([[a]], dtype=np.uint32).view(np.int32))
                if c.shape != (1, 8) or c[0].tolist() != b:
                    return False
    return True


def pin_gptq_roundtrips(gptq, seed=5):
    rng = np.random.default_rng(seed)
    Q = rng.integers(0, 16, (64, 24), dtype=np.uint8)
    if not np.array_equal(gptq.unpack_gptq_weight(gptq.pack_gptq_weight(Q)), Q):
        return False
    W = rng.integers(0, 2**32, (5, 24), dtype=np.uint32).view(np.int32)
    if not np.array_equal(gptq.pack_gptq_weight(gptq.unpack_gptq_weight(W)), W):
        return False
    Z = rng.integers(0, 16, (3, 40), dtype=np.uint8)
    if not np.array_equal(gptq.unpack_gptq_zeros(gptq.pack_gptq_zeros(Z)), Z):
        return False
    return True


def pin_gptq_row_moves_one_nibble(gptq):
    """A single code in row r of a column block lands in word r // 8, nibble r % 8."""
    for r in range(16):
        Q = np.zeros((16, 8), dtype=np.uint8)
        Q[r, 3] = 9
        w = gptq.pack_gptq_weight(Q).view(np.uint32)
        want = np.zeros((2, 8), dtype=np.uint32)
        want[r // 8, 3] = 9 << (4 * (r % 8))
        if not np.array_equal(w, want):
            return False
    return True


def run_gptq_pins(gptq):
    return {"golden": pin_gptq_golden(gptq), "roundtrips": pin_gptq_roundtrips(gptq),
            "one nibble": pin_gptq_row_moves_one_nibble(gptq)}


# ---------------------------------------------------------------- W4A8 (fp8 activations)
# Facts fixed by the E4M3 format (OCP 8-bit floating point, "fn" variant): bias 7,
# 3 mantissa bits, subnormals m * 2^-9, largest finite 448, S.1111.111 NaN.
E4M3_SPEC = [
    (0.0, 0x00), (2.0 ** -9, 0x01), (7 * 2.0 ** -9, 0x07), (2.0 ** -6, 0x08), (0.5, 0x30),
    (1.0, 0x38), (1.125, 0x39), (2.0, 0x40), (-2.0, 0xC0), (240.0, 0x77), (256.0, 0x78),
    (448.0, 0x7E), (-448.0, 0xFE),
]
# ties go to the even mantissa; values past 448 below the midpoint 464 round to 448
E4M3_TIES = [
    (1.0625, 0x38), (1.1875, 0x3A), (0.5 * 2.0 ** -9, 0x00), (1.5 * 2.0 ** -9, 0x02),
    (2.5 * 2.0 ** -9, 0x02), (7.5 * 2.0 ** -9, 0x08), (456.0, 0x7E), (-1.0625, 0xB8),
]


def pin_e4m3_spec(w):
    for v, c in E4M3_SPEC:
        if int(w.e4m3_encode_rne(np.array([v]))[0]) != c or float(w.e4m3_decode(np.array([c]))[0]) != v:
            return False
    for v, c in E4M3_TIES:
        if int(w.e4m3_encode_rne(np.array([v]))[0]) != c:
            return False
    if int(w.e4m3_encode_rne(np.array([-0.0]))[0]) != 0x80:
        return False
    d = w.e4m3_decode(np.arange(256, dtype=np.uint8))
    if not (np.isnan(d[0x7F]) and np.isnan(d[0xFF]) and np.sum(np.isnan(d)) == 2):
        return False
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    return bool(np.array_equal(w.e4m3_encode_rne(w.e4m3_decode(finite)), finite))


def _all_bf16_within(limit):
    with np.errstate(invalid="ignore"):       # NaN patterns among the 65536
        v = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    return v[np.isfinite(v) & (np.abs(v) <= limit)]


def pin_e4m3_against_torch(w):
    """Decode of all 256 codes and encode of every bf16 value in [-448, 448] agree
    with torch's float8_e4m3fn conversions (an independent implementation)."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = w.e4m3_decode(codes)
    if not np.array_equal(np.isnan(ref), np.isnan(got)) or not np.array_equal(ref[~np.isnan(ref)], got[~np.isnan(got)]):
        return False
    v = _all_bf16_within(448.0)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return bool(np.array_equal(w.e4m3_encode_rne(v), ref))


def _nearest_even_bruteforce(v):
    """Nearest finite E4M3 code by exhaustive search, ties to the even code."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.int64)
    vals = np.empty(codes.shape)
    for t, c in enumerate(codes):            # decode written out again, field by field
        s = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 15, c & 7
        vals[t] = s * (m / 512.0 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))
    out = np.empty(v.shape, dtype=np.int64)
    for a in range(0, v.size, 4096):
        x = v[a:a + 4096, None]
        # codes of the value's own sign (so -0.0 and small negatives go to 0x80)
        same_sign = (codes[None, :] >= 128) == np.signbit(x)
        dist = np.where(same_sign, np.abs(vals[None, :] - x), np.inf)
        cand = dist == dist.min(axis=1, keepdims=True)
        # of equally near codes, the even one (mantissa bit 0 clear)
        pick = np.where(cand & (codes[None, :] % 2 == 0), codes[None, :], 1 << 20).min(axis=1)
        pick = np.where(pick == 1 << 20, np.where(cand, codes[None, :], 1 << 20).min(axis=1), pick)
        out[a:a + 4096] = pick
    return out


def pin_e4m3_bruteforce(w):
    v = _all_bf16_within(460.0)
    v = np.concatenate([v, np.array([E4M3_TIES[i][0] for i in range(len(E4M3_TIES))])])
    return bool(np.array_equal(w.e4m3_encode_rne(v).astype(np.int64), _nearest_even_bruteforce(v)))


def pin_nibble_reading(w):
    """A code q in the low nibble of an E4M3 byte reads q * 2^-9: the factor 512."""
    return bool(np.array_equal(w.e4m3_decode(np.arange(16, dtype=np.uint8)), np.arange(16) / 512.0))


def pin_quantize_rows(w, seed=3):
    rng = np.random.default_rng(seed)
    M, K = 6, 256
    X = rng.standard_normal((M, K)).astype(np.float32)
    X[1] = 0.0                                    # a row of zeros
    X[2] = 0.0
    X[2, 17] = -3.5                               # one non-zero
    X[3] *= 1e-3                                  # small values (subnormal codes)
    bits = (X.view(np.uint32) >> 16).astype(np.uint16)      # truncate to bf16 bit patterns
    codes, scale = w.quantize_rows(bits, "bf16")
    Xb = (bits.astype(np.uint32) << 16).view(np.float32)
    amax = np.abs(Xb).max(axis=1)
    want_scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    if not np.array_equal(scale, want_scale):
        return False
    if np.any(codes[1] != 0) or scale[1] != 1.0:
        return False
    # the largest magnitude of each non-zero row lands on +-448
    for m in (0, 2, 3, 4, 5):
        k = int(np.argmax(np.abs(Xb[m])))
        if codes[m, k] & 0x7F != 0x7E:
            return False
    # every code is the nearest-even E4M3 value of the float32 quotient
    q = (Xb / scale[:, None]).astype(np.float32).astype(np.float64)
    if not np.array_equal(codes.reshape(-1).astype(np.int64), _nearest_even_bruteforce(q.reshape(-1))):
        return False
    # on-grid rows come back unchanged: x = dec(c) / 8 with a +-448 / 8 entry
    c = rng.integers(0, 0x7F, size=(2, 128)).astype(np.uint8) | (rng.integers(0, 2, size=(2, 128)) << 7).astype(np.uint8)
    c[c == 0xFF] = 0xFE
    c[:, 5] = 0x7E
    vals = (w.e4m3_decode(c) / 8.0).astype(np.float32)
    g_bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    gc, gs = w.quantize_rows(g_bits, "bf16")
    return bool(np.array_equal(gc, c) and np.all(gs == np.float32(1.0 / 8.0)))


def pin_operand_order(w, tile_layout, seed=4):
    """The operand order pairs each activation byte with the weight code of the
    same row: for every lane (c, h) of a weight block, byte 8 i + j of the lane's
    expanded codes (word i, byte j of (word & 0x0F0F0F0F) for j < 4, of
    ((word >> 4) & 0x0F0F0F0F) for j >= 4) meets activation byte 32 h + 8 i + j,
    and the products summed over the block's lanes give sum_k a[k] * Q[k, c]."""
    rng = np.random.default_rng(seed)
    K, N = 256, 16
    a = rng.integers(0, 256, size=(3, K)).astype(np.uint8)
    if not np.array_equal(w.element_order(w.operand_order(a)), a):
        return False
    Q = rng.integers(0, 16, size=(K, N)).astype(np.uint8)
    packed = tile_layout.repack(Q, np.zeros((K // 128, N), np.uint8), np.zeros((K // 128, N), np.uint16), 128)
    words = packed[:K * N // 2].view(np.uint32).reshape(K // 128, 64, 4)    # one column block: [kb, lane, i]
    ops = w.operand_order(a).astype(np.int64)
    want = a.astype(np.int64) @ Q.astype(np.int64)
    got = np.zeros_like(want)
    for kb in range(K // 128):
        for lane in range(64):
            c, h = lane % 16, lane // 16
            for i in range(4):
                wd = int(words[kb, lane, i])
                for j in range(8):
                    code = (wd >> (8 * j)) & 0xF if j < 4 else (wd >> (8 * (j - 4) + 4)) & 0xF
                    got[:, c] += ops[:, kb * 128 + 32 * h + 8 * i + j] * code
    return bool(np.array_equal(got, want))


def _bf16_bits_rne(v):
    """float array -> bf16 bit patterns, nearest even (finite values)."""
    b = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def pin_w4a8_bruteforce(w, awq, seed=8):
    """Tiny layer in exact rationals: y = a[m] * sum_k dec(e) (q - z) s (+ bias)."""
    rng = np.random.default_rng(seed)
    M, K, N, G = 2, 256, 8, 128
    Q = rng.integers(0, 16, size=(K, N)).astype(np.uint8)
    Z = rng.integers(0, 16, size=(K // G, N)).astype(np.uint8)
    S = _bf16_bits_rne(rng.uniform(0.005, 0.02, size=(K // G, N)))
    e = rng.integers(0, 0x7F, size=(M, K)).astype(np.uint8) | (rng.integers(0, 2, size=(M, K)) << 7).astype(np.uint8)
    scale = np.array([0.0078125, 0.013], dtype=np.float32)
    bias = _bf16_bits_rne(np.array([0.25, -1.5, 0, 0, 3.0, 0, 0, 0.125]))
    y = w.w4a8_reference(e, scale, Q, Z, S, "bf16", G, bias)

    def frac_e4m3(c):
        c = int(c)
        s = -1 if c & 0x80 else 1
        ex, m = (c >> 3) & 15, c & 7
        return s * (Fraction(m, 512) if ex == 0 else Fraction(8 + m, 8) * Fraction(2) ** (ex - 7))

    def frac_bf16(b):
        return Fraction(float((np.array([b], np.uint32) << 16).view(np.float32)[0]))

    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += frac_e4m3(e[m, k]) * (int(Q[k, n]) - int(Z[k // G, n])) * frac_bf16(S[k // G, n])
            ref = Fraction(float(scale[m])) * acc + frac_bf16(bias[n])
            if abs(float(ref) - y[m, n]) > 1e-12 * max(1.0, abs(float(ref))):
                return False
    return True


def pin_w4a8_on_grid_equals_w4a16(w, gemm_mod, awq, seed=9):
    """Activations already on the E4M3 grid of their row scale quantise without
    error, so the W4A8 layer equals the (separately pinned) W4A16 layer."""
    rng = np.random.default_rng(seed)
    M, K, N, G = 3, 512, 16, 128
    c = rng.integers(0, 0x7F, size=(M, K)).astype(np.uint8) | (rng.integers(0, 2, size=(M, K)) << 7).astype(np.uint8)
    c[:, 0] = 0x7E
    x = (w.e4m3_decode(c) * 2.0 ** -5).astype(np.float32)
    x_bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    Q = rng.integers(0, 16, size=(K, N)).astype(np.uint8)
    Z = rng.integers(0, 16, size=(K // G, N)).astype(np.uint8)
    S = _bf16_bits_rne(rng.uniform(0.005, 0.02, size=(K // G, N)))
    qw, qz = awq.pack_awq(Q), awq.pack_awq(Z)
    y8 = w.w4a8_layer(x_bits, qw, qz, S, "bf16", G)
    y16 = gemm_mod.w4a16_reference(x_bits, qw, qz, S, "bf16", G)
    return bool(np.max(np.abs(y8 - y16)) <= 1e-12 * np.max(np.abs(y16)))


def pin_w4a8_block_sums(w, seed=10):
    rng = np.random.default_rng(seed)
    e = rng.integers(0, 0x7F, size=(2, 384)).astype(np.uint8)
    s = w.block_sums(e)
    want = np.array([[sum(float(w.e4m3_decode(np.array([e[m, k]]))[0]) for k in range(128 * b, 128 * b + 128))
                      for b in range(3)] for m in range(2)])
    return s.shape == (2, 3) and bool(np.array_equal(s, want))


def run_w4a8_pins(w, gemm_mod, awq, tile_layout):
    return {
        "spec": pin_e4m3_spec(w),
        "torch": pin_e4m3_against_torch(w),
        "bruteforce": pin_e4m3_bruteforce(w),
        "nibble": pin_nibble_reading(w),
        "quantize": pin_quantize_rows(w),
        "operand_order": pin_operand_order(w, tile_layout),
        "gemm_bruteforce": pin_w4a8_bruteforce(w, awq),
        "on_grid": pin_w4a8_on_grid_equals_w4a16(w, gemm_mod, awq),
        "block_sums": pin_w4a8_block_sums(w),
    }
