"""The CPU oracle against facts fixed independently of it (host only).

Every pin is also run against copies of the oracle with one planted mistake, and
each planted mistake must trip at least one pin.
"""

import importlib
import os
import types

import numpy as np
import pytest

from oracle import awq, embedding, gemm, gptq, numerics, tile_layout
import oracle_pins as pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


# ---------------------------------------------------------------- AWQ packing

def test_awq_golden_words():
    assert pins.pin_awq_golden(awq)


def test_awq_sign_word_minus_one_is_all_fifteen():
    assert awq.unpack_awq(np.array([[-1]], dtype=np.int32)).tolist() == [[15] * 8]


def test_awq_roundtrip_random():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, (37, 64), dtype=np.uint8)
    assert np.array_equal(awq.unpack_awq(awq.pack_awq(codes)), codes)
    words = rng.integers(0, 2**32, (13, 24), dtype=np.uint32).view(np.int32)
    assert np.array_equal(awq.pack_awq(awq.unpack_awq(words)), words)


def test_awq_each_slot_moves_one_column():
    # a word with one nonzero nibble unpacks to exactly one nonzero column, and the
    # eight slots reach eight different columns (the packing is a bijection of slots)
    seen = set()
    for s in range(8):
        for v in range(1, 16):
            word = np.array([[v << (4 * s)]], dtype=np.uint32).view(np.int32)
            codes = awq.unpack_awq(word)[0]
            nz = np.nonzero(codes)[0]
            assert len(nz) == 1 and codes[nz[0]] == v
            seen.add(int(nz[0]))
    assert seen == set(range(8))


def test_awq_rejects_bad_input():
    with pytest.raises(ValueError):
        awq.pack_awq(np.zeros((2, 7), dtype=np.uint8))
    with pytest.raises(ValueError):
        awq.pack_awq(np.full((1, 8), 16))


def test_unpacked_sizes_match_printed_int32_transients():
    assert pins.pin_page3_transients(awq)


# ---------------------------------------------------------------- numerics

def test_bf16_decoding_known_values():
    bits = np.array([0x3F80, 0xBF80, 0x4300, 0x0000, 0x8000, 0x3C00, 0x7F7F], dtype=np.uint16)
    vals = numerics.half_bits_to_f64(bits, "bf16")
    assert vals[:6].tolist() == [1.0, -1.0, 128.0, 0.0, -0.0, 2.0 ** -7]
    assert vals[6] == (2 - 2 ** -7) * 2.0 ** 127


def test_fp16_decoding_known_values():
    bits = np.array([0x3C00, 0xC000, 0x6400, 0x0001, 0x7BFF], dtype=np.uint16)
    assert numerics.half_bits_to_f64(bits, "fp16").tolist() == [1.0, -2.0, 1024.0, 2.0 ** -24, 65504.0]


def test_rne_rounding_ties_and_neighbours():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1 + 2^-7: ties to the even mantissa (1.0)
    r = numerics.f64_to_half_bits_rne([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -30, -3.0], "bf16")
    assert r.tolist() == [0x3F80, 0x3F82, 0x3F81, 0xC040]
    r = numerics.f64_to_half_bits_rne([1 + 2 ** -11, 1 + 3 * 2 ** -11], "fp16")
    assert r.tolist() == [0x3C00, 0x3C02]


# ---------------------------------------------------------------- GEMM

def test_worked_example():
    assert pins.pin_worked_example(gemm)


def test_fraction_bruteforce():
    assert pins.pin_fraction_bruteforce(gemm)


def test_closed_form_constant_codes():
    assert pins.pin_closed_form_constant_codes(gemm, awq)


def test_integer_special_case():
    assert pins.pin_integer_special_case(gemm, awq)


def test_zero_point_cancels():
    assert pins.pin_zero_point_cancels(gemm, awq)


def test_group_index():
    assert pins.pin_group_index(gemm, awq)


def test_linearity_in_activations():
    rng = np.random.default_rng(2)
    M, K, N = 3, 256, 32
    Q = rng.integers(0, 16, (K, N), dtype=np.uint8)
    Z = rng.integers(0, 16, (2, N), dtype=np.uint8)
    S = rng.uniform(0.005, 0.02, (2, N))
    W = gemm.dequant(Q, Z, S, 128)
    x1, x2 = rng.standard_normal((M, K)), rng.standard_normal((M, K))
    assert np.allclose(gemm.gemm(x1 + x2, W), gemm.gemm(x1, W) + gemm.gemm(x2, W), rtol=1e-12, atol=1e-12)


def test_group_size_minus_one_is_per_channel():
    rng = np.random.default_rng(4)
    K, N = 256, 16
    Q = rng.integers(0, 16, (K, N), dtype=np.uint8)
    Z = rng.integers(0, 16, (1, N), dtype=np.uint8)
    S = rng.uniform(0.005, 0.02, (1, N))
    assert np.array_equal(gemm.dequant(Q, Z, S, -1), gemm.dequant(Q, Z, S, K))
    with pytest.raises(ValueError):
        gemm.dequant(Q, Z, S, 100)


def test_tolerance_measure():
    ref = np.array([[1.0, -4.0], [2.0, 0.5]])
    assert gemm.max_rel_error(ref, ref) == 0.0
    assert gemm.max_rel_error(ref + 0.04, ref) == pytest.approx(0.01)
    assert gemm.within_tolerance(ref + 0.039, ref)
    assert not gemm.within_tolerance(ref + 0.041, ref)


# ---------------------------------------------------------------- tile layout

def test_layout_array_form_equals_loop_form():
    rng = np.random.default_rng(6)
    for K, N, G in [(128, 16, 128), (256, 48, 128), (512, 32, 256), (256, 16, -1)]:
        Gr = K if G == -1 else G
        Q = rng.integers(0, 16, (K, N), dtype=np.uint8)
        Z = rng.integers(0, 16, (K // Gr, N), dtype=np.uint8)
        S = rng.integers(0, 2**16, (K // Gr, N), dtype=np.uint16)
        assert np.array_equal(tile_layout.repack(Q, Z, S, G), tile_layout.repack_loops(Q, Z, S, G))


def test_layout_index_patterns():
    assert pins.pin_layout_index_patterns(tile_layout)


def test_layout_metadata_pattern():
    assert pins.pin_layout_metadata(tile_layout)


def test_layout_decode_roundtrip():
    rng = np.random.default_rng(8)
    K, N, G = 384, 64, 128
    Q = rng.integers(0, 16, (K, N), dtype=np.uint8)
    Z = rng.integers(0, 16, (K // G, N), dtype=np.uint8)
    S = rng.integers(0, 2**16, (K // G, N), dtype=np.uint16)
    q, z, s = tile_layout.decode(tile_layout.repack(Q, Z, S, G), K, N, G)
    assert np.array_equal(q, Q) and np.array_equal(z, Z) and np.array_equal(s, S)


def test_layout_column_chunks_are_independent():
    # repacking column ranges of whole 16-column blocks separately gives exactly the
    # bytes of those ranges in both planes, including a ragged last chunk
    rng = np.random.default_rng(10)
    K, N, G = 256, 112, 128
    Q = rng.integers(0, 16, (K, N), dtype=np.uint8)
    Z = rng.integers(0, 16, (K // G, N), dtype=np.uint8)
    S = rng.integers(0, 2**16, (K // G, N), dtype=np.uint16)
    whole = tile_layout.repack(Q, Z, S, G)
    wb = K * N // 2
    w_parts, m_parts = [], []
    for n0, n1 in [(0, 48), (48, 96), (96, 112)]:
        part = tile_layout.repack(Q[:, n0:n1], Z[:, n0:n1], S[:, n0:n1], G)
        pw = K * (n1 - n0) // 2
        w_parts.append(part[:pw])
        m_parts.append(part[pw:])
    assert np.array_equal(np.concatenate(w_parts), whole[:wb])
    assert np.array_equal(np.concatenate(m_parts), whole[wb:])


def test_layout_sizes_and_rejections():
    assert tile_layout.packed_bytes(2048, 13312, 128) == 2048 * 13312 // 2 + 4 * 16 * 13312
    assert tile_layout.packed_bytes(6656, 2048, 128) == 6656 * 2048 // 2 + 4 * 52 * 2048
    assert tile_layout.packed_bytes(384, 16, 128) == 384 * 16 // 2 + 4 * 4 * 16      # 3 row blocks padded to 4
    assert tile_layout.packed_bytes(256, 24, 128) == 256 * 32 // 2 + 4 * 4 * 32      # half block padded to 16
    assert tile_layout.packed_bytes(384, 16, 64) == 384 * 16 // 2 + 4 * 8 * 16       # 6 units of 64 rows -> 8
    assert tile_layout.packed_bytes(384, 16, 32) == 384 * 16 // 2 + 4 * 12 * 16      # 12 units of 32 rows
    for K, N, G in [(100, 16, 128), (256, 20, 128), (256, 16, 96), (256, 16, 16), (384, 16, 256)]:
        with pytest.raises(ValueError):
            tile_layout.packed_bytes(K, N, G)


def test_layout_decode_rejects_reserved_bits():
    K, N, G = 128, 16, 128
    buf = tile_layout.repack(np.zeros((K, N), np.uint8), np.zeros((1, N), np.uint8),
                             np.zeros((1, N), np.uint16), G).copy()
    buf[K * N // 2 + 3] = 0x10
    with pytest.raises(ValueError):
        tile_layout.decode(buf, K, N, G)
    buf = tile_layout.repack(np.zeros((K, N), np.uint8), np.zeros((1, N), np.uint8),
                             np.zeros((1, N), np.uint16), G).copy()
    buf[K * N // 2 + 4] = 1            # padding word kb = 1 of column 0 (KB = 1, KBP = 4)
    with pytest.raises(ValueError):
        tile_layout.decode(buf, K, N, G)


# ---------------------------------------------------------------- planted mistakes

def _mutant(modname, old, new):
    """A copy of oracle/<modname>.py with `old` replaced by `new`. A target string
    that is no longer in the source fails the test outright (pytest.fail is not an
    AssertionError, so no caller's except clause can count it as a caught mistake)."""
    path = os.path.join(ORACLE_DIR, modname + ".py")
    with open(path) as f:
        src = f.read()
    if old not in src or old == new:
        pytest.fail(f"planted mistake is stale: {old!r} is not in oracle/{modname}.py")
    mod = types.ModuleType(f"oracle.{modname}_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), path, "exec"), mod.__dict__)
    return mod


AWQ_MUTANTS = [
    ("other reading of the interleave", "AWQ_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)", "AWQ_ORDER = (0, 4, 1, 5, 2, 6, 3, 7)"),
    ("plain order", "AWQ_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)", "AWQ_ORDER = (0, 1, 2, 3, 4, 5, 6, 7)"),
    ("nibbles read from the top", "codes[:, :, AWQ_ORDER[s]] = ((w >> np.uint32(4 * s))",
     "codes[:, :, AWQ_ORDER[s]] = ((w >> np.uint32(28 - 4 * s))"),
]


@pytest.mark.parametrize("desc,old,new", AWQ_MUTANTS, ids=[m[0] for m in AWQ_MUTANTS])
def test_planted_awq_mistakes_are_caught(desc, old, new):
    mut = _mutant("awq", old, new)
    assert not pins.pin_awq_golden(mut)


GEMM_MUTANTS = [
    ("sign of zero point", "(Q.astype(np.float64) - Z[group_of_row].astype(np.float64))",
     "(Z[group_of_row].astype(np.float64) - Q.astype(np.float64))"),
    ("zero point dropped", "(Q.astype(np.float64) - Z[group_of_row].astype(np.float64))",
     "(Q.astype(np.float64) - 0 * Z[group_of_row].astype(np.float64))"),
    ("groups interleaved instead of contiguous", "group_of_row = np.arange(K) // G",
     "group_of_row = np.arange(K) % (K // G)"),
    ("scale of the next group", "* S[group_of_row]", "* S[(group_of_row + 1) % (K // G)]"),
    ("scale not applied", "* S[group_of_row]", "* 1.0"),
    ("activation row reversed", "return X @ W", "return X[:, ::-1] @ W"),
    ("bias-free product scaled", "return X @ W", "return 2.0 * (X @ W)"),
]


@pytest.mark.parametrize("desc,old,new", GEMM_MUTANTS, ids=[m[0] for m in GEMM_MUTANTS])
def test_planted_gemm_mistakes_are_caught(desc, old, new):
    mut = _mutant("gemm", old, new)
    results = pins.run_gemm_pins(mut, awq)
    assert not all(results.values()), results


def test_planted_numerics_mistake_is_caught():
    mut_num = _mutant("numerics", "(bits.astype(np.uint32) << 16)", "(bits.astype(np.uint32) << 15)")
    mut_gemm = types.ModuleType("oracle.gemm_mutant")
    mut_gemm.__dict__.update(gemm.__dict__)
    mut_gemm.half_bits_to_f64 = mut_num.half_bits_to_f64
    # w4a16_reference looks half_bits_to_f64 up in its own globals; rebuild it there
    src = open(os.path.join(ORACLE_DIR, "gemm.py")).read()
    mod = types.ModuleType("oracle.gemm_mutant2")
    mod.__package__ = "oracle"
    exec(compile(src, "gemm.py", "exec"), mod.__dict__)
    mod.half_bits_to_f64 = mut_num.half_bits_to_f64
    assert not pins.pin_worked_example(mod)


LAYOUT_MUTANTS = [
    ("slot order identity", "TILE_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)", "TILE_ORDER = (0, 1, 2, 3, 4, 5, 6, 7)"),
    ("word index and lane group swapped", "codes = codes.transpose(3, 0, 2, 4, 1)           # [nb, kb, h, c, i]",
     "codes = codes.transpose(3, 0, 1, 4, 2)"),
    ("lane = 4c + h instead of 16h + c", "codes = codes.transpose(3, 0, 2, 4, 1)           # [nb, kb, h, c, i]",
     "codes = codes.transpose(3, 0, 4, 2, 1)"),
    ("blocks kb-major", "words = np.zeros((NB, KB, 4, 16, 4), dtype=np.uint32)   # [nb, kb, h, c, i]",
     "words = np.zeros((KB, NB, 4, 16, 4), dtype=np.uint32)"),
    ("metadata zero in bits 12..15", "(s_u | (z_u << np.uint32(16))).T", "(s_u | (z_u << np.uint32(12))).T"),
    ("metadata row-block-major", "meta[:, :U] = (s_u | (z_u << np.uint32(16))).T",
     "meta[:, :U] = (s_u | (z_u << np.uint32(16))).reshape(N, U)"),
    ("metadata unpadded", "meta = np.zeros((N, padded_units(K, G)), dtype=np.uint32)          # [n, b], padding 0",
     "meta = np.zeros((N, U), dtype=np.uint32)"),
]


@pytest.mark.parametrize("desc,old,new", LAYOUT_MUTANTS, ids=[m[0] for m in LAYOUT_MUTANTS])
def test_planted_layout_mistakes_are_caught(desc, old, new):
    mut = _mutant("tile_layout", old, new)
    try:
        ok = pins.pin_layout_index_patterns(mut) and pins.pin_layout_metadata(mut)
    except (ValueError, AssertionError):
        ok = False    # a mutant that breaks the layout's own size check is caught too
    assert not ok


# ---------------------------------------------------------------- tied embedding

def test_embedding_worked_example():
    assert pins.pin_embedding_worked_example(embedding)


def test_embedding_rounding_by_hand():
    assert pins.pin_embedding_rounding(embedding)


def test_embedding_is_the_identity_product():
    assert pins.pin_embedding_matches_gemm(embedding, gemm)


def test_embedding_empty_and_all_out_of_range():
    ex = pins.worked_example()
    assert embedding.embedding(np.array([], dtype=np.int64), ex["qweight"], ex["qzeros"], ex["scale_bits"],
                               "bf16", 128).shape == (0, 128)
    e = embedding.embedding(np.array([16, -1, 1 << 40]), ex["qweight"], ex["qzeros"], ex["scale_bits"],
                            "bf16", 128)
    assert e.shape == (3, 128) and not e.any()


EMBEDDING_MUTANTS = [
    ("neighbouring column", "where = np.searchsorted(words, ids[valid] // 8) * 8 + ids[valid] % 8",
     "where = np.searchsorted(words, ids[valid] // 8) * 8 + (ids[valid] + 1) % 8"),
    ("negative ids wrap around", "valid = (ids >= 0) & (ids < N)", "valid = (ids >= -N) & (ids < N)"),
    ("truncation instead of rounding",
     "return f64_to_half_bits_rne(embedding_f64(ids, qweight, qzeros, scale_bits, dtype, group_size), dtype)",
     "return (embedding_f64(ids, qweight, qzeros, scale_bits, dtype, group_size).astype(np.float32)"
     ".view(np.uint32) >> 16).astype(np.uint16) if dtype == 'bf16' else "
     "f64_to_half_bits_rne(embedding_f64(ids, qweight, qzeros, scale_bits, dtype, group_size), dtype)"),
    ("row of W instead of column", "E[valid] = W[:, where].T", "E[valid] = W[where % W.shape[0], :K]"),
]


@pytest.mark.parametrize("desc,old,new", EMBEDDING_MUTANTS, ids=[m[0] for m in EMBEDDING_MUTANTS])
def test_planted_embedding_mistakes_are_caught(desc, old, new):
    mut = _mutant("embedding", old, new)
    try:
        results = pins.run_embedding_pins(mut, gemm)
        ok = all(results.values())
    except (ValueError, IndexError):
        ok = False    # a mutant that breaks the gather's shapes is caught too
    assert not ok


# ---------------------------------------------------------------- GPTQ-standard packing

def test_gptq_golden_words():
    assert pins.pin_gptq_golden(gptq)


def test_gptq_roundtrips():
    assert pins.pin_gptq_roundtrips(gptq)


def test_gptq_row_moves_one_nibble():
    assert pins.pin_gptq_row_moves_one_nibble(gptq)


def test_gptq_and_awq_repack_to_the_same_layout():
    # the tile layout is a function of the codes alone: the same codes, zero points
    # and scales reach the same packed buffer through either checkpoint format
    rng = np.random.default_rng(3)
    K, N, G = 256, 48, 128
    Q = rng.integers(0, 16, (K, N), dtype=np.uint8)
    Z = rng.integers(0, 16, (K // G, N), dtype=np.uint8)
    S = rng.integers(0, 2**16, (K // G, N), dtype=np.uint16)
    via_gptq = tile_layout.repack(gptq.unpack_gptq_weight(gptq.pack_gptq_weight(Q)),
                                  gptq.unpack_gptq_zeros(gptq.pack_gptq_zeros(Z)), S, G)
    via_awq = tile_layout.repack(awq.unpack_awq(awq.pack_awq(Q)), awq.unpack_awq(awq.pack_awq(Z)), S, G)
    assert np.array_equal(via_gptq, via_awq)


def test_gptq_rejects_bad_input():
    with pytest.raises(ValueError):
        gptq.pack_gptq_weight(np.zeros((12, 8), dtype=np.uint8))     # K not a multiple of 8
    with pytest.raises(ValueError):
        gptq.pack_gptq_zeros(np.zeros((1, 12), dtype=np.uint8))      # N not a multiple of 8
    with pytest.raises(ValueError):
        gptq.pack_gptq_weight(np.full((8, 8), 16, dtype=np.uint8))


GPTQ_MUTANTS = [
    ("weight nibbles from the top", "words |= grouped[:, j, :] << np.uint32(4 * j)",
     "words |= grouped[:, j, :] << np.uint32(28 - 4 * j)"),
    ("weight unpacked from the top", "codes[:, j, :] = ((w >> np.uint32(4 * j))",
     "codes[:, j, :] = ((w >> np.uint32(28 - 4 * j))"),
    ("zeros in AWQ's interleaved order", "words |= grouped[:, :, j] << np.uint32(4 * j)",
     "words |= grouped[:, :, (0, 2, 4, 6, 1, 3, 5, 7)[j]] << np.uint32(4 * j)"),
    ("zero point stored with a +1 offset", "codes[:, :, j] = ((w >> np.uint32(4 * j)) & np.uint32(0xF)).astype(np.uint8)",
     "codes[:, :, j] = (((w >> np.uint32(4 * j)) & np.uint32(0xF)) + 1).astype(np.uint8)"),
    ("rows of a word strided by K/8", "grouped = codes.astype(np.uint32).reshape(K // 8, 8, N)",
     "grouped = codes.astype(np.uint32).reshape(8, K // 8, N).transpose(1, 0, 2)"),
]


@pytest.mark.parametrize("desc,old,new", GPTQ_MUTANTS, ids=[m[0] for m in GPTQ_MUTANTS])
def test_planted_gptq_mistakes_are_caught(desc, old, new):
    mut = _mutant("gptq", old, new)
    assert not all(pins.run_gptq_pins(mut).values())


# ---------------------------------------------------------------- N % 16 == 8

def test_layout_half_block_padding():
    assert pins.pin_layout_half_block(tile_layout)


def test_layout_half_block_decode_roundtrip():
    rng = np.random.default_rng(12)
    K, N, G = 384, 40, 128
    Q = rng.integers(0, 16, (K, N), dtype=np.uint8)
    Z = rng.integers(0, 16, (K // G, N), dtype=np.uint8)
    S = rng.integers(0, 2**16, (K // G, N), dtype=np.uint16)
    out = tile_layout.repack(Q, Z, S, G)
    assert np.array_equal(out, tile_layout.repack_loops(Q, Z, S, G))
    Q2, Z2, S2 = tile_layout.decode(out, K, N, G)
    assert np.array_equal(Q2, Q) and np.array_equal(Z2, Z) and np.array_equal(S2, S)
    bad = out.copy()
    bad[(K * 48 // 2) + 4 * 4 * 47] = 1          # metadata word of padding column 47
    with pytest.raises(ValueError):
        tile_layout.decode(bad, K, N, G)


HALF_BLOCK_MUTANTS = [
    ("padding repeats the last column", "Q, Z, scale_bits = np.pad(Q, pad), np.pad(Z, pad), np.pad(scale_bits, pad)",
     "Q, Z, scale_bits = np.pad(Q, pad, mode='edge'), np.pad(Z, pad), np.pad(scale_bits, pad)"),
    ("padding metadata repeats the last column",
     "Q, Z, scale_bits = np.pad(Q, pad), np.pad(Z, pad), np.pad(scale_bits, pad)",
     "Q, Z, scale_bits = np.pad(Q, pad), np.pad(Z, pad), np.pad(scale_bits, pad, mode='edge')"),
    ("metadata plane placed after K*N/2 (padding codes moved to the end, same size)",
     "reshape(-1),\n        np.ascontiguousarray(meta).astype(\"<u4\").view(np.uint8).reshape(-1),\n    ])",
     "reshape(-1)[:K * N_real // 2],\n        np.ascontiguousarray(meta).astype(\"<u4\").view(np.uint8).reshape(-1),\n"
     "        np.zeros(K * (N - N_real) // 2, dtype=np.uint8),\n    ])"),
    ("metadata rows only for the real columns",
     "meta = np.zeros((N, padded_units(K, G)), dtype=np.uint32)          # [n, b], padding 0",
     "meta = np.zeros((N_real, padded_units(K, G)), dtype=np.uint32)"),
]


@pytest.mark.parametrize("desc,old,new", HALF_BLOCK_MUTANTS, ids=[m[0] for m in HALF_BLOCK_MUTANTS])
def test_planted_half_block_mistakes_are_caught(desc, old, new):
    mut = _mutant("tile_layout", old, new)
    try:
        ok = pins.pin_layout_half_block(mut)
    except (ValueError, AssertionError, IndexError):
        ok = False
    assert not ok


# ---------------------------------------------------------------- group sizes 32 and 64

@pytest.mark.parametrize("G", [32, 64])
def test_layout_small_group_metadata(G):
    assert pins.pin_layout_small_groups(tile_layout, G)


@pytest.mark.parametrize("G", [32, 64])
def test_layout_small_group_roundtrip(G):
    rng = np.random.default_rng(G)
    K, N = 384, 40
    Q = rng.integers(0, 16, (K, N), dtype=np.uint8)
    Z = rng.integers(0, 16, (K // G, N), dtype=np.uint8)
    S = rng.integers(0, 2**16, (K // G, N), dtype=np.uint16)
    out = tile_layout.repack(Q, Z, S, G)
    assert np.array_equal(out, tile_layout.repack_loops(Q, Z, S, G))
    Q2, Z2, S2 = tile_layout.decode(out, K, N, G)
    assert np.array_equal(Q2, Q) and np.array_equal(Z2, Z) and np.array_equal(S2, S)


SMALL_GROUP_MUTANTS = [
    ("one word per row block", "    return min(G, ROWS_PER_BLOCK)", "    return ROWS_PER_BLOCK"),
    ("unit groups from 128-row blocks", "group_of_unit = (np.arange(U) * Gu) // G",
     "group_of_unit = (np.arange(U) * ROWS_PER_BLOCK) // G % (K // G)"),
    ("units unpadded", "    return (U + 3) // 4 * 4", "    return U"),
]


@pytest.mark.parametrize("desc,old,new", SMALL_GROUP_MUTANTS, ids=[m[0] for m in SMALL_GROUP_MUTANTS])
def test_planted_small_group_mistakes_are_caught(desc, old, new):
    mut = _mutant("tile_layout", old, new)
    try:
        ok = pins.pin_layout_small_groups(mut, 32) and pins.pin_layout_small_groups(mut, 64)
    except (ValueError, AssertionError, IndexError):
        ok = False
    assert not ok
