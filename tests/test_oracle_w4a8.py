"""Pins of the W4A8 oracle (fp8 E4M3 activations, int4 weights) against the E4M3
format, torch's independent fp8 conversions, exhaustive nearest-even search, the
pinned weight tile layout and exact rational arithmetic; planted mistakes in the
oracle must trip at least one pin."""

import os
import types

import numpy as np
import pytest

import oracle_pins as pins
from oracle import awq, gemm, tile_layout, w4a8

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def test_e4m3_spec_values():
    assert pins.pin_e4m3_spec(w4a8)


def test_e4m3_agrees_with_torch():
    assert pins.pin_e4m3_against_torch(w4a8)


def test_e4m3_nearest_even_bruteforce():
    assert pins.pin_e4m3_bruteforce(w4a8)


def test_nibble_reads_as_code_over_512():
    assert pins.pin_nibble_reading(w4a8)


def test_quantize_rows():
    assert pins.pin_quantize_rows(w4a8)


def test_operand_order_pairs_with_tile_layout():
    assert pins.pin_operand_order(w4a8, tile_layout)


def test_w4a8_bruteforce():
    assert pins.pin_w4a8_bruteforce(w4a8, awq)


def test_w4a8_on_grid_equals_w4a16():
    assert pins.pin_w4a8_on_grid_equals_w4a16(w4a8, gemm, awq)


def test_block_sums():
    assert pins.pin_w4a8_block_sums(w4a8)


def test_encode_rejects_out_of_range():
    for v in (464.0, -500.0, np.nan, np.inf):
        with pytest.raises(ValueError):
            w4a8.e4m3_encode_rne(np.array([v]))


def test_quantisation_error_is_bounded():
    # |dec(e) * a - x| <= a * 2^-4 * 2^floor(log2 |x / a|) for normal codes, a * 2^-10 below
    rng = np.random.default_rng(12)
    x = rng.standard_normal((4, 1024)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    codes, scale = w4a8.quantize_rows(bits, "bf16")
    xb = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q = xb / scale[:, None]
    err = np.abs(w4a8.e4m3_decode(codes) - q)
    bound = np.where(np.abs(q) >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(q), 1e-300))) - 4), 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-6))


def _mutant(old, new):
    path = os.path.join(ORACLE_DIR, "w4a8.py")
    src = open(path).read()
    if old not in src or old == new:
        pytest.fail(f"planted mistake is stale: {old!r} is not in oracle/w4a8.py")
    mod = types.ModuleType("oracle.w4a8_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new, 1), path, "exec"), mod.__dict__)
    return mod


W4A8_MUTANTS = [
    ("subnormals truncated", "sub_code = np.rint(a * 512.0)", "sub_code = np.floor(a * 512.0)"),
    ("mantissa truncated", "mant = np.rint((2.0 * frac - 1.0) * 8.0)", "mant = np.floor((2.0 * frac - 1.0) * 8.0)"),
    ("exponent bias 8", "np.exp2(e - 10.0)", "np.exp2(e - 11.0)"),
    ("largest value of the fnuz variant", "E4M3_MAX = 448.0", "E4M3_MAX = 240.0"),
    ("scale multiplied, not divided", "(X / scale[:, None])", "(X * scale[:, None])"),
    ("subnormal threshold", "code = np.where(a < 2.0 ** -6", "code = np.where(a < 2.0 ** -7"),
    ("operand order: step and lane group swapped", "src.transpose(0, 1, 3, 2, 4)).reshape(M, K)   # [m, kb, h, i, j]",
     "src).reshape(M, K)"),
    ("operand order: bytes in row order", "ROW_OF_BYTE = (0, 4, 1, 5, 2, 6, 3, 7)", "ROW_OF_BYTE = (0, 1, 2, 3, 4, 5, 6, 7)"),
    ("row scale dropped", "np.asarray(scale, dtype=np.float64)[:, None] * (A @ W)", "(A @ W)"),
    ("block sums over the wrong axis", ".sum(axis=2)", ".sum(axis=1)"),
]


@pytest.mark.parametrize("desc,old,new", W4A8_MUTANTS, ids=[m[0] for m in W4A8_MUTANTS])
def test_planted_w4a8_mistakes_are_caught(desc, old, new):
    mut = _mutant(old, new)
    results = {}
    for name, fn in [("spec", lambda: pins.pin_e4m3_spec(mut)), ("bruteforce", lambda: pins.pin_e4m3_bruteforce(mut)),
                     ("quantize", lambda: pins.pin_quantize_rows(mut)),
                     ("operand_order", lambda: pins.pin_operand_order(mut, tile_layout)),
                     ("gemm", lambda: pins.pin_w4a8_bruteforce(mut, awq)),
                     ("on_grid", lambda: pins.pin_w4a8_on_grid_equals_w4a16(mut, gemm, awq)),
                     ("block_sums", lambda: pins.pin_w4a8_block_sums(mut))]:
        try:
            results[name] = fn()
        except (ValueError, IndexError, AssertionError):
            results[name] = False
    assert not all(results.values()), results
