"""GPU W4A8 (fp8 E4M3 activations, int4 weights) against the oracle.

Quantisation: codes, row scales and block sums bit-exact (the integer decision is
taken on the same float32 quotient on both sides). Product: max |y_gpu - y_ref| <=
1e-2 * max |y_ref| over each output tensor, y_ref the oracle's float64 W4A8 product of
the same quantised activations; at the LM-head size on sampled column blocks.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import awq, gemm as ogemm, w4a8 as ow4a8
from gpu_util import (DEV, TORCH_DTYPE, bits_to_device, device_to_bits, weights_to_device, whole_output_error,
                      y_to_f64)

pytestmark = pytest.mark.gpu
TOL = ogemm.TOLERANCE


@pytest.fixture(scope="module")
def w():
    import w4a16_int4_weight_amd as mod
    return mod


def quantize_on_gpu(w, x_bits, dtype):
    M, K = x_bits.shape
    act = w.w4a8_quantize(bits_to_device(x_bits, dtype))
    torch.cuda.synchronize()
    codes, scale, sums = w.w4a8_act_parts(act, M, K)
    return act, codes.cpu().numpy(), scale.cpu().numpy(), sums.cpu().numpy()


def oracle_w4a8_y(ws, x_bits, cols=None, bias_bits=None):
    codes, scale = ow4a8.quantize_rows(x_bits, ws.dtype)
    qweight, qzeros, scale_bits = ws.qweight, ws.qzeros, ws.scale_bits
    if cols is not None:
        words = np.unique(cols // 8)
        qweight, qzeros, scale_bits = qweight[:, words], qzeros[:, words], scale_bits[:, cols]
        if bias_bits is not None:
            bias_bits = bias_bits[cols]
    return ow4a8.w4a8_reference(codes, scale, awq.unpack_awq(qweight), awq.unpack_awq(qzeros), scale_bits,
                                ws.dtype, ws.group_size, bias_bits)


@pytest.mark.parametrize("M,K,dtype", [(1, 2048, "bf16"), (5, 384, "fp16"), (512, 2048, "bf16"), (8, 6656, "bf16"),
                                       (300, 128, "fp16"),
                                       # long rows: several 16-byte chunks per thread in both passes
                                       (3, 16384, "bf16"), (2, 10240, "fp16")])
def test_quantize_matches_oracle(w, M, K, dtype):
    print(f"w4a8 quantize M={M} K={K} {dtype}", flush=True)
    rng = np.random.default_rng(600 + M)
    x_bits = synth.draw_activations(rng, M, K, dtype)
    _, codes, scale, sums = quantize_on_gpu(w, x_bits, dtype)
    want_codes, want_scale = ow4a8.quantize_rows(x_bits, dtype)
    assert np.array_equal(scale, want_scale)
    assert np.array_equal(codes, ow4a8.operand_order(want_codes))
    assert np.array_equal(sums, ow4a8.block_sums(want_codes).astype(np.float32))


def test_quantize_every_bf16_value(w):
    # rows holding +448 have scale 1, so each code is the E4M3 rounding of the value itself
    v = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    K = 1024
    per_row = K - 1
    rows = (v.size + per_row - 1) // per_row
    x = np.zeros(rows * per_row, np.float32)
    x[:v.size] = v
    x = np.concatenate([np.full((rows, 1), 448.0, np.float32), x.reshape(rows, per_row)], axis=1)
    x_bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    _, codes, scale, _ = quantize_on_gpu(w, x_bits, "bf16")
    assert np.all(scale == 1.0)
    got = ow4a8.element_order(codes)
    assert np.array_equal(got, ow4a8.e4m3_encode_rne(x.astype(np.float64)))


def test_quantize_zero_and_tiny_rows(w):
    x = np.zeros((4, 256), np.float32)
    x[1, 3] = 1e-30                      # one tiny value: scale tiny, code 448
    x[2] = np.linspace(-1e-3, 1e-3, 256)
    x[3, ::2] = 2.0 ** -16               # values far below the row maximum: subnormal codes
    x[3, 1] = 1.0
    x_bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    _, codes, scale, sums = quantize_on_gpu(w, x_bits, "bf16")
    want_codes, want_scale = ow4a8.quantize_rows(x_bits, "bf16")
    assert scale[0] == 1.0 and np.all(codes[0] == 0)
    assert np.array_equal(scale, want_scale)
    assert np.array_equal(codes, ow4a8.operand_order(want_codes))
    assert np.array_equal(sums, ow4a8.block_sums(want_codes).astype(np.float32))


def guarded_w4a8(w, ws, M, bias_bits=None):
    x = bits_to_device(ws.x_bits[M], ws.dtype)
    qw, qz, sc = weights_to_device(ws)
    packed = w.w4a16_repack(qw, qz, sc, ws.group_size)
    pad = 4096
    buf = torch.full((M * ws.N + 2 * pad,), -7.0, dtype=TORCH_DTYPE[ws.dtype], device=DEV)
    y = buf[pad:pad + M * ws.N].view(M, ws.N)
    bias = None if bias_bits is None else bits_to_device(bias_bits, ws.dtype)
    w.w4a8_linear(x, packed, ws.N, ws.group_size, bias=bias, y=y)
    torch.cuda.synchronize()
    b = buf.cpu()
    assert torch.all(b[:pad] == -7.0) and torch.all(b[-pad:] == -7.0), "write outside y"
    return y_to_f64(y, ws.dtype)


W4A8_CASES = [
    # decode-sized rows (16-row tiles, K split over workgroups), prefill tiles of 64 and
    # 128 rows, ragged M, a half last column block, per-channel and 256-row groups
    (1, 2048, 13312, 128, "bf16"), (8, 6656, 2048, 128, "bf16"), (16, 2048, 3072, 128, "fp16"),
    (40, 384, 40, 128, "bf16"), (100, 2048, 1040, -1, "fp16"), (300, 512, 520, 256, "bf16"),
    (512, 2048, 3072, 128, "bf16"), (512, 2048, 13312, 128, "bf16"), (129, 1024, 13288, 128, "bf16"),
    (33, 6656, 2048, 128, "bf16"),
    # 64 x 128 tiles as 8 waves of one column block: ragged M, a half last column block
    (480, 512, 3080, 128, "fp16"),
    # 256 x 256 tiles (outputs of at least two rounds of them): ragged M, a half last
    # column block, fp16 with one group per column
    (257, 256, 65544, 128, "bf16"), (512, 384, 65536, -1, "fp16"),
    # the zero-point operands staged in the ring (8 to 16 k blocks per workgroup): 16
    # blocks per K split of 4, ragged M, a half last column block
    (120, 8192, 2056, 128, "fp16"),
    # staged, with the term on the bf16 matrix cores (128 x 256 tiles, 16 fragments per
    # wave) from fp16 scales: ragged M, a half last column block
    (400, 2048, 10248, 128, "fp16"),
]


@pytest.mark.parametrize("M,K,N,G,dtype", W4A8_CASES)
def test_w4a8_gemm_matches_oracle(w, M, K, N, G, dtype):
    print(f"w4a8 gemm M={M} K={K} N={N} G={G} {dtype}", flush=True)
    ws = synth.make_custom(700 + M + N % 97, M, K, N, dtype, G)
    got = guarded_w4a8(w, ws, M)
    err = ogemm.max_rel_error(got, oracle_w4a8_y(ws, ws.x_bits[M]))
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= TOL


@pytest.mark.parametrize("M,K,N,dtype", [
    (24, 512, 48, "bf16"),
    (130, 2048, 8200, "fp16"),     # zero-point operands and row scales staged in the ring
])
def test_w4a8_bias(w, M, K, N, dtype):
    print(f"w4a8 bias M={M} K={K} N={N} {dtype}", flush=True)
    ws = synth.make_custom(750 + M, M, K, N, dtype, 128)
    rng = np.random.default_rng(7)
    bias_bits = synth.f32_to_half_bits(rng.standard_normal(N, dtype=np.float32), dtype)
    got = guarded_w4a8(w, ws, M, bias_bits)
    err = ogemm.max_rel_error(got, oracle_w4a8_y(ws, ws.x_bits[M], bias_bits=bias_bits))
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= TOL


def test_w4a8_lm_head_whole_output(w):
    # the LM-head prefill at full size (M = 512, K = 2048, N = 131072), every output
    # checked (the oracle in column chunks, the activations quantised once)
    print("w4a8 lm_head M=512", flush=True)
    ws = synth.make("lm_head", Ms=(512,))
    M = 512
    x = bits_to_device(ws.x_bits[M], ws.dtype)
    qw, qz, sc = weights_to_device(ws)
    packed = w.w4a16_repack(qw, qz, sc, ws.group_size)
    y = w.w4a8_linear(x, packed, ws.N, ws.group_size)
    torch.cuda.synchronize()
    got = y_to_f64(y, ws.dtype)
    codes, scale = ow4a8.quantize_rows(ws.x_bits[M], ws.dtype)

    def ref(cols):
        words = np.unique(cols // 8)
        return ow4a8.w4a8_reference(codes, scale, awq.unpack_awq(ws.qweight[:, words]),
                                    awq.unpack_awq(ws.qzeros[:, words]), ws.scale_bits[:, cols], ws.dtype,
                                    ws.group_size)

    err, _ = whole_output_error(got, ref)
    print(f"  max rel err over all {M} x {ws.N} outputs {err:.3e}", flush=True)
    assert err <= TOL


def test_w4a8_deterministic(w):
    ws = synth.make_custom(760, 16, 6656, 2048, "bf16", 128)     # K split over workgroups
    x = bits_to_device(ws.x_bits[16], "bf16")
    qw, qz, sc = weights_to_device(ws)
    packed = w.w4a16_repack(qw, qz, sc, 128)
    y0 = w.w4a8_linear(x, packed, ws.N, 128)
    y1 = w.w4a8_linear(x, packed, ws.N, 128)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_w4a8_rejects_small_groups(w):
    ws = synth.make_custom(770, 4, 256, 32, "bf16", 64)
    qw, qz, sc = weights_to_device(ws)
    packed = w.w4a16_repack(qw, qz, sc, 64)
    x = bits_to_device(ws.x_bits[4], "bf16")
    with pytest.raises(w.W4A16Error):
        w.w4a8_linear(x, packed, ws.N, 64)


def test_w4a8_empty_batch(w):
    # M = 0: quantisation and product launch nothing and return empty results
    ws = synth.make_custom(770, 2, 512, 48, "bf16", 128)
    qw, qz, sc = weights_to_device(ws)
    packed = w.w4a16_repack(qw, qz, sc, ws.group_size)
    x0 = torch.empty((0, 512), dtype=torch.bfloat16, device=DEV)
    act = w.w4a8_quantize(x0)
    y = w.w4a8_gemm(act, packed, 0, 512, 48, 128)
    assert tuple(y.shape) == (0, 48)
    y2 = w.w4a8_linear(x0, packed, 48, 128)
    torch.cuda.synchronize()
    assert tuple(y2.shape) == (0, 48)
