"""GPU repack of GPTQ-standard tensors against the oracle: bit-exact, and the same
packed buffer as the AWQ repack of the same codes."""

import numpy as np
import pytest
import torch

import synth
from oracle import awq, gemm as ogemm, gptq, tile_layout
from gpu_util import DEV, bits_to_device, int32_to_device, y_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w():
    import w4a16_int4_weight_amd as mod
    return mod


def gptq_on_gpu(w, gs):
    packed = w.w4a16_repack_gptq(int32_to_device(gs.qweight), int32_to_device(gs.qzeros),
                                 bits_to_device(gs.scale_bits, gs.dtype), gs.group_size)
    torch.cuda.synchronize()
    return packed


def oracle_gptq_repack(gs):
    return tile_layout.repack(gptq.unpack_gptq_weight(gs.qweight), gptq.unpack_gptq_zeros(gs.qzeros),
                              gs.scale_bits, gs.group_size)


SHAPES = [(2048, 13312, 128, "bf16"), (6656, 2048, 128, "bf16"), (2048, 3072, 128, "bf16"),
          (512, 512, 128, "fp16"), (128, 16, 128, "bf16"), (384, 272, -1, "fp16"), (1024, 48, 256, "bf16"),
          (8192, 40, 128, "bf16")]


@pytest.mark.parametrize("K,N,G,dtype", SHAPES)
def test_gptq_repack_bit_exact(w, K, N, G, dtype):
    # the layer shapes, one row block and one column block, a ragged column
    # workgroup (272 columns), per-channel and wide groups
    print(f"gptq repack K={K} N={N} G={G} {dtype}", flush=True)
    gs = synth.draw_gptq_weights(2000 + K // 128 + N // 16, K, N, dtype, G)
    got = gptq_on_gpu(w, gs).cpu().numpy()
    assert np.array_equal(got, oracle_gptq_repack(gs))


def test_gptq_lm_head_bit_exact(w):
    print("gptq repack lm_head", flush=True)
    gs = synth.draw_gptq_weights(2100, 2048, 131072, "bf16", 128)
    got = gptq_on_gpu(w, gs).cpu().numpy()
    assert np.array_equal(got, oracle_gptq_repack(gs))


def test_gptq_and_awq_give_the_same_buffer(w):
    # the same codes, zero points and scales, packed both ways on the CPU oracle,
    # repacked on the GPU by both entry points
    gs = synth.draw_gptq_weights(2200, 1024, 528, "bf16", 128)
    Q = gptq.unpack_gptq_weight(gs.qweight)
    Z = gptq.unpack_gptq_zeros(gs.qzeros)
    from_gptq = gptq_on_gpu(w, gs)
    from_awq = w.w4a16_repack(int32_to_device(awq.pack_awq(Q)), int32_to_device(awq.pack_awq(Z)),
                              bits_to_device(gs.scale_bits, "bf16"), 128)
    torch.cuda.synchronize()
    assert torch.equal(from_gptq, from_awq)


def test_gemm_from_gptq_buffer(w):
    gs = synth.draw_gptq_weights(2300, 2048, 1040, "bf16", 128)
    packed = gptq_on_gpu(w, gs)
    rng = np.random.default_rng(5)
    x_bits = synth.f32_to_half_bits(rng.standard_normal((24, 2048), dtype=np.float32), "bf16")
    y = w.w4a16_gemm(bits_to_device(x_bits, "bf16"), packed, 1040, 128)
    torch.cuda.synchronize()
    ref = ogemm.w4a16_reference(x_bits, awq.pack_awq(gptq.unpack_gptq_weight(gs.qweight)),
                                awq.pack_awq(gptq.unpack_gptq_zeros(gs.qzeros)), gs.scale_bits, "bf16", 128)
    assert ogemm.max_rel_error(y_to_f64(y, "bf16"), ref) <= ogemm.TOLERANCE
