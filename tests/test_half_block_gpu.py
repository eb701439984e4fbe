"""N % 16 == 8: a last column block of 8 real columns (N only needs the checkpoint
pack factor 8). The packed buffer pads that block with zero columns; every entry
point must match the oracle on the real columns and write nothing past them."""

import numpy as np
import pytest
import torch

import synth
from oracle import awq, embedding as oemb, gemm as ogemm, gptq, tile_layout
from gpu_util import (DEV, TORCH_DTYPE, bits_to_device, device_to_bits, int32_to_device, oracle_repack,
                      oracle_y, weights_to_device, y_to_f64)

pytestmark = pytest.mark.gpu
TOL = ogemm.TOLERANCE


@pytest.fixture(scope="module")
def w():
    import w4a16_int4_weight_amd as mod
    return mod


def pack_on_gpu(w, ws):
    qw, qz, sc = weights_to_device(ws)
    packed = w.w4a16_repack(qw, qz, sc, ws.group_size)
    torch.cuda.synchronize()
    return packed


@pytest.mark.parametrize("K,N,G,dtype", [(256, 24, 128, "bf16"), (2048, 13288, 128, "bf16"),
                                         (384, 40, -1, "fp16"), (1024, 520, 256, "bf16")])
def test_repack_half_block(w, K, N, G, dtype):
    print(f"repack half block K={K} N={N}", flush=True)
    ws = synth.make_custom(3000 + N % 97, 1, K, N, dtype, G)
    got = pack_on_gpu(w, ws).cpu().numpy()
    assert got.size == tile_layout.packed_bytes(K, N, G)
    assert np.array_equal(got, oracle_repack(ws))


@pytest.mark.parametrize("K,N", [(256, 24), (2048, 13288)])
def test_repack_gptq_half_block(w, K, N):
    gs = synth.draw_gptq_weights(3100 + N % 97, K, N, "bf16", 128)
    got = w.w4a16_repack_gptq(int32_to_device(gs.qweight), int32_to_device(gs.qzeros),
                              bits_to_device(gs.scale_bits, "bf16"), 128).cpu().numpy()
    want = tile_layout.repack(gptq.unpack_gptq_weight(gs.qweight), gptq.unpack_gptq_zeros(gs.qzeros),
                              gs.scale_bits, 128)
    assert np.array_equal(got, want)


def guarded_gemm(w, ws, M, path, bias_bits=None):
    x = bits_to_device(ws.x_bits[M], ws.dtype)
    pad = 4096
    buf = torch.full((M * ws.N + 2 * pad,), -7.0, dtype=TORCH_DTYPE[ws.dtype], device=DEV)
    y = buf[pad:pad + M * ws.N].view(M, ws.N)
    bias = None if bias_bits is None else bits_to_device(bias_bits, ws.dtype)
    w.w4a16_gemm_ex(x, pack_on_gpu(w, ws), ws.N, ws.group_size, bias=bias, y=y, path=path)
    torch.cuda.synchronize()
    b = buf.cpu()
    assert torch.all(b[:pad] == -7.0) and torch.all(b[-pad:] == -7.0), "write outside y"
    return y_to_f64(y, ws.dtype)


@pytest.mark.parametrize("M,N,path,dtype", [(1, 13288, "gemv", "bf16"), (3, 13288, "gemv", "fp16"),
                                            (8, 24, "gemv", "bf16"), (16, 13288, "mfma", "bf16"),
                                            (100, 40, "mfma", "fp16"), (512, 13288, "mfma", "bf16"),
                                            (5, 40, "mfma", "bf16"), (300, 520, "mfma", "bf16")])
def test_gemm_half_block(w, M, N, path, dtype):
    # both paths; the MFMA GEMM with 128 x 256 tiles (M = 512), small tiles and a K
    # split (N = 40, 520), the 16-row tile (M = 16)
    print(f"gemm half block M={M} N={N} {path} {dtype}", flush=True)
    ws = synth.make_custom(3200 + M + N % 97, M, 2048, N, dtype, 128)
    got = guarded_gemm(w, ws, M, path)
    assert ogemm.max_rel_error(got, oracle_y(ws, ws.x_bits[M])) <= TOL


@pytest.mark.parametrize("path", ["gemv", "mfma"])
def test_bias_half_block(w, path):
    ws = synth.make_custom(3300, 4, 512, 40, "bf16", 128)
    rng = np.random.default_rng(3)
    bias_bits = synth.f32_to_half_bits(rng.standard_normal(40, dtype=np.float32), "bf16")
    got = guarded_gemm(w, ws, 4, path, bias_bits)
    assert ogemm.max_rel_error(got, oracle_y(ws, ws.x_bits[4], bias_bits=bias_bits)) <= TOL


def test_embedding_half_block(w):
    ws = synth.make_custom(3400, 1, 2048, 13288, "bf16", 128)
    packed = pack_on_gpu(w, ws)
    ids = np.concatenate([synth.draw_token_ids(3401, 64, 13288), [13287, 13280, 13279, 13288, 13295]])
    out = w.w4a16_embedding(int32_to_device(ids.astype(np.int32)), packed, 2048, 13288, 128, torch.bfloat16)
    torch.cuda.synchronize()
    want = oemb.embedding(ids, ws.qweight, ws.qzeros, ws.scale_bits, "bf16", 128)
    assert np.array_equal(device_to_bits(out), want)
