"""Group sizes 32 and 64 (a scale and zero point per 32 or 64 rows: 4 or 2 metadata
words per 128-row block). Repack bit-exact; GEMV and MFMA GEMM within tolerance of
the oracle; the embedding gather bit-exact."""

import numpy as np
import pytest
import torch

import synth
from oracle import embedding as oemb, gemm as ogemm, gptq, tile_layout
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


@pytest.mark.parametrize("K,N,G,dtype", [(384, 40, 32, "bf16"), (384, 40, 64, "fp16"), (2048, 3072, 32, "bf16"),
                                         (6656, 2048, 64, "bf16")])
def test_repack_small_groups(w, K, N, G, dtype):
    print(f"repack K={K} N={N} G={G}", flush=True)
    ws = synth.make_custom(5000 + G + N % 97, 1, K, N, dtype, G)
    got = pack_on_gpu(w, ws).cpu().numpy()
    assert got.size == tile_layout.packed_bytes(K, N, G)
    assert np.array_equal(got, oracle_repack(ws))


@pytest.mark.parametrize("G", [32, 64])
def test_gptq_and_chunked_repack_small_groups(w, G):
    K, N = 1024, 520
    gs = synth.draw_gptq_weights(5100 + G, K, N, "bf16", G)
    want = tile_layout.repack(gptq.unpack_gptq_weight(gs.qweight), gptq.unpack_gptq_zeros(gs.qzeros),
                              gs.scale_bits, G)
    got = w.w4a16_repack_gptq(int32_to_device(gs.qweight), int32_to_device(gs.qzeros),
                              bits_to_device(gs.scale_bits, "bf16"), G)
    assert np.array_equal(got.cpu().numpy(), want)
    packed = torch.full((want.size,), 0xAB, dtype=torch.uint8, device=DEV)
    for n0 in range(0, N, 64):
        nc = min(64, N - n0)
        w.w4a16_repack_gptq_columns(int32_to_device(np.ascontiguousarray(gs.qweight[:, n0:n0 + nc])),
                                    int32_to_device(np.ascontiguousarray(gs.qzeros[:, n0 // 8:(n0 + nc) // 8])),
                                    bits_to_device(np.ascontiguousarray(gs.scale_bits[:, n0:n0 + nc]), "bf16"),
                                    N, n0, G, packed)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), want)


def guarded(w, ws, M, path, bias_bits=None):
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


@pytest.mark.parametrize("G", [32, 64])
@pytest.mark.parametrize("M,K,N,path,dtype", [(1, 2048, 13312, "gemv", "bf16"), (3, 2048, 3072, "gemv", "fp16"),
                                              (8, 6656, 2048, "gemv", "bf16"), (16, 6656, 2048, "gemv", "bf16"),
                                              (1, 9216, 256, "gemv", "bf16"),
                                              (16, 6656, 2048, "mfma", "bf16"), (100, 2048, 1040, "mfma", "fp16"),
                                              (512, 2048, 3072, "mfma", "bf16"), (40, 384, 40, "mfma", "bf16")])
def test_gemm_small_groups(w, G, M, K, N, path, dtype):
    # GEMV staged (M <= 8) and direct (M = 16, activations not staged), a long K
    # (72 row blocks: several runs per wave); MFMA GEMM with a K split (M = 16,
    # N = 2048), ragged tiles, 128-row tiles and a half last column block (N = 40)
    print(f"gemm G={G} M={M} K={K} N={N} {path} {dtype}", flush=True)
    ws = synth.make_custom(5200 + G + M + K // 128, M, K, N, dtype, G)
    got = guarded(w, ws, M, path)
    assert ogemm.max_rel_error(got, oracle_y(ws, ws.x_bits[M])) <= TOL


@pytest.mark.parametrize("path", ["gemv", "mfma"])
def test_bias_small_groups(w, path):
    ws = synth.make_custom(5300, 4, 512, 48, "bf16", 32)
    rng = np.random.default_rng(9)
    bias_bits = synth.f32_to_half_bits(rng.standard_normal(48, dtype=np.float32), "bf16")
    got = guarded(w, ws, 4, path, bias_bits)
    assert ogemm.max_rel_error(got, oracle_y(ws, ws.x_bits[4], bias_bits=bias_bits)) <= TOL


@pytest.mark.parametrize("G,dtype", [(32, "bf16"), (64, "fp16")])
def test_embedding_small_groups(w, G, dtype):
    ws = synth.make_custom(5400 + G, 1, 2048, 1040, dtype, G)
    packed = pack_on_gpu(w, ws)
    ids = np.concatenate([synth.draw_token_ids(5401, 40, 1040), [0, 1039, 1040, -1]])
    out = w.w4a16_embedding(int32_to_device(ids.astype(np.int32)), packed, 2048, 1040, G, TORCH_DTYPE[dtype])
    torch.cuda.synchronize()
    want = oemb.embedding(ids, ws.qweight, ws.qzeros, ws.scale_bits, dtype, G)
    assert np.array_equal(device_to_bits(out), want)
