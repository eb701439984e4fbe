"""Load path on the GPU: column-chunked repack (AWQ and GPTQ input) gives the bytes
of the whole-matrix repack and touches only its columns; the host-chunked loader and
a saved-then-loaded buffer give the same bytes and the same GEMM results."""

import numpy as np
import pytest
import torch

import synth
from oracle import gptq, tile_layout
from gpu_util import DEV, bits_to_device, int32_to_device, oracle_repack, weights_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w():
    import w4a16_int4_weight_amd as mod
    return mod


def chunks(N, step):
    return [(n0, min(step, N - n0)) for n0 in range(0, N, step)]


@pytest.mark.parametrize("K,N,step", [(2048, 131072, 4096), (2048, 13288, 1024), (6656, 2048, 48), (384, 40, 16)])
def test_awq_chunks_equal_whole(w, K, N, step):
    # LM head in 32 chunks; a last chunk ending in a half block; chunks of 3 blocks
    print(f"awq chunks K={K} N={N} step={step}", flush=True)
    ws = synth.make_custom(4000 + N % 97, 1, K, N, "bf16", 128)
    want = torch.from_numpy(oracle_repack(ws))
    packed = torch.full((tile_layout.packed_bytes(K, N, 128),), 0xAB, dtype=torch.uint8, device=DEV)
    for n0, nc in chunks(N, step):
        qw = int32_to_device(np.ascontiguousarray(ws.qweight[:, n0 // 8:(n0 + nc) // 8]))
        qz = int32_to_device(np.ascontiguousarray(ws.qzeros[:, n0 // 8:(n0 + nc) // 8]))
        sc = bits_to_device(np.ascontiguousarray(ws.scale_bits[:, n0:n0 + nc]), "bf16")
        w.w4a16_repack_columns(qw, qz, sc, N, n0, 128, packed)
    torch.cuda.synchronize()
    assert torch.equal(packed.cpu(), want)


@pytest.mark.parametrize("K,N,step", [(2048, 13288, 2048), (1024, 520, 64)])
def test_gptq_chunks_equal_whole(w, K, N, step):
    gs = synth.draw_gptq_weights(4100 + N % 97, K, N, "bf16", 128)
    want = tile_layout.repack(gptq.unpack_gptq_weight(gs.qweight), gptq.unpack_gptq_zeros(gs.qzeros),
                              gs.scale_bits, 128)
    packed = torch.full((want.size,), 0xAB, dtype=torch.uint8, device=DEV)
    for n0, nc in chunks(N, step):
        qw = int32_to_device(np.ascontiguousarray(gs.qweight[:, n0:n0 + nc]))
        qz = int32_to_device(np.ascontiguousarray(gs.qzeros[:, n0 // 8:(n0 + nc) // 8]))
        sc = bits_to_device(np.ascontiguousarray(gs.scale_bits[:, n0:n0 + nc]), "bf16")
        w.w4a16_repack_gptq_columns(qw, qz, sc, N, n0, 128, packed)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), want)


def test_chunk_touches_only_its_columns(w):
    K, N, G = 512, 96, 128
    ws = synth.make_custom(4200, 1, K, N, "fp16", G)
    whole = oracle_repack(ws)
    n0, nc = 32, 48
    packed = torch.full((whole.size,), 0xAB, dtype=torch.uint8, device=DEV)
    qw = int32_to_device(np.ascontiguousarray(ws.qweight[:, n0 // 8:(n0 + nc) // 8]))
    qz = int32_to_device(np.ascontiguousarray(ws.qzeros[:, n0 // 8:(n0 + nc) // 8]))
    sc = bits_to_device(np.ascontiguousarray(ws.scale_bits[:, n0:n0 + nc]), "fp16")
    w.w4a16_repack_columns(qw, qz, sc, N, n0, G, packed)
    torch.cuda.synchronize()
    got = packed.cpu().numpy()
    KB, KBP = K // 128, 4
    mine = np.zeros(whole.size, dtype=bool)
    for nb in range(n0 // 16, (n0 + nc) // 16):            # weight blocks of the chunk
        mine[nb * KB * 1024:(nb + 1) * KB * 1024] = True
    meta0 = K * N // 2
    mine[meta0 + 4 * KBP * n0:meta0 + 4 * KBP * (n0 + nc)] = True
    assert np.array_equal(got[mine], whole[mine])
    assert np.all(got[~mine] == 0xAB)


@pytest.mark.parametrize("fmt", ["awq", "gptq"])
def test_repack_from_host(w, fmt):
    K, N = 2048, 13288
    if fmt == "awq":
        ws = synth.make_custom(4300, 1, K, N, "bf16", 128)
        qw, qz = torch.from_numpy(ws.qweight), torch.from_numpy(ws.qzeros)
        want = oracle_repack(ws)
    else:
        ws = synth.draw_gptq_weights(4301, K, N, "bf16", 128)
        qw, qz = torch.from_numpy(ws.qweight), torch.from_numpy(ws.qzeros)
        want = tile_layout.repack(gptq.unpack_gptq_weight(ws.qweight), gptq.unpack_gptq_zeros(ws.qzeros),
                                  ws.scale_bits, 128)
    sc = torch.from_numpy(ws.scale_bits.view(np.int16)).view(torch.bfloat16)
    packed = w.repack_from_host(qw, qz, sc, 128, fmt=fmt, chunk_columns=3072, device=DEV)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), want)


def test_saved_buffer_loads_and_runs(w, tmp_path):
    ws = synth.make_custom(4400, 8, 2048, 3072, "bf16", 128)
    qw, qz, sc = weights_to_device(ws)
    packed = w.w4a16_repack(qw, qz, sc, 128)
    path = str(tmp_path / "qkv.w4a16")
    w.save_packed(path, packed, 2048, 3072, 128, torch.bfloat16)
    loaded, K, N, G, dtype = w.load_packed(path, device=DEV)
    assert (K, N, G, dtype) == (2048, 3072, 128, torch.bfloat16)
    assert torch.equal(loaded, packed[:loaded.numel()])
    x = bits_to_device(ws.x_bits[8], "bf16")
    y0 = w.w4a16_gemm(x, packed, 3072, 128)
    y1 = w.w4a16_gemm(x, loaded, 3072, 128)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
