"""The path on a weight past 4 GiB of packed codes (K = 65536, N = 135176, bf16, G = 128).

Byte offsets into the packed buffer then pass 2^32 in the codes (column blocks from
8192 on start at 8192 x 512 KiB = 4 GiB) as well as in the metadata plane after them,
so the repack, the GEMV (M = 1), the MFMA GEMM (M = 48), the W4A8 GEMM (M = 48, 512 k
blocks: 32 batches of the zero-point term) and the gather all run their address
arithmetic past 32 bits. The products are checked against the oracle on column blocks
on both sides of the 4 GiB line and the last block (a half block, N % 16 == 8); the
gather bit-exactly, on ids in the same blocks.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import awq, embedding as oemb, gemm as ogemm, w4a8 as ow4a8
from gpu_util import DEV, TORCH_DTYPE, bits_to_device, device_to_bits, int32_to_device, oracle_y, weights_to_device, \
    y_to_f64

pytestmark = pytest.mark.gpu
TOL = ogemm.TOLERANCE
K, N, G, M = 65536, 135176, 128, 48
# first block, blocks just below and at the 4 GiB line, beyond it, the last (half) block
BLOCKS = [0, 4095, 8191, 8192, 8193, 8320, 8447, 8448]


@pytest.fixture(scope="module")
def w():
    import w4a16_int4_weight_amd as mod
    return mod


@pytest.fixture(scope="module")
def big(w):
    print(f"large weight K={K} N={N}: drawing and repacking", flush=True)
    ws = synth.make_custom(1900, M, K, N, "bf16", G)
    qw, qz, sc = weights_to_device(ws)
    packed = w.w4a16_repack(qw, qz, sc, G)
    torch.cuda.synchronize()
    del qw, qz, sc
    torch.cuda.empty_cache()
    assert packed.numel() == w.w4a16_packed_bytes(K, N, G) and packed.numel() > 2**32
    return ws, packed


def sampled_cols():
    cols = np.concatenate([np.arange(16 * b, min(16 * b + 16, N)) for b in BLOCKS])
    assert cols[-1] == N - 1
    return cols


def check(got, ref):
    err = ogemm.max_rel_error(got, ref)
    print(f"  max rel err {err:.3e}", flush=True)
    assert err <= TOL


def test_large_gemv_m1(w, big):
    ws, packed = big
    print("large GEMV M=1", flush=True)
    x = bits_to_device(ws.x_bits[M][:1], ws.dtype)
    y = w.w4a16_gemm(x, packed, N, G)
    torch.cuda.synchronize()
    cols = sampled_cols()
    check(y_to_f64(y, ws.dtype)[:, cols], oracle_y(ws, ws.x_bits[M][:1], cols))


def test_large_mfma_gemm(w, big):
    ws, packed = big
    print(f"large MFMA GEMM M={M}", flush=True)
    x = bits_to_device(ws.x_bits[M], ws.dtype)
    y = w.w4a16_gemm_ex(x, packed, N, G, path="mfma")
    torch.cuda.synchronize()
    cols = sampled_cols()
    check(y_to_f64(y, ws.dtype)[:, cols], oracle_y(ws, ws.x_bits[M], cols))


def test_large_w4a8_gemm(w, big):
    ws, packed = big
    print(f"large W4A8 GEMM M={M}", flush=True)
    x = bits_to_device(ws.x_bits[M], ws.dtype)
    y = w.w4a8_linear(x, packed, N, G)
    torch.cuda.synchronize()
    cols = sampled_cols()
    words = np.unique(cols // 8)
    codes, scale = ow4a8.quantize_rows(ws.x_bits[M], ws.dtype)
    ref = ow4a8.w4a8_reference(codes, scale, awq.unpack_awq(ws.qweight[:, words]), awq.unpack_awq(ws.qzeros[:, words]),
                               ws.scale_bits[:, cols], ws.dtype, G)
    check(y_to_f64(y, ws.dtype)[:, cols], ref)


def test_large_gather(w, big):
    ws, packed = big
    print("large gather", flush=True)
    ids = np.array([0, 16 * 8192 - 1, 16 * 8192, 16 * 8320 + 5, N - 8, N - 1], dtype=np.int64)
    out = w.w4a16_embedding(int32_to_device(ids.astype(np.int32)), packed, K, N, G, TORCH_DTYPE[ws.dtype])
    torch.cuda.synchronize()
    got = device_to_bits(out)
    want = oemb.embedding(ids, ws.qweight, ws.qzeros, ws.scale_bits, ws.dtype, G)
    assert got.shape == want.shape
    assert np.array_equal(got, want)
