"""GPU tied-embedding gather against the oracle.

Bar: bit-exact. Every output value is (q - z) * s, exact before one rounding to
the 16-bit dtype, so the correctly rounded value is unique and both sides must
produce it (rows for ids outside [0, N) are zeros).
"""

import numpy as np
import pytest
import torch

import oracle_pins as pins
import synth
from oracle import embedding as oemb
from gpu_util import DEV, TORCH_DTYPE, device_to_bits, int32_to_device, weights_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w():
    import w4a16_int4_weight_amd as mod
    return mod


def pack_on_gpu(w, ws):
    qw, qz, sc = weights_to_device(ws)
    return w.w4a16_repack(qw, qz, sc, ws.group_size)


def gather(w, ids, packed, K, N, G, dtype):
    out = w.w4a16_embedding(int32_to_device(np.asarray(ids, dtype=np.int32)), packed, K, N, G, TORCH_DTYPE[dtype])
    torch.cuda.synchronize()
    return device_to_bits(out)


def edge_ids(N):
    return np.array([0, N - 1, N - 1, 15, 16, N // 2, -1, N, -(2**31), 2**31 - 1], dtype=np.int64)


def test_lm_head_tied_embedding(w):
    # the tied 131072 x 2048 head: 512 prompt tokens plus edge ids (first and last
    # column, a repeat, column-block edges, ids out of range both ways)
    print("embedding lm_head T=522", flush=True)
    ws = synth.make("lm_head", Ms=())
    packed = pack_on_gpu(w, ws)
    ids = np.concatenate([synth.draw_token_ids(601, 512, ws.N), edge_ids(ws.N)])
    got = gather(w, ids, packed, ws.K, ws.N, ws.group_size, ws.dtype)
    want = oemb.embedding(ids, ws.qweight, ws.qzeros, ws.scale_bits, ws.dtype, ws.group_size)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


def test_worked_example(w):
    ex = pins.worked_example()
    weights, _ = pins.embedding_golden()
    ws = synth.WeightSet(128, 16, 128, "bf16", ex["qweight"], ex["qzeros"], ex["scale_bits"])
    packed = pack_on_gpu(w, ws)
    ids = [r[0] for r in weights]
    got = gather(w, ids, packed, 128, 16, 128, "bf16")
    assert np.array_equal(got, oemb.embedding(ids, ws.qweight, ws.qzeros, ws.scale_bits, "bf16", 128))


def test_rounding_ties_by_hand(w):
    _, rounding = pins.embedding_golden()
    for dtype, sbits, q, z, want in rounding:
        qweight = np.full((128, 2), q * 0x11111111, dtype=np.uint32).view(np.int32)
        qzeros = np.full((1, 2), z * 0x11111111, dtype=np.uint32).view(np.int32)
        scale_bits = np.full((1, 16), sbits, dtype=np.uint16)
        ws = synth.WeightSet(128, 16, 128, dtype, qweight, qzeros, scale_bits)
        got = gather(w, [0, 7, 15], pack_on_gpu(w, ws), 128, 16, 128, dtype)
        assert np.all(got == want), (dtype, hex(sbits), q, z)


@pytest.mark.parametrize("K,N,G,dtype,T", [(256, 16, 128, "fp16", 1), (384, 48, -1, "bf16", 5),
                                           (1024, 272, 256, "bf16", 9), (2048, 2048, 128, "fp16", 64),
                                           (6656, 32, 128, "bf16", 3)])
def test_shapes(w, K, N, G, dtype, T):
    # one row block to 52 (more (row block, lane group) pairs than lanes), per-channel
    # and wide groups, both dtypes, token counts that leave the last workgroup ragged
    print(f"embedding K={K} N={N} G={G} {dtype} T={T}", flush=True)
    ws = synth.make_custom(1100 + K // 128 + N // 16, 1, K, N, dtype, G)
    packed = pack_on_gpu(w, ws)
    ids = np.concatenate([synth.draw_token_ids(1200 + T, T, N), edge_ids(N)])
    got = gather(w, ids, packed, K, N, G, dtype)
    assert np.array_equal(got, oemb.embedding(ids, ws.qweight, ws.qzeros, ws.scale_bits, dtype, G))


def test_writes_only_its_rows_and_zero_tokens(w):
    ws = synth.make_custom(1300, 1, 512, 64, "bf16", 128)
    packed = pack_on_gpu(w, ws)
    ids = int32_to_device(np.array([3, 63, 0, 64, 17], dtype=np.int32))
    pad = 4096
    buf = torch.full((5 * 512 + 2 * pad,), -7.0, dtype=torch.bfloat16, device=DEV)
    out = buf[pad:pad + 5 * 512].view(5, 512)
    w.w4a16_embedding(ids, packed, 512, 64, 128, torch.bfloat16, out=out)
    torch.cuda.synchronize()
    b = buf.cpu()
    assert torch.all(b[:pad] == -7.0) and torch.all(b[-pad:] == -7.0), "write outside out"
    want = oemb.embedding([3, 63, 0, 64, 17], ws.qweight, ws.qzeros, ws.scale_bits, "bf16", 128)
    assert np.array_equal(device_to_bits(out), want)
    empty = w.w4a16_embedding(int32_to_device(np.zeros(0, dtype=np.int32)), packed, 512, 64, 128, torch.bfloat16)
    assert tuple(empty.shape) == (0, 512)


def test_rejects_bad_calls(w):
    ws = synth.make_custom(1400, 1, 256, 32, "bf16", 128)
    packed = pack_on_gpu(w, ws)
    ids = int32_to_device(np.array([1, 2], dtype=np.int32))
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_embedding(ids, packed[:1000], 256, 32, 128, torch.bfloat16)
    assert e.value.status == "W4A16_ERR_BUFFER_SIZE"
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_embedding(ids, packed, 256, 32, 96, torch.bfloat16)
    assert e.value.status == "W4A16_ERR_GROUP"
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_embedding(ids, packed, 256, 32, 128, torch.float32)
    assert e.value.status == "W4A16_ERR_DTYPE"
