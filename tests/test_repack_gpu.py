"""GPU repack against the oracle: the packed buffer must be bit-exact, whole."""

import numpy as np
import pytest
import torch

import synth
from oracle import awq, tile_layout
import oracle_pins
from gpu_util import DEV, weights_to_device, oracle_repack, int32_to_device, bits_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w():
    import w4a16_int4_weight_amd as mod
    return mod


def gpu_repack(w, ws, canary=0):
    qw, qz, sc = weights_to_device(ws)
    nbytes = w.w4a16_packed_bytes(ws.K, ws.N, ws.group_size)
    buf = torch.full((nbytes + 2 * canary,), 0xA5, dtype=torch.uint8, device=DEV)
    packed = buf[canary:canary + nbytes] if canary else buf
    w.w4a16_repack(qw, qz, sc, ws.group_size, packed=packed)
    torch.cuda.synchronize()
    return buf.cpu().numpy()


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_repack_bit_exact_on_workloads(w, name):
    print(f"repack workload {name}", flush=True)
    ws = synth.make(name, Ms=())
    got = gpu_repack(w, ws)
    want = oracle_repack(ws)
    assert got.size == want.size
    mism = np.nonzero(got != want)[0]
    assert mism.size == 0, f"{mism.size} bytes differ, first at {mism[:8]}"


@pytest.mark.parametrize("K,N,G,dtype", [(128, 16, 128, "bf16"), (256, 272, 128, "bf16"), (512, 48, 256, "fp16"),
                                         (384, 4112, -1, "bf16"), (1024, 64, 512, "fp16"), (2048, 2048, 128, "bf16"),
                                         # more row blocks (65) than the tile has columns (24): the
                                         # metadata rows are dealt to the first row blocks only
                                         (8320, 24, 128, "bf16")])
def test_repack_bit_exact_shapes_and_groups(w, K, N, G, dtype):
    print(f"repack K={K} N={N} G={G} {dtype}", flush=True)
    ws = synth.make_custom(1000 + K + N, 1, K, N, dtype, G)
    got = gpu_repack(w, ws, canary=4096)
    want = oracle_repack(ws)
    assert np.all(got[:4096] == 0xA5) and np.all(got[-4096:] == 0xA5), "write outside the packed buffer"
    assert np.array_equal(got[4096:-4096], want)


def test_repack_index_patterns(w):
    K, N, G = 256, 48, 128
    for desc, Q, expect in oracle_pins.layout_index_pattern_cases(K, N):
        qweight = awq.pack_awq(Q)
        qzeros = awq.pack_awq(np.zeros((K // G, N), np.uint8))
        sbits = np.zeros((K // G, N), np.uint16)
        packed = w.w4a16_repack(int32_to_device(qweight), int32_to_device(qzeros), bits_to_device(sbits, "bf16"), G)
        got = packed.cpu().numpy()
        assert np.array_equal(got[:K * N // 2], expect), desc


def test_repack_decodes_to_inputs_and_is_deterministic(w):
    ws = synth.make_custom(77, 1, 1024, 528, "bf16", 128)
    a = gpu_repack(w, ws)
    b = gpu_repack(w, ws)
    assert np.array_equal(a, b)
    Q, Z, S = tile_layout.decode(a, ws.K, ws.N, ws.group_size)
    assert np.array_equal(Q, awq.unpack_awq(ws.qweight))
    assert np.array_equal(Z, awq.unpack_awq(ws.qzeros))
    assert np.array_equal(S, ws.scale_bits)


def test_repack_on_side_stream(w):
    ws = synth.make_custom(78, 1, 512, 512, "fp16", 128)
    qw, qz, sc = weights_to_device(ws)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        packed = w.w4a16_repack(qw, qz, sc, 128, stream=s)
    s.synchronize()
    assert np.array_equal(packed.cpu().numpy(), oracle_repack(ws))


def test_repack_rejects_bad_calls(w):
    ws = synth.make_custom(79, 1, 256, 32, "bf16", 128)
    qw, qz, sc = weights_to_device(ws)
    small = torch.empty(100, dtype=torch.uint8, device=DEV)
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_repack(qw, qz, sc, 128, packed=small)
    assert e.value.status == "W4A16_ERR_BUFFER_SIZE"
    assert torch.all(small == small)  # untouched buffer still readable
    big = torch.empty(w.w4a16_packed_bytes(256, 32, 128) + 1, dtype=torch.uint8, device=DEV)
    with pytest.raises(w.W4A16Error) as e:
        w.w4a16_repack(qw, qz, sc, 128, packed=big[1:])
    assert e.value.status == "W4A16_ERR_ALIGN"
