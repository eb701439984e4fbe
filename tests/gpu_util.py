"""Helpers shared by the GPU tests: move seeded inputs to the device, read results
back as 16-bit bit patterns, compute oracle references."""

import numpy as np
import torch

from oracle import awq, gemm as ogemm, numerics, tile_layout

TORCH_DTYPE = {"fp16": torch.float16, "bf16": torch.bfloat16}
DEV = "cuda:0"


def bits_to_device(bits, dtype, device=DEV):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(TORCH_DTYPE[dtype]).to(device)


def int32_to_device(a, device=DEV):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(device)


def device_to_bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def weights_to_device(ws, device=DEV):
    return (int32_to_device(ws.qweight, device), int32_to_device(ws.qzeros, device),
            bits_to_device(ws.scale_bits, ws.dtype, device))


def oracle_repack(ws):
    Q = awq.unpack_awq(ws.qweight)
    Z = awq.unpack_awq(ws.qzeros)
    return tile_layout.repack(Q, Z, ws.scale_bits, ws.group_size)


def oracle_y(ws, x_bits, cols=None, bias_bits=None):
    """float64 reference; `cols` (a sorted array of whole 16-column blocks' column
    indices) restricts it to a subset of output columns."""
    qweight, qzeros, scale_bits = ws.qweight, ws.qzeros, ws.scale_bits
    if cols is not None:
        words = np.unique(cols // 8)
        assert np.array_equal(np.repeat(words, 8) * 8 + np.tile(np.arange(8), len(words)), cols)
        qweight, qzeros, scale_bits = qweight[:, words], qzeros[:, words], scale_bits[:, cols]
        if bias_bits is not None:
            bias_bits = bias_bits[cols]
    return ogemm.w4a16_reference(x_bits, qweight, qzeros, scale_bits, ws.dtype, ws.group_size, bias_bits)


def y_to_f64(y, dtype):
    return numerics.half_bits_to_f64(device_to_bits(y), dtype)


def sample_column_blocks(N, count, seed):
    rng = np.random.default_rng(seed)
    nb = N // 16
    pick = np.unique(np.concatenate([rng.choice(nb, size=min(count, nb), replace=False), [0, nb - 1]]))
    return (pick[:, None] * 16 + np.arange(16)[None, :]).reshape(-1)
