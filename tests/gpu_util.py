"""Helpers shared by the GPU tests: move seeded inputs to the device, read results
back as 16-bit bit patterns, compute oracle references."""

from concurrent.futures import ThreadPoolExecutor

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


def whole_output_error(got, ref_cols, chunk=8192, workers=8):
    """max |got - ref| / max |ref| over the whole [M, N] output, the reference computed
    in column chunks of `chunk` (a multiple of 16) by ref_cols(cols) -> float64
    [M, len(cols)], `workers` chunks at a time (NumPy releases the interpreter lock in
    its array work). Returns (error, max |ref|): the same measure as
    oracle.gemm.max_rel_error on the whole tensor, with one max over all chunks."""
    N = got.shape[1]
    assert chunk % 16 == 0

    def one(n0):
        cols = np.arange(n0, min(n0 + chunk, N))
        ref = ref_cols(cols)
        return float(np.max(np.abs(got[:, cols] - ref))), float(np.max(np.abs(ref)))

    with ThreadPoolExecutor(max_workers=workers) as pool:
        parts = list(pool.map(one, range(0, N, chunk)))
    num = max(p[0] for p in parts)
    den = max(p[1] for p in parts)
    if den == 0.0:
        return (0.0 if num == 0.0 else np.inf), den
    return num / den, den
